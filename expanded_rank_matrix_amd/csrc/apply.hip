// Inference from the packed factors: Y = (B diag(D) C X^T)^T for a batch of vectors x.
//
// The factorisation stays free of multiplications at inference: ternary additions and
// subtractions plus one scale per component (ExTernD review, Significance); the factors are
// read in the 2-bit mask+sign format (pith.science report, the storage assumption of Eq. 5).
//   s_i = D_i sum_j C_ij x_j   (one wave per component, the lanes over the packed words of row i)
//   y_r = sum_i B_ri s_i       (a thread per packed word of B's rows, i.e. 16 outputs, over a chunk
//                               of components, with s in 62-bit fixed point: exact integer sums,
//                               combined across chunks by integer atomics)
// t_i is an fp64 sum in a fixed order; y is exact for the fixed-point s (one unit is
// 2^(E + ceil(log2(k + 1)) - 62) for max |s| < 2^E, below 2^-46 of it) and rounded once to fp32.
// Both are deterministic.
#include <mutex>

#include "common.hpp"
#include "externd_internal.hpp"

namespace externd {

// the 2-bit code at bit offset off of word: 0, 1 or 3 (= -1) -> 0, 1, -1
__device__ __forceinline__ int tcode_at(unsigned word, int off) { return __builtin_amdgcn_sbfe(word, off, 2); }


constexpr int kSWords = 64;    // words over which max |s| is spread (one per lane) ...
constexpr int kSStride = 32;   // ... each on its own 128-byte line

__global__ void infer_zero_kernel(unsigned* smax) { smax[threadIdx.x * kSStride] = 0u; }

// the high 32 bits of |v| (sign cleared): monotonic in |v|, so their maximum bounds max |v|
__device__ __forceinline__ unsigned hi_abs(double v) {
  return (unsigned)((u64)__double_as_longlong(v) >> 32) & 0x7FFFFFFFu;
}

// acc + c x for the 2-bit codes c of one packed word and x[0..15] (zero past n): adds and
// subtracts only
__device__ __forceinline__ double tacc16(double acc, unsigned word, const float (&xv)[16]) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int c = tcode_at(word, 2 * t);
    const double xd = (double)xv[t];
    acc = c == 0 ? acc : (c > 0 ? acc + xd : acc - xd);
  }
  return acc;
}

// s_bi = D_i sum_j C_ij x_bj: wave v of workgroup g takes component 4 g + v, its lanes the packed
// words of that row (x read as float4 when rows of X are 16-byte aligned).  Also zeroes Yacc and
// records max |s| (one atomic per workgroup).
__global__ void __launch_bounds__(256) infer_c_kernel(const uint32_t* C, int wn, int n, const float* D, int k,
                                                      const float* X, int batch, int x_vec4, double* S,
                                                      unsigned* smax, long long* Yacc, long long nY) {
  __shared__ unsigned wmx[4];
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < nY; x += (long long)gridDim.x * 256) Yacc[x] = 0;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wid;
  unsigned mx = 0u;
  if (i < k) {  // uniform within the wave
    const uint32_t* row = C + (size_t)i * wn;
    for (int b = 0; b < batch; ++b) {
      const float* x = X + (size_t)b * n;
      double acc = 0.0;
      for (int w = lane; w < wn; w += 64) {
        const unsigned word = row[w];
        if (word == 0u) continue;
        const int j0 = w * 16;
        float xv[16];
        if (x_vec4 && j0 + 16 <= n) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(x + j0 + 4 * q);
            xv[4 * q] = v.x;
            xv[4 * q + 1] = v.y;
            xv[4 * q + 2] = v.z;
            xv[4 * q + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int t = 0; t < 16; ++t) xv[t] = j0 + t < n ? x[j0 + t] : 0.0f;
        }
        acc = tacc16(acc, word, xv);
      }
      acc = wave_sum_f64(acc);
      const double si = (double)D[i] * acc;
      if (lane == 0) S[(size_t)b * k + i] = si;
      const unsigned hb = hi_abs(si);
      mx = hb > mx ? hb : mx;
    }
  }
  if (lane == 0) wmx[wid] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned v = wmx[0] > wmx[1] ? wmx[0] : wmx[1];
    v = wmx[2] > v ? wmx[2] : v;
    v = wmx[3] > v ? wmx[3] : v;
    if (v != 0u) atomicMax(smax + (blockIdx.x % kSWords) * kSStride, v);
  }
}

// Fixed-point scale of y's sums: one unit is 2^-f, f = 62 - E - ceil(log2(k + 1)) with
// max |s| < 2^E, so a sum of k terms stays below 2^62 in magnitude.
__device__ __forceinline__ int infer_scale(const unsigned* smax, int k) {
  const unsigned hb = wave_max_u32(smax[(threadIdx.x & 63) * kSStride]);
  if (hb == 0u) return 0;
  const double bound = __longlong_as_double((long long)(((u64)hb << 32) | 0xFFFFFFFFull));  // >= max |s|
  int E;
  frexp(bound, &E);
  const int lk = 32 - __clz((unsigned)k);
  return 62 - E - lk;
}

// Yacc[b][r] += sum over the components of this workgroup's chunk of B_ri S_bi, with
// S_bi = rint(s_bi 2^f) as int64: exact, so the integer atomics of the chunks give the same sum in
// any order.  Thread (wave v, lane l): packed word 64 blockIdx.x + l, components
// c0 + v kc .. c0 + (v + 1) kc - 1; the four waves add in LDS before one atomic per output.
__global__ void __launch_bounds__(256) infer_b_kernel(const uint32_t* B, int wm, int m, int k, const double* S,
                                                      int batch, int kc, const unsigned* smax, long long* Yacc) {
  __shared__ long long red[4][64][17];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int w = blockIdx.x * 64 + lane;
  const int b = blockIdx.z;
  const int f = infer_scale(smax, k);
  const int c0 = blockIdx.y * 4 * kc + wid * kc;
  const int c1 = c0 + kc < k ? c0 + kc : k;
  long long acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0;
  const double* s = S + (size_t)b * k;
  if (w < wm) {
    for (int i = c0; i < c1; ++i) {
      const unsigned word = B[(size_t)i * wm + w];
      if (word == 0u) continue;
      const long long si = llrint(ldexp(s[i], f));
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int c = tcode_at(word, 2 * t);
        acc[t] = c == 0 ? acc[t] : (c > 0 ? acc[t] + si : acc[t] - si);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) red[wid][lane][t] = acc[t];
  __syncthreads();
  for (int x = tid; x < 64 * 16; x += 256) {
    const int wl = x >> 4, t = x & 15;
    const int r = (blockIdx.x * 64 + wl) * 16 + t;
    if (r < m) {
      const long long v = red[0][wl][t] + red[1][wl][t] + red[2][wl][t] + red[3][wl][t];
      if (v != 0) atomicAdd(reinterpret_cast<unsigned long long*>(Yacc + (size_t)b * m + r), (unsigned long long)v);
    }
  }
}

// Y = fp32(Yacc 2^-f)
__global__ void __launch_bounds__(256) infer_fin_kernel(const long long* Yacc, long long count, int k,
                                                        const unsigned* smax, float* Y) {
  const int f = infer_scale(smax, k);
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < count; x += (long long)gridDim.x * 256)
    Y[x] = (float)ldexp((double)Yacc[x], -f);
}

int infer_kc(int k, int m) {
  // components per wave: about 512 workgroups of the B pass for one vector, at least 8
  const int xb = (m + 1023) / 1024;
  int per = (k + 511 * xb) / (512 * xb);  // components per workgroup / 4 rounded
  per = (per + 3) / 4;
  return per < 8 ? 8 : per;
}

size_t infer_workspace_bytes(int k, int m, int batch) {
  return (((size_t)batch * k * 8 + 255) & ~(size_t)255) + (((size_t)batch * m * 8 + 255) & ~(size_t)255) +
         4 * kSWords * kSStride;
}

hipError_t infer_run(const uint32_t* B, const uint32_t* C, const float* D, int k, int m, int n, const float* X,
                     int batch, float* Y, void* ws, hipStream_t st) {
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  char* base = static_cast<char*>(ws);
  double* S = reinterpret_cast<double*>(base);
  const size_t oS = ((size_t)batch * k * 8 + 255) & ~(size_t)255;
  long long* Yacc = reinterpret_cast<long long*>(base + oS);
  unsigned* smax = reinterpret_cast<unsigned*>(base + oS + (((size_t)batch * m * 8 + 255) & ~(size_t)255));
  hipLaunchKernelGGL(infer_zero_kernel, dim3(1), dim3(64), 0, st, smax);
  const long long nY = (long long)batch * m;
  const int x_vec4 = (n % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 15u) == 0) ? 1 : 0;
  hipLaunchKernelGGL(infer_c_kernel, dim3((k + 3) / 4), dim3(256), 0, st, C, wn, n, D, k, X, batch, x_vec4, S, smax,
                     Yacc, nY);
  const int kc = infer_kc(k, m);
  const int nch = (k + 4 * kc - 1) / (4 * kc);
  hipLaunchKernelGGL(infer_b_kernel, dim3((wm + 63) / 64, nch, batch), dim3(256), 0, st, B, wm, m, k, S, batch, kc,
                     smax, Yacc);
  const long long nb = (nY + 255) / 256;
  hipLaunchKernelGGL(infer_fin_kernel, dim3((unsigned)(nb < 4096 ? nb : 4096)), dim3(256), 0, st, Yacc, nY, k, smax,
                     Y);
  return hipGetLastError();
}

// ---- allocation-free inference: the workspace in a file-scope device array -------------------
// One array per GPU, held until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a host-side stand-in); it passes the device address that
// hipGetSymbolAddress returns, fetched once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kInferStaticBytes];

hipError_t infer_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace externd
