// Inference from the packed factors: Y = (B diag(D) C X^T)^T for a batch of vectors x.
//
// The factorisation stays free of multiplications at inference: ternary additions and
// subtractions plus one scale per component (ExTernD review, Significance); the factors are
// read in the 2-bit mask+sign format (pith.science report, the storage assumption of Eq. 5).
//   s_i = D_i sum_j C_ij x_j   (one wave per component, the lanes over the packed words of row i)
//   y_r = sum_i B_ri s_i       (a thread per packed word of B's rows, i.e. 16 outputs, over a chunk
//                               of components; the chunks' partial sums are then added in chunk
//                               order)
// Every sum is fp64 in a fixed order (deterministic); y is rounded once to fp32.
#include "common.hpp"
#include "externd_internal.hpp"

namespace externd {

// the 2-bit code at bit offset off of word: 0, 1 or 3 (= -1) -> 0, 1, -1
__device__ __forceinline__ int tcode_at(unsigned word, int off) { return __builtin_amdgcn_sbfe(word, off, 2); }

// ternary accumulate: acc + c x for c in {-1, 0, 1}, as an add, a subtract or nothing
__device__ __forceinline__ double tacc(double acc, int c, double x) { return c == 0 ? acc : (c > 0 ? acc + x : acc - x); }

__global__ void __launch_bounds__(256) infer_c_kernel(const uint32_t* C, int wn, int n, const float* D, int k,
                                                      const float* X, int batch, double* S) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= k) return;  // uniform within the wave; the kernel has no barriers
  const uint32_t* row = C + (size_t)i * wn;
  for (int b = 0; b < batch; ++b) {
    const float* x = X + (size_t)b * n;
    double acc = 0.0;
    for (int w = lane; w < wn; w += 64) {
      const unsigned word = row[w];
      if (word == 0u) continue;
      const int j0 = w * 16;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int c = tcode_at(word, 2 * t);
        if (c != 0 && j0 + t < n) acc = tacc(acc, c, (double)x[j0 + t]);
      }
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) S[(size_t)b * k + i] = (double)D[i] * acc;
  }
}

// part[chunk][b][r] = sum over components i of the chunk of B_ri s_bi (thread = one packed word)
__global__ void __launch_bounds__(256) infer_b_kernel(const uint32_t* B, int wm, int m, int k, const double* S,
                                                      int batch, int kchunk, double* part) {
  const int w = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.z;
  const int c0 = blockIdx.y * kchunk, c1 = c0 + kchunk < k ? c0 + kchunk : k;
  if (w >= wm) return;  // no barriers in the kernel
  double acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0.0;
  const double* s = S + (size_t)b * k;
  for (int i = c0; i < c1; ++i) {
    const unsigned word = B[(size_t)i * wm + w];
    if (word == 0u) continue;
    const double si = s[i];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = tacc(acc[t], tcode_at(word, 2 * t), si);
  }
  double* out = part + ((size_t)blockIdx.y * batch + b) * m;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int r = w * 16 + t;
    if (r < m) out[r] = acc[t];
  }
}

// Y[x] = fp32(sum over chunks, in chunk order, of part[chunk][x]), x over batch x m
__global__ void __launch_bounds__(256) infer_reduce_kernel(const double* part, int nchunk, long long count, float* Y) {
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < count; x += (long long)gridDim.x * 256) {
    double acc = 0.0;
    for (int c = 0; c < nchunk; ++c) acc += part[(size_t)c * count + x];
    Y[x] = (float)acc;
  }
}

int infer_chunks(int k, int m) {
  // about 512 workgroups of the B pass for one vector, chunks of at least 16 components
  const int xb = (m / 16 + 1 + 255) / 256;
  int nch = (512 + xb - 1) / xb;
  const int maxc = (k + 15) / 16;
  nch = nch > maxc ? maxc : nch;
  return nch < 1 ? 1 : nch;
}

size_t infer_workspace_bytes(int k, int m, int batch) {
  const size_t s = (size_t)batch * k * 8, p = (size_t)infer_chunks(k, m) * batch * m * 8;
  return ((s + 255) & ~(size_t)255) + p;
}

hipError_t infer_run(const uint32_t* B, const uint32_t* C, const float* D, int k, int m, int n, const float* X,
                     int batch, float* Y, void* ws, hipStream_t st) {
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  double* S = static_cast<double*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + (((size_t)batch * k * 8 + 255) & ~(size_t)255));
  const int nch = infer_chunks(k, m);
  const int kchunk = (k + nch - 1) / nch;
  const int nchunk = (k + kchunk - 1) / kchunk;
  hipLaunchKernelGGL(infer_c_kernel, dim3((k + 3) / 4), dim3(256), 0, st, C, wn, n, D, k, X, batch, S);
  hipLaunchKernelGGL(infer_b_kernel, dim3((wm + 255) / 256, nchunk, batch), dim3(256), 0, st, B, wm, m, k, S, batch,
                     kchunk, part);
  const long long count = (long long)batch * m;
  const long long nb = (count + 255) / 256;
  hipLaunchKernelGGL(infer_reduce_kernel, dim3((unsigned)(nb < 4096 ? nb : 4096)), dim3(256), 0, st, part, nchunk,
                     count, Y);
  return hipGetLastError();
}

}  // namespace externd
