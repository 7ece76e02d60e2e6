// Inference from the packed factors: Y = (B diag(D) C X^T)^T for a batch of vectors x.
//
// At inference the factorisation needs only ternary additions and subtractions plus one scale per
// component (ExTernD review, Significance); the factors are read in the 2-bit mask+sign format
// (pith.science report, the storage assumption of Eq. 5):
//   t_i = sum_j C_ij x_j,   s_i = D_i t_i,   y_r = sum_i B_ri s_i.
// Both sums run on v_mfma_i32_16x16x64_i8 over exact integer images.  x enters as
// X_j = rint(x_j 2^e), one power-of-two scale per vector chosen from max |x| so that |X_j| <= 2^50
// and n |X_j| <= 2^62, split into seven signed 8-bit digits; the ternary codes are exact int8.
// The products of codes and digits are additions and subtractions of the digits, summed exactly in
// int32 and recombined exactly in int64, so t_i 2^e is the exact sum over the image of x.  Then
// s_i = D_i t_i in fp64, and s enters the second sum the same way: S_i = rint(s_i 2^f) with
// |S_i| <= 2^50 and k |S_i| <= 2^62; y_r 2^f = sum_i B_ri S_i is exact, its chunk sums added with
// 64-bit integer atomics (exact, so in any order), and y_r is rounded once to fp32.  Each image is
// within 2^-50 of the vector's max |x| (|s|) per element, and the result does not depend on the
// launch shape.
//
// Two launches: the t pass (infer_t_kernel: 32 components x two vectors per workgroup; also clears
// the y accumulator and stores each workgroup's max |s|) and the y pass (infer_y_kernel: 256 outputs
// x 512 components x two vectors per workgroup; the last workgroup of each output group rounds it).
#include <mutex>

#include "common.hpp"
#include "externd_internal.hpp"

namespace externd {

typedef int iv4 __attribute__((ext_vector_type(4)));

constexpr int kIDig = 7;   // signed 8-bit digits of a fixed-point image (|N| <= 2^50)
constexpr int kIBits = 50; // largest magnitude exponent of an image (the rounding below is exact to 2^51)
// bits of 1.5 2^52 minus the digit bias 0x0080808080808080 (128 in bytes 0..6)
constexpr unsigned long long kIMagic = 0x42B77F7F7F7F7F80ull;
constexpr int kTComp = 32;          // components per workgroup of the t pass (two tiles of 16)
constexpr int kTKh = 4;             // waves of the t pass that split the columns of one tile
constexpr int kTThreads = 128 * kTKh;
constexpr int kTWords = 192;        // packed words of x per chunk of digit operands in LDS (3072 columns)
constexpr int kYWords = 16;         // packed words of B (256 outputs) per workgroup of the y pass
constexpr int kYWpw = 2;            // words per wave of the y pass
constexpr int kYThreads = 64 * kYWords / kYWpw;
constexpr int kYComp = 512;         // components per workgroup of the y pass
constexpr int kYPitch = kYComp + 4; // LDS pitch (words) of the staged B words: rows 16 bytes apart in banks

// bits P of an image that is summed over len terms: len 2^P <= 2^62, at most kIBits
__device__ __forceinline__ int inf_bits(int len) {
  const int L = 32 - __clz((unsigned)len);
  return 62 - L < kIBits ? 62 - L : kIBits;
}

// E with |v| < 2^E for the fp32 bit pattern hb of |v| > 0 (normal or subnormal)
__device__ __forceinline__ int f32_bound_exp(unsigned hb) {
  const int ex = (int)(hb >> 23);
  return ex == 0 ? -126 : ex - 126;
}

// E with |v| < 2^E for the high word hb of the fp64 bit pattern of |v| > 0
__device__ __forceinline__ int f64_bound_exp(unsigned hb) {
  const int ex = (int)(hb >> 20);
  return ex == 0 ? -1022 : ex - 1022;
}

// the high 32 bits of |v| (sign cleared): monotonic in |v|
__device__ __forceinline__ unsigned hi_abs(double v) {
  return (unsigned)((u64)__double_as_longlong(v) >> 32) & 0x7FFFFFFFu;
}

// N + 0x0080808080808080 for N = rint(v 2^e), |v 2^e| < 2^51: v 2^e is exact (a power-of-two
// scale), and adding 1.5 2^52 rounds it to the nearest integer (ties to even, as rint) in the low
// mantissa bits, so the bit pattern minus the constant's is N.
__device__ __forceinline__ unsigned long long fx_biased(double v, int e) {
  return (unsigned long long)__double_as_longlong(ldexp(v, e) + 0x1.8p52) - kIMagic;
}

// Digits of four biased images: word t holds digit t of values 0..3 in bytes 0..3, each byte t of
// the biased value minus 128, so that N = sum_t 256^t digit_t.
__device__ __forceinline__ void fx_digits7(const unsigned long long (&b)[4], unsigned (&w)[kIDig]) {
  const unsigned l0 = (unsigned)b[0], l1 = (unsigned)b[1], l2 = (unsigned)b[2], l3 = (unsigned)b[3];
  const unsigned h0 = (unsigned)(b[0] >> 32), h1 = (unsigned)(b[1] >> 32), h2 = (unsigned)(b[2] >> 32),
                 h3 = (unsigned)(b[3] >> 32);
  // v_perm_b32: selector bytes 0..3 pick bytes of the second source, 4..7 of the first
  const unsigned x01lo = __builtin_amdgcn_perm(l1, l0, 0x05010400u);  // b0.0 b1.0 b0.1 b1.1
  const unsigned x01hi = __builtin_amdgcn_perm(l1, l0, 0x07030602u);  // b0.2 b1.2 b0.3 b1.3
  const unsigned x23lo = __builtin_amdgcn_perm(l3, l2, 0x05010400u);
  const unsigned x23hi = __builtin_amdgcn_perm(l3, l2, 0x07030602u);
  const unsigned y01lo = __builtin_amdgcn_perm(h1, h0, 0x05010400u);  // b0.4 b1.4 b0.5 b1.5
  const unsigned y01hi = __builtin_amdgcn_perm(h1, h0, 0x07030602u);  // b0.6 b1.6 b0.7 b1.7
  const unsigned y23lo = __builtin_amdgcn_perm(h3, h2, 0x05010400u);
  const unsigned y23hi = __builtin_amdgcn_perm(h3, h2, 0x07030602u);
  w[0] = __builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u) ^ 0x80808080u;
  w[1] = __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u) ^ 0x80808080u;
  w[2] = __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u) ^ 0x80808080u;
  w[3] = __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u) ^ 0x80808080u;
  w[4] = __builtin_amdgcn_perm(y23lo, y01lo, 0x05040100u) ^ 0x80808080u;
  w[5] = __builtin_amdgcn_perm(y23lo, y01lo, 0x07060302u) ^ 0x80808080u;
  w[6] = __builtin_amdgcn_perm(y23hi, y01hi, 0x05040100u) ^ 0x80808080u;
}

// ---- t pass: s_bi = D_i sum_j C_ij x_bj -------------------------------------------------------
// Workgroup (blockIdx.x, blockIdx.y): components 32 x .. 32 x + 31, vectors 2 y and 2 y + 1.
// MFMA D(16 x 16) += A(16 x 64) B(64 x 16): A row = component (the codes of one packed word of C
// per lane, 16 columns, unpacked to signed bytes through a 256-entry table), B column c = digit
// column 7 v + t (digit t of vector v's image; columns 14, 15 zero), k = the 64 columns of four
// packed words.  Eight waves: wave w takes component tile w & 1 and every fourth group of 16
// words, from group w >> 1; the four partial tiles add in LDS.
// The digit operands are built in LDS for up to kTWords words at a time: word W, column c holds
// the 16 bytes of digit c for x[16 W .. 16 W + 15] at slot c ^ (W % 16) of the word's 256 bytes
// (the 16 lanes of a group still read the word's 256 contiguous bytes; the builders' stores of one
// column for 16 words fall in distinct banks).
// smax[b gridDim.x + blockIdx.x] receives the workgroup's max |s_b| (high word of the fp64 bits).
__global__ void __launch_bounds__(kTThreads) infer_t_kernel(const uint32_t* __restrict__ C, int wn, int n,
                                                      const float* __restrict__ D, int k, const float* __restrict__ X,
                                                      int batch, int x_vec4, int c_vec4, double* __restrict__ S,
                                                      unsigned* __restrict__ smax, long long* __restrict__ Yacc,
                                                      long long nY, unsigned* __restrict__ cnt, int ncnt) {
  // every argument fetched at once (else the compiler waits for them one after another)
  asm volatile("" ::"s"(C), "s"(wn), "s"(n), "s"(D), "s"(k), "s"(X), "s"(batch), "s"(x_vec4), "s"(c_vec4), "s"(S),
               "s"(smax), "s"(Yacc), "s"(nY), "s"(cnt), "s"(ncnt));
  constexpr int kSS = (kTWords / 16 + kTKh - 1) / kTKh;     // super-steps (16 words) of a wave per chunk
  constexpr int kXI = (kTWords * 4 + kTThreads - 1) / kTThreads;  // quads of x per thread per chunk
  constexpr int kNW = kTThreads / 64;
  __shared__ unsigned lut[256];
  __shared__ __attribute__((aligned(16))) unsigned char xop[kTWords * 256];
  __shared__ int red[kNW][256];
  __shared__ unsigned wmx[2][kNW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tile = wv & 1, kh = wv >> 1, gg = lane >> 4, lr = lane & 15;
  const int ci = blockIdx.x * kTComp + 16 * tile + lr;  // this lane's component (row of A)
  const bool crow = ci < k;
  const uint32_t* cp = C + (size_t)(crow ? ci : 0) * wn;
  const int b0 = 2 * blockIdx.y;
  const bool two = b0 + 1 < batch;
  const float* x0 = X + (size_t)b0 * n;
  const float* x1 = two ? x0 + n : x0;
  const int wnp = (wn + 15) & ~15;
  // threads 0..63 finish (tile tid >> 5, row (tid >> 1) & 15, vector tid & 1): their scale, early
  const int fi = blockIdx.x * kTComp + 16 * ((tid >> 5) & 1) + ((tid >> 1) & 15);
  const float dfin = D[fi < k ? fi : 0];  // an unconditional load: nothing waits for it until the end
  int e0 = 0, e1 = 0;
  long long T = 0;  // threads 0..63: (tile tid >> 5, row (tid >> 1) & 15, vector tid & 1)
  for (int cw0 = 0; cw0 < wnp; cw0 += kTWords) {
    const int cwn = wnp - cw0 < kTWords ? wnp - cw0 : kTWords;  // multiple of 16
    const int ns = cwn / 16;
    // every global load of the chunk first: this lane's words of C, this thread's quads of x
    uint4 cv[kSS];
#pragma unroll
    for (int u = 0; u < kSS; ++u) {
      const int s = kh + kTKh * u, wg = cw0 + 16 * s + 4 * gg;
      if (s < ns && crow && wg + 4 <= wn && c_vec4) {
        cv[u] = *reinterpret_cast<const uint4*>(cp + wg);
      } else {
        const bool ok = s < ns && crow;
        cv[u].x = (ok && wg < wn) ? cp[wg] : 0u;
        cv[u].y = (ok && wg + 1 < wn) ? cp[wg + 1] : 0u;
        cv[u].z = (ok && wg + 2 < wn) ? cp[wg + 2] : 0u;
        cv[u].w = (ok && wg + 3 < wn) ? cp[wg + 3] : 0u;
      }
    }
    float4 xa[kXI], xb[kXI];
#pragma unroll
    for (int u = 0; u < kXI; ++u) {
      const int it = tid + kTThreads * u;
      const int j = 16 * (cw0 + (it >> 2)) + 4 * (it & 3);
      if (it < cwn * 4 && x_vec4 && j + 4 <= n) {
        xa[u] = *reinterpret_cast<const float4*>(x0 + j);
        xb[u] = *reinterpret_cast<const float4*>(x1 + j);
      } else {
        const bool ok = it < cwn * 4;
        xa[u].x = (ok && j < n) ? x0[j] : 0.0f;
        xa[u].y = (ok && j + 1 < n) ? x0[j + 1] : 0.0f;
        xa[u].z = (ok && j + 2 < n) ? x0[j + 2] : 0.0f;
        xa[u].w = (ok && j + 3 < n) ? x0[j + 3] : 0.0f;
        xb[u].x = (ok && j < n) ? x1[j] : 0.0f;
        xb[u].y = (ok && j + 1 < n) ? x1[j + 1] : 0.0f;
        xb[u].z = (ok && j + 2 < n) ? x1[j + 2] : 0.0f;
        xb[u].w = (ok && j + 3 < n) ? x1[j + 3] : 0.0f;
      }
    }
    if (cw0 == 0) {
      for (long long x = ((long long)blockIdx.y * gridDim.x + blockIdx.x) * kTThreads + tid; x < nY;
           x += (long long)gridDim.x * gridDim.y * kTThreads)
        Yacc[x] = 0;  // the y pass adds into it after this launch
      for (int x = (blockIdx.y * gridDim.x + blockIdx.x) * kTThreads + tid; x < ncnt; x += gridDim.x * gridDim.y * kTThreads)
        cnt[x] = 0u;  // and counts its finished workgroups here
      if (tid < 256) {  // byte value -> its four 2-bit codes as signed bytes (0 -> 0, 1 -> 1, 3 -> -1)
        unsigned v = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned c = (tid >> (2 * q)) & 3u;
          v |= (c >= 2 ? (c | 0xFCu) : c) << (8 * q);
        }
        lut[tid] = v;
      }
      // max |x| of both vectors: the quads in registers, and the rest of x when it spans chunks
      unsigned m0 = 0u, m1 = 0u;
#pragma unroll
      for (int u = 0; u < kXI; ++u) {
        const unsigned a[4] = {__float_as_uint(xa[u].x), __float_as_uint(xa[u].y), __float_as_uint(xa[u].z),
                               __float_as_uint(xa[u].w)};
        const unsigned c[4] = {__float_as_uint(xb[u].x), __float_as_uint(xb[u].y), __float_as_uint(xb[u].z),
                               __float_as_uint(xb[u].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned aa = a[e] & 0x7FFFFFFFu, cc = c[e] & 0x7FFFFFFFu;
          m0 = aa > m0 ? aa : m0;
          m1 = cc > m1 ? cc : m1;
        }
      }
      for (int j = 16 * kTWords + tid; j < n; j += kTThreads) {
        const unsigned aa = __float_as_uint(x0[j]) & 0x7FFFFFFFu, cc = __float_as_uint(x1[j]) & 0x7FFFFFFFu;
        m0 = aa > m0 ? aa : m0;
        m1 = cc > m1 ? cc : m1;
      }
      if (!two) m1 = 0u;
      m0 = wave_max_u32(m0);
      m1 = wave_max_u32(m1);
      if (lane == 0) {
        wmx[0][wv] = m0;
        wmx[1][wv] = m1;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kNW; ++q) {
        m0 = wmx[0][q] > m0 ? wmx[0][q] : m0;
        m1 = wmx[1][q] > m1 ? wmx[1][q] : m1;
      }
      const int px = inf_bits(n);
      e0 = m0 ? px - f32_bound_exp(m0) : 0;
      e1 = m1 ? px - f32_bound_exp(m1) : 0;
    } else {
      __syncthreads();  // the last chunk's operands are read
    }
    // digit operands of the chunk
#pragma unroll
    for (int u = 0; u < kXI; ++u) {
      const int it = tid + kTThreads * u;
      if (it < cwn * 4) {
        const int W = it >> 2, q = it & 3;
        const float a[4] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w};
        const float c[4] = {xb[u].x, xb[u].y, xb[u].z, xb[u].w};
        unsigned long long ba[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ba[e] = fx_biased((double)a[e], e0);
        unsigned da[kIDig], db[kIDig];
        fx_digits7(ba, da);
        if (two) {  // uniform
          unsigned long long bb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) bb[e] = fx_biased((double)c[e], e1);
          fx_digits7(bb, db);
        } else {
#pragma unroll
          for (int t = 0; t < kIDig; ++t) db[t] = 0u;
        }
        unsigned* o = reinterpret_cast<unsigned*>(xop + W * 256 + 4 * q);  // column c at slot c ^ (W % 16)
        const int sw = W & 15;
#pragma unroll
        for (int t = 0; t < kIDig; ++t) {
          o[4 * (t ^ sw)] = da[t];
          o[4 * ((kIDig + t) ^ sw)] = db[t];
        }
        o[4 * (14 ^ sw)] = 0u;
        o[4 * (15 ^ sw)] = 0u;
      }
    }
    __syncthreads();
    iv4 acc4[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};  // one chain per word slot
#pragma unroll
    for (int u = 0; u < kSS; ++u) {
      const int s = kh + kTKh * u;
      if (s < ns) {
        const int wl = 16 * s + 4 * gg;  // chunk-local index of this lane group's first word
        const unsigned cw[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
        iv4 av[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          av[e][0] = (int)lut[cw[e] & 0xFFu];
          av[e][1] = (int)lut[(cw[e] >> 8) & 0xFFu];
          av[e][2] = (int)lut[(cw[e] >> 16) & 0xFFu];
          av[e][3] = (int)lut[cw[e] >> 24];
          bv[e] = *reinterpret_cast<const iv4*>(xop + ((wl + e) * 16 + (lr ^ ((wl + e) & 15))) * 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc4[e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[e], bv[e], acc4[e], 0, 0, 0);
      }
    }
    const iv4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    // acc[q] = D(component 4 gg + q, column lr)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wv][(4 * gg + q) * 16 + lr] = acc[q];
    __syncthreads();
    if (tid < 64) {
      const int tl = tid >> 5, rr = (tid >> 1) & 15, v = tid & 1;
      long long sum = 0;  // Horner over the digits: sum_t 256^t (column 7 v + t)
#pragma unroll
      for (int t = kIDig - 1; t >= 0; --t) {
        const int c = kIDig * v + t;
        int d = 0;
#pragma unroll
        for (int h = 0; h < kTKh; ++h) d += red[tl + 2 * h][rr * 16 + c];
        sum = sum * 256 + d;
      }
      T += sum;
    }
  }
  if (tid < 64) {
    const int tl = tid >> 5, rr = (tid >> 1) & 15, v = tid & 1;
    const int i = blockIdx.x * kTComp + 16 * tl + rr;
    const int b = b0 + v;
    unsigned hb = 0u;
    if (i < k && b < batch) {
      const double s = (double)dfin * ldexp((double)T, -(v ? e1 : e0));
      S[(size_t)b * k + i] = s;
      hb = hi_abs(s);
    }
    const unsigned h0 = wave_max_u32(v == 0 ? hb : 0u), h1 = wave_max_u32(v == 1 ? hb : 0u);
    if (tid == 0) {
      smax[(size_t)b0 * gridDim.x + blockIdx.x] = h0;
      if (two) smax[(size_t)(b0 + 1) * gridDim.x + blockIdx.x] = h1;
    }
  }
}

// this thread's part of max |s_b| over the t pass's per-workgroup maxima (high words of the bits)
__device__ __forceinline__ unsigned infer_smax_part(const unsigned* smax, int gxt, int b) {
  unsigned h = 0u;
  for (int x = threadIdx.x; x < gxt; x += blockDim.x) {
    const unsigned v = smax[(size_t)b * gxt + x];
    h = v > h ? v : h;
  }
  return h;
}

// the workgroup's max of h0 (and h1) -> fixed-point scales f (k |S| <= 2^62); wmx: 2 x 16 words
__device__ __forceinline__ void infer_s_scales(unsigned h0, unsigned h1, int k, unsigned* wmx, int& f0, int& f1) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = (int)(blockDim.x >> 6);
  h0 = wave_max_u32(h0);
  h1 = wave_max_u32(h1);
  if (lane == 0) {
    wmx[wv] = h0;
    wmx[16 + wv] = h1;
  }
  __syncthreads();
  for (int q = 0; q < nw; ++q) {
    h0 = wmx[q] > h0 ? wmx[q] : h0;
    h1 = wmx[16 + q] > h1 ? wmx[16 + q] : h1;
  }
  const int ps = inf_bits(k);
  f0 = h0 ? ps - f64_bound_exp(h0) : 0;
  f1 = h1 ? ps - f64_bound_exp(h1) : 0;
}

// ---- y pass: Yacc[b][r] += sum over a chunk of components of B_ri S_bi --------------------------
// Workgroup (x, y), x = nwg c + g: packed words 16 g .. 16 g + 15 of B's rows (outputs 256 g ..),
// components 256 c .. 256 c + 255, vectors 2 y and 2 y + 1.  MFMA D(16 x 16) += A(16 x 64) B(64 x 16): A row
// c = digit column 7 v + t of S (16 bytes = 16 consecutive components), B column = output, k = 64
// components.  The B words of the chunk are staged in LDS word-major, so that a lane reads the 16
// words of its 16 components as 64 contiguous bytes and extracts its output's 2-bit code from each
// (signed bit-field extracts, packed into bytes by byte permutes).  Eight waves, wave w on words
// w and w + 8; each output's chunk sum is added with one 64-bit atomic per vector.  The last
// workgroup of an output group to finish (a counter per group and vector pair, cleared by the t
// pass) rounds the group's outputs to fp32: every workgroup's adds have returned before it counts
// itself, and the last one reads the sums back with atomic adds of zero, at the same place the
// adds were made.
// Every global load of the workgroup is issued before the first is used.
__global__ void __launch_bounds__(kYThreads) infer_y_kernel(const uint32_t* __restrict__ B, int wm, int m, int k,
                                                      const double* __restrict__ S, int batch,
                                                      const unsigned* __restrict__ smax, int gxt, int nwg,
                                                      int b_vec4, long long* __restrict__ Yacc,
                                                      unsigned* __restrict__ cnt, float* __restrict__ Y) {
  asm volatile("" ::"s"(B), "s"(wm), "s"(m), "s"(k), "s"(S), "s"(batch), "s"(smax), "s"(gxt), "s"(nwg), "s"(b_vec4),
               "s"(Yacc), "s"(cnt), "s"(Y));
  __shared__ int last;
  constexpr int kBI = kYComp * (kYWords / 4) / kYThreads;  // quads of B words per thread
  __shared__ __attribute__((aligned(16))) uint32_t bw[kYWords * kYPitch];
  __shared__ __attribute__((aligned(16))) unsigned char sop[kYComp / 64 * 4 * 256];
  __shared__ unsigned wmx[32];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int w0 = (int)(blockIdx.x % nwg) * kYWords, i0 = (int)(blockIdx.x / nwg) * kYComp, b0 = 2 * blockIdx.y;
  const bool two = b0 + 1 < batch;
  // the chunk's B words (item: words 4 wq .. 4 wq + 3 of component il)
  uint4 bq[kBI];
#pragma unroll
  for (int u = 0; u < kBI; ++u) {
    const int it = tid + kYThreads * u, wq = it & 3, il = it >> 2;
    const int i = i0 + il, w = w0 + 4 * wq;
    const uint32_t* src = B + (size_t)(i < k ? i : 0) * wm + w;
    if (i < k && w + 4 <= wm && b_vec4) {
      bq[u] = *reinterpret_cast<const uint4*>(src);
    } else {
      bq[u].x = (i < k && w < wm) ? src[0] : 0u;
      bq[u].y = (i < k && w + 1 < wm) ? src[1] : 0u;
      bq[u].z = (i < k && w + 2 < wm) ? src[2] : 0u;
      bq[u].w = (i < k && w + 3 < wm) ? src[3] : 0u;
    }
  }
  // s of the digit item (component quad p = tid >> 1, vector tid & 1; threads below kYComp / 2)
  const int dp = tid >> 1, dv = tid & 1, dil = 4 * dp, db = b0 + dv;
  double sv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + dil + e;
    sv[e] = (tid < kYComp / 2 && i < k && db < batch) ? S[(size_t)db * k + i] : 0.0;
  }
  const unsigned h0 = infer_smax_part(smax, gxt, b0), h1 = two ? infer_smax_part(smax, gxt, b0 + 1) : 0u;
  // stage the B words transposed: bw[w][i]
#pragma unroll
  for (int u = 0; u < kBI; ++u) {
    const int it = tid + kYThreads * u, wq = it & 3, il = it >> 2;
    bw[(4 * wq) * kYPitch + il] = bq[u].x;
    bw[(4 * wq + 1) * kYPitch + il] = bq[u].y;
    bw[(4 * wq + 2) * kYPitch + il] = bq[u].z;
    bw[(4 * wq + 3) * kYPitch + il] = bq[u].w;
  }
  int f0, f1;
  infer_s_scales(h0, h1, k, wmx, f0, f1);
  // digit operands of S: component il = 4 p + e sits at step il / 64, lane group (il / 16) % 4,
  // byte il % 16 of row c = 7 v + t
  if (tid < kYComp / 2) {
    unsigned long long bs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bs[e] = fx_biased(sv[e], dv ? f1 : f0);
    unsigned d[kIDig];
    fx_digits7(bs, d);
    unsigned char* o = sop + (((dil >> 6) * 4 + ((dil >> 4) & 3)) * 16) * 16 + (dil & 15);
#pragma unroll
    for (int t = 0; t < kIDig; ++t) *reinterpret_cast<unsigned*>(o + 16 * (kIDig * dv + t)) = d[t];
    if (dv == 1) {
      *reinterpret_cast<unsigned*>(o + 16 * 14) = 0u;
      *reinterpret_cast<unsigned*>(o + 16 * 15) = 0u;
    }
  }
  __syncthreads();
  const int gg = lane >> 4, lr = lane & 15;
  iv4 av[kYComp / 64];
#pragma unroll
  for (int st = 0; st < kYComp / 64; ++st) av[st] = *reinterpret_cast<const iv4*>(sop + ((st * 4 + gg) * 16 + lr) * 16);
  const int sh = 2 * lr;
  // weights 256^t of the four digit rows 4 gg + q this lane's accumulator holds, per vector
  long long wt0[4], wt1[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = 4 * gg + q;
    wt0[q] = c < kIDig ? (1ll << (8 * c)) : 0ll;
    wt1[q] = (c >= kIDig && c < 2 * kIDig) ? (1ll << (8 * (c - kIDig))) : 0ll;
  }
  iv4 accw[kYWpw];
#pragma unroll
  for (int wq = 0; wq < kYWpw; ++wq) accw[wq] = iv4{0, 0, 0, 0};
#pragma unroll
  for (int st = 0; st < kYComp / 64; ++st) {
    uint4 q[kYWpw][4];
#pragma unroll
    for (int wq = 0; wq < kYWpw; ++wq) {
      const uint4* src = reinterpret_cast<const uint4*>(bw + (wv + (kYWords / kYWpw) * wq) * kYPitch + 64 * st + 16 * gg);
#pragma unroll
      for (int h = 0; h < 4; ++h) q[wq][h] = src[h];
    }
#pragma unroll
    for (int wq = 0; wq < kYWpw; ++wq) {
      const unsigned wd[16] = {q[wq][0].x, q[wq][0].y, q[wq][0].z, q[wq][0].w, q[wq][1].x, q[wq][1].y,
                               q[wq][1].z, q[wq][1].w, q[wq][2].x, q[wq][2].y, q[wq][2].z, q[wq][2].w,
                               q[wq][3].x, q[wq][3].y, q[wq][3].z, q[wq][3].w};
      iv4 bv;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const unsigned c0 = (unsigned)__builtin_amdgcn_sbfe((int)wd[4 * h], sh, 2);
        const unsigned c1 = (unsigned)__builtin_amdgcn_sbfe((int)wd[4 * h + 1], sh, 2);
        const unsigned c2 = (unsigned)__builtin_amdgcn_sbfe((int)wd[4 * h + 2], sh, 2);
        const unsigned c3 = (unsigned)__builtin_amdgcn_sbfe((int)wd[4 * h + 3], sh, 2);
        const unsigned p01 = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);  // c0.0 c1.0 0 0
        const unsigned p23 = __builtin_amdgcn_perm(c3, c2, 0x0c0c0400u);
        bv[h] = (int)__builtin_amdgcn_perm(p23, p01, 0x05040100u);
      }
      accw[wq] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[st], bv, accw[wq], 0, 0, 0);
    }
  }
  unsigned long long got = 0ull;  // the returned old values, so that the adds are waited for
#pragma unroll
  for (int wq = 0; wq < kYWpw; ++wq) {
    const int wl = wv + (kYWords / kYWpw) * wq;
    const iv4 acc = accw[wq];
    // acc[q] = D(digit row 4 gg + q, output lr): recombine per vector, then over the lane groups
    long long y0 = 0, y1 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y0 += (long long)acc[q] * wt0[q];
      y1 += (long long)acc[q] * wt1[q];
    }
    y0 += __shfl_xor(y0, 16);
    y1 += __shfl_xor(y1, 16);
    y0 += __shfl_xor(y0, 32);
    y1 += __shfl_xor(y1, 32);
    const int r = 16 * (w0 + wl) + lr;
    if (gg == 0 && r < m) {
      if (y0 != 0)
        got |= atomicAdd(reinterpret_cast<unsigned long long*>(Yacc + (size_t)b0 * m + r), (unsigned long long)y0);
      if (two && y1 != 0)
        got |= atomicAdd(reinterpret_cast<unsigned long long*>(Yacc + (size_t)(b0 + 1) * m + r), (unsigned long long)y1);
    }
  }
  asm volatile("" ::"v"(got));  // this thread's adds have returned
  __syncthreads();
  const int grp = (int)(blockIdx.x % nwg), nch = (int)((k + kYComp - 1) / kYComp);
  if (tid == 0) last = atomicAdd(cnt + (size_t)blockIdx.y * nwg + grp, 1u) == (unsigned)(nch - 1);
  __syncthreads();
  if (last) {  // every chunk of this output group has been added: round its outputs
    for (int x = tid; x < 2 * 16 * kYWords; x += kYThreads) {
      const int v = x / (16 * kYWords), r = 16 * w0 + x % (16 * kYWords), b = b0 + v;
      if (r < m && b < batch) {
        const long long val =
            (long long)atomicAdd(reinterpret_cast<unsigned long long*>(Yacc + (size_t)b * m + r), 0ull);
        Y[(size_t)b * m + r] = (float)ldexp((double)val, -(v ? f1 : f0));
      }
    }
  }
}

static int infer_gxt(int k) { return (k + kTComp - 1) / kTComp; }

static int infer_groups(int m) { return ((m + 15) / 16 + kYWords - 1) / kYWords; }  // output groups of the y pass

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// S (batch x k fp64), Yacc (batch x m int64), smax (batch x gxt), counters (pairs of vectors x groups)
size_t infer_workspace_bytes(int k, int m, int batch) {
  return al256((size_t)batch * k * 8) + al256((size_t)batch * m * 8) + al256((size_t)batch * infer_gxt(k) * 4) +
         al256((size_t)((batch + 1) / 2) * infer_groups(m) * 4);
}

hipError_t infer_run(const uint32_t* B, const uint32_t* C, const float* D, int k, int m, int n, const float* X,
                     int batch, float* Y, void* ws, hipStream_t st) {
  const int wm = (m + 15) / 16, wn = (n + 15) / 16, gxt = infer_gxt(k);
  char* base = static_cast<char*>(ws);
  double* S = reinterpret_cast<double*>(base);
  base += al256((size_t)batch * k * 8);
  long long* Yacc = reinterpret_cast<long long*>(base);
  base += al256((size_t)batch * m * 8);
  unsigned* smax = reinterpret_cast<unsigned*>(base);
  base += al256((size_t)batch * gxt * 4);
  unsigned* cnt = reinterpret_cast<unsigned*>(base);
  const long long nY = (long long)batch * m;
  const int x_vec4 = (n % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 15u) == 0) ? 1 : 0;
  const int c_vec4 = (wn % 4 == 0 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0) ? 1 : 0;
  const int b_vec4 = (wm % 4 == 0 && (reinterpret_cast<uintptr_t>(B) & 15u) == 0) ? 1 : 0;
  const int gb = (batch + 1) / 2;
  const long long nwg = infer_groups(m), nch = (k + kYComp - 1) / kYComp;
  if (nwg * nch > 2147483647ll || nwg * gb > 2147483647ll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(infer_t_kernel, dim3(gxt, gb), dim3(kTThreads), 0, st, C, wn, n, D, k, X, batch, x_vec4, c_vec4, S,
                     smax, Yacc, nY, cnt, (int)(nwg * gb));
  hipLaunchKernelGGL(infer_y_kernel, dim3((unsigned)(nwg * nch), gb), dim3(kYThreads), 0, st, B, wm, m, k, S, batch, smax,
                     gxt, (int)nwg, b_vec4, Yacc, cnt, Y);
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
