// Block-ALS path: b components per block with dense contractions on fp64 MFMA (gfx950).
//
// Method (ExTernD review, Method: "a batched block-ALS GPU algorithm with a decorrelated
// least-squares target"; pith.science minor comment 1, Eq. 3: V <- T_tau((U^T U + eps I)^-1
// U^T R)^T).  Per block of b components:
//   U  = T_tau(R Omega) column by column (Omega: column 0 all ones, the rest Rademacher signs
//        from splitmix64, so b = 1 starts from the row sums like the sequential engine);
//   als_iters times:
//     G = (U^T U + eps I)^-1 U^T R,  V[c] = T_tau(G[c]; h)          (corrected weighted V-step)
//     F = R H V (V^T H V + eps I)^-1, U[:,c] = T_tau(F[:,c])         (U-step)
//   d_c = (u_c^T R H v_c - sum_{c'<c} d_c' (u_c^T u_c')(v_c'^T H v_c)) / (|u_c|^2 v_c^T H v_c),
//        the sequential scale of each component against the residual left by the earlier ones;
//   R <- fl32(R - U diag(d) V^T).
// eps = 1e-6 trace(Gram) / b.
//
// MI355X mapping.  The three residual contractions per half-step (R Omega / R H V with K = n,
// U^T R with K = m, and the rank-b update with K = b) run on v_mfma_f64_16x16x4f64: R is
// converted fp32 -> fp64 exactly, the ternary operand is exact, accumulation is fp64, so the
// contractions agree with the fp64 sums of a plain implementation to rounding order.  Split-K
// partial results are summed in a fixed order (deterministic).  The small b x b work (Grams,
// Cholesky, triangular solves, scales) runs in dedicated kernels with the same operation order as
// a textbook implementation.  Selections use the same exact projection as the sequential path,
// one workgroup per component.
#include "externd_internal.hpp"
#include "select.hpp"

namespace externd {

typedef double dbl4 __attribute__((ext_vector_type(4)));

constexpr int kGramSplit = 8;    // most K splits of the weighted Gram
constexpr int kGramTiles = 136;  // lower 16 x 16 tiles of a Gram with b <= 256

struct BlockWs {
  int ldu, ldv;    // row lengths of Ut / Vt: m and n rounded up to 16 (zero padding)
  int8_t* Ut;      // b x ldu, component-major
  int8_t* Vt;      // b x ldv (also holds Omega for the sketch)
  double* Yt;      // b x m: sketch / (R H V)^T
  double* Ft;      // b x m: F^T
  double* X;       // b x n: U^T R
  double* Z;       // b x max(m, n): G (V-step target)
  double* Tmp;     // b x max(m, n): L^-1 times the right-hand sides
  double* GU;      // b x b
  double* GV;      // b x b
  double* Li;      // b x b: (G + eps I)^-1 for b <= kSpdMax, else the inverse Cholesky factor
  double* Md;      // b: u_c^T Q_c (diagonal of U^T R H V)
  double* PHC;     // b x 3 selection results
  float* d;        // b
  double* st;      // [0] E, [1] E0, [2] E before a refit's add-back, [3] E with it restored
  int* flags;      // [0] dead, [1] empty sketch columns, [2] fallbacks, [3] energy target reached,
                   // [4] components of the block kept (emitted), [5] refit discarded (sweeps)
  int* used;       // m: rows used by sketch fallbacks within the block
  unsigned* rmax;  // [64 (s & 1) + w]: max |R| (fp32 bits) at the start of block s, spread over 64
                   // words w to keep the atomics of one update uncontended
  uint8_t* hdig;   // kHDig x ldv: 7-bit digits of the fixed-point column weights (weighted only)
  double* gpart;   // kGramSplit x kGramTiles x 256: split-K partial tiles of the weighted Gram
  unsigned* gcnt;  // kGramTiles: workgroups of each tile done (zero between launches)
  double* GUo;     // b x b: Gram of the old U (refinement sweeps)
  double* GVo;     // b x b: weighted Gram of the old V
  double* ppo;     // b: u_c^T (R + X) H v_c of the old components
  float* dold;     // b: old scales
};

constexpr int kMaxWords = 64;      // words per residual-max slot (one per lane of a wave)
constexpr int kHDig = 5;           // 7-bit digits of the fixed-point weights (35 bits)

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// One layout for both sizing and carving.
template <typename F>
static void ws_layout(int m, int n, int b, F&& take) {
  const size_t mx = (size_t)(m > n ? m : n), bb = (size_t)b;
  take((void**)nullptr, bb * (size_t)((m + 15) & ~15));  // Ut
  take((void**)nullptr, bb * (size_t)((n + 15) & ~15));  // Vt
  take((void**)nullptr, bb * m * 8);
  take((void**)nullptr, bb * m * 8);
  take((void**)nullptr, bb * n * 8);
  take((void**)nullptr, bb * mx * 8);
  take((void**)nullptr, bb * mx * 8);
  take((void**)nullptr, bb * bb * 8);
  take((void**)nullptr, bb * bb * 8);
  take((void**)nullptr, bb * bb * 8);
  take((void**)nullptr, bb * 8);
  take((void**)nullptr, bb * 3 * 8);
  take((void**)nullptr, bb * 4);
  take((void**)nullptr, 64);
  take((void**)nullptr, 64);
  take((void**)nullptr, (size_t)m * 4);
  take((void**)nullptr, 2 * kMaxWords * 4);
  take((void**)nullptr, (size_t)kHDig * (size_t)((n + 15) & ~15));
  take((void**)nullptr, bb * bb * 8);
  take((void**)nullptr, bb * bb * 8);
  take((void**)nullptr, bb * 8);
  take((void**)nullptr, bb * 4);
  take((void**)nullptr, (size_t)kGramSplit * kGramTiles * 256 * 8);  // split-K Gram partial tiles
  take((void**)nullptr, (size_t)kGramTiles * 4);                     // their arrival counters
}

static BlockWs carve(void* base, int m, int n, int b) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  void* ptrs[32];
  int np = 0;
  ws_layout(m, n, b, [&](void**, size_t bytes) {
    ptrs[np++] = p + o;
    o = al(o + bytes);
  });
  BlockWs w;
  w.ldu = (m + 15) & ~15;
  w.ldv = (n + 15) & ~15;
  int q = 0;
  w.Ut = static_cast<int8_t*>(ptrs[q++]);
  w.Vt = static_cast<int8_t*>(ptrs[q++]);
  w.Yt = static_cast<double*>(ptrs[q++]);
  w.Ft = static_cast<double*>(ptrs[q++]);
  w.X = static_cast<double*>(ptrs[q++]);
  w.Z = static_cast<double*>(ptrs[q++]);
  w.Tmp = static_cast<double*>(ptrs[q++]);
  w.GU = static_cast<double*>(ptrs[q++]);
  w.GV = static_cast<double*>(ptrs[q++]);
  w.Li = static_cast<double*>(ptrs[q++]);
  w.Md = static_cast<double*>(ptrs[q++]);
  w.PHC = static_cast<double*>(ptrs[q++]);
  w.d = static_cast<float*>(ptrs[q++]);
  w.st = static_cast<double*>(ptrs[q++]);
  w.flags = static_cast<int*>(ptrs[q++]);
  w.used = static_cast<int*>(ptrs[q++]);
  w.rmax = static_cast<unsigned*>(ptrs[q++]);
  w.hdig = static_cast<uint8_t*>(ptrs[q++]);
  w.GUo = static_cast<double*>(ptrs[q++]);
  w.GVo = static_cast<double*>(ptrs[q++]);
  w.ppo = static_cast<double*>(ptrs[q++]);
  w.dold = static_cast<float*>(ptrs[q++]);
  w.gpart = static_cast<double*>(ptrs[q++]);
  w.gcnt = static_cast<unsigned*>(ptrs[q++]);
  return w;
}

size_t block_workspace_bytes(int m, int n, int b) {
  size_t o = 0;
  ws_layout(m, n, b, [&](void**, size_t bytes) { o = al(o + bytes); });
  return o;
}

// ---- splitmix64 sketch signs (S. Vigna's splitmix64: golden-gamma step, then the mix) ----
__device__ __forceinline__ u64 splitmix64(u64 key) {
  u64 z = key + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) omega_kernel(int8_t* Vt, int ldv, int bs, int n, long long s, int* flags,
                                                    unsigned* rmax, double* Z0, long long zcount) {
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < zcount; x += (long long)gridDim.x * 256) Z0[x] = 0.0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    flags[1] = 0;  // empty sketch columns of this block
    flags[2] = 0;  // fallback starts of this block
  }
  if (blockIdx.x == 0 && threadIdx.x < kMaxWords) rmax[kMaxWords * ((s + 1) & 1) + threadIdx.x] = 0u;
  const long long total = (long long)bs * ldv;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < total; x += (long long)gridDim.x * 256) {
    const int c = (int)(x / ldv), j = (int)(x - (long long)c * ldv);
    int8_t v = j < n ? (int8_t)1 : (int8_t)0;
    if (c > 0 && j < n) {
      const u64 key = (((u64)s << 16) + (u64)c) * (1ull << 32) + (u64)j;
      v = (splitmix64(key) >> 63) ? (int8_t)-1 : (int8_t)1;
    }
    Vt[x] = v;
  }
}

// ---- residual contractions on v_mfma_i32_16x16x64_i8 with R in fixed point ------------------
// D(16x16) += A(16x64) B(64x16) in int32: lane l supplies 16 bytes of row l % 16 of A and 16 bytes
// of column l % 16 of B, paired on the same k; D(i, j) lands in lane j + 16 (i / 4), register i % 4.
// Lane group g = l / 16 takes k = k0 + 16 g .. k0 + 16 g + 15 of each 64-wide k chunk.
//
// R enters as N = rint(x 2^f), x = R_ij (times h_j where weighted), with one power-of-two scale per
// block chosen from max |R| so that |N| <= 2^30, split into four signed 8-bit digits
// N = sum_s 2^(8 s) d_s.  The ternary operand is exact in int8, each digit product sums exactly
// in int32 (|sum| <= 2^7 K), the digits recombine exactly in fp64 and splits of K add exactly
// (every partial is an integer times 2^-f below 2^53).  The result is therefore the exact
// contraction of the fixed-point image of R, whatever the launch shape or the order of the
// atomic adds: its only error is the rounding of each x to the grid 2^-f, at most 2^-31 of the
// largest |x|.
typedef int v4i __attribute__((ext_vector_type(4)));

// exponent E of the fixed-point range: |x| < 2^E for every x entering a contraction (each wave
// reduces the 64 words of block s's slot itself)
__device__ __forceinline__ int fx_exponent(const unsigned* rmax, int s, int ehm) {
  const unsigned bits = wave_max_u32(rmax[kMaxWords * (s & 1) + (threadIdx.x & 63)]);
  if (bits == 0u) return 0;
  return exp_bound(__uint_as_float(bits)) + ehm;
}

// Digits of four fixed-point values: word t holds digit t of n[0..3] in bytes 0..3.  With
// B = n + 0x808080, digits 0..2 are B's bytes minus 128 (byte ^ 0x80) and digit 3 is B >> 24.
__device__ __forceinline__ void fx_digits4(int n0, int n1, int n2, int n3, unsigned (&w)[4]) {
  const unsigned b0 = (unsigned)(n0 + 0x808080), b1 = (unsigned)(n1 + 0x808080);
  const unsigned b2 = (unsigned)(n2 + 0x808080), b3 = (unsigned)(n3 + 0x808080);
  // v_perm_b32: selector bytes 0..3 pick bytes of the second source, 4..7 of the first
  const unsigned x01lo = __builtin_amdgcn_perm(b1, b0, 0x05010400u);  // b0.0 b1.0 b0.1 b1.1
  const unsigned x01hi = __builtin_amdgcn_perm(b1, b0, 0x07030602u);  // b0.2 b1.2 b0.3 b1.3
  const unsigned x23lo = __builtin_amdgcn_perm(b3, b2, 0x05010400u);
  const unsigned x23hi = __builtin_amdgcn_perm(b3, b2, 0x07030602u);
  w[0] = __builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u) ^ 0x80808080u;
  w[1] = __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u) ^ 0x80808080u;
  w[2] = __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u) ^ 0x80808080u;
  w[3] = __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u);
}

// 16 fixed-point values -> the four digit operands (operand t = digit t of values 0..15)
__device__ __forceinline__ void fx_operands(const int (&nv)[16], v4i (&op)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    unsigned w[4];
    fx_digits4(nv[4 * q], nv[4 * q + 1], nv[4 * q + 2], nv[4 * q + 3], w);
#pragma unroll
    for (int t = 0; t < 4; ++t) op[t][q] = (int)w[t];
  }
}

__device__ __forceinline__ v4i load16(const int8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// (G + eps I)^-1 by one workgroup of NT threads over `smem` (spd_lds_bytes(bs) bytes); below.
template <int NT>
__device__ __forceinline__ void spd_inv_body(const double* G, int bs, double* Gi, char* smem);
__host__ __device__ inline size_t spd_lds_bytes(int bs);

// The residual tile of each 64-wide k chunk is loaded by the whole workgroup as float4 rows
// (256 contiguous bytes per tile row: full cache lines), converted to its fixed-point image
// once, and staged in LDS; each lane then reads its 16 values of the MFMA layout from there.  The
// next chunk's loads are issued before the current chunk is consumed.
constexpr int kTileP = 68;  // int32 pitch of a [64 rows][64 k] tile (rows 16 B aligned)
constexpr int kTileQ = 65;  // int32 pitch of a [64 k][64 cols] tile (column reads conflict-free)

// out[c][i] (+)= sum_{k in this split} x_ik T[c][k], x_ik = R[i][k] (h_k): rows of R x components.
// Workgroup: 64 rows (16 per wave) x 16 NCT components (blockIdx.y), K range blockIdx.z.
template <int NCT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) rv_i8_kernel(const float* R, int ldr, int rows, int K, const int8_t* T,
                                                    int ldt, const float* h, int ehm, int bs, const unsigned* rmax,
                                                    int sblk, int kspan, double* out, const double* spdG,
                                                    double* spdGi) {
  extern __shared__ __align__(16) char dsm[];
  if (spdG && blockIdx.x == gridDim.x - 1) {  // the extra column of workgroups: one inverts spdG
    if (blockIdx.y == 0 && blockIdx.z == 0) spd_inv_body<256>(spdG, bs, spdGi, dsm);
    return;
  }
  int* tile = reinterpret_cast<int*>(dsm);  // 64 x kTileP
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.y * 16 * NCT;
  const int kb = blockIdx.z * kspan, ke = kb + kspan < K ? kb + kspan : K;
  const int E = fx_exponent(rmax, sblk, h ? ehm : 0);
  const int sc = 30 - E < 126 ? (30 - E > -126 ? 30 - E : -126) : 126;  // scale 2^sc, a normal float
  const float fscale = ldexpf(1.0f, sc);
  const double dscale = ldexp(1.0, sc);
  // staging role: thread t loads tile rows t / 16 + 16 q, k columns 4 (t % 16) .. + 3
  const int srow = tid >> 4, scol = 4 * (tid & 15);
  v4i acc[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[ct][t] = (v4i){0, 0, 0, 0};
  float4 pre[4];
  float4 hpre = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fetch = [&](int k0) {
    const int k = k0 + scol;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = blockIdx.x * 64 + srow + 16 * q;
      pre[q] = (i < rows && k < ke) ? *reinterpret_cast<const float4*>(R + (size_t)i * ldr + k)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (h && k < ke)  // the caller's weights: scalar loads, each inside [0, K)
      hpre = make_float4(h[k], k + 1 < K ? h[k + 1] : 0.f, k + 2 < K ? h[k + 2] : 0.f, k + 3 < K ? h[k + 3] : 0.f);
  };
  if (kb < ke) fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += 64) {
    __syncthreads();  // the previous chunk's tile is consumed
    {
      const int k = k0 + scol;
      const float hv[4] = {hpre.x, hpre.y, hpre.z, hpre.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float xv[4] = {pre[q].x, pre[q].y, pre[q].z, pre[q].w};
        int nv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool in = k + e < ke;
          if (h) nv[e] = in ? __double2int_rn((double)xv[e] * (double)hv[e] * dscale) : 0;
          else nv[e] = in ? __float2int_rn(xv[e] * fscale) : 0;
        }
        *reinterpret_cast<int4*>(&tile[(srow + 16 * q) * kTileP + scol]) = make_int4(nv[0], nv[1], nv[2], nv[3]);
      }
    }
    __syncthreads();
    if (k0 + 64 < ke) fetch(k0 + 64);
    const int k = k0 + 16 * g;
    v4i tb[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = c0 + ct * 16 + lr;
      tb[ct] = (c < bs && k < ke) ? load16(T + (size_t)c * ldt + k) : (v4i){0, 0, 0, 0};
    }
    int nv[16];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int4 v = *reinterpret_cast<const int4*>(&tile[(wid * 16 + lr) * kTileP + 16 * g + 4 * p]);
      nv[4 * p] = v.x;
      nv[4 * p + 1] = v.y;
      nv[4 * p + 2] = v.z;
      nv[4 * p + 3] = v.w;
    }
    v4i da[4];
    fx_operands(nv, da);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[ct][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(tb[ct], da[t], acc[ct][t], 0, 0, 0);
  }
  // D = T x^T: lane l, register q holds component 4 g + q of the tile for row lr, so each store
  // instruction covers four components x 16 consecutive rows
  const double unit = ldexp(1.0, -sc);
  const bool split = gridDim.z > 1;
  const int r = blockIdx.x * 64 + wid * 16 + lr;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + ct * 16 + 4 * g + q;
      if (c < bs && r < rows) {
        const double v = ((double)acc[ct][0][q] + 256.0 * (double)acc[ct][1][q] + 65536.0 * (double)acc[ct][2][q] +
                          16777216.0 * (double)acc[ct][3][q]) * unit;
        double* o = out + (size_t)c * rows + r;
        if (split) atomicAdd(o, v);
        else *o = v;
      }
    }
  }
}

// out[c][j] (+)= sum_{i in this split} U[c][i] R[i][j]: components x columns of R.
// Workgroup: 64 columns (16 per wave) x 16 NCT components (blockIdx.y), K = m range blockIdx.z.
template <int NCT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) utr_i8_kernel(const float* R, int ldr, int m, int n, const int8_t* U, int ldu,
                                                     int bs, const unsigned* rmax, int sblk, int kspan, double* out,
                                                     const double* spdG, double* spdGi) {
  extern __shared__ __align__(16) char dsm[];
  if (spdG && blockIdx.x == gridDim.x - 1) {  // the extra column of workgroups: one inverts spdG
    if (blockIdx.y == 0 && blockIdx.z == 0) spd_inv_body<256>(spdG, bs, spdGi, dsm);
    return;
  }
  int* tile = reinterpret_cast<int*>(dsm);  // 64 x kTileQ
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const int j = blockIdx.x * 64 + wid * 16 + lr;  // column supplied by this lane
  const int c0 = blockIdx.y * 16 * NCT;
  const int kb = blockIdx.z * kspan, ke = kb + kspan < m ? kb + kspan : m;
  const int E = fx_exponent(rmax, sblk, 0);
  const int sc = 30 - E < 126 ? (30 - E > -126 ? 30 - E : -126) : 126;  // scale 2^sc, a normal float
  const float fscale = ldexpf(1.0f, sc);
  const bool jok = j < n;
  // staging role: thread t loads tile rows (k) t / 16 + 16 q, columns 4 (t % 16) .. + 3
  const int srow = tid >> 4, scol = 4 * (tid & 15), sj = blockIdx.x * 64 + scol;
  v4i acc[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[ct][t] = (v4i){0, 0, 0, 0};
  float4 pre[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = k0 + srow + 16 * q;
      pre[q] = (i < ke && sj < ldr) ? *reinterpret_cast<const float4*>(R + (size_t)i * ldr + sj)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (kb < ke) fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += 64) {
    __syncthreads();  // the previous chunk's tile is consumed
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // columns past n hold R's zero padding (or nothing: zero)
      int* trow = &tile[(srow + 16 * q) * kTileQ + scol];
      trow[0] = __float2int_rn(pre[q].x * fscale);
      trow[1] = __float2int_rn(pre[q].y * fscale);
      trow[2] = __float2int_rn(pre[q].z * fscale);
      trow[3] = __float2int_rn(pre[q].w * fscale);
    }
    __syncthreads();
    if (k0 + 64 < ke) fetch(k0 + 64);
    const int k = k0 + 16 * g;
    v4i ua[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = c0 + ct * 16 + lr;
      ua[ct] = (c < bs && k < ke) ? load16(U + (size_t)c * ldu + k) : (v4i){0, 0, 0, 0};
    }
    int nv[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) nv[t] = tile[(16 * g + t) * kTileQ + wid * 16 + lr];
    v4i db[4];
    fx_operands(nv, db);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[ct][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua[ct], db[t], acc[ct][t], 0, 0, 0);
  }
  const double unit = ldexp(1.0, -sc);
  const bool split = gridDim.z > 1;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + ct * 16 + 4 * g + q;
      if (c < bs && jok) {
        const double v = ((double)acc[ct][0][q] + 256.0 * (double)acc[ct][1][q] + 65536.0 * (double)acc[ct][2][q] +
                          16777216.0 * (double)acc[ct][3][q]) * unit;
        double* o = out + (size_t)c * n + j;
        if (split) atomicAdd(o, v);
        else *o = v;
      }
    }
  }
}

// G = T T^T for ternary rows T (bs x K, ld ldt, zero-padded to ldt): integer-exact.  One
// workgroup of 16 waves per lower 16 x 16 tile; the waves split K (four 64-wide chunks in flight
// per wave) and add their int32 sums in LDS in wave order.
__global__ void __launch_bounds__(1024) gram_i8_kernel(const int8_t* T, int ldt, int K, int bs, double* G) {
  __shared__ int red[16][256];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= (int)blockIdx.x) ++ti;
  const int tj = (int)blockIdx.x - ti * (ti + 1) / 2;
  const int ra = ti * 16 + lr, rb = tj * 16 + lr;
  const int nch = (K + 63) / 64;
  v4i acc = (v4i){0, 0, 0, 0};
  constexpr int CH = 8;  // chunks per wave and round, all their loads issued before the products
  for (int c0 = wid; c0 < nch; c0 += CH * 16) {
    v4i a[CH], b[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int k = (c0 + 16 * u) * 64 + 16 * g;
      const bool ok = c0 + 16 * u < nch && k < ldt;
      a[u] = (ok && ra < bs) ? load16(T + (size_t)ra * ldt + k) : (v4i){0, 0, 0, 0};
      b[u] = (ok && rb < bs) ? load16(T + (size_t)rb * ldt + k) : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u], acc, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wid][q * 64 + lane] = acc[q];
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int v = 0;
#pragma unroll
      for (int w2 = 0; w2 < 16; ++w2) v += red[w2][q * 64 + lane];
      const int r = ti * 16 + 4 * g + q, c = tj * 16 + lr;
      if (r < bs && c < bs) {
        G[(size_t)r * bs + c] = (double)v;
        G[(size_t)c * bs + r] = (double)v;
      }
    }
  }
}

// Column weights in fixed point: H_j = rint(h_j 2^(35 - EHm)) < 2^35 (h < 2^EHm), stored as five
// unsigned 7-bit digits hdig[t][j] (zero past n, up to the padded length ldv).
__global__ void __launch_bounds__(256) hdig_kernel(const float* h, int n, int ldv, int ehm, uint8_t* hdig) {
  for (int j = blockIdx.x * 256 + threadIdx.x; j < ldv; j += gridDim.x * 256) {
    const u64 H = j < n ? (u64)llrint(ldexp((double)h[j], kHDig * 7 - ehm)) : 0ull;
#pragma unroll
    for (int t = 0; t < kHDig; ++t) hdig[(size_t)t * ldv + j] = (uint8_t)((H >> (7 * t)) & 0x7Fu);
  }
}

// bytes of t (each 0, 1 or -1) times bytes of d (each 0..127), as signed bytes
__device__ __forceinline__ unsigned tmul_bytes(unsigned t, unsigned d) {
  const unsigned nz = (t & 0x01010101u) * 0xFFu;         // 0xFF where t != 0
  const unsigned ng = ((t >> 7) & 0x01010101u) * 0xFFu;  // 0xFF where t == -1
  const unsigned nd = (0x80808080u - d) ^ 0x80808080u;   // per-byte -d (no borrows: d <= 0x7F)
  return (d & nz & ~ng) | (nd & ng);
}

// G = T diag(h) T^T for ternary rows T with h in fixed point (hdig): sum_t 2^(7 t) T (T o dig_t)^T,
// each digit product exact in int32, recombined exactly in fp64, times 2^-(35 - EHm).  The only
// difference from the fp64 sum is the rounding of each h_j to the grid.  Workgroup: 16 waves on
// one lower 16 x 16 tile (blockIdx.x) and one of gridDim.y ranges of K; the waves add in LDS in
// wave order.  With several ranges each workgroup stores its partial tile, and the last one of the
// tile to arrive adds them in range order; every partial is an integer below 2^53 (in units of
// the grid), so the sums are exact and the result does not depend on the split.
__global__ void __launch_bounds__(1024) gram_w_i8_kernel(const int8_t* T, int ldt, int K, int bs, const uint8_t* hdig,
                                                         int ehm, double* G, double* gpart, unsigned* gcnt) {
  __shared__ double red[16][256];
  __shared__ unsigned last_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= (int)blockIdx.x) ++ti;
  const int tj = (int)blockIdx.x - ti * (ti + 1) / 2;
  const int ra = ti * 16 + lr, rb = tj * 16 + lr;
  const int nch = (K + 63) / 64, S = (int)gridDim.y, y = (int)blockIdx.y;
  const int cb = (int)((long long)nch * y / S), ce = (int)((long long)nch * (y + 1) / S);
  v4i acc[kHDig];
#pragma unroll
  for (int t = 0; t < kHDig; ++t) acc[t] = (v4i){0, 0, 0, 0};
  constexpr int CH = 3;  // chunks per wave and round, all their loads issued before the products
  for (int c0 = cb + wid; c0 < ce; c0 += CH * 16) {
    v4i a[CH], b[CH], d[CH][kHDig];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int k = (c0 + 16 * u) * 64 + 16 * g;
      const bool ok = c0 + 16 * u < ce && k < ldt;
      a[u] = (ok && ra < bs) ? load16(T + (size_t)ra * ldt + k) : (v4i){0, 0, 0, 0};
      b[u] = (ok && rb < bs) ? load16(T + (size_t)rb * ldt + k) : (v4i){0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < kHDig; ++t)
        d[u][t] = ok ? load16(reinterpret_cast<const int8_t*>(hdig) + (size_t)t * ldt + k) : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
#pragma unroll
      for (int t = 0; t < kHDig; ++t) {
        v4i bd;
#pragma unroll
        for (int q = 0; q < 4; ++q) bd[q] = (int)tmul_bytes((unsigned)b[u][q], (unsigned)d[u][t][q]);
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], bd, acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    double v = 0.0;
#pragma unroll
    for (int t = kHDig - 1; t >= 0; --t) v = v * 128.0 + (double)acc[t][q];
    red[wid][q * 64 + lane] = v;
  }
  __syncthreads();
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  if (wid == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w2 = 0; w2 < 16; ++w2) v[q] += red[w2][q * 64 + lane];
  }
  if (S > 1) {
    const int ntile = (int)gridDim.x;
    if (wid == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) st_dev(gpart + ((size_t)y * ntile + blockIdx.x) * 256 + q * 64 + lane, v[q]);
    }
    // the partials go through agent-coherent stores and loads (no L2 writeback or invalidate);
    // each store has completed before the arrival is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) last_s = add_dev(&gcnt[blockIdx.x], 1u) == (unsigned)(S - 1) ? 1u : 0u;
    __syncthreads();
    if (!last_s) return;
    if (wid == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = 0.0;
        for (int y2 = 0; y2 < S; ++y2) v[q] += ld_dev(gpart + ((size_t)y2 * ntile + blockIdx.x) * 256 + q * 64 + lane);
      }
    }
    if (tid == 0) st_dev(&gcnt[blockIdx.x], 0u);  // ready for the next launch
  }
  if (wid == 0) {
    const double unit = ldexp(1.0, ehm - kHDig * 7);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double x = v[q] * unit;
      const int r = ti * 16 + 4 * g + q, c = tj * 16 + lr;
      if (r < bs && c < bs) {
        G[(size_t)r * bs + c] = x;
        G[(size_t)c * bs + r] = x;
      }
    }
  }
}

__global__ void __launch_bounds__(256) zero_kernel(double* p, long long count) {
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < count; x += (long long)gridDim.x * 256) p[x] = 0.0;
}

// max |R| over the m x n residual into words[0..kMaxWords) (fp32 bits; the words start at zero)
__global__ void __launch_bounds__(256) rmax_kernel(const float* R, int ldr, int m, int n, unsigned* words) {
  __shared__ unsigned wm[4];
  unsigned mx = 0u;
  const long long total = (long long)m * n;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < total; x += (long long)gridDim.x * 256) {
    const int i = (int)(x / n), j = (int)(x - (long long)i * n);
    const unsigned b = __float_as_uint(R[(size_t)i * ldr + j]) & 0x7FFFFFFFu;
    mx = b > mx ? b : mx;
  }
  mx = wave_max_u32(mx);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = wm[0] > wm[1] ? wm[0] : wm[1];
    mx = wm[2] > mx ? wm[2] : mx;
    mx = wm[3] > mx ? wm[3] : mx;
    if (mx != 0u) atomicMax(words + blockIdx.x % kMaxWords, mx);
  }
}

// ---- inverse Cholesky factor of G + eps I, eps = 1e-6 trace(G) / bs, by one workgroup of NT
// threads.  The packed lower triangle (element e = i (i + 1) / 2 + k) lives in registers: slot q
// of thread t holds element q * NT + t.
//   1. Cholesky, right-looking: after step j every entry (i, k), k > j, has had L_ij L_kj
//      subtracted, so each entry sees its subtractions in ascending order (the column is scaled
//      by the reciprocal of the pivot: one division per step);
//   2. X = L^-1 in place, right-looking: at step t row t of X is finished (divided by L_tt) and
//      every later row i takes X_ik -= L_it X_tk for k <= t; entry (i, t) turns from L_it into
//      X_it = -L_it X_tt at that step, just after its last use as an L entry.
// Columns / rows broadcast through LDS are double-buffered by step parity, so two barriers per
// step suffice.  Writes Li = L^-1 (row-major, zeros above the diagonal).
template <int NT, int SLOTS>
__global__ void __launch_bounds__(NT) chol_inv_kernel(const double* G, int bs, double* Li) {
#pragma clang fp contract(off)
  __shared__ double colb[2][256];
  __shared__ double rowb[2][256];
  __shared__ double eps_s;
  const int tid = threadIdx.x;
  const int ne = bs * (bs + 1) / 2;
  if (tid == 0) {
    double tr = 0.0;
    for (int c = 0; c < bs; ++c) tr += G[(size_t)c * bs + c];
    eps_s = 1e-6 * tr / (double)bs;
  }
  for (int x = tid; x < bs * bs; x += NT) {
    const int i = x / bs, k = x - i * bs;
    if (k > i) Li[x] = 0.0;
  }
  __syncthreads();
  const double eps = eps_s;
  double a[SLOTS];
  int ik[SLOTS];  // (i << 16) | k, or -1 for an unused slot
#pragma unroll
  for (int q = 0; q < SLOTS; ++q) {
    const int e = q * NT + tid;
    if (e < ne) {
      int i = (int)((sqrt(8.0 * (double)e + 1.0) - 1.0) * 0.5);
      while ((i + 1) * (i + 2) / 2 <= e) ++i;
      while (i * (i + 1) / 2 > e) --i;
      const int k = e - i * (i + 1) / 2;
      ik[q] = (i << 16) | k;
      a[q] = G[(size_t)i * bs + k] + (i == k ? eps : 0.0);
    } else {
      ik[q] = -1;
      a[q] = 0.0;
    }
  }
  // 1. Cholesky
  for (int j = 0; j < bs; ++j) {
    double* col = colb[j & 1];
#pragma unroll
    for (int q = 0; q < SLOTS; ++q)
      if (ik[q] == ((j << 16) | j)) {
        a[q] = a[q] > 0.0 ? sqrt(a[q]) : 0.0;
        col[j] = a[q];
      }
    __syncthreads();
    const double ljj = col[j];
    const double rj = ljj > 0.0 ? 1.0 / ljj : 0.0;  // one division per step, then products
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      if (ik[q] >= 0 && k == j && i > j) {
        a[q] = a[q] * rj;
        col[i] = a[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      if (ik[q] >= 0 && k > j) a[q] -= col[i] * col[k];
    }
  }
  __syncthreads();
  // 2. X = L^-1
  for (int t = 0; t < bs; ++t) {
    double* lc = colb[t & 1];
    double* xr = rowb[t & 1];
#pragma unroll
    for (int q = 0; q < SLOTS; ++q)
      if (ik[q] == ((t << 16) | t)) lc[t] = a[q];  // L_tt
    __syncthreads();
    const double ltt = lc[t];
    const double rt = ltt > 0.0 ? 1.0 / ltt : 0.0;
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
      if (ik[q] < 0) continue;
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      if (i == t) {  // row t of X: finished
        a[q] = k == t ? rt : a[q] * rt;
        xr[k] = a[q];
      } else if (k == t && i > t) {
        lc[i] = a[q];  // L_it
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
      if (ik[q] < 0) continue;
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      if (i > t && k < t) a[q] -= lc[i] * xr[k];
      else if (i > t && k == t) a[q] = 0.0 - lc[i] * xr[t];
    }
  }
#pragma unroll
  for (int q = 0; q < SLOTS; ++q)
    if (ik[q] >= 0) {
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      Li[(size_t)i * bs + k] = a[q];
    }
}

// ---- Gi = (G + eps I)^-1 for bs <= 128, eps = 1e-6 trace(G) / bs (the regularised Gram of the
// pages' Eq. 3), by a blocked Cholesky factorisation on 16 x 16 tiles, the block inverse of the
// factor and the product X^T X (X = L^-1), all in LDS.  The tile products run on fp64 MFMA; the
// 16 x 16 diagonal blocks are factored and inverted by one wave with a row per lane.  Pivots that
// are not positive give zero rows, as in a plain Cholesky solve.  The matrix is padded to a
// multiple of 16 with an identity block, which keeps it block diagonal and leaves the real part of
// the inverse unchanged.  One workgroup; about 4 (nb - 1) + 2 barriers for nb tiles per side.
constexpr int kSpdMax = 128;
constexpr int kSpdFused = 64;  // largest b whose inverse runs inside the contraction launch
__host__ __device__ inline size_t spd_lds_bytes(int bs) {
  const int bp = (bs + 15) & ~15, ld = bp + 1;
  return 8 * ((size_t)bp * ld + (size_t)(bp / 16) * 256 + 16);
}
// NT threads share the tile products (256 for b <= 64, where four waves cover the few tiles and
// the body fits a contraction's workgroup; 1024 above); wave 0 factors the diagonal blocks.
// The body runs in its own launch (spd_inv_kernel) or as one extra workgroup of a residual
// contraction (rv_i8_kernel, utr_i8_kernel), which overlaps the two without a second stream.
template <int NT>
__device__ __forceinline__ void spd_inv_body(const double* G, int bs, double* Gi, char* smem) {
  constexpr int NWV = NT / 64;
  const int bp = (bs + 15) & ~15, nb = bp / 16, ld = bp + 1;
  double* A = reinterpret_cast<double*>(smem);  // bp x ld
  double* Dg = A + (size_t)bp * ld;             // nb diagonal-block inverses, 16 x 16 row-major
  double* misc = Dg + (size_t)nb * 256;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;  // MFMA operand coordinates: row / column lr, k 4 s + lk
  if (wid == 0) {
    double tr = 0.0;
    for (int c = lane; c < bs; c += 64) tr += G[(size_t)c * bs + c];
    tr = wave_sum_f64(tr);
    if (lane == 0) misc[0] = 1e-6 * tr / (double)bs;
  }
  __syncthreads();
  const double eps = misc[0];
  for (int x0 = 0; x0 < bp * bp; x0 += 8 * NT) {  // 8 loads in flight per thread, then the stores
    double v8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int x = x0 + tid + NT * q, i = x / bp, j = x - i * bp;
      if (x < bp * bp && i < bs && j < bs) v8[q] = G[(size_t)i * bs + j] + (i == j ? eps : 0.0);
      else v8[q] = i == j ? 1.0 : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int x = x0 + tid + NT * q, i = x / bp, j = x - i * bp;
      if (x < bp * bp) A[(size_t)i * ld + j] = v8[q];
    }
  }
  __syncthreads();
  auto at = [&](int bi, int bj) -> double* { return A + (size_t)(16 * bi) * ld + 16 * bj; };
  // operand "row lr, column 4 s + lk" of a row-major 16 x 16 tile (P of P Q^T, or Q^T's Q)
  auto opr = [&](const double* t, int tld, int sl) -> double { return t[(size_t)lr * tld + 4 * sl + lk]; };
  // operand "row 4 s + lk, column lr" (B of P Q with Q row-major)
  auto opc = [&](const double* t, int tld, int sl) -> double { return t[(size_t)(4 * sl + lk) * tld + lr]; };
  // ---------------- Cholesky, one 16-column panel at a time.  Look-ahead: after the panel of p,
  // wave 0 updates diagonal block p + 1 first and factors it while the other waves finish the
  // trailing update, so the serial 16 x 16 factorisation leaves the critical path.
  // 16 x 16 diagonal block: Cholesky factor and its inverse by wave 0, lane r (mod 16) holding row r
  auto factor_diag = [&](int p) {  // wave 0
    const int r = lr;
    double* T = at(p, p);
    double a[16], x[16], rk[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) a[c] = T[(size_t)r * ld + c];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const double piv = readlane_f64(a[k], k);
      const double lkk = piv > 0.0 ? sqrt(piv) : 0.0;
      const double rr = lkk > 0.0 ? 1.0 / lkk : 0.0;
      rk[k] = rr;
      a[k] = r > k ? a[k] * rr : (r == k ? lkk : a[k]);
#pragma unroll
      for (int j = k + 1; j < 16; ++j) {
        const double ljk = readlane_f64(a[k], j);
        a[j] = fma(-a[k], ljk, a[j]);  // meaningful for rows r >= j
      }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) x[c] = 0.0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      // row t of X = L^-1 is finished: x[c] held -sum_{j<t} L_tj X_jc (one scale per lane
      // instead of a select per entry)
      const double sc = r == t ? rk[t] : 1.0;
#pragma unroll
      for (int c = 0; c < t; ++c) x[c] *= sc;
      x[t] = r == t ? rk[t] : x[t];
      // later rows r > t take -L_rt X_tc; the multiplier is zero for rows r <= t
      const double lrt = r > t ? a[t] : 0.0;
#pragma unroll
      for (int c = 0; c <= t; ++c) x[c] = fma(-lrt, readlane_f64(x[c], t), x[c]);
    }
    if (lane < 16) {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        T[(size_t)r * ld + c] = c <= r ? a[c] : 0.0;
        Dg[p * 256 + r * 16 + c] = c <= r ? x[c] : 0.0;
      }
    }
  };
  auto trailing_tile = [&](int p, int t) {  // A_ij -= L_ip L_jp^T, tile t of the p-th update
    int ii = 0;
    while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
    const int jj = t - ii * (ii + 1) / 2;
    const int i = p + 1 + ii, j = p + 1 + jj;
    double* T = at(i, j);
    const double* Li_ = at(i, p);
    const double* Lj_ = at(j, p);
    dbl4 acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = T[(size_t)(4 * q + lk) * ld + lr];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(-opr(Li_, ld, sl), opr(Lj_, ld, sl), acc, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) T[(size_t)(4 * q + lk) * ld + lr] = acc[q];
  };
  if (wid == 0) factor_diag(0);
  __syncthreads();
  for (int p = 0; p < nb; ++p) {
    // panel below: L_ip = A_ip D_p^T (in place)
    for (int i = p + 1 + wid; i < nb; i += NWV) {
      double* T = at(i, p);
      dbl4 acc = (dbl4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(opr(T, ld, sl), opr(Dg + p * 256, 16, sl), acc, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) T[(size_t)(4 * q + lk) * ld + lr] = acc[q];
    }
    __syncthreads();
    if (p + 1 == nb) break;
    // trailing update; tile 0 is diagonal block p + 1
    const int rem = nb - 1 - p, ntile = rem * (rem + 1) / 2;
    if (wid == 0) {
      trailing_tile(p, 0);
      factor_diag(p + 1);
    } else {
      for (int t = wid; t < ntile; t += NWV - 1) trailing_tile(p, t);
    }
    __syncthreads();
  }
  // ---------------- X = L^-1 by block rows: X_ii = D_i, X_ij = -D_i sum_{k=j}^{i-1} L_ik X_kj.
  // X_ij (i > j) is stored transposed in the free upper block (j, i) of A.
  for (int i = 1; i < nb; ++i) {
    for (int j = wid; j < i; j += NWV) {
      dbl4 sacc = (dbl4){0.0, 0.0, 0.0, 0.0};
      for (int k = j; k < i; ++k) {
        const double* P = at(i, k);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          // X_kj[4 s + lk][lr]: D_j for k == j, else transposed storage in block (j, k)
          const double bq = k == j ? opc(Dg + j * 256, 16, sl) : opr(at(j, k), ld, sl);
          sacc = __builtin_amdgcn_mfma_f64_16x16x4f64(opr(P, ld, sl), bq, sacc, 0, 0, 0);
        }
      }
      dbl4 xacc = (dbl4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)  // an MFMA result in lane l, register s is operand B[4 s + lk][lr]
        xacc = __builtin_amdgcn_mfma_f64_16x16x4f64(-opr(Dg + i * 256, 16, sl), sacc[sl], xacc, 0, 0, 0);
      double* T = at(j, i);
#pragma unroll
      for (int q = 0; q < 4; ++q) T[(size_t)lr * ld + 4 * q + lk] = xacc[q];
    }
    __syncthreads();
  }
  // ---------------- Gi = X^T X: tile (i, j), i >= j, is sum_{k >= i} X_ki^T X_kj
  for (int t = wid; t < nb * (nb + 1) / 2; t += NWV) {
    int i = 0;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    const int j = t - i * (i + 1) / 2;
    dbl4 acc = (dbl4){0.0, 0.0, 0.0, 0.0};
    for (int k = i; k < nb; ++k) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        // X_ki[4 s + lk][lr] and X_kj[4 s + lk][lr]
        const double av = k == i ? opc(Dg + i * 256, 16, sl) : opr(at(i, k), ld, sl);
        const double bv = k == j ? opc(Dg + j * 256, 16, sl) : opr(at(j, k), ld, sl);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * q + lk, c = 16 * j + lr;
      if (r < bs && c < bs) {
        Gi[(size_t)r * bs + c] = acc[q];
        if (i != j) Gi[(size_t)c * bs + r] = acc[q];
      }
    }
  }
}

template <int NT>
__global__ void __launch_bounds__(NT) spd_inv_kernel(const double* G, int bs, double* Gi) {
  extern __shared__ __align__(16) char smem[];
  spd_inv_body<NT>(G, bs, Gi, smem);
}

// ---- out (bs x ncols) = op(A) B with A bs x bs (op: A or A^T), B bs x ncols, fp64 MFMA, K = bs.
// Workgroup: 64 columns; wave w: columns 16 w .. 16 w + 15, all bs rows (NRT tiles of 16).
template <int NRT, bool TA>
__global__ void __launch_bounds__(256) apply_kernel(const double* __restrict__ A, int bs, const double* Bm,
                                                    double* out, int ncols) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = blockIdx.x * 64 + wid * 16 + (lane & 15);
  const bool okc = col < ncols;
  dbl4 acc[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t] = (dbl4){0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < bs; k0 += 4) {
    const int k = k0 + (lane >> 4);
    const double bv = (k < bs && okc) ? Bm[(size_t)k * ncols + col] : 0.0;
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      const int r = t * 16 + (lane & 15);
      double av = 0.0;
      if (r < bs && k < bs) av = TA ? A[(size_t)k * bs + r] : A[(size_t)r * bs + k];
      acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[t], 0, 0, 0);
    }
  }
  if (okc) {
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = t * 16 + (lane >> 4) + 4 * q;
        if (r < bs) out[(size_t)r * ncols + col] = acc[t][q];
      }
  }
}

// ---- out (bs x ncols) = A B for bs <= kSpdMax (A bs x bs, B bs x ncols), fp64 MFMA, K = bs.
// Workgroup: NCT 16-column strips of B (staged in LDS) x all bs rows; wave w takes the row tiles
// w, w + 4, ...  Every A operand of the whole K range (NKS k-steps of 4) is loaded into registers
// before the strips are staged, so the workgroup waits for one round of loads, then runs its MFMAs
// back to back, each A operand serving the NCT strips.
template <int NRW, int NKS, int NCT>
__global__ void __launch_bounds__(256) apply_strip_kernel(const double* __restrict__ A, int bs, const double* Bm,
                                                          double* out, int ncols) {
  __shared__ double Bs[kSpdMax][16 * NCT];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int col0 = blockIdx.x * 16 * NCT;
  const int ntiles = (bs + 15) / 16;
  dbl4 acc[NRW][NCT];
  double av[NKS][NRW];
#pragma unroll
  for (int u = 0; u < NRW; ++u) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[u][ct] = (dbl4){0.0, 0.0, 0.0, 0.0};
    const int r = (wid + 4 * u) * 16 + lr;
    const bool rok = wid + 4 * u < ntiles && r < bs;
    const double* ap = A + (size_t)(rok ? r : 0) * bs;
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      const int k = 4 * st + lk;
      av[st][u] = (rok && k < bs) ? ap[k] : 0.0;
    }
  }
  // the strips: (4 NKS) x 16 NCT values, NKS NCT / 4 per thread, all loads issued before the
  // first store
  constexpr int NB = NKS * NCT / 4, W = 16 * NCT;
  double bl[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int x = tid + 256 * i, k = x / W, c = x % W;
    bl[i] = (k < bs && col0 + c < ncols) ? Bm[(size_t)k * ncols + col0 + c] : 0.0;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int x = tid + 256 * i;
    Bs[x / W][x % W] = bl[i];
  }
  __syncthreads();
#pragma unroll
  for (int st = 0; st < NKS; ++st) {
    const int k = 4 * st + lk;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const double bv = k < bs ? Bs[k][16 * ct + lr] : 0.0;
#pragma unroll
      for (int u = 0; u < NRW; ++u)
        acc[u][ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[st][u], bv, acc[u][ct], 0, 0, 0);
    }
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = col0 + 16 * ct + lr;
    if (col >= ncols) continue;
#pragma unroll
    for (int u = 0; u < NRW; ++u) {
      if (wid + 4 * u >= ntiles) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = (wid + 4 * u) * 16 + lk + 4 * q;
        if (r < bs) out[(size_t)r * ncols + col] = acc[u][ct][q];
      }
    }
  }
}

// ---- one workgroup per component row: T[c] = T_tau(fp32(X[c]); h) -----------------------------
template <bool W, int NT>
// Z0 (nullable): row c of the next split-K contraction's output is cleared here (zlen doubles),
// which saves that contraction a separate clearing launch.  Md (nullable): Md[c] = T[c] . Yd[c]
// over the L entries (the last U-step's u_c^T Q_c for the scales), fixed reduction order.
__global__ void __launch_bounds__(NT) select_rows_kernel(const double* X, int L, int ldT, float tau,
                                                          const float* h, int EHm, int8_t* T, double* PHC,
                                                          int* flags, int flag_empty, double* Z0, int zlen,
                                                          const double* Yd, double* Md) {
  __shared__ SelScratchT<W> s;
  __shared__ double red[NT / 64];
  const int c = blockIdx.x;
  const double* x = X + (size_t)c * L;
  if (Z0)
    for (int j = threadIdx.x; j < zlen; j += NT) Z0[(size_t)c * zlen + j] = 0.0;
  if (flags[0]) {  // residual is zero: nothing to select
    for (int j = threadIdx.x; j < ldT; j += NT) T[(size_t)c * ldT + j] = 0;
    return;
  }
  const SelResult r = ternary_select<NT, W>(x, h, L, tau, EHm, s);
  double dot = 0.0;
  for (int j = threadIdx.x; j < ldT; j += NT) {  // the padding [L, ldT) stays zero
    const float xv = j < L ? (float)x[j] : 0.0f;
    const int8_t t = selected(xv, r) ? (xv > 0.0f ? (int8_t)1 : (int8_t)-1) : (int8_t)0;
    T[(size_t)c * ldT + j] = t;
    if (Md && t) dot += (double)t * Yd[(size_t)c * L + j];
  }
  if (Md) {
    dot = wave_sum_f64(dot);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dot;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
      for (int w = 0; w < NT / 64; ++w) t += red[w];
      Md[c] = t;
    }
  }
  if (threadIdx.x == 0) {
    PHC[3 * c + 0] = r.P;
    PHC[3 * c + 1] = r.H;
    PHC[3 * c + 2] = (double)r.count;
    if (flag_empty && r.count == 0u) atomicAdd(&flags[1], 1);
  }
}

// ---- sketch columns that came out empty start from the largest |R_ij| (smallest row-major index
// on ties) in a row not used yet by this block; one workgroup, and it only does work when such a
// column exists (the sketch of a nonzero residual is almost never empty) ----
__global__ void __launch_bounds__(512) fallback_kernel(const float* R, int ldr, int m, int n, int bs, int8_t* Ut,
                                                       int ldu, const double* PHC, int* flags, int* used) {
  __shared__ float bv[8];
  __shared__ long long bi[8];
  if (flags[1] == 0 || flags[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const long long none = 0x7fffffffffffffffll;
  for (int i = tid; i < m; i += 512) used[i] = 0;
  __syncthreads();
  for (int c = 0; c < bs; ++c) {
    if (PHC[3 * c + 2] != 0.0) continue;
    float best = 0.0f;
    long long bidx = none;
    for (long long x = tid; x < (long long)m * n; x += 512) {
      const int i = (int)(x / n), j = (int)(x - (long long)i * n);
      if (used[i]) continue;
      const float v = fabsf(R[(size_t)i * ldr + j]);
      if (v > best) {
        best = v;
        bidx = x;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float b2 = __shfl_xor(best, o);
      const long long i2 = __shfl_xor(bidx, o);
      if (b2 > best || (b2 == best && i2 < bidx)) {
        best = b2;
        bidx = i2;
      }
    }
    if (lane == 0) {
      bv[wid] = best;
      bi[wid] = bidx;
    }
    __syncthreads();
    float bb = 0.0f;
    long long bix = none;
    for (int w = 0; w < 8; ++w)
      if (bv[w] > bb || (bv[w] == bb && bi[w] < bix)) {
        bb = bv[w];
        bix = bi[w];
      }
    if (bb > 0.0f) {  // else every row holding a nonzero entry is taken: the column stays empty
      const int r = (int)(bix / n);
      for (int i = tid; i < m; i += 512) Ut[(size_t)c * ldu + i] = (i == r) ? (int8_t)1 : (int8_t)0;
      if (tid == 0) {
        used[r] = 1;
        flags[2] += 1;
      }
    }
    __syncthreads();
  }
}

// Rows of GU and GV staged at a time by scales_kernel: 96 KB of dynamic LDS at most.
__host__ __device__ inline int scales_window(int bs) {
  const int w = (96 * 1024) / (16 * bs);
  return w < bs ? w : bs;
}
__host__ inline size_t scales_lds_bytes(int bs) { return (size_t)16 * scales_window(bs) * bs; }

// ---- scales and energy: one workgroup; one wave walks, lane l owning components l + 64 s for
// the NS = ceil(bs / 64) slots s.  The sequential scale of each component against the residual
// left by the earlier ones of the block:
//   p_t = Md_t - sum_{c < t} d_c (u_t . u_c) (v_c^T H v_t),   d_t = fp32(p_t / q_t),
// the subtractions applied in ascending c (as the textbook loop does); the Gram of U is exactly
// symmetric (integer entries), so row c is read for column c.
// With target > 0 the energy walk ends at the first component whose energy reaches the target:
// the later components of the block get d = 0 (not applied, emitted as zero) and the energy of
// the last kept one.
template <int NS>
__global__ void __launch_bounds__(256) scales_kernel(const double* Md, const double* GU, const double* GV, int bs,
                                                     int k0, int T, float* dvec, float* D, double* energy,
                                                     double* st, int* flags, u64* stats, double target) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  if (tid == 0) {
    if (flags[0]) {
      // zero components (none counted when A = 0); with a target only the first is fitted
      if (st[1] > 0.0) stats[3] += (u64)(target > 0.0 ? 1 : bs);
    } else {
      stats[0] += (u64)(2 * T);   // ALS half-steps
      stats[2] += (u64)flags[2];  // sketch columns started from the largest entry
    }
  }
  if (flags[0]) {
    if (tid < bs) {
      dvec[tid] = 0.0f;
      D[k0 + tid] = 0.0f;
      energy[k0 + tid] = 1.0;
    }
    if (tid == 0 && target > 0.0) {
      flags[3] = 1;
      stats[5] = (u64)(k0 + 1);
    }
    return;
  }
  // Component c's running value comes to every lane by readlane, so no workgroup barrier per
  // step.  The rows of GU and GV the walk reads are staged in LDS by the whole workgroup, `wr`
  // rows at a time, so that it waits on no global load.
  extern __shared__ __align__(16) double sg[];  // wr x bs of GU, then wr x bs of GV
  const int wr = scales_window(bs);
  double* sgu = sg;
  double* sgv = sg + (size_t)wr * bs;
  const int lane = tid & 63;
  double acc[NS], q[NS];
  if (tid < 64) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int c2 = lane + 64 * sl;
      const bool o = c2 < bs;
      acc[sl] = o ? Md[c2] : 0.0;
      q[sl] = o ? GU[(size_t)c2 * bs + c2] * GV[(size_t)c2 * bs + c2] : 0.0;
    }
  }
  for (int w0 = 0; w0 < bs; w0 += wr) {
    const int rows = bs - w0 < wr ? bs - w0 : wr;
    __syncthreads();  // the previous window is consumed
    const int tot = rows * bs;
    for (int x0 = 0; x0 < tot; x0 += 8 * 256) {  // 16 loads in flight per thread, then the stores
      double u8[8], v8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int x = x0 + tid + 256 * q;
        u8[q] = x < tot ? GU[(size_t)w0 * bs + x] : 0.0;
        v8[q] = x < tot ? GV[(size_t)w0 * bs + x] : 0.0;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int x = x0 + tid + 256 * q;
        if (x < tot) {
          sgu[x] = u8[q];
          sgv[x] = v8[q];
        }
      }
    }
    __syncthreads();
    if (tid < 64) {
#pragma unroll
      for (int sc = 0; sc < NS; ++sc) {  // the slot of the current component, static
        const int cb = w0 > 64 * sc ? w0 : 64 * sc;
        const int ce = w0 + rows < 64 * sc + 64 ? w0 + rows : 64 * sc + 64;
        for (int c = cb; c < ce; ++c) {
          const double* gur = sgu + (size_t)(c - w0) * bs;
          const double* gvr = sgv + (size_t)(c - w0) * bs;
          double gu[NS], gv[NS];
#pragma unroll
          for (int sl = sc; sl < NS; ++sl) {  // read before the scale: the reads overlap the division
            const int c2 = lane + 64 * sl;
            const int ci = c2 < bs ? c2 : bs - 1;
            gu[sl] = gur[ci];
            gv[sl] = gvr[ci];
          }
          const double ac = readlane_f64(acc[sc], c & 63), qc = readlane_f64(q[sc], c & 63);
          const double dd = (double)(qc > 0.0 ? (float)(ac / qc) : 0.0f);
#pragma unroll
          for (int sl = sc; sl < NS; ++sl) {
            const int c2 = lane + 64 * sl;
            const double t = dd * gu[sl] * gv[sl];
            acc[sl] = (c2 > c && c2 < bs) ? acc[sl] - t : acc[sl];
          }
        }
      }
    }
  }
  if (tid >= 64) return;
  // acc now holds each component's final p (no later step touches it), so the owner lane forms
  // its scale again (the same operands, the same value) and the term 2 d p - d^2 q it removes
  // from the residual energy.  The energy chain E_c = E_{c-1} - term_c runs in ascending c.
  float dl[NS];
  double tl[NS], el[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    dl[sl] = q[sl] > 0.0 ? (float)(acc[sl] / q[sl]) : 0.0f;
    const double dd = (double)dl[sl];
    tl[sl] = 2.0 * dd * acc[sl] - dd * dd * q[sl];
    el[sl] = 0.0;
  }
  double E = st[0];
  const double E0 = st[1];
  // (a lane past bs holds the term +0, which leaves E as it is, so every slot runs 64 steps)
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
#pragma unroll 16
    for (int lc = 0; lc < 64; ++lc) {
      E = E - readlane_f64(tl[sl], lc);
      el[sl] = lane == lc ? E : el[sl];
    }
  }
  // energies and the first component that reaches the target
  int first = bs;
  double en[NS];
#pragma unroll
  for (int sl = NS - 1; sl >= 0; --sl) {
    en[sl] = 1.0 - el[sl] / E0;
    const u64 hit = __ballot(target > 0.0 && lane + 64 * sl < bs && en[sl] >= target);
    if (hit) first = 64 * sl + __ffsll((unsigned long long)hit) - 1;
  }
  const int kept = first < bs ? first + 1 : bs;
  const int ks = (kept - 1) >> 6, kl = (kept - 1) & 63;
  double e_last = 0.0, E_last = 0.0;
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
    if (sl == ks) {
      e_last = readlane_f64(en[sl], kl);
      E_last = readlane_f64(el[sl], kl);
    }
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int c = lane + 64 * sl;
    if (c < bs) {
      energy[k0 + c] = c < kept ? en[sl] : e_last;
      const float d = c < kept ? dl[sl] : 0.0f;
      dvec[c] = d;
      D[k0 + c] = d;
    }
  }
  if (lane == 0) {
    if (first < bs) {
      flags[3] = 1;
      stats[5] = (u64)(k0 + kept);
    }
    st[0] = E_last;
    flags[4] = kept;
  }
}

// ---- update: R <- fl32(R - U diag(d) V^T), fp64 MFMA with K = bs ----------------------------
// Tile 64 x 64 of R; wave w owns rows 16w..16w+15 and four 16-column strips.
// A[i][k] = d_k U[k][i], B[k][j] = V[k][j].  The operands are staged 64 components at a time
// (10 KB of LDS), so that many workgroups share a CU: the kernel streams R once each way and
// needs many loads in flight.  Each lane's 16 entries of R are loaded before anything else
// (the dead-residual flag included), in the MFMA output layout: lane l of wave w holds rows
// 16 w + l / 16 + 4 r, column 16 t + l % 16 of strip t.  Entries whose product is zero are not
// written back.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) update_kernel(float* R, int ldr, int m, int n, const int8_t* Ut, int ldu,
                                                     const int8_t* Vt, int ldv, const float* dvec, int bs,
                                                     const int* flags, unsigned* rmax_next) {
  __shared__ __align__(16) int8_t Us[64][64 + 16];
  __shared__ __align__(16) int8_t Vs[64][64 + 16];
  __shared__ float ds[64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  float rv[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wid * 16 + (lane >> 4) + 4 * r;
      rv[t][r] = (i < m && j < n) ? R[(size_t)i * ldr + j] : 0.0f;
    }
  }
  if (flags[0]) return;
  const int bs4 = (bs + 3) & ~3;
  dbl4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (dbl4){0.0, 0.0, 0.0, 0.0};
  for (int kc = 0; kc < bs4; kc += 64) {
    const int kn = bs4 - kc < 64 ? bs4 - kc : 64;
    if (kc > 0) __syncthreads();  // the previous chunk's operands are consumed
    // 16-byte pieces: rows of Ut / Vt are zero-padded to a multiple of 16, and i0, j0 are
    // multiples of 64, so a piece is either inside the padded row or past it
    {
      const int x = tid, c = x >> 2, q = (x & 3) * 16, cg = kc + c;
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      if (c < kn) {
        *reinterpret_cast<uint4*>(&Us[c][q]) =
            (cg < bs && i0 + q < ldu) ? *reinterpret_cast<const uint4*>(Ut + (size_t)cg * ldu + i0 + q) : z;
        *reinterpret_cast<uint4*>(&Vs[c][q]) =
            (cg < bs && j0 + q < ldv) ? *reinterpret_cast<const uint4*>(Vt + (size_t)cg * ldv + j0 + q) : z;
      }
    }
    if (tid < kn) ds[tid] = kc + tid < bs ? dvec[kc + tid] : 0.0f;
    __syncthreads();
    for (int k0 = 0; k0 < kn; k0 += 4) {
      const int k = k0 + (lane >> 4);
      const double a = (double)ds[k] * (double)Us[k][wid * 16 + (lane & 15)];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const double bv = (double)Vs[k][t * 16 + (lane & 15)];
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc[t], 0, 0, 0);
      }
    }
  }
  unsigned mx = 0u;  // largest |R| of the tile after the update (fp32 bits)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wid * 16 + (lane >> 4) + 4 * r;
      if (i < m && j < n) {
        const double sv = acc[t][r];
        float x = rv[t][r];
        if (sv != 0.0) {
          x = (float)((double)x - sv);
          R[(size_t)i * ldr + j] = x;
        }
        const unsigned b = __float_as_uint(x) & 0x7FFFFFFFu;
        mx = b > mx ? b : mx;
      }
    }
  }
  __shared__ unsigned wm[4];
  mx = wave_max_u32(mx);
  if (lane == 0) wm[wid] = mx;
  __syncthreads();
  if (tid == 0) {
    mx = wm[0] > wm[1] ? wm[0] : wm[1];
    mx = wm[2] > mx ? wm[2] : mx;
    mx = wm[3] > mx ? wm[3] : mx;
    if (mx != 0u) atomicMax(rmax_next + (blockIdx.x + blockIdx.y) % kMaxWords, mx);
  }
}

// ---- emit: pack the block's components into B and C rows ----------------------------------
__global__ void __launch_bounds__(256) emit_kernel(const int8_t* Ut, int ldu, const int8_t* Vt, int ldv, int m, int n,
                                                   int bs, int k0, uint32_t* Bp, uint32_t* Cp, const int* flags) {
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  const bool dead = flags[0] != 0;
  const int kept = flags[4];  // components past an energy-target stop are emitted as zero
  const long long totB = (long long)bs * wm, totC = (long long)bs * wn;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < totB + totC; x += (long long)gridDim.x * 256) {
    const bool isB = x < totB;
    const long long y = isB ? x : x - totB;
    const int words = isB ? wm : wn, len = isB ? m : n;
    const int c = (int)(y / words), w = (int)(y - (long long)c * words);
    const int8_t* src = isB ? Ut + (size_t)c * ldu : Vt + (size_t)c * ldv;
    unsigned word = 0u;
    if (!dead && c < kept)
      for (int q = 0; q < 16; ++q) {
        const int i = w * 16 + q;
        if (i < len) word |= tcode(src[i]) << (2 * q);
      }
    (isB ? Bp : Cp)[(size_t)(k0 + c) * words + w] = word;
  }
}

// components [from, k) after an energy-target stop: zero codes and scale, the energy of
// component from - 1 held
__global__ void __launch_bounds__(256) stop_fill_kernel(uint32_t* Bp, uint32_t* Cp, float* D, double* energy, int m,
                                                        int n, int from, int k) {
  const long long wm = (m + 15) / 16, wn = (n + 15) / 16;
  const long long nb = (long long)(k - from) * wm, nc = (long long)(k - from) * wn;
  const double held = energy[from - 1];
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < nb + nc + (k - from); x += (long long)gridDim.x * 256) {
    if (x < nb) Bp[(size_t)from * wm + x] = 0u;
    else if (x < nb + nc) Cp[(size_t)from * wn + (x - nb)] = 0u;
    else {
      const int c = from + (int)(x - nb - nc);
      D[c] = 0.0f;
      energy[c] = held;
    }
  }
}

// ---- refinement sweeps: refit block [k0, k0 + bs) from its previous factors ----------------
// Unpack the block's codes into Ut / Vt (zero padded), dvec = -D (its add-back through the update
// kernel), reset the per-block flags and clear the residual-max slot the add-back writes.
// (restore = true: the same unpacking, done only when the refit was discarded, flags[5].)
__global__ void __launch_bounds__(256) refit_load_kernel(const uint32_t* Bp, const uint32_t* Cp, const float* D, int m,
                                                         int n, int k0, int bs, int8_t* Ut, int ldu, int8_t* Vt,
                                                         int ldv, float* dvec, float* dold, double* st, int* flags,
                                                         unsigned* rmax_slot, bool restore, double* Z0,
                                                         long long zcount) {
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  if (restore) {
    if (!flags[5]) return;
  } else {
    for (long long x = blockIdx.x * 256ll + threadIdx.x; x < zcount; x += (long long)gridDim.x * 256) Z0[x] = 0.0;
  }
  if (!restore && blockIdx.x == 0) {
    if (threadIdx.x < kMaxWords) rmax_slot[threadIdx.x] = 0u;
    if (threadIdx.x < bs) {
      dvec[threadIdx.x] = -D[k0 + threadIdx.x];
      dold[threadIdx.x] = D[k0 + threadIdx.x];
    }
    if (threadIdx.x == 0) {
      flags[0] = 0;
      flags[1] = 0;
      flags[2] = 0;
      flags[5] = 0;
      st[2] = st[0];  // the energy before the add-back
    }
  }
  const long long tu = (long long)bs * ldu, tv = (long long)bs * ldv;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < tu + tv; x += (long long)gridDim.x * 256) {
    const bool isU = x < tu;
    const long long y = isU ? x : x - tu;
    const int ld = isU ? ldu : ldv, len = isU ? m : n, words = isU ? wm : wn;
    const int c = (int)(y / ld), i = (int)(y - (long long)c * ld);
    int8_t t = 0;
    if (i < len) {
      const unsigned code = ((isU ? Bp : Cp)[(size_t)(k0 + c) * words + (i >> 4)] >> (2 * (i & 15))) & 3u;
      t = code == 1u ? (int8_t)1 : (code == 3u ? (int8_t)-1 : (int8_t)0);
    }
    (isU ? Ut : Vt)[y] = t;
  }
}

// pp[c] = v_c^T H X[c] for the first V-step's X = U^T (R + X_blk) and the block's old V: one
// workgroup per component, fixed reduction order.
__global__ void __launch_bounds__(256) addback_dot_kernel(const double* X, int n, const int8_t* Vt, int ldv,
                                                          const float* h, double* pp) {
  __shared__ double red[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double acc = 0.0;
  for (int j = tid; j < n; j += 256) {
    const int v = Vt[(size_t)c * ldv + j];
    if (v) acc += (double)v * (h ? (double)h[j] : 1.0) * X[(size_t)c * n + j];
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) red[wid] = acc;
  __syncthreads();
  if (tid == 0) pp[c] = (red[0] + red[1]) + (red[2] + red[3]);
}

// E <- E + 2 sum_c d_c pp_c - sum_{c,c'} d_c d_c' (u_c . u_c') (v_c^T H v_c'): the energy of the
// residual with the block's contribution X_blk restored, |R + X|^2 = |R|^2 + 2 <R + X, X> - |X|^2
// (kept in st[3] too).  GU holds the Gram of the old U (copied to GUo), GV the weighted Gram of
// the old V.  Also clears the residual-max slot the refit's own update will write.
__global__ void __launch_bounds__(256) addback_energy_kernel(const double* pp, const double* GU, const double* GV,
                                                             const float* D, int k0, int bs, double* st,
                                                             unsigned* rmax_slot, double* GUo) {
  __shared__ double red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid < kMaxWords) rmax_slot[tid] = 0u;
  for (int x = tid; x < bs * bs; x += 256) GUo[x] = GU[x];
  double cr = 0.0, xx = 0.0;
  if (tid < bs) {
    const double dc = (double)D[k0 + tid];
    cr = dc * pp[tid];
    for (int c2 = 0; c2 < bs; ++c2)
      xx += dc * (double)D[k0 + c2] * GU[(size_t)tid * bs + c2] * GV[(size_t)tid * bs + c2];
  }
  cr = wave_sum_f64(cr);
  xx = wave_sum_f64(xx);
  if (lane == 0) {
    red[0][wid] = cr;
    red[1][wid] = xx;
  }
  __syncthreads();
  if (tid == 0) {
    const double c = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    const double x = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    st[0] = st[0] + 2.0 * c - x;
    st[3] = st[0];
  }
}

// After the refit's scales: if the refit leaves the residual larger than before the add-back by
// more than 1e-9 |A|^2_H, keep the old block instead (flags[5] = 1): its scales go back to D and
// dvec, and its own sequential energy walk on the restored residual, from st[3], replaces the
// refit's energies (thread t forms p_t = pp_t - sum_{c < t} d_c (u_t . u_c)(v_c^T H v_t)).
__global__ void __launch_bounds__(256) refit_choose_kernel(const double* ppo, const double* GUo, const double* GVo,
                                                           const float* dold, int k0, int bs, float* dvec, float* D,
                                                           double* energy, double* st, int* flags, u64* stats) {
#pragma clang fp contract(off)
  __shared__ double ps[256], qs[256];
  __shared__ int revert;
  const int tid = threadIdx.x;
  if (tid == 0) revert = st[0] > st[2] + 1e-9 * st[1] ? 1 : 0;
  __syncthreads();
  if (!revert) return;
  if (tid < bs) {
    double p = ppo[tid];
    for (int c2 = 0; c2 < tid; ++c2)
      p -= (double)dold[c2] * GUo[(size_t)tid * bs + c2] * GVo[(size_t)c2 * bs + tid];
    ps[tid] = p;
    qs[tid] = GUo[(size_t)tid * bs + tid] * GVo[(size_t)tid * bs + tid];
    dvec[tid] = dold[tid];
    D[k0 + tid] = dold[tid];
  }
  __syncthreads();
  if (tid == 0) {
    double E = st[3];
    const double E0 = st[1];
    for (int c = 0; c < bs; ++c) {
      const double dd = (double)dold[c];
      E = E - (2.0 * dd * ps[c] - dd * dd * qs[c]);
      energy[k0 + c] = 1.0 - E / E0;
    }
    st[0] = E;
    flags[5] = 1;
    stats[6] += 1ull;
  }
}

// E0 from the per-row energies (fixed order), dead flag for A = 0
__global__ void block_init_kernel(const double* rowE, int m, double* st, int* flags, unsigned* rmax,
                                  unsigned* gcnt) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid < kGramTiles) gcnt[tid] = 0u;
  double e = 0.0;
  for (int i = tid; i < m; i += 256) e += rowE[i];
  e = wave_sum_f64(e);
  if (lane == 0) red[wid] = e;
  __syncthreads();
  if (tid == 0) {
    const double E0 = red[0] + red[1] + red[2] + red[3];
    st[0] = E0;
    st[1] = E0;
    flags[0] = E0 > 0.0 ? 0 : 1;
    flags[1] = 0;
    flags[2] = 0;
    flags[3] = 0;
    flags[4] = 0;
    for (int x = 0; x < 2 * kMaxWords; ++x) rmax[x] = 0u;
  }
}

// residual exactly zero: mark dead (checked after a sketch found only empty columns)
__global__ void __launch_bounds__(256) zero_check_kernel(const float* R, int ldr, int m, int n, int* flags,
                                                         double* st) {
  __shared__ int nz;
  if (flags[1] == 0 || flags[0]) return;
  if (threadIdx.x == 0) nz = 0;
  __syncthreads();
  int any = 0;
  for (long long x = threadIdx.x; x < (long long)m * n && !any; x += 256) {
    const int i = (int)(x / n), j = (int)(x - (long long)i * n);
    if (R[(size_t)i * ldr + j] != 0.0f) any = 1;
  }
  if (any) atomicOr(&nz, 1);
  __syncthreads();
  if (threadIdx.x == 0 && !nz) {
    flags[0] = 1;
    st[0] = 0.0;
  }
}

// K splits of an int8 contraction with `tiles` workgroups per split: about 512 workgroups, at
// least 256 of K per split, at most 16 splits; kspan is a multiple of the 64-wide k chunk.
static int i8_splits(int tiles, int K, int* kspan) {
  int z = (512 + tiles - 1) / tiles;
  const int maxz = (K + 255) / 256;
  z = z > maxz ? maxz : z;
  z = z > 16 ? 16 : z;
  z = z < 1 ? 1 : z;
  *kspan = ((K + z - 1) / z + 63) / 64 * 64;
  return (K + *kspan - 1) / *kspan;
}

static void zero_fill(double* p, long long count, hipStream_t st) {
  const long long nb = (count + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, st, p, count);
}

// Y^T (bs x m) = (R diag(h) V^T)^T for V = Vt rows, on int8 MFMA with R in fixed point
// Whether the contraction of R (rows or columns) with bs ternary vectors splits K, so that its
// output must be cleared first.
static bool rw_splits(const BlockLaunch& L, int bs) {
  const int nct = bs <= 16 ? 1 : (bs <= 32 ? 2 : 4);
  int kspan = 0;
  return i8_splits(((L.m + 63) / 64) * ((bs + 16 * nct - 1) / (16 * nct)), L.n, &kspan) > 1;
}
static bool utr_splits(const BlockLaunch& L, int bs) {
  const int nct = bs <= 16 ? 1 : (bs <= 32 ? 2 : 4);
  int kspan = 0;
  return i8_splits(((L.n + 63) / 64) * ((bs + 16 * nct - 1) / (16 * nct)), L.m, &kspan) > 1;
}

static void rw_product(const BlockLaunch& L, const BlockWs& w, const float* h, int bs, int sblk, double* outT,
                       hipStream_t st, bool prezeroed = false, const double* spdG = nullptr,
                       double* spdGi = nullptr) {
  const int nct = bs <= 16 ? 1 : (bs <= 32 ? 2 : 4);  // 8 tiles: one wave per SIMD, slower
  const int gx = (L.m + 63) / 64, gy = (bs + 16 * nct - 1) / (16 * nct);
  int kspan = 0;
  const int gz = i8_splits(gx * gy, L.n, &kspan);
  if (gz > 1 && !prezeroed) zero_fill(outT, (long long)bs * L.m, st);
  // with spdG, one more column of workgroups, one of which inverts spdG
  const dim3 grid(gx + (spdG ? 1 : 0), gy, gz);
  size_t lds = (size_t)4 * 64 * kTileP;
  if (spdG && spd_lds_bytes(bs) > lds) lds = spd_lds_bytes(bs);
  if (nct == 1)
    hipLaunchKernelGGL(rv_i8_kernel<1>, grid, dim3(256), lds, st, L.R, L.ldr, L.m, L.n, w.Vt, w.ldv, h, L.EHm, bs,
                       w.rmax, sblk, kspan, outT, spdG, spdGi);
  else if (nct == 2)
    hipLaunchKernelGGL(rv_i8_kernel<2>, grid, dim3(256), lds, st, L.R, L.ldr, L.m, L.n, w.Vt, w.ldv, h, L.EHm, bs,
                       w.rmax, sblk, kspan, outT, spdG, spdGi);
  else
    hipLaunchKernelGGL(rv_i8_kernel<4>, grid, dim3(256), lds, st, L.R, L.ldr, L.m, L.n, w.Vt, w.ldv, h, L.EHm, bs,
                       w.rmax, sblk, kspan, outT, spdG, spdGi);
}

// G (bs x bs) = T diag(w) T^T for ternary rows T (bs x len, ld ldt); integer-exact without weights
static void gram_product(const BlockWs& w, const int8_t* T, int len, int ldt, const float* wt, int ehm, int bs,
                         double* G, hipStream_t st) {
  const int nt = (bs + 15) / 16;
  if (!wt) {
    hipLaunchKernelGGL(gram_i8_kernel, dim3(nt * (nt + 1) / 2), dim3(1024), 0, st, T, ldt, len, bs, G);
    return;
  }
  // K split so that each wave takes about one round of chunks (16 waves x 3 chunks per range)
  const int nch = (len + 63) / 64;
  int split = (nch + 47) / 48;
  split = split < 1 ? 1 : (split > kGramSplit ? kGramSplit : split);
  hipLaunchKernelGGL(gram_w_i8_kernel, dim3(nt * (nt + 1) / 2, split), dim3(1024), 0, st, T, ldt, len, bs, w.hdig,
                     ehm, G, w.gpart, w.gcnt);
}

// X (bs x n) = U^T R, on int8 MFMA with R in fixed point
static void utr_product(const BlockLaunch& L, const BlockWs& w, int bs, int sblk, hipStream_t st,
                        bool prezeroed = false, const double* spdG = nullptr, double* spdGi = nullptr) {
  const int nct = bs <= 16 ? 1 : (bs <= 32 ? 2 : 4);  // 8 tiles: one wave per SIMD, slower
  const int gx = (L.n + 63) / 64, gy = (bs + 16 * nct - 1) / (16 * nct);
  int kspan = 0;
  const int gz = i8_splits(gx * gy, L.m, &kspan);
  if (gz > 1 && !prezeroed) zero_fill(w.X, (long long)bs * L.n, st);
  // with spdG, one more column of workgroups, one of which inverts spdG
  const dim3 grid(gx + (spdG ? 1 : 0), gy, gz);
  size_t lds = (size_t)4 * 64 * kTileQ;
  if (spdG && spd_lds_bytes(bs) > lds) lds = spd_lds_bytes(bs);
  if (nct == 1)
    hipLaunchKernelGGL(utr_i8_kernel<1>, grid, dim3(256), lds, st, L.R, L.ldr, L.m, L.n, w.Ut, w.ldu, bs, w.rmax,
                       sblk, kspan, w.X, spdG, spdGi);
  else if (nct == 2)
    hipLaunchKernelGGL(utr_i8_kernel<2>, grid, dim3(256), lds, st, L.R, L.ldr, L.m, L.n, w.Ut, w.ldu, bs, w.rmax,
                       sblk, kspan, w.X, spdG, spdGi);
  else
    hipLaunchKernelGGL(utr_i8_kernel<4>, grid, dim3(256), lds, st, L.R, L.ldr, L.m, L.n, w.Ut, w.ldu, bs, w.rmax,
                       sblk, kspan, w.X, spdG, spdGi);
}

// Li = (G + eps I)^-1 for bs <= kSpdMax, else Li = L^-1 for L L^T = G + eps I
static void chol_inverse(const BlockWs& w, const double* G, int bs, hipStream_t st) {
  if (bs <= kSpdMax) {
    static bool attr_set[64] = {};  // once per device: dynamic LDS above 64 KB
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr_set[dev] &&
        hipFuncSetAttribute((const void*)spd_inv_kernel<256>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)spd_lds_bytes(kSpdMax)) == hipSuccess &&
        hipFuncSetAttribute((const void*)spd_inv_kernel<1024>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)spd_lds_bytes(kSpdMax)) == hipSuccess)
      attr_set[dev] = true;  // a failure shows up as a launch error, checked by the caller
    if (bs <= 64)
      hipLaunchKernelGGL(spd_inv_kernel<256>, dim3(1), dim3(256), spd_lds_bytes(bs), st, G, bs, w.Li);
    else
      hipLaunchKernelGGL(spd_inv_kernel<1024>, dim3(1), dim3(1024), spd_lds_bytes(bs), st, G, bs, w.Li);
    return;
  }
  const int ne = bs * (bs + 1) / 2;
  if (ne <= 256 * 2)
    hipLaunchKernelGGL((chol_inv_kernel<256, 2>), dim3(1), dim3(256), 0, st, G, bs, w.Li);
  else if (ne <= 256 * 5)
    hipLaunchKernelGGL((chol_inv_kernel<256, 5>), dim3(1), dim3(256), 0, st, G, bs, w.Li);
  else if (ne <= 256 * 9)
    hipLaunchKernelGGL((chol_inv_kernel<256, 9>), dim3(1), dim3(256), 0, st, G, bs, w.Li);
  else if (ne <= 1024 * 5)
    hipLaunchKernelGGL((chol_inv_kernel<1024, 5>), dim3(1), dim3(1024), 0, st, G, bs, w.Li);
  else if (ne <= 1024 * 9)
    hipLaunchKernelGGL((chol_inv_kernel<1024, 9>), dim3(1), dim3(1024), 0, st, G, bs, w.Li);
  else if (ne <= 1024 * 17)
    hipLaunchKernelGGL((chol_inv_kernel<1024, 17>), dim3(1), dim3(1024), 0, st, G, bs, w.Li);
  else
    hipLaunchKernelGGL((chol_inv_kernel<1024, 33>), dim3(1), dim3(1024), 0, st, G, bs, w.Li);
}

template <bool TA>
static void apply(const double* A, int bs, const double* Bm, double* out, int ncols, hipStream_t st) {
  const dim3 grid((ncols + 63) / 64);
  const int nrt = (bs + 15) / 16;
  if (nrt <= 1) hipLaunchKernelGGL((apply_kernel<1, TA>), grid, dim3(256), 0, st, A, bs, Bm, out, ncols);
  else if (nrt <= 2) hipLaunchKernelGGL((apply_kernel<2, TA>), grid, dim3(256), 0, st, A, bs, Bm, out, ncols);
  else if (nrt <= 4) hipLaunchKernelGGL((apply_kernel<4, TA>), grid, dim3(256), 0, st, A, bs, Bm, out, ncols);
  else if (nrt <= 8) hipLaunchKernelGGL((apply_kernel<8, TA>), grid, dim3(256), 0, st, A, bs, Bm, out, ncols);
  else hipLaunchKernelGGL((apply_kernel<16, TA>), grid, dim3(256), 0, st, A, bs, Bm, out, ncols);
}

// out (bs x ncols) = (G + eps I)^-1 in: one product with the inverse, or L^-T (L^-1 in) for
// bs > kSpdMax; in and out may not alias
static void solve(const BlockWs& w, int bs, const double* in, double* out, int ncols, hipStream_t st) {
  if (bs <= kSpdMax) {
    // two strips per workgroup once that still leaves a workgroup per CU or more
    const bool two = ncols >= 2 * 16 * 256;
    const dim3 grid(two ? (ncols + 31) / 32 : (ncols + 15) / 16);
    if (bs <= 64) {
      if (two) hipLaunchKernelGGL((apply_strip_kernel<1, 16, 2>), grid, dim3(256), 0, st, w.Li, bs, in, out, ncols);
      else hipLaunchKernelGGL((apply_strip_kernel<1, 16, 1>), grid, dim3(256), 0, st, w.Li, bs, in, out, ncols);
    } else {
      if (two) hipLaunchKernelGGL((apply_strip_kernel<2, 32, 2>), grid, dim3(256), 0, st, w.Li, bs, in, out, ncols);
      else hipLaunchKernelGGL((apply_strip_kernel<2, 32, 1>), grid, dim3(256), 0, st, w.Li, bs, in, out, ncols);
    }
    return;
  }
  apply<false>(w.Li, bs, in, w.Tmp, ncols, st);
  apply<true>(w.Li, bs, w.Tmp, out, ncols, st);
}

static void select_rows(const double* X, int L, int ldT, int bs, float tau, const float* h, int EHm, int8_t* T,
                        double* PHC, int* flags, int flag_empty, hipStream_t st, double* Z0 = nullptr,
                        int zlen = 0, const double* Yd = nullptr, double* Md = nullptr) {
  // long rows take 1024 threads (only bs workgroups run, so the CUs have room)
  if (L > 4096) {
    if (h)
      hipLaunchKernelGGL((select_rows_kernel<true, 1024>), dim3(bs), dim3(1024), 0, st, X, L, ldT, tau, h, EHm, T,
                         PHC, flags, flag_empty, Z0, zlen, Yd, Md);
    else
      hipLaunchKernelGGL((select_rows_kernel<false, 1024>), dim3(bs), dim3(1024), 0, st, X, L, ldT, tau, h, EHm, T,
                         PHC, flags, flag_empty, Z0, zlen, Yd, Md);
    return;
  }
  if (h)
    hipLaunchKernelGGL((select_rows_kernel<true, 512>), dim3(bs), dim3(512), 0, st, X, L, ldT, tau, h, EHm, T, PHC,
                       flags, flag_empty, Z0, zlen, Yd, Md);
  else
    hipLaunchKernelGGL((select_rows_kernel<false, 512>), dim3(bs), dim3(512), 0, st, X, L, ldT, tau, h, EHm, T, PHC,
                       flags, flag_empty, Z0, zlen, Yd, Md);
}

hipError_t block_run(const BlockLaunch& L, hipStream_t st, double* flops, double* bytes) {
  if (L.b > 256) return hipErrorInvalidValue;
  {
    static bool scales_attr[64] = {};  // once per device: dynamic LDS above 64 KB
    int dev = 0;
    hipError_t ea = hipGetDevice(&dev);
    if (ea != hipSuccess) return ea;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!scales_attr[dev]) {
      const void* kernels[4] = {(const void*)scales_kernel<1>, (const void*)scales_kernel<2>,
                                (const void*)scales_kernel<3>, (const void*)scales_kernel<4>};
      for (const void* kf : kernels) {
        ea = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(96 * 1024));
        if (ea != hipSuccess) return ea;
      }
      scales_attr[dev] = true;
    }
  }
  const BlockWs w = carve(L.ws, L.m, L.n, L.b);
  const int m = L.m, n = L.n;
  hipError_t e = hipSuccess;
  hipLaunchKernelGGL(block_init_kernel, dim3(1), dim3(256), 0, st, L.rowE, m, w.st, w.flags, w.rmax, w.gcnt);
  {
    const long long nb = ((long long)m * n + 255) / 256;
    hipLaunchKernelGGL(rmax_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, st, L.R, L.ldr, m, n,
                       w.rmax);
  }
  if (L.h)
    hipLaunchKernelGGL(hdig_kernel, dim3((w.ldv + 255) / 256), dim3(256), 0, st, L.h, n, w.ldv, L.EHm, w.hdig);
  const int nblocks = (L.k + L.b - 1) / L.b;
  double fl = 0.0, by = 0.0;  // multiply-adds of R by ternary operands; residual bytes read/written
  const double rbytes = 4.0 * m * n;
  int used = L.k;  // components fitted before an energy-target stop
  // ALS iterations of one block from its current Ut, then the scales, the update and the outputs.
  // sblk: residual updates so far (which max slot holds max |R|); addback: the first V-step also
  // yields the energy of the residual with the block's old contribution restored.
  // Ablations: naive_t drops Eq. 3's decorrelation (the targets are U^T R and R H V themselves),
  // hsel = nullptr projects the V-step without the weights.
  const bool naive_t = (L.ablation & 1) != 0;
  const float* hsel = (L.ablation & 2) ? nullptr : L.h;
  const int ehsel = (L.ablation & 2) ? 0 : L.EHm;
  // Split-K outputs are cleared by the kernel before their contraction: X by the selection of U
  // (or the sketch's, or the refit's load), Yt by the selection of V (or the sketch's Omega).
  auto als_fit = [&](int sblk, int bs, int k0, double target, bool addback) -> hipError_t {
    const bool xz = utr_splits(L, bs), yz = rw_splits(L, bs);
    const bool fused = bs <= kSpdFused;
    for (int t = 0; t < L.T; ++t) {
      double* x0 = (xz && t + 1 < L.T) ? w.X : nullptr;  // for the next V-step
      double* y0 = yz ? w.Yt : nullptr;                  // for this U-step
      if (naive_t) {
        if (addback && t == 0) gram_product(w, w.Ut, m, w.ldu, nullptr, 0, bs, w.GU, st);
        utr_product(L, w, bs, sblk, st, true);
        if (addback && t == 0) {
          hipLaunchKernelGGL(addback_dot_kernel, dim3(bs), dim3(256), 0, st, w.X, n, w.Vt, w.ldv, L.h, w.ppo);
          hipLaunchKernelGGL(addback_energy_kernel, dim3(1), dim3(256), 0, st, w.ppo, w.GU, w.GVo, L.D, k0, bs,
                             w.st, w.rmax + kMaxWords * ((sblk + 1) & 1), w.GUo);
        }
        select_rows(w.X, n, w.ldv, bs, L.tau, hsel, ehsel, w.Vt, w.PHC, w.flags, 0, st, y0, m);
        gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GV, st);  // for the scales
        rw_product(L, w, L.h, bs, sblk, w.Yt, st, true);
        select_rows(w.Yt, m, w.ldu, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 0, st, x0, n,
                    t + 1 == L.T ? w.Yt : nullptr, t + 1 == L.T ? w.Md : nullptr);
        fl += 4.0 * m * n * bs;
        by += 2.0 * rbytes;
        continue;
      }
      // V-step: G = (U^T U + eps I)^-1 U^T R, rows ternarized with weights h.  For b <= 64 the
      // inverse runs inside the contraction's launch; above, before it on the same stream (beside
      // a contraction on a second stream it ran ~1.6x slower, and the events cost more again).
      if (fused) {
        gram_product(w, w.Ut, m, w.ldu, nullptr, 0, bs, w.GU, st);
        utr_product(L, w, bs, sblk, st, true, w.GU, w.Li);
      } else {
        gram_product(w, w.Ut, m, w.ldu, nullptr, 0, bs, w.GU, st);
        chol_inverse(w, w.GU, bs, st);
        utr_product(L, w, bs, sblk, st, true);
      }
      if (addback && t == 0) {
        hipLaunchKernelGGL(addback_dot_kernel, dim3(bs), dim3(256), 0, st, w.X, n, w.Vt, w.ldv, L.h, w.ppo);
        hipLaunchKernelGGL(addback_energy_kernel, dim3(1), dim3(256), 0, st, w.ppo, w.GU, w.GVo, L.D, k0, bs, w.st,
                           w.rmax + kMaxWords * ((sblk + 1) & 1), w.GUo);
      }
      solve(w, bs, w.X, w.Z, n, st);
      select_rows(w.Z, n, w.ldv, bs, L.tau, hsel, ehsel, w.Vt, w.PHC, w.flags, 0, st, y0, m);
      // U-step: F^T = (V^T H V + eps I)^-1 (R H V)^T, columns ternarized without weights
      if (fused) {
        gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GV, st);
        rw_product(L, w, L.h, bs, sblk, w.Yt, st, true, w.GV, w.Li);
      } else {
        gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GV, st);
        chol_inverse(w, w.GV, bs, st);
        rw_product(L, w, L.h, bs, sblk, w.Yt, st, true);
      }
      solve(w, bs, w.Yt, w.Ft, m, st);
      select_rows(w.Ft, m, w.ldu, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 0, st, x0, n,
                  t + 1 == L.T ? w.Yt : nullptr, t + 1 == L.T ? w.Md : nullptr);
      fl += 4.0 * m * n * bs;
      by += 2.0 * rbytes;
    }
    // scales against Q = R H V of the last U-step, then the update and the outputs
    gram_product(w, w.Ut, m, w.ldu, nullptr, 0, bs, w.GU, st);  // Md came with the last selection
    {
      auto kern = bs <= 64 ? scales_kernel<1> : bs <= 128 ? scales_kernel<2> : bs <= 192 ? scales_kernel<3> : scales_kernel<4>;
      hipLaunchKernelGGL(kern, dim3(1), dim3(256), scales_lds_bytes(bs), st, w.Md, w.GU, w.GV, bs, k0, L.T, w.d, L.D,
                         L.energy, w.st, w.flags, L.stats, target);
    }
    if (addback) {  // keep the better of the refit and the old block
      hipLaunchKernelGGL(refit_choose_kernel, dim3(1), dim3(256), 0, st, w.ppo, w.GUo, w.GVo, w.dold, k0, bs, w.d,
                         L.D, L.energy, w.st, w.flags, L.stats);
      const long long nb = ((long long)bs * (w.ldu + w.ldv) + 255) / 256;
      hipLaunchKernelGGL(refit_load_kernel, dim3((unsigned)(nb < 1024 ? nb : 1024)), dim3(256), 0, st, L.Bp, L.Cp,
                         L.D, m, n, k0, bs, w.Ut, w.ldu, w.Vt, w.ldv, w.d, w.dold, w.st, w.flags, w.rmax, true,
                         nullptr, 0ll);
    }
    hipLaunchKernelGGL(update_kernel, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, st, L.R, L.ldr, m, n, w.Ut,
                       w.ldu, w.Vt, w.ldv, w.d, bs, w.flags, w.rmax + kMaxWords * ((sblk + 1) & 1));
    hipLaunchKernelGGL(emit_kernel, dim3(256), dim3(256), 0, st, w.Ut, w.ldu, w.Vt, w.ldv, m, n, bs, k0, L.Bp, L.Cp,
                       w.flags);
    fl += 2.0 * m * n * bs;
    by += 2.0 * rbytes;
    return hipGetLastError();
  };
  for (int s = 0; s < nblocks; ++s) {
    const int bs = (L.k - s * L.b) < L.b ? (L.k - s * L.b) : L.b;
    const int k0 = s * L.b;
    // sketch
    hipLaunchKernelGGL(omega_kernel, dim3(256), dim3(256), 0, st, w.Vt, w.ldv, bs, n, (long long)s, w.flags,
                       w.rmax, w.Yt, rw_splits(L, bs) ? (long long)bs * m : 0ll);
    rw_product(L, w, nullptr, bs, s, w.Yt, st, true);
    select_rows(w.Yt, m, w.ldu, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 1, st,
                utr_splits(L, bs) ? w.X : nullptr, n);
    hipLaunchKernelGGL(zero_check_kernel, dim3(1), dim3(256), 0, st, L.R, L.ldr, m, n, w.flags, w.st);
    hipLaunchKernelGGL(fallback_kernel, dim3(1), dim3(512), 0, st, L.R, L.ldr, m, n, bs, w.Ut, w.ldu, w.PHC,
                       w.flags, w.used);
    fl += 2.0 * m * n * bs;
    by += rbytes;
    if ((e = als_fit(s, bs, k0, L.target, false)) != hipSuccess) return e;
    if (L.target > 0.0 && k0 + bs < L.k) {
      // the host learns of a stop before queueing the next block (one 4-byte read per block)
      int reached = 0;
      if ((e = hipMemcpyAsync(&reached, w.flags + 3, sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
      if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
      if (reached) {
        u64 u = 0;
        if ((e = hipMemcpyAsync(&u, L.stats + 5, sizeof(u64), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
        if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
        used = (int)u;
        hipLaunchKernelGGL(stop_fill_kernel, dim3(256), dim3(256), 0, st, L.Bp, L.Cp, L.D, L.energy, m, n, k0 + bs,
                           L.k);
        break;
      }
    }
  }
  // refinement sweeps: refit each block of the first `used` components from its previous
  // factors (backfitting).  step numbers the residual updates: update number t writes the max
  // slot (t + 1) & 1 that the contractions after it read; every refit starts with an add-back
  // update, so the slot history before the sweeps does not matter.
  int step = nblocks;
  bool zero_start = false;  // A == 0: nothing to refit
  if (L.sweeps > 0) {
    double e0h[2] = {0.0, 0.0};
    u64 u = 0;  // a stop inside the last block is not seen by the per-block check
    if ((e = hipMemcpyAsync(e0h, w.st, 2 * sizeof(double), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(&u, L.stats + 5, sizeof(u64), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    zero_start = !(e0h[1] > 0.0);
    if (L.target > 0.0 && u > 0) used = (int)u;
  }
  for (int sw = 0; sw < L.sweeps && !zero_start; ++sw) {
    for (int k0 = 0; k0 < used; k0 += L.b) {
      int bs = L.k - k0 < L.b ? L.k - k0 : L.b;
      if (used - k0 < bs) bs = used - k0;
      const long long tot = (long long)bs * (w.ldu + w.ldv);
      const long long nb = (tot + 255) / 256;
      hipLaunchKernelGGL(refit_load_kernel, dim3((unsigned)(nb < 1024 ? nb : 1024)), dim3(256), 0, st, L.Bp, L.Cp,
                         L.D, m, n, k0, bs, w.Ut, w.ldu, w.Vt, w.ldv, w.d, w.dold, w.st, w.flags,
                         w.rmax + kMaxWords * ((step + 1) & 1), false, w.X,
                         utr_splits(L, bs) ? (long long)bs * n : 0ll);
      // add the block back: R <- fl32(R + U diag(d) V^T), the new residual max into the next slot
      hipLaunchKernelGGL(update_kernel, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, st, L.R, L.ldr, m, n,
                         w.Ut, w.ldu, w.Vt, w.ldv, w.d, bs, w.flags, w.rmax + kMaxWords * ((step + 1) & 1));
      ++step;
      // the old V's weighted Gram for the add-back energy (the U-step overwrites GV)
      gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GVo, st);
      by += 2.0 * rbytes;
      if ((e = als_fit(step, bs, k0, 0.0, true)) != hipSuccess) return e;
      ++step;
    }
  }
  if (L.sweeps > 0 && !zero_start && used < L.k)  // the held energy after the stop is the final one
    hipLaunchKernelGGL(stop_fill_kernel, dim3(256), dim3(256), 0, st, L.Bp, L.Cp, L.D, L.energy, m, n, used, L.k);
  *flops = fl;
  *bytes = by;
  return hipGetLastError();
}

}  // namespace externd
