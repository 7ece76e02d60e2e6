// Block-ALS path: b components per block with dense contractions on int8 and fp64 MFMA (gfx950).
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
// MI355X mapping.  The residual contractions (R Omega and R H V with K = n, U^T R with K = m) run
// on v_mfma_i32_16x16x64_i8: the ternary operand is exact int8, and R (times h_j, formed in fp64,
// in the weighted U-step) enters as its 48-bit fixed-point image split into six signed 8-bit
// digits, one power-of-two grid per block chosen from max |R| (and max h).  Digit products sum
// exactly in int32 and recombine exactly in int64; split-K partials add with 64-bit integer
// atomics, so each contraction is the exact contraction of the image, independent of launch shape
// and atomic order, within 2^-47 of max |R| per entry of the fp64 sums of a plain implementation.
// The contraction outputs stay integers (with their grid unit) until the kernels that read them.
// The contractions split their work evenly over one workgroup per CU (stream-K); the residual is
// kept twice, R and R^T, so that both read rows.  Grams are the same int8 MFMA on the ternary
// rows (integer-exact; the weighted Gram takes h in 35-bit fixed point).  The b x b solves use
// (G + eps I)^-1 from a blocked Cholesky (fp64 MFMA tiles; for b <= 128 one workgroup of the
// contraction launch computes it) and one fp64 MFMA product per solve.  The rank-b update forms
// the exact fp64 value of sum_c d_c u_ic v_jc on int8 MFMA from a fixed-point image of the scales
// (fp64 MFMA when the scales do not fit one grid), rounds once to fp32 and writes R and R^T.
// Selections use the same exact projection as the sequential path, one workgroup per component
// row, and write the ternary operand of the next contraction in its load order.
#include "externd_internal.hpp"
#include <type_traits>
#include "select.hpp"

namespace externd {

typedef double dbl4 __attribute__((ext_vector_type(4)));

constexpr int kGramSplit = 8;    // most K splits of the weighted Gram
constexpr int kGramTiles = 136;  // lower 16 x 16 tiles of a Gram with b <= 256

struct BlockWs {
  int ldu, ldv;    // row lengths of Ut / Vt: m and n rounded up to 16 (zero padding)
  int8_t* Ut;      // b x ldu, component-major
  int8_t* Vt;      // b x ldv (also holds Omega for the sketch)
  double* Yt;      // b x m: sketch / (R H V)^T, int64 in units of unit[1] (see Yi)
  double* Ft;      // b x m: F^T
  double* X;       // b x n: U^T R, int64 in units of unit[0] (see Xi)
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
  double* unit;    // [0] unit of X, [1] unit of Yt: the fixed-point grid of the last contraction
  long long* Xi;   // X and Yt as the contractions write them (exact integers)
  long long* Yi;
  float* hpad;     // the column weights, zero-padded to a multiple of 64 (weighted only)
  int ncu;         // compute units of the device (contraction workgroups per launch)
  int8_t* Ts;      // the ternary operand of a contraction, swizzled (b rounded up to 64 x max(m, n)
                   // rounded up to 64)
};

constexpr int kMaxWords = 64;      // words per residual-max slot (one per lane of a wave)
constexpr int kHDig = 5;           // 7-bit digits of the fixed-point weights (35 bits)

// (G + eps I)^-1 for bs <= 128 is stored in the order the solves read it (apply_strip_kernel): the
// operand "row r, k" of a lane (lane group lk, lane lr of row tile t = r / 16, k = 4 st + lk)
// sits at ((((t NKS / 2 + st / 2) 4 + lk) 16 + lr) 2 + st % 2, so that a wave's 16-byte loads of
// a k-step pair read 1 KB contiguous.  NKS = 32 k-steps for bs > 64, else 16.
__host__ __device__ inline int spd_nks(int bs) { return bs > 64 ? 32 : 16; }
__host__ __device__ inline size_t spd_sw(int r, int k, int nks) {
  const int t = r >> 4, lr = r & 15, lk = k & 3, st = k >> 2;
  (void)nks;
  return ((((size_t)t * (nks / 2) + (st >> 1)) * 4 + lk) * 16 + lr) * 2 + (st & 1);
}
// doubles of that storage: the row tiles times the 4 NKS k-steps
__host__ __device__ inline size_t spd_sw_size(int bs) { return (size_t)((bs + 15) & ~15) * 4 * spd_nks(bs); }

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// One layout for both sizing and carving.
template <typename F>
static void ws_layout(int m, int n, int b, bool weighted, F&& take) {
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
  // Li: (G + eps I)^-1 in the solves' order for b <= 128, else L^-1 (b x b)
  take((void**)nullptr, (b <= 128 ? spd_sw_size(b) : ((bb + 15) & ~(size_t)15) * ((bb + 15) & ~(size_t)15)) * 8);
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
  take((void**)nullptr, 64);                                         // contraction units
  take((void**)nullptr, weighted ? (size_t)((n + 63) & ~63) * 4 : 0);            // padded weights
  take((void**)nullptr, (size_t)((b + 63) & ~63) * ((mx + 63) & ~(size_t)63));  // swizzled T
}

static BlockWs carve(void* base, int m, int n, int b, bool weighted) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  void* ptrs[32];
  int np = 0;
  ws_layout(m, n, b, weighted, [&](void**, size_t bytes) {
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
  w.unit = static_cast<double*>(ptrs[q++]);
  w.hpad = weighted ? static_cast<float*>(ptrs[q]) : nullptr;
  ++q;
  w.Ts = static_cast<int8_t*>(ptrs[q++]);
  w.Xi = reinterpret_cast<long long*>(w.X);
  w.Yi = reinterpret_cast<long long*>(w.Yt);
  return w;
}

size_t block_workspace_bytes(int m, int n, int b, bool weighted) {
  size_t o = 0;
  ws_layout(m, n, b, weighted, [&](void**, size_t bytes) { o = al(o + bytes); });
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
// R enters as N = rint(x 2^f), x = R_ij (times h_j where weighted, formed in fp64), with one
// power-of-two scale per block chosen from max |R| (and max h) so that |N| <= 2^46, split into six
// signed 8-bit digits N = sum_s 2^(8 s) d_s.  The ternary operand is exact in int8, each digit
// product sums exactly in int32 (|sum| <= 2^7 K), the digits recombine exactly in int64
// (|sum| <= 2^46 K < 2^61 for K <= 16384) and splits of K add exactly with 64-bit integer
// atomics.  The result is the exact contraction of the fixed-point image of R, whatever the launch
// shape or the order of the atomic adds; its only error is the rounding of each x to the grid
// 2^-f, at most 2^-47 of the largest |x| (a 32-bit image, 2^-31, left the weighted targets of the
// 2560 x 9728 down projection within ~1e-7 of their fp64 values, one or two fp32 ulps, enough to
// flip near-tied selections).  The outputs are these integers (int64, in units of 2^-f); each
// launch also stores the unit 2^-f, and every kernel that reads an output scales it by that unit.
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kFxBits = 46;  // |N| <= 2^kFxBits
constexpr int kDig = 6;      // signed 8-bit digits of N

// exponent E of the fixed-point range: |x| < 2^E for every x entering a contraction (each wave
// reduces the 64 words of block s's slot itself)
__device__ __forceinline__ int fx_exponent(const unsigned* rmax, int s, int ehm) {
  const unsigned bits = wave_max_u32(rmax[kMaxWords * (s & 1) + (threadIdx.x & 63)]);
  if (bits == 0u) return 0;
  return exp_bound(__uint_as_float(bits)) + ehm;
}

// scale exponent f with |x 2^f| <= 2^kFxBits, inside fp64's normal range
__device__ __forceinline__ int fx_scale(const unsigned* rmax, int s, int ehm) {
  const int f = kFxBits - fx_exponent(rmax, s, ehm);
  return f < 1000 ? (f > -1000 ? f : -1000) : 1000;
}

// rint of an fp64 value of magnitude <= 2^46 (exact conversion of the integral result)
__device__ __forceinline__ long long fx_round(double v) { return (long long)rint(v); }

// Digits of four fixed-point values: word t holds digit t of n[0..3] in bytes 0..3.  With
// B = n + 0x8080808080 (128 in bytes 0..4), digits 0..4 are B's bytes minus 128 (byte ^ 0x80) and
// digit 5 is B >> 40, in [-64, 64] for |n| <= 2^46 (B's byte 5 read as a signed byte).
__device__ __forceinline__ void fx_digits6(long long n0, long long n1, long long n2, long long n3,
                                           unsigned (&w)[kDig]) {
  const long long bias = 0x8080808080ll;
  const unsigned long long b0 = (unsigned long long)(n0 + bias), b1 = (unsigned long long)(n1 + bias);
  const unsigned long long b2 = (unsigned long long)(n2 + bias), b3 = (unsigned long long)(n3 + bias);
  const unsigned l0 = (unsigned)b0, l1 = (unsigned)b1, l2 = (unsigned)b2, l3 = (unsigned)b3;
  const unsigned h0 = (unsigned)(b0 >> 32), h1 = (unsigned)(b1 >> 32), h2 = (unsigned)(b2 >> 32),
                 h3 = (unsigned)(b3 >> 32);
  // v_perm_b32: selector bytes 0..3 pick bytes of the second source, 4..7 of the first
  const unsigned x01lo = __builtin_amdgcn_perm(l1, l0, 0x05010400u);  // b0.0 b1.0 b0.1 b1.1
  const unsigned x01hi = __builtin_amdgcn_perm(l1, l0, 0x07030602u);  // b0.2 b1.2 b0.3 b1.3
  const unsigned x23lo = __builtin_amdgcn_perm(l3, l2, 0x05010400u);
  const unsigned x23hi = __builtin_amdgcn_perm(l3, l2, 0x07030602u);
  const unsigned y01 = __builtin_amdgcn_perm(h1, h0, 0x05010400u);    // b0.4 b1.4 b0.5 b1.5
  const unsigned y23 = __builtin_amdgcn_perm(h3, h2, 0x05010400u);
  w[0] = __builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u) ^ 0x80808080u;
  w[1] = __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u) ^ 0x80808080u;
  w[2] = __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u) ^ 0x80808080u;
  w[3] = __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u) ^ 0x80808080u;
  w[4] = __builtin_amdgcn_perm(y23, y01, 0x05040100u) ^ 0x80808080u;
  w[5] = __builtin_amdgcn_perm(y23, y01, 0x07060302u);
}

// 16 fixed-point values -> the six digit operands (operand t = digit t of values 0..15)
__device__ __forceinline__ void fx_operands(const long long (&nv)[16], v4i (&op)[kDig]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    unsigned w[kDig];
    fx_digits6(nv[4 * q], nv[4 * q + 1], nv[4 * q + 2], nv[4 * q + 3], w);
#pragma unroll
    for (int t = 0; t < kDig; ++t) op[t][q] = (int)w[t];
  }
}

// the digit sums of one output recombined: sum_t 256^t acc_t, exact in int64
__device__ __forceinline__ long long fx_combine(const v4i (&acc)[kDig], int q) {
  long long v = 0;
#pragma unroll
  for (int t = kDig - 1; t >= 0; --t) v = v * 256ll + (long long)acc[t][q];
  return v;
}

__device__ __forceinline__ v4i load16(const int8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// (G + eps I)^-1 by one workgroup of NT threads over `smem` (spd_lds_bytes(bs) bytes); below.
template <int NT>
__device__ __forceinline__ void spd_inv_body(const double* G, int bs, double* Gi, char* smem);
__host__ __device__ inline size_t spd_lds_bytes(int bs);




__host__ __device__ inline int pad64(int x) { return (x + 63) & ~63; }

// ---- contraction operands.  The k order inside each 64-wide chunk is free (the products are
// summed over it), so it is chosen for the loads: lane group g of a wave takes, for each of the
// four 16-wide quarters q of the chunk, the 4 consecutive k = 16 q + 4 g .. + 3; byte 4 q + e of
// the lane's 16-byte MFMA operand is then k = 16 q + 4 g + e.  A wave's float4 loads of R read 64
// contiguous bytes of each of its 16 rows per instruction.
//
// The ternary operand in that order, swizzled so that each operand load of a wave reads 1 KB
// contiguous: one 1 KB block per 16 components and chunk, lane l = 16 g + cc holding the operand
// of component 16 p + cc (block (p, c)); components past bs and k past ldt are zero.
__global__ void __launch_bounds__(256) swizzle_t_kernel(const int8_t* T, int ldt, int bs, int nct, int nchunk,
                                                        int8_t* Ts) {
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blk >= nct * nchunk) return;
  const int p = blk / nchunk, ch = blk - p * nchunk;
  const int c = 16 * p + (lane & 15), g = lane >> 4;
  v4i v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = 64 * ch + 16 * q + 4 * g;  // ldt is a multiple of 16: the word is inside or past
    v[q] = (c < bs && k < ldt) ? *reinterpret_cast<const int*>(T + (size_t)c * ldt + k) : 0;
  }
  *reinterpret_cast<v4i*>(Ts + (size_t)blk * 1024 + 16 * lane) = v;
}

// The six digit words of four fp32 values x (times weights w, all in fp64): fma(x, w 2^f, 1.5 2^52)
// rounds x w 2^f to the nearest integer N (ties to even, as rint) in the low bits of the mantissa,
// exactly for |N| < 2^51; the bit pattern minus the constant's is N, and adding the digit bias of
// fx_digits6 gives its biased form directly.
__device__ __forceinline__ void fx_digits_of(const float (&x)[4], const double (&ws)[4], unsigned (&w)[kDig]) {
  constexpr double kMagic = 6755399441055744.0;                        // 1.5 2^52
  constexpr unsigned long long kOff = 0x4338000000000000ull - 0x8080808080ull;  // its bits, less the bias
  unsigned long long bv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) bv[e] = (unsigned long long)__double_as_longlong(fma((double)x[e], ws[e], kMagic)) - kOff;
  const unsigned l0 = (unsigned)bv[0], l1 = (unsigned)bv[1], l2 = (unsigned)bv[2], l3 = (unsigned)bv[3];
  const unsigned h0 = (unsigned)(bv[0] >> 32), h1 = (unsigned)(bv[1] >> 32), h2 = (unsigned)(bv[2] >> 32),
                 h3 = (unsigned)(bv[3] >> 32);
  const unsigned x01lo = __builtin_amdgcn_perm(l1, l0, 0x05010400u);
  const unsigned x01hi = __builtin_amdgcn_perm(l1, l0, 0x07030602u);
  const unsigned x23lo = __builtin_amdgcn_perm(l3, l2, 0x05010400u);
  const unsigned x23hi = __builtin_amdgcn_perm(l3, l2, 0x07030602u);
  const unsigned y01 = __builtin_amdgcn_perm(h1, h0, 0x05010400u);
  const unsigned y23 = __builtin_amdgcn_perm(h3, h2, 0x05010400u);
  w[0] = __builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u) ^ 0x80808080u;
  w[1] = __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u) ^ 0x80808080u;
  w[2] = __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u) ^ 0x80808080u;
  w[3] = __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u) ^ 0x80808080u;
  w[4] = __builtin_amdgcn_perm(y23, y01, 0x05040100u) ^ 0x80808080u;
  w[5] = __builtin_amdgcn_perm(y23, y01, 0x07060302u);
}

// out[c][r] += sum_k N(x_rk) T[c][k] for the rows r of X (R, or R^T), with x_rk = X_rk (times
// h_k when HW) and N the fixed-point image at the scale of residual-max slot sblk, in units
// *unit = 2^-f; out starts at zero.  Work is split evenly ("stream-K"): the units (row tile of 64,
// component group of 16 NCT, 64-wide k chunk) are dealt to nwg workgroups in contiguous runs of
// chunks, so that one launch round fills the CUs whatever the shape, and each run's partial sums
// are added into out with 64-bit integer atomics (exact, in any order).  With gy >= 2 component
// groups, the two halves of a workgroup (four waves each, 16 rows per wave) take the groups 2 j and
// 2 j + 1 of the same rows and chunks, so the rows are read once into the CU's caches; with a
// single group the halves take separate runs.  Per chunk a lane loads 64 bytes of its row (and of
// the weights) and 16 NCT bytes of the swizzled T, the next chunk's rows in flight while the
// current one is converted and multiplied.  Columns past ldx read as zero (the rows' padding up to
// ldx is zero).
// HW: 0 unweighted, 1 weights staged in LDS (Kp floats, the launch's dynamic LDS), 2 weights read
// from global memory (Kp too large for LDS).
template <int NCT, int HW>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
fx_contract_kernel(const float* X, int ldx, int rows, int Kp, const float* hp, int ehm, const unsigned* rmax,
                   int sblk, const int8_t* Ts, int bs, int gx, int gy, int nwg, long long* out, double* unit,
                   const double* spdG, double* spdGi) {
  extern __shared__ __align__(16) char dsm[];
  int w = (int)blockIdx.x;
  if (spdG) {  // workgroup 0, dispatched first, inverts spdG beside the contraction
    if (w == 0) {
      spd_inv_body<512>(spdG, bs, spdGi, dsm);
      return;
    }
    --w;
  }
  const int half = (int)threadIdx.x >> 8;
  const int tid = threadIdx.x & 255, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const float* hsrc = hp;
  if (HW == 1) {  // every workgroup stages the weights once (all its threads, before any run)
    float* hs = reinterpret_cast<float*>(dsm);
    for (int k = 4 * (int)threadIdx.x; k < Kp; k += 4 * 512)
      *reinterpret_cast<float4*>(hs + k) = *reinterpret_cast<const float4*>(hp + k);
    __syncthreads();
    hsrc = hs;
  }
  const int sc = fx_scale(rmax, sblk, HW ? ehm : 0);
  const double dsc = ldexp(1.0, sc);
  if (w == 0 && threadIdx.x == 0) *unit = ldexp(1.0, -sc);
  const int nch = Kp / 64;
  const int per = gy == 1 ? 2 : 1;  // workers per workgroup
  const long long span = (long long)(gy == 1 ? 1 : (gy + 1) / 2) * gx * nch;
  const long long nwk = (long long)nwg * per, wk = (long long)w * per + (per == 2 ? half : 0);
  long long u = wk * span / nwk;
  const long long uend = (wk + 1) * span / nwk;
  v4i acc[NCT][kDig];
  while (u < uend) {  // one run: consecutive chunks of one (row tile, component group)
    const long long tile = u / nch;
    const int cs = (int)(u - tile * nch);
    const int ce = (long long)(nch - cs) < uend - u ? nch : cs + (int)(uend - u);
    u += ce - cs;
    const int jg = (int)(tile / gx), bx = (int)(tile - (long long)jg * gx);
    const int by = gy == 1 ? 0 : 2 * jg + half;
    if (by >= gy) continue;  // the idle half of an odd count of groups
    const int c0 = by * 16 * NCT;
    const int r = bx * 64 + wid * 16 + lr;
    // rows past `rows` only reach outputs that are not stored: they read row 0
    const float* xrow = X + (size_t)(r < rows ? r : 0) * ldx + 4 * g;
    const int8_t* tsrc = Ts + (size_t)(c0 / 16) * (Kp / 64) * 1024 + 16 * lane;  // tile ct: + ct Kp 16
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int t = 0; t < kDig; ++t) acc[ct][t] = (v4i){0, 0, 0, 0};
    // Every lane issues every load (past ldx it reads its row's start and the value is dropped
    // at use), so the chunk loop has no branches and the products wait only for the older
    // chunk's loads.  The T operands (L2-resident) are loaded as a chunk's conversion starts,
    // which covers their latency and keeps one register set.
    auto load = [&](int k0, float4(&xv)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = k0 + 16 * q + 4 * g;
        xv[q] = *reinterpret_cast<const float4*>(xrow + (k < ldx ? k0 + 16 * q : -4 * g));
      }
    };
    auto products = [&](int k0, const float4(&xv)[4]) {
      v4i tt[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) tt[ct] = load16(tsrc + (size_t)16 * k0 + (size_t)ct * Kp * 16);
      float4 hv[4];  // the weights (padded to Kp with zeros), from LDS or global memory
      if (HW) {
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = *reinterpret_cast<const float4*>(hsrc + k0 + 16 * q + 4 * g);
      }
      v4i da[kDig];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = k0 + 16 * q + 4 * g < ldx;
        const float x[4] = {in ? xv[q].x : 0.f, in ? xv[q].y : 0.f, in ? xv[q].z : 0.f, in ? xv[q].w : 0.f};
        double ws[4] = {dsc, dsc, dsc, dsc};
        if (HW) {
          ws[0] = (double)hv[q].x * dsc;
          ws[1] = (double)hv[q].y * dsc;
          ws[2] = (double)hv[q].z * dsc;
          ws[3] = (double)hv[q].w * dsc;
        }
        unsigned wd[kDig];
        fx_digits_of(x, ws, wd);
#pragma unroll
        for (int t = 0; t < kDig; ++t) da[t][q] = (int)wd[t];
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int t = 0; t < kDig; ++t)
          acc[ct][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(tt[ct], da[t], acc[ct][t], 0, 0, 0);
    };
    // Two register sets of rows in turn (no copies between them)
    const int kb = 64 * cs, nk = ce - cs;
    float4 xa[4], xb[4];
    load(kb, xa);
    int it = 1;
    for (; it + 1 < nk; it += 2) {
      load(kb + 64 * it, xb);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
      products(kb + 64 * (it - 1), xa);
      load(kb + 64 * (it + 1), xa);
      __builtin_amdgcn_sched_barrier(0);
      products(kb + 64 * it, xb);
    }
    if (it < nk) {
      load(kb + 64 * it, xb);
      __builtin_amdgcn_sched_barrier(0);
      products(kb + 64 * (it - 1), xa);
      products(kb + 64 * it, xb);
    } else {
      products(kb + 64 * (it - 1), xa);
    }
    // D = T x^T: lane l, register q holds component 4 g + q of the tile for row lr, so each
    // atomic instruction covers four components x 16 consecutive rows
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + ct * 16 + 4 * g + q;
        if (c < bs && r < rows)
          atomicAdd(reinterpret_cast<unsigned long long*>(out + (size_t)c * rows + r),
                    (unsigned long long)fx_combine(acc[ct], q));
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

// hp[j] = h_j for j < n, 0 up to np
__global__ void __launch_bounds__(256) hpad_kernel(const float* h, int n, int np, float* hp) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < np) hp[j] = j < n ? h[j] : 0.0f;
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

// compile-time loop: f(integral_constant<int, I>) for I = B .. E - 1
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// lane N's value of each 16-lane row, in every lane of that row (DPP row_newbcast: a VALU move,
// where a readlane would go through a scalar register; every lane is written, so no old value is
// needed and the move is not preceded by a copy)
template <int N>
__device__ __forceinline__ double bcast16(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)b, 0x150 + N, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), 0x150 + N, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// ---- Gi = (G + eps I)^-1 for bs <= 128, eps = 1e-6 trace(G) / bs (the regularised Gram of the
// pages' Eq. 3), by a blocked Cholesky factorisation on 16 x 16 tiles, the block inverse of the
// factor and the product X^T X (X = L^-1), all in LDS.  The tile products run on fp64 MFMA; the
// 16 x 16 diagonal blocks are factored and inverted by one wave with a row per lane.  Pivots that
// are not positive give zero rows, as in a plain Cholesky solve.  The matrix is padded to a
// multiple of 16 with an identity block, which keeps it block diagonal and leaves the real part of
// the inverse unchanged.  One workgroup; 2 nb + 1 barriers for nb tiles per side.
constexpr int kSpdMax = 128;
constexpr int kSpdFused = kSpdMax;  // largest b whose inverse runs inside the contraction launch
constexpr size_t kContractLds = 160 * 1024;  // dynamic LDS limit of the contraction launches
__host__ __device__ inline size_t spd_lds_bytes(int bs) {
  const int bp = (bs + 15) & ~15, ld = bp + 1;
  return 8 * ((size_t)bp * ld + (size_t)(bp / 16) * 256);
}
// NT threads share the tile products; wave 0 factors the diagonal blocks.  The body runs as
// workgroup 0 (512 threads) of the residual contraction of the same half-step, which overlaps the
// two without a second stream, or in its own launch (spd_inv_kernel).
template <int NT>
__device__ __forceinline__ void spd_inv_body(const double* G, int bs, double* Gi, char* smem) {
  constexpr int NWV = NT / 64;
  const int bp = (bs + 15) & ~15, nb = bp / 16, ld = bp + 1;
  double* A = reinterpret_cast<double*>(smem);  // bp x ld
  double* Dg = A + (size_t)bp * ld;             // nb diagonal-block inverses, 16 x 16 row-major
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;  // MFMA operand coordinates: row / column lr, k 4 s + lk
  for (int x0 = 0; x0 < bp * bp; x0 += 16 * NT) {  // 16 loads in flight per thread, then the stores
    double v16[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int x = x0 + tid + NT * q, i = x / bp, j = x - i * bp;
      if (x < bp * bp && i < bs && j < bs) v16[q] = G[(size_t)i * bs + j];
      else v16[q] = i == j ? 1.0 : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int x = x0 + tid + NT * q, i = x / bp, j = x - i * bp;
      if (x < bp * bp) A[(size_t)i * ld + j] = v16[q];
    }
  }
  __syncthreads();
  if (wid == 0) {  // eps from the trace (summed per lane in c order, then across the wave)
    double tr = 0.0;
    for (int c = lane; c < bs; c += 64) tr += A[(size_t)c * ld + c];
    tr = wave_sum_f64(tr);
    const double eps = 1e-6 * tr / (double)bs;
    for (int c = lane; c < bs; c += 64) A[(size_t)c * ld + c] += eps;
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
  // 16 x 16 diagonal block: Cholesky factor and its inverse by wave 0.  Every 16-lane row of the
  // wave factors the block (lane r holding row r); the inverse X = L^-1 is split by columns, lane
  // group g computing columns g, g + 4, g + 8 and g + 12 of every row.
  auto factor_diag = [&](int p) {  // wave 0
    const int r = lr;
    double* T = at(p, p);
    double a[16], rk[16], x[4];
#pragma unroll
    for (int c = 0; c < 16; ++c) a[c] = T[(size_t)r * ld + c];
    static_for<0, 16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const double piv = bcast16<k>(a[k]);
      // 1 / sqrt(piv): the hardware estimate and two Newton steps (each squares the relative
      // error), then sqrt(piv) = piv / sqrt(piv); far shorter than a rounded sqrt and divide.  A
      // pivot that is not positive gives a zero row (computed on 1 and then dropped: no branch).
      const bool pos = piv > 0.0;
      const double pv = pos ? piv : 1.0;
      double y = __builtin_amdgcn_rsq(pv);
      y = y * fma(-0.5 * pv * y, y, 1.5);
      y = y * fma(-0.5 * pv * y, y, 1.5);
      const double rr = pos ? y : 0.0;
      const double lkk = piv * rr;
      rk[k] = rr;
      a[k] = r > k ? a[k] * rr : (r == k ? lkk : a[k]);
      static_for<k + 1, 16>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        a[j] = fma(-a[k], bcast16<j>(a[k]), a[j]);  // meaningful for rows r >= j
      });
    });
    // X = L^-1 row by row with the scales deferred: u_t = row t of L_tt X, so that a later row r
    // takes u_r[c] -= (L_rt / L_tt) u_t[c], and X_rc = u_r[c] / L_rr at the end.  Column c = g + 4 q
    // sits in x[q]; u_r starts as the unit row e_r.
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = (lk + 4 * q == r) ? 1.0 : 0.0;
    double myrk = 0.0;
    static_for<0, 16>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      myrk = r == t ? rk[t] : myrk;
      const double mrt = r > t ? a[t] * rk[t] : 0.0;  // zero for the rows r <= t
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = fma(-mrt, bcast16<t>(x[q]), x[q]);  // u_t[c] = 0 for c > t
    });
    if (lane < 16) {
#pragma unroll
      for (int c = 0; c < 16; ++c) T[(size_t)r * ld + c] = c <= r ? a[c] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lk + 4 * q;
      Dg[p * 256 + r * 16 + c] = c <= r ? x[q] * myrk : 0.0;
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
    dbl4 acc, c[4];  // the four k-steps in independent chains
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = T[(size_t)(4 * q + lk) * ld + lr];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      c[sl] = __builtin_amdgcn_mfma_f64_16x16x4f64(-opr(Li_, ld, sl), opr(Lj_, ld, sl), (dbl4){0.0, 0.0, 0.0, 0.0},
                                                   0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) T[(size_t)(4 * q + lk) * ld + lr] = acc[q] + ((c[0][q] + c[1][q]) + (c[2][q] + c[3][q]));
  };
  if (wid == 0) factor_diag(0);
  __syncthreads();
  for (int p = 0; p < nb; ++p) {
    // panel below: L_ip = A_ip D_p^T (in place)
    for (int i = p + 1 + wid; i < nb; i += NWV) {
      double* T = at(i, p);
      dbl4 c[4];  // the four k-steps in independent chains
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        c[sl] = __builtin_amdgcn_mfma_f64_16x16x4f64(opr(T, ld, sl), opr(Dg + p * 256, 16, sl),
                                                     (dbl4){0.0, 0.0, 0.0, 0.0}, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) T[(size_t)(4 * q + lk) * ld + lr] = (c[0][q] + c[1][q]) + (c[2][q] + c[3][q]);
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
  // ---------------- X = L^-1, one column block per wave and no barrier: a wave reads only L's
  // tiles, the D_i and the blocks of its own column written before.  X_jj = D_j and
  // X_ij = -D_i sum_{k=j}^{i-1} L_ik X_kj for i > j, the four k-steps of each tile product in
  // independent accumulator chains; X_ij is stored transposed in the free upper block (j, i) of A.
  for (int j = wid; j < nb - 1; j += NWV) {
    for (int i = j + 1; i < nb; ++i) {
      dbl4 sc[4];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) sc[sl] = (dbl4){0.0, 0.0, 0.0, 0.0};
      for (int k = j; k < i; ++k) {
        const double* P = at(i, k);
        double pa[4], pb[4];
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          // X_kj[4 s + lk][lr]: D_j for k == j, else transposed storage in block (j, k)
          pa[sl] = opr(P, ld, sl);
          pb[sl] = k == j ? opc(Dg + j * 256, 16, sl) : opr(at(j, k), ld, sl);
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) sc[sl] = __builtin_amdgcn_mfma_f64_16x16x4f64(pa[sl], pb[sl], sc[sl], 0, 0, 0);
      }
      const dbl4 sum = (sc[0] + sc[1]) + (sc[2] + sc[3]);
      dbl4 xc[4];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)  // an MFMA result in lane l, register s is operand B[4 s + lk][lr]
        xc[sl] = __builtin_amdgcn_mfma_f64_16x16x4f64(-opr(Dg + i * 256, 16, sl), sum[sl], (dbl4){0.0, 0.0, 0.0, 0.0},
                                                      0, 0, 0);
      const dbl4 xacc = (xc[0] + xc[1]) + (xc[2] + xc[3]);
      double* T = at(j, i);
#pragma unroll
      for (int q = 0; q < 4; ++q) T[(size_t)lr * ld + 4 * q + lk] = xacc[q];
    }
  }
  __syncthreads();
  // ---------------- Gi = X^T X: tile (i, j), i >= j, is sum_{k >= i} X_ki^T X_kj (four chains)
  for (int t = wid; t < nb * (nb + 1) / 2; t += NWV) {
    int i = 0;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    const int j = t - i * (i + 1) / 2;
    dbl4 ac[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) ac[sl] = (dbl4){0.0, 0.0, 0.0, 0.0};
    for (int k = i; k < nb; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        // X_ki[4 s + lk][lr] and X_kj[4 s + lk][lr]
        av[sl] = k == i ? opc(Dg + i * 256, 16, sl) : opr(at(i, k), ld, sl);
        bv[sl] = k == j ? opc(Dg + j * 256, 16, sl) : opr(at(j, k), ld, sl);
      }
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) ac[sl] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[sl], bv[sl], ac[sl], 0, 0, 0);
    }
    const dbl4 acc = (ac[0] + ac[1]) + (ac[2] + ac[3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * q + lk, c = 16 * j + lr;
      if (r < bs && c < bs) {
        const double v = acc[q];
        const int nks = spd_nks(bs);
        Gi[spd_sw(r, c, nks)] = v;
        if (i != j) Gi[spd_sw(c, r, nks)] = v;
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
// bunit (nullable): Bm holds a contraction's int64 output in units of *bunit.
template <int NRT, bool TA>
__global__ void __launch_bounds__(256) apply_kernel(const double* __restrict__ A, int bs, const double* Bm,
                                                    const double* bunit, double* out, int ncols) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const double bu = bunit ? *bunit : 1.0;
  const long long* Bi = reinterpret_cast<const long long*>(Bm);
  const int col = blockIdx.x * 64 + wid * 16 + (lane & 15);
  const bool okc = col < ncols;
  dbl4 acc[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t] = (dbl4){0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < bs; k0 += 4) {
    const int k = k0 + (lane >> 4);
    const double bv = (k < bs && okc) ? (bunit ? (double)Bi[(size_t)k * ncols + col] * bu : Bm[(size_t)k * ncols + col])
                                      : 0.0;
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
// back to back, each A operand serving the NCT strips.  K is walked in the order k = 4 st + lk
// (step st, lane group lk): the four lane groups read adjacent rows of the staged strips (distinct
// LDS banks as far as the wave's 512 bytes allow).  A is (G + eps I)^-1 as the SPD
// inverse stores it (spd_sw): each 16-byte load of a wave reads 1 KB contiguous.
// Bm holds a contraction's int64 output in units of *bunit.
template <int NRW, int NKS, int NCT>
__global__ void __launch_bounds__(256) apply_strip_kernel(const double* __restrict__ A, int bs, const long long* Bm,
                                                          const double* bunit, double* out, int ncols) {
  // rows 4 st .. 4 st + 3 feed the four lane groups: a row pitch of 32 mod 64 words (NCT odd) keeps
  // them on two bank halves
  __shared__ double Bs[kSpdMax][16 * NCT + (NCT % 2 == 0 ? 16 : 0)];
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
    const int t = wid + 4 * u, r = t * 16 + lr;
    const bool rok = t < ntiles && r < bs;
    // the stored order (spd_sw): each 16-byte load of the wave reads 1 KB contiguous
    const double* ap = A + spd_sw(rok ? r : 0, lk, NKS);
#pragma unroll
    for (int st = 0; st < NKS; st += 2) {
      const double2 v = *reinterpret_cast<const double2*>(ap + (size_t)st * 64);
      const int k = 4 * st + lk;
      av[st][u] = (rok && k < bs) ? v.x : 0.0;
      av[st + 1][u] = (rok && k + 4 < bs) ? v.y : 0.0;
    }
  }
  // the strips: (4 NKS) x 16 NCT values, NKS NCT / 4 per thread, all loads issued before the
  // first store
  constexpr int NB = NKS * NCT / 4, W = 16 * NCT;
  double bl[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int x = tid + 256 * i, k = x / W, c = x % W;
    const bool ok = k < bs && col0 + c < ncols;
    const double bv = (double)Bm[ok ? (size_t)k * ncols + col0 + c : 0];  // issued unconditionally
    bl[i] = ok ? bv : 0.0;
  }
  const double bu = *bunit;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int x = tid + 256 * i;
    Bs[x / W][x % W] = bl[i] * bu;
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
// X holds fp64 rows, or (xunit set) a contraction's int64 rows in units of *xunit, whose fp32
// roundings are formed in LDS first.  Z0 (nullable): row c of the next split-K contraction's
// output is cleared here (zlen values), which saves that contraction a separate clearing launch.
// Md (nullable): Md[c] = T[c] . Yd[c] over the L entries (the last U-step's u_c^T Q_c for the
// scales); Yd is a contraction's int64 output in units of *ydunit, so the sum is exact in int64 and
// scaled once.
template <bool W, int NT>
__global__ void __launch_bounds__(NT) select_rows_kernel(const double* X, const double* xunit, int L, int ldT,
                                                          float tau, const float* h, int EHm, int8_t* T, double* PHC,
                                                          int* flags, int flag_empty, double* Z0, int zlen,
                                                          const long long* Yd, const double* ydunit, double* Md,
                                                          int8_t* Ts) {
  __shared__ SelScratchT<W> s;
  __shared__ u64 red[NT / 64];
  extern __shared__ float xs[];  // L values when xunit is set
  const int c = blockIdx.x;
  const double* x = X + (size_t)c * L;
  if (Z0)
    for (int j = threadIdx.x; j < zlen; j += NT) Z0[(size_t)c * zlen + j] = 0.0;
  if (flags[0]) {  // residual is zero: nothing to select
    for (int j = threadIdx.x; j < ldT; j += NT) T[(size_t)c * ldT + j] = 0;
    return;
  }
  SelResult r;
  if (xunit) {
    const long long* xi = reinterpret_cast<const long long*>(x);
    const double u = *xunit;
    for (int j = threadIdx.x; j < L; j += NT) xs[j] = (float)((double)xi[j] * u);
    __syncthreads();
    r = ternary_select<NT, W>(xs, h, L, tau, EHm, s);
  } else {
    r = ternary_select<NT, W>(x, h, L, tau, EHm, s);
  }
  long long dot = 0;
  // four entries per thread and store; ldT is a multiple of 16 and the padding [L, ldT) stays
  // zero.  Ts (nullable): the same words in the swizzled operand order of the next contraction
  // (K = L), written here so that it needs no swizzle launch; its words past L are not needed.
  const int nch = (L + 63) >> 6;
  for (int j4 = 4 * (int)threadIdx.x; j4 < ldT; j4 += 4 * NT) {
    unsigned word = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j4 + e;
      const int jc = j < L ? j : L - 1;  // clamped: the loads do not wait for the bounds test
      const float xr = xunit ? xs[jc] : (float)x[jc];
      const float xv = j < L ? xr : 0.0f;
      const int t = selected(xv, r) ? (xv > 0.0f ? 1 : -1) : 0;
      word |= (unsigned)(t & 0xFF) << (8 * e);
      if (Md) {
        const long long yv = Yd[(size_t)c * L + jc];
        dot += t > 0 ? yv : (t < 0 ? -yv : 0ll);
      }
    }
    *reinterpret_cast<unsigned*>(T + (size_t)c * ldT + j4) = word;
    if (Ts && j4 < L)  // block (c / 16, j / 64), lane 16 g + c % 16, word q: j % 64 = 16 q + 4 g
      *reinterpret_cast<unsigned*>(Ts + ((size_t)(c >> 4) * nch + (j4 >> 6)) * 1024 +
                                   (16 * ((j4 >> 2) & 3) + (c & 15)) * 16 + 4 * ((j4 >> 4) & 3)) = word;
  }
  if (Md) {
    const u64 wsum = wave_sum_u64((u64)dot);  // two's complement: exact in any order
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wsum;
    __syncthreads();
    if (threadIdx.x == 0) {
      u64 t = 0;
      for (int w = 0; w < NT / 64; ++w) t += red[w];
      Md[c] = (double)(long long)t * *ydunit;
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

// ---- update: R <- fl32(R - U diag(d) V^T) -----------------------------------------------------
// The inner sum s_ij = sum_c d_c u_ic v_jc is exact whenever every d_c is an integer multiple of
// 2^(E - 45) with max |d_c| < 2^E: its partial sums, in any order, are then multiples of that
// unit below 2^(E + 7) for b <= 128 components (2^(E + 8) for 256), within fp64's 53 bits.  In
// that case (always, unless the block's scales span more than 2^22 or so) the kernel forms
// D_c = d_c 2^(45 - E) in int64 and takes the sum on int8 MFMA: six signed 8-bit digits of D_c
// (of -D_c where u_ic = -1) times the ternary operands, recombined exactly in int64; otherwise it
// sums on fp64 MFMA.  Both give the exact s_ij, the same value as a sum in fp64 in any order.
// Tile 64 x 64 of R; wave w owns rows 16w..16w+15 and four 16-column strips.  The ternary
// operands are staged 64 components at a time, transposed (component index fastest) for the int8
// products.  Each lane's 16 entries of R are loaded before anything else (the dead-residual flag
// included), in the MFMA output layout: lane l of wave w holds rows 16 w + 4 (l / 16) + r, column
// 16 t + l % 16 of strip t.  Entries whose sum is zero are not written back.
constexpr int kUpdPitch = 80;    // bytes per staged row of the fp64 path (64 components + padding)
constexpr int kUpdPitch2 = 144;  // bytes per staged row of the int8 path (128 components + padding)

// signed 8-bit digits of n (|n| < 2^45): n = sum_t 256^t d_t
__device__ __forceinline__ void fx_digits_one(long long n, int8_t (&d)[kDig]) {
  const unsigned long long bv = (unsigned long long)(n + 0x8080808080ll);
#pragma unroll
  for (int t = 0; t < kDig - 1; ++t) d[t] = (int8_t)((unsigned)((bv >> (8 * t)) & 0xFFu) ^ 0x80u);
  d[kDig - 1] = (int8_t)(unsigned)((bv >> 40) & 0xFFu);
}

// 4 x 4 byte transpose: out[q] byte e = in[e] byte q
__device__ __forceinline__ void transpose4x4(const unsigned (&w)[4], unsigned (&o)[4]) {
  const unsigned a = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u), b = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
  const unsigned c = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u), d = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  o[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) update_kernel(float* R, int ldr, float* RT, int ldt, int m, int n,
                                                     const int8_t* Ut, int ldu, const int8_t* Vt, int ldv,
                                                     const float* dvec, int bs, const int* flags,
                                                     unsigned* rmax_next) {
  // int8 path: [i][c] for 128 components; fp64 path: [c][i] for 64
  __shared__ __align__(16) int8_t Us[64 * kUpdPitch2];
  __shared__ __align__(16) int8_t Vs[64 * kUpdPitch2];
  __shared__ __align__(16) int8_t dg[2][kDig][256];  // digits of D_c and of -D_c
  __shared__ float ds[64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  // every global load the int8 path needs for its first 128 components is issued here, before
  // anything waits: R, the scales, and the ternary pieces (thread (cq, pq): components
  // 4 cq .. + 3 of each 64-chunk, positions 4 pq .. + 3 of the tile; rows of Ut / Vt are
  // zero-padded to a multiple of 16, so a 4-byte piece is inside them or past them)
  float rv[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wid * 16 + (lane >> 4) * 4 + r;
      rv[t][r] = (i < m && j < n) ? R[(size_t)i * ldr + j] : 0.0f;
    }
  }
  float dl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) dl[q] = lane + 64 * q < bs ? dvec[lane + 64 * q] : 0.0f;
  const int cq = tid >> 4, pq = tid & 15;
  unsigned wu[2][4], wv[2][4];
  auto stage_loads = [&](int kc) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = kc + 64 * h + 4 * cq + e;
        const bool oku = c < bs && i0 + 4 * pq < ldu, okv = c < bs && j0 + 4 * pq < ldv;
        const unsigned a = *reinterpret_cast<const unsigned*>(oku ? Ut + (size_t)c * ldu + i0 + 4 * pq : Ut);
        const unsigned b = *reinterpret_cast<const unsigned*>(okv ? Vt + (size_t)c * ldv + j0 + 4 * pq : Vt);
        wu[h][e] = oku ? a : 0u;
        wv[h][e] = okv ? b : 0u;
      }
  };
  stage_loads(0);
  if (flags[0]) return;
  // the scales' exponent and whether they are exact on the grid 2^(E - 45) (every wave alike)
  unsigned mb = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned b = __float_as_uint(dl[q]) & 0x7FFFFFFFu;
    mb = b > mb ? b : mb;
  }
  mb = wave_max_u32(mb);
  int E = 0;
  if (mb != 0u) frexp((double)__uint_as_float(mb), &E);  // max |d| < 2^E
  const int f = 45 - E;
  unsigned inexact = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double x = ldexp((double)dl[q], f);
    inexact |= x != rint(x) ? 1u : 0u;
  }
  const bool use_i8 = mb != 0u && wave_sum_u32(inexact) == 0u;
  const int bs4 = (bs + 3) & ~3;
  double sv[4][4];
  if (use_i8) {
    // digit tables: dg[0][t][c] of D_c, dg[1][t][c] of -D_c (zero past bs); wave w fills
    // components 64 w .. 64 w + 63 from its lanes' scales (dl[w] of lane c - 64 w)
    {
      int8_t dp[kDig], dn[kDig];
      float dw = dl[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) dw = wid == q ? dl[q] : dw;
      const long long D = (long long)ldexp((double)dw, f);
      fx_digits_one(D, dp);
      fx_digits_one(-D, dn);
#pragma unroll
      for (int t = 0; t < kDig; ++t) {
        dg[0][t][tid] = dp[t];
        dg[1][t][tid] = dn[t];
      }
    }
    v4i acc[4][kDig];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
      for (int t = 0; t < kDig; ++t) acc[s2][t] = (v4i){0, 0, 0, 0};
    const int lr = lane & 15, g = lane >> 4;
    for (int kc = 0; kc < bs; kc += 128) {
      if (kc > 0) {
        __syncthreads();  // the previous 128 components' operands are consumed
        stage_loads(kc);
      }
      // transposed into [position][component] (128 components per row)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned ou[4], ov[4];
        transpose4x4(wu[h], ou);
        transpose4x4(wv[h], ov);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<unsigned*>(&Us[(4 * pq + q) * kUpdPitch2 + 64 * h + 4 * cq]) = ou[q];
          *reinterpret_cast<unsigned*>(&Vs[(4 * pq + q) * kUpdPitch2 + 64 * h + 4 * cq]) = ov[q];
        }
      }
      __syncthreads();
      const int nsub = bs - kc < 128 ? (bs - kc + 63) / 64 : 2;
      for (int h = 0; h < nsub; ++h) {
        // A_t[i][c] = digit t of u_ic D_c (row i = 16 w + lr, c = kc + 64 h + 16 g ..): the bytes
        // of u (1, -1 = 0xFF, 0) as masks over the digit bytes of D_c and -D_c
        const v4i u4 = *reinterpret_cast<const v4i*>(&Us[(wid * 16 + lr) * kUpdPitch2 + 64 * h + 16 * g]);
        unsigned pm[4], nm[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned u = (unsigned)u4[q];
          const unsigned nb = (u >> 1) & 0x01010101u, pb = (u & 0x01010101u) ^ nb;
          nm[q] = (nb << 8) - nb;  // 0xFF in the bytes where u = -1
          pm[q] = (pb << 8) - pb;  // 0xFF where u = 1
        }
        v4i bv[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          bv[s2] = *reinterpret_cast<const v4i*>(&Vs[(s2 * 16 + lr) * kUpdPitch2 + 64 * h + 16 * g]);
        const int cb = kc + 64 * h + 16 * g;
#pragma unroll
        for (int t = 0; t < kDig; ++t) {
          const v4i dp = *reinterpret_cast<const v4i*>(&dg[0][t][cb]);
          const v4i dn = *reinterpret_cast<const v4i*>(&dg[1][t][cb]);
          v4i at;
#pragma unroll
          for (int q = 0; q < 4; ++q) at[q] = (int)(((unsigned)dp[q] & pm[q]) | ((unsigned)dn[q] & nm[q]));
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            acc[s2][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(at, bv[s2], acc[s2][t], 0, 0, 0);
        }
      }
    }
    // D(i, j) = sum_c A[i][c] V[j][c]: lane l, register r holds row 4 (l / 16) + r, column l % 16
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[s2][r] = ldexp((double)fx_combine(acc[s2], r), -f);
  } else {
    dbl4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = (dbl4){0.0, 0.0, 0.0, 0.0};
    for (int kc = 0; kc < bs4; kc += 64) {
      const int kn = bs4 - kc < 64 ? bs4 - kc : 64;
      __syncthreads();  // the previous chunk's operands are consumed
      // 16-byte pieces: rows of Ut / Vt are zero-padded to a multiple of 16, and i0, j0 are
      // multiples of 64, so a piece is either inside the padded row or past it
      {
        const int x = tid, c = x >> 2, q = (x & 3) * 16, cg = kc + c;
        if (c < kn) {
          // an out-of-range piece reads row 0's first bytes and is replaced by zeros
          const bool oku = cg < bs && i0 + q < ldu, okv = cg < bs && j0 + q < ldv;
          uint4 a = *reinterpret_cast<const uint4*>(oku ? Ut + (size_t)cg * ldu + i0 + q : Ut);
          uint4 b = *reinterpret_cast<const uint4*>(okv ? Vt + (size_t)cg * ldv + j0 + q : Vt);
          if (!oku) a = make_uint4(0u, 0u, 0u, 0u);
          if (!okv) b = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(&Us[c * kUpdPitch + q]) = a;
          *reinterpret_cast<uint4*>(&Vs[c * kUpdPitch + q]) = b;
        }
      }
      if (tid < kn) ds[tid] = kc + tid < bs ? dvec[kc + tid] : 0.0f;
      __syncthreads();
      // A[i][k] = d_k U[k][i], B[k][j] = V[k][j].  This MFMA leaves row a + 4 r of its output in
      // lane 16 a + j, register r; A's rows are supplied permuted (sigma(x) = 4 (x % 4) + x / 4)
      // so that lane l, register r holds row 4 (l / 16) + r, the layout of R's values above
      for (int k0 = 0; k0 < kn; k0 += 4) {
        const int k = k0 + (lane >> 4), x = lane & 15;
        const double a = (double)ds[k] * (double)Us[k * kUpdPitch + wid * 16 + 4 * (x & 3) + (x >> 2)];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const double bvv = (double)Vs[k * kUpdPitch + t * 16 + (lane & 15)];
          acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bvv, acc[t], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[t][r] = acc[t][r];
  }
  __shared__ float tt[64][65];  // the updated tile, transposed, for R^T
  unsigned mx = 0u;              // largest |R| of the tile after the update (fp32 bits)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int il = wid * 16 + (lane >> 4) * 4 + r, i = i0 + il;
      float x = rv[t][r];  // zero outside the matrix
      if (i < m && j < n) {
        if (sv[t][r] != 0.0) {
          x = (float)((double)x - sv[t][r]);
          R[(size_t)i * ldr + j] = x;
        }
        const unsigned b = __float_as_uint(x) & 0x7FFFFFFFu;
        mx = b > mx ? b : mx;
      }
      tt[t * 16 + (lane & 15)][il] = x;
    }
  }
  __shared__ unsigned wm[4];
  mx = wave_max_u32(mx);
  if (lane == 0) wm[wid] = mx;
  __syncthreads();
  // R^T rows j0 .. j0 + 63, entries i0 .. i0 + 63 (past m: zeros, R^T's padding up to ldt)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = tid + 256 * q, jl = x >> 4, iq = 4 * (x & 15);
    if (j0 + jl < n && i0 + iq < ldt)
      *reinterpret_cast<float4*>(RT + (size_t)(j0 + jl) * ldt + i0 + iq) =
          make_float4(tt[jl][iq], tt[jl][iq + 1], tt[jl][iq + 2], tt[jl][iq + 3]);
  }
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

// pp[c] = v_c^T H X[c] for the first V-step's X = U^T (R + X_blk) (int64 in units of *xunit) and
// the block's old V: one workgroup per component, fixed reduction order.
__global__ void __launch_bounds__(256) addback_dot_kernel(const long long* X, const double* xunit, int n,
                                                          const int8_t* Vt, int ldv, const float* h, double* pp) {
  __shared__ double red[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const double u = *xunit;
  double acc = 0.0;
  for (int j = tid; j < n; j += 256) {
    const int v = Vt[(size_t)c * ldv + j];
    if (v) acc += (double)v * (h ? (double)h[j] : 1.0) * ((double)X[(size_t)c * n + j] * u);
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

static void zero_fill(double* p, long long count, hipStream_t st) {
  const long long nb = (count + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, st, p, count);
}

// 16-component tiles per contraction workgroup (six digit accumulators each)
static int contract_nct(int bs) { return bs <= 16 ? 1 : bs <= 32 ? 2 : 4; }

// The contractions add their partial sums into outputs that start at zero (the selection before
// each clears the next one's output, or zero_fill does)
static bool rw_splits(const BlockLaunch&, int) { return true; }
static bool utr_splits(const BlockLaunch&, int) { return true; }

// out (bs x rows, int64) = T N(X)^T for the rows of X (ld ldx, K columns; hp: the padded weights
// or null), at the fixed-point scale of residual-max slot sblk; with spdG one more workgroup
// inverts spdG
static void contract(const BlockLaunch& L, const BlockWs& w, const float* X, int ldx, int rows, int K,
                     const float* hp, int sblk, const int8_t* T, int ldt, int bs, long long* out, double* unit,
                     hipStream_t st, bool prezeroed, const double* spdG, double* spdGi, bool ts_ready) {
  const int nct = contract_nct(bs), Kp = pad64(K);
  const int gx = (rows + 63) / 64, gy = (bs + 16 * nct - 1) / (16 * nct);
  if (!prezeroed) zero_fill(reinterpret_cast<double*>(out), (long long)bs * rows, st);
  if (!ts_ready) {  // else the selection that produced T wrote its swizzled copy
    const int nblk = gy * nct * (Kp / 64);  // every component tile the launch reads
    hipLaunchKernelGGL(swizzle_t_kernel, dim3((nblk + 3) / 4), dim3(256), 0, st, T, ldt, bs, gy * nct, Kp / 64, w.Ts);
  }
  // one workgroup per CU (their registers allow no more), one CU left to a fused inverse
  const int nwg = w.ncu - (spdG ? 1 : 0);
  const dim3 grid(nwg + (spdG ? 1 : 0));
  // weights in LDS when they fit beside nothing else (the inverse's LDS is its workgroup's own)
  const bool hlds = hp && (size_t)Kp * 4 <= kContractLds;
  size_t lds = spdG ? spd_lds_bytes(bs) : 0;
  if (hlds && (size_t)Kp * 4 > lds) lds = (size_t)Kp * 4;
#define EXTERND_CONTRACT(NCT, HW)                                                                             \
  hipLaunchKernelGGL((fx_contract_kernel<NCT, HW>), grid, dim3(512), lds, st, X, ldx, rows, Kp, hp, L.EHm, w.rmax, \
                     sblk, w.Ts, bs, gx, gy, nwg, out, unit, spdG, spdGi)
  if (hlds) {
    if (nct == 1) EXTERND_CONTRACT(1, 1);
    else if (nct == 2) EXTERND_CONTRACT(2, 1);
    else EXTERND_CONTRACT(4, 1);
  } else if (hp) {
    if (nct == 1) EXTERND_CONTRACT(1, 2);
    else if (nct == 2) EXTERND_CONTRACT(2, 2);
    else EXTERND_CONTRACT(4, 2);
  } else {
    if (nct == 1) EXTERND_CONTRACT(1, 0);
    else if (nct == 2) EXTERND_CONTRACT(2, 0);
    else EXTERND_CONTRACT(4, 0);
  }
#undef EXTERND_CONTRACT
}

// Y^T (bs x m) = (R diag(h) V^T)^T for V = Vt rows (h may be null: R V^T)
static void rw_product(const BlockLaunch& L, const BlockWs& w, const float* h, int bs, int sblk, long long* outT,
                       hipStream_t st, bool prezeroed, const double* spdG, double* spdGi, bool ts_ready) {
  contract(L, w, L.R, L.ldr, L.m, L.n, h ? w.hpad : nullptr, sblk, w.Vt, w.ldv, bs, outT, w.unit + 1, st, prezeroed,
           spdG, spdGi, ts_ready);
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

// X (bs x n) = U^T R, from the rows of R^T
static void utr_product(const BlockLaunch& L, const BlockWs& w, int bs, int sblk, hipStream_t st, bool prezeroed,
                        const double* spdG, double* spdGi, bool ts_ready) {
  contract(L, w, L.RT, L.ldt, L.n, L.m, nullptr, sblk, w.Ut, w.ldu, bs, w.Xi, w.unit, st, prezeroed, spdG, spdGi,
           ts_ready);
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

// bunit (nullable): Bm is a contraction's int64 output in units of *bunit
template <bool TA>
static void apply(const double* A, int bs, const double* Bm, const double* bunit, double* out, int ncols,
                  hipStream_t st) {
  const dim3 grid((ncols + 63) / 64);
  const int nrt = (bs + 15) / 16;
  if (nrt <= 1) hipLaunchKernelGGL((apply_kernel<1, TA>), grid, dim3(256), 0, st, A, bs, Bm, bunit, out, ncols);
  else if (nrt <= 2) hipLaunchKernelGGL((apply_kernel<2, TA>), grid, dim3(256), 0, st, A, bs, Bm, bunit, out, ncols);
  else if (nrt <= 4) hipLaunchKernelGGL((apply_kernel<4, TA>), grid, dim3(256), 0, st, A, bs, Bm, bunit, out, ncols);
  else if (nrt <= 8) hipLaunchKernelGGL((apply_kernel<8, TA>), grid, dim3(256), 0, st, A, bs, Bm, bunit, out, ncols);
  else hipLaunchKernelGGL((apply_kernel<16, TA>), grid, dim3(256), 0, st, A, bs, Bm, bunit, out, ncols);
}

// out (bs x ncols) = (G + eps I)^-1 in: one product with the inverse, or L^-T (L^-1 in) for
// bs > kSpdMax; in is a contraction's int64 output in units of *in_unit; in and out may not alias
static void solve(const BlockWs& w, int bs, const long long* in, const double* in_unit, double* out, int ncols,
                  hipStream_t st) {
  if (bs <= kSpdMax) {
    // one 16-column strip per workgroup: with several workgroups per CU one's loads overlap
    // another's products (measured faster than two or three strips per workgroup at every size)
    const dim3 grid((ncols + 15) / 16);
    if (bs <= 64)
      hipLaunchKernelGGL((apply_strip_kernel<1, 16, 1>), grid, dim3(256), 0, st, w.Li, bs, in, in_unit, out, ncols);
    else
      hipLaunchKernelGGL((apply_strip_kernel<2, 32, 1>), grid, dim3(256), 0, st, w.Li, bs, in, in_unit, out, ncols);
    return;
  }
  apply<false>(w.Li, bs, reinterpret_cast<const double*>(in), in_unit, w.Tmp, ncols, st);
  apply<true>(w.Li, bs, w.Tmp, nullptr, out, ncols, st);
}

// X: fp64 rows, or with xunit a contraction's int64 rows; Yd/ydunit: the int64 output whose row
// products with the selection give Md (see select_rows_kernel)
static void select_rows(const double* X, const double* xunit, int L, int ldT, int bs, float tau, const float* h,
                        int EHm, int8_t* T, double* PHC, int* flags, int flag_empty, hipStream_t st,
                        double* Z0 = nullptr, int zlen = 0, const long long* Yd = nullptr,
                        const double* ydunit = nullptr, double* Md = nullptr, int8_t* Ts = nullptr) {
  const size_t dyn = xunit ? sizeof(float) * (size_t)L : 0;
  // long rows take 1024 threads (only bs workgroups run, so the CUs have room)
  if (L > 4096) {
    if (h)
      hipLaunchKernelGGL((select_rows_kernel<true, 1024>), dim3(bs), dim3(1024), dyn, st, X, xunit, L, ldT, tau, h,
                         EHm, T, PHC, flags, flag_empty, Z0, zlen, Yd, ydunit, Md, Ts);
    else
      hipLaunchKernelGGL((select_rows_kernel<false, 1024>), dim3(bs), dim3(1024), dyn, st, X, xunit, L, ldT, tau, h,
                         EHm, T, PHC, flags, flag_empty, Z0, zlen, Yd, ydunit, Md, Ts);
    return;
  }
  if (h)
    hipLaunchKernelGGL((select_rows_kernel<true, 512>), dim3(bs), dim3(512), dyn, st, X, xunit, L, ldT, tau, h, EHm,
                       T, PHC, flags, flag_empty, Z0, zlen, Yd, ydunit, Md, Ts);
  else
    hipLaunchKernelGGL((select_rows_kernel<false, 512>), dim3(bs), dim3(512), dyn, st, X, xunit, L, ldT, tau, h, EHm,
                       T, PHC, flags, flag_empty, Z0, zlen, Yd, ydunit, Md, Ts);
}

hipError_t block_run(const BlockLaunch& L, hipStream_t st, double* flops, double* bytes) {
  if (L.b > 256) return hipErrorInvalidValue;
  static int ncu_of[64] = {};  // compute units of each device
  int dev = 0;
  {
    static bool scales_attr[64] = {};  // once per device: dynamic LDS above 64 KB
    hipError_t ea = hipGetDevice(&dev);
    if (ea != hipSuccess) return ea;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!scales_attr[dev]) {
      ea = hipDeviceGetAttribute(&ncu_of[dev], hipDeviceAttributeMultiprocessorCount, dev);
      if (ea != hipSuccess) return ea;
      if (ncu_of[dev] < 2) return hipErrorInvalidDevice;
      const void* kernels[4] = {(const void*)scales_kernel<1>, (const void*)scales_kernel<2>,
                                (const void*)scales_kernel<3>, (const void*)scales_kernel<4>};
      for (const void* kf : kernels) {
        ea = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(96 * 1024));
        if (ea != hipSuccess) return ea;
      }
      // the fp32 copy of an int64 row (up to 16384 values) beside the selection scratch
      const void* sel[4] = {(const void*)select_rows_kernel<true, 1024>, (const void*)select_rows_kernel<false, 1024>,
                            (const void*)select_rows_kernel<true, 512>, (const void*)select_rows_kernel<false, 512>};
      for (const void* kf : sel) {
        ea = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(64 * 1024));
        if (ea != hipSuccess) return ea;
      }
      // a contraction launch may carry the inverse of a b <= kSpdMax Gram (its LDS for all groups)
      const void* con[9] = {(const void*)fx_contract_kernel<1, 0>, (const void*)fx_contract_kernel<2, 0>,
                            (const void*)fx_contract_kernel<4, 0>, (const void*)fx_contract_kernel<1, 1>,
                            (const void*)fx_contract_kernel<2, 1>, (const void*)fx_contract_kernel<4, 1>,
                            (const void*)fx_contract_kernel<1, 2>, (const void*)fx_contract_kernel<2, 2>,
                            (const void*)fx_contract_kernel<4, 2>};
      for (const void* kf : con) {
        ea = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kContractLds);
        if (ea != hipSuccess) return ea;
      }

      scales_attr[dev] = true;
    }
  }
  BlockWs w = carve(L.ws, L.m, L.n, L.b, L.h != nullptr);
  w.ncu = ncu_of[dev];
  const int m = L.m, n = L.n;
  hipError_t e = hipSuccess;
  hipLaunchKernelGGL(block_init_kernel, dim3(1), dim3(256), 0, st, L.rowE, m, w.st, w.flags, w.rmax, w.gcnt);
  {
    const long long nb = ((long long)m * n + 255) / 256;
    hipLaunchKernelGGL(rmax_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, st, L.R, L.ldr, m, n,
                       w.rmax);
  }
  if (L.h) {
    hipLaunchKernelGGL(hdig_kernel, dim3((w.ldv + 255) / 256), dim3(256), 0, st, L.h, n, w.ldv, L.EHm, w.hdig);
    hipLaunchKernelGGL(hpad_kernel, dim3((pad64(n) + 255) / 256), dim3(256), 0, st, L.h, n, pad64(n), w.hpad);
  }
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
        utr_product(L, w, bs, sblk, st, true, nullptr, nullptr, t > 0);
        if (addback && t == 0) {
          hipLaunchKernelGGL(addback_dot_kernel, dim3(bs), dim3(256), 0, st, w.Xi, w.unit, n, w.Vt, w.ldv, L.h,
                             w.ppo);
          hipLaunchKernelGGL(addback_energy_kernel, dim3(1), dim3(256), 0, st, w.ppo, w.GU, w.GVo, L.D, k0, bs,
                             w.st, w.rmax + kMaxWords * ((sblk + 1) & 1), w.GUo);
        }
        select_rows(w.X, w.unit, n, w.ldv, bs, L.tau, hsel, ehsel, w.Vt, w.PHC, w.flags, 0, st, y0, m, nullptr,
                    nullptr, nullptr, w.Ts);
        gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GV, st);  // for the scales
        rw_product(L, w, L.h, bs, sblk, w.Yi, st, true, nullptr, nullptr, true);
        // the selection reads Yt while the last one also forms Md from it: Md reads the integers
        // (the selection converts its own copy in LDS)
        select_rows(w.Yt, w.unit + 1, m, w.ldu, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 0, st, x0, n,
                    t + 1 == L.T ? w.Yi : nullptr, w.unit + 1, t + 1 == L.T ? w.Md : nullptr, w.Ts);
        fl += 4.0 * m * n * bs;
        by += 2.0 * rbytes;
        continue;
      }
      // V-step: G = (U^T U + eps I)^-1 U^T R, rows ternarized with weights h.  For b <= kSpdMax the
      // inverse runs inside the contraction's launch, beside it; above, before it on the stream.
      if (fused) {
        gram_product(w, w.Ut, m, w.ldu, nullptr, 0, bs, w.GU, st);
        utr_product(L, w, bs, sblk, st, true, w.GU, w.Li, t > 0);
      } else {
        gram_product(w, w.Ut, m, w.ldu, nullptr, 0, bs, w.GU, st);
        chol_inverse(w, w.GU, bs, st);
        utr_product(L, w, bs, sblk, st, true, nullptr, nullptr, t > 0);
      }
      if (addback && t == 0) {
        hipLaunchKernelGGL(addback_dot_kernel, dim3(bs), dim3(256), 0, st, w.Xi, w.unit, n, w.Vt, w.ldv, L.h,
                           w.ppo);
        hipLaunchKernelGGL(addback_energy_kernel, dim3(1), dim3(256), 0, st, w.ppo, w.GU, w.GVo, L.D, k0, bs, w.st,
                           w.rmax + kMaxWords * ((sblk + 1) & 1), w.GUo);
      }
      solve(w, bs, w.Xi, w.unit, w.Z, n, st);
      select_rows(w.Z, nullptr, n, w.ldv, bs, L.tau, hsel, ehsel, w.Vt, w.PHC, w.flags, 0, st, y0, m, nullptr,
                  nullptr, nullptr, w.Ts);
      // U-step: F^T = (V^T H V + eps I)^-1 (R H V)^T, columns ternarized without weights
      if (fused) {
        gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GV, st);
        rw_product(L, w, L.h, bs, sblk, w.Yi, st, true, w.GV, w.Li, true);
      } else {
        gram_product(w, w.Vt, n, w.ldv, L.h, L.EHm, bs, w.GV, st);
        chol_inverse(w, w.GV, bs, st);
        rw_product(L, w, L.h, bs, sblk, w.Yi, st, true, nullptr, nullptr, true);
      }
      solve(w, bs, w.Yi, w.unit + 1, w.Ft, m, st);
      select_rows(w.Ft, nullptr, m, w.ldu, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 0, st, x0, n,
                  t + 1 == L.T ? w.Yi : nullptr, w.unit + 1, t + 1 == L.T ? w.Md : nullptr, w.Ts);
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
    hipLaunchKernelGGL(update_kernel, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, st, L.R, L.ldr, L.RT, L.ldt, m, n, w.Ut,
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
    rw_product(L, w, nullptr, bs, s, w.Yi, st, true, nullptr, nullptr, false);
    select_rows(w.Yt, w.unit + 1, m, w.ldu, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 1, st,
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
      hipLaunchKernelGGL(update_kernel, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, st, L.R, L.ldr, L.RT, L.ldt, m, n,
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
