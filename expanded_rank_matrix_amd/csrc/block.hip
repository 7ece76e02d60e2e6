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

struct BlockWs {
  int8_t* Ut;      // b x m, component-major
  int8_t* Vt;      // b x n (also holds Omega for the sketch)
  double* Yt;      // b x m: sketch / (R H V)^T
  double* Ft;      // b x m: F^T
  double* X;       // b x n: U^T R, then G
  double* part;    // split-K partials
  double* GU;      // b x b
  double* GV;      // b x b
  double* Lc;      // b x b Cholesky factor (lower triangle)
  double* LT;      // its transpose
  double* Md;      // b: u_c^T Q_c (diagonal of U^T R H V)
  double* PHC;     // b x 3 selection results
  float* d;        // b
  double* st;      // [0] E, [1] E0
  int* flags;      // [0] dead, [1] empty sketch columns, [2] fallbacks
  int* used;       // m: rows used by sketch fallbacks within the block
};

constexpr int kMaxSplit = 8;

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

static BlockWs carve(void* base, int m, int n, int b) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* r = p + o;
    o = al(o + bytes);
    return r;
  };
  BlockWs w;
  w.Ut = reinterpret_cast<int8_t*>(take((size_t)b * m));
  w.Vt = reinterpret_cast<int8_t*>(take((size_t)b * n));
  w.Yt = reinterpret_cast<double*>(take((size_t)b * m * 8));
  w.Ft = reinterpret_cast<double*>(take((size_t)b * m * 8));
  w.X = reinterpret_cast<double*>(take((size_t)b * n * 8));
  w.part = reinterpret_cast<double*>(take((size_t)kMaxSplit * b * (m > n ? m : n) * 8));
  w.GU = reinterpret_cast<double*>(take((size_t)b * b * 8));
  w.GV = reinterpret_cast<double*>(take((size_t)b * b * 8));
  w.Lc = reinterpret_cast<double*>(take((size_t)b * b * 8));
  w.LT = reinterpret_cast<double*>(take((size_t)b * b * 8));
  w.Md = reinterpret_cast<double*>(take((size_t)b * 8));
  w.PHC = reinterpret_cast<double*>(take((size_t)b * 3 * 8));
  w.d = reinterpret_cast<float*>(take((size_t)b * 4));
  w.st = reinterpret_cast<double*>(take(64));
  w.flags = reinterpret_cast<int*>(take(64));
  w.used = reinterpret_cast<int*>(take((size_t)m * 4));
  return w;
}

size_t block_workspace_bytes(int m, int n, int b) {
  size_t o = 0;
  auto take = [&](size_t bytes) { o = al(o + bytes); };
  take((size_t)b * m);
  take((size_t)b * n);
  take((size_t)b * m * 8);
  take((size_t)b * m * 8);
  take((size_t)b * n * 8);
  take((size_t)kMaxSplit * b * (m > n ? m : n) * 8);
  take((size_t)b * b * 8);
  take((size_t)b * b * 8);
  take((size_t)b * b * 8);
  take((size_t)b * b * 8);
  take((size_t)b * 8);
  take((size_t)b * 3 * 8);
  take((size_t)b * 4);
  take(64);
  take(64);
  take((size_t)m * 4);
  return o;
}

// ---- splitmix64 sketch signs (S. Vigna's splitmix64: golden-gamma step, then the mix) ----
__device__ __forceinline__ u64 splitmix64(u64 key) {
  u64 z = key + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) omega_kernel(int8_t* Vt, int bs, int n, long long s, int* flags) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    flags[1] = 0;  // empty sketch columns of this block
    flags[2] = 0;  // fallback starts of this block
  }
  const long long total = (long long)bs * n;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < total; x += (long long)gridDim.x * 256) {
    const int c = (int)(x / n), j = (int)(x - (long long)c * n);
    int8_t v = 1;
    if (c > 0) {
      const u64 key = (((u64)s << 16) + (u64)c) * (1ull << 32) + (u64)j;
      v = (splitmix64(key) >> 63) ? (int8_t)-1 : (int8_t)1;
    }
    Vt[x] = v;
  }
}

// ---- contraction 1: part[split][c][i] = sum_{j in split} R[i][j] * h_j * T[c][j] ------------
// MFMA f64 16x16x4: D(16x16) += A(16x4) B(4x16).  Lane l: A[l%16][l/16], B[l/16][l%16];
// D(i, j) in lane j + 16 (i % 4), register i / 4 (rows interleaved, unlike the fp32 forms).
// Tile: 64 rows of R (one 16-row strip per wave) x all components (NCT tiles of 16); K chunks
// of 32 columns staged in LDS.
template <int NCT, typename TR>
__global__ void __launch_bounds__(256) contract_rw_kernel(const TR* R, int ldr, int m, int n, const int8_t* T,
                                                          const float* h, int bs, int kspan, double* part) {
  constexpr int KC = 32;
  __shared__ float Rs[64][KC + 1];
  __shared__ int8_t Ts[16 * NCT][KC + 4];
  __shared__ float hs[KC];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int kb = split * kspan, ke = (kb + kspan < n) ? kb + kspan : n;
  dbl4 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = (dbl4){0.0, 0.0, 0.0, 0.0};
  for (int k0 = kb; k0 < ke; k0 += KC) {
    // stage R[i0 .. i0+63][k0 .. k0+31] (zero outside)
    for (int x = tid; x < 64 * KC; x += 256) {
      const int r = x / KC, c = x % KC;
      const int i = i0 + r, j = k0 + c;
      Rs[r][c] = (i < m && j < ke) ? (float)R[(size_t)i * ldr + j] : 0.0f;
    }
    for (int x = tid; x < 16 * NCT * KC; x += 256) {
      const int cc = x / KC, c = x % KC;
      const int j = k0 + c;
      Ts[cc][c] = (cc < bs && j < ke) ? T[(size_t)cc * n + j] : (int8_t)0;
    }
    if (tid < KC) {
      const int j = k0 + tid;
      hs[tid] = (j < ke) ? (h ? h[j] : 1.0f) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; kk += 4) {
      const int kq = kk + (lane >> 4);
      const double a = (double)Rs[wid * 16 + (lane & 15)][kq];
      const float hw = hs[kq];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const double bv = (double)(hw * (float)Ts[ct * 16 + (lane & 15)][kq]);
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc[ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  double* out = part + (size_t)split * bs * m;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = ct * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wid * 16 + (lane >> 4) + 4 * r;
      if (c < bs && i < m) out[(size_t)c * m + i] = acc[ct][r];
    }
  }
}

// ---- contraction 2: part[split][c][j] = sum_{i in split} U[c][i] * R[i][j] ----------------
// D rows = components (16 per tile), columns = j.  A[c][k] = U[c][i0+k], B[k][j] = R[i0+k][j].
// Tile: all components x 64 columns (one 16-column strip per wave); K chunks of 32 rows.
template <int NCT>
__global__ void __launch_bounds__(256) contract_utr_kernel(const float* R, int ldr, int m, int n, const int8_t* U,
                                                           int bs, int kspan, double* part) {
  constexpr int KC = 32;
  __shared__ float Rs[KC][64 + 1];
  __shared__ int8_t Us[16 * NCT][KC + 4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int j0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int kb = split * kspan, ke = (kb + kspan < m) ? kb + kspan : m;
  dbl4 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = (dbl4){0.0, 0.0, 0.0, 0.0};
  for (int k0 = kb; k0 < ke; k0 += KC) {
    for (int x = tid; x < KC * 64; x += 256) {
      const int r = x / 64, c = x % 64;
      const int i = k0 + r, j = j0 + c;
      Rs[r][c] = (i < ke && j < n) ? R[(size_t)i * ldr + j] : 0.0f;
    }
    for (int x = tid; x < 16 * NCT * KC; x += 256) {
      const int cc = x / KC, r = x % KC;
      const int i = k0 + r;
      Us[cc][r] = (cc < bs && i < ke) ? U[(size_t)cc * m + i] : (int8_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; kk += 4) {
      const int kq = kk + (lane >> 4);
      const double bv = (double)Rs[kq][wid * 16 + (lane & 15)];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const double a = (double)Us[ct * 16 + (lane & 15)][kq];
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc[ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  double* out = part + (size_t)split * bs * n;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int j = j0 + wid * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = ct * 16 + (lane >> 4) + 4 * r;
      if (c < bs && j < n) out[(size_t)c * n + j] = acc[ct][r];
    }
  }
}

// out[x] = sum over splits (ascending) of part[s][x]
__global__ void __launch_bounds__(256) reduce_splits_kernel(const double* part, int nsplit, long long count,
                                                            double* out) {
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < count; x += (long long)gridDim.x * 256) {
    double acc = 0.0;
    for (int s = 0; s < nsplit; ++s) acc += part[(size_t)s * count + x];
    out[x] = acc;
  }
}

// ---- Cholesky of G + eps I, eps = 1e-6 trace(G) / bs, by one workgroup of NT threads.  The
// lower triangle (packed, element e = i (i + 1) / 2 + k) is held in registers: slot q of thread t
// holds element q * NT + t.  Right-looking order: after step j every entry (i, k), k > j, has had
// L_ij L_kj subtracted, so each entry sees its subtractions in ascending t, as in the textbook
// left-looking formula.  Writes L (row-major) and its transpose.
constexpr int kCholSlots = 33;  // ceil(128 * 129 / 2 / 256) = ceil(256 * 257 / 2 / 1024) = 33
template <int NT>
__global__ void __launch_bounds__(NT) chol_kernel(const double* G, int bs, double* L, double* LT) {
#pragma clang fp contract(off)
  __shared__ double colb[2][256];  // column j in buffer j % 2 (no barrier needed between steps)
  __shared__ double eps_s;
  const int tid = threadIdx.x;
  const int ne = bs * (bs + 1) / 2;
  if (tid == 0) {
    double tr = 0.0;
    for (int c = 0; c < bs; ++c) tr += G[(size_t)c * bs + c];
    eps_s = 1e-6 * tr / (double)bs;
  }
  __syncthreads();
  const double eps = eps_s;
  double a[kCholSlots];
  int ik[kCholSlots];  // (i << 16) | k, or -1 for an unused slot
#pragma unroll
  for (int q = 0; q < kCholSlots; ++q) {
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
  for (int j = 0; j < bs; ++j) {
    double* col = colb[j & 1];
#pragma unroll
    for (int q = 0; q < kCholSlots; ++q)
      if (ik[q] == ((j << 16) | j)) {
        a[q] = a[q] > 0.0 ? sqrt(a[q]) : 0.0;
        col[j] = a[q];
      }
    __syncthreads();
    const double ljj = col[j];
#pragma unroll
    for (int q = 0; q < kCholSlots; ++q) {
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      if (ik[q] >= 0 && k == j && i > j) {
        a[q] = ljj > 0.0 ? a[q] / ljj : 0.0;
        col[i] = a[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCholSlots; ++q) {
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      if (ik[q] >= 0 && k > j) a[q] -= col[i] * col[k];
    }
  }
#pragma unroll
  for (int q = 0; q < kCholSlots; ++q)
    if (ik[q] >= 0) {
      const int i = ik[q] >> 16, k = ik[q] & 0xFFFF;
      L[(size_t)i * bs + k] = a[q];
      LT[(size_t)k * bs + i] = a[q];
    }
}

// ---- out[:, col] = (L L^T)^-1 in[:, col]: one column per lane, 64 columns per workgroup, the
// column in LDS (bs x 64 doubles); L and L^T are read at workgroup-uniform addresses.  The inner
// sums run in four interleaved partial sums.  in and out may alias.
__global__ void __launch_bounds__(64) solve_kernel(const double* __restrict__ L, const double* __restrict__ LT,
                                                   int bs, const double* in, double* out, int ncols) {
  extern __shared__ double xs[];
  const int lane = threadIdx.x;
  const int col = blockIdx.x * 64 + lane;
  const bool ok = col < ncols;
  for (int i = 0; i < bs; ++i) xs[i * 64 + lane] = ok ? in[(size_t)i * ncols + col] : 0.0;
  for (int i = 0; i < bs; ++i) {
    const double* Li = L + (size_t)i * bs;
    double p0 = 0.0, p1 = 0.0, p2 = 0.0, p3 = 0.0;
    int t = 0;
    for (; t + 4 <= i; t += 4) {
      p0 += Li[t] * xs[t * 64 + lane];
      p1 += Li[t + 1] * xs[(t + 1) * 64 + lane];
      p2 += Li[t + 2] * xs[(t + 2) * 64 + lane];
      p3 += Li[t + 3] * xs[(t + 3) * 64 + lane];
    }
    for (; t < i; ++t) p0 += Li[t] * xs[t * 64 + lane];
    const double s = xs[i * 64 + lane] - ((p0 + p1) + (p2 + p3));
    const double lii = Li[i];
    xs[i * 64 + lane] = lii > 0.0 ? s / lii : 0.0;
  }
  for (int i = bs - 1; i >= 0; --i) {
    const double* Ci = LT + (size_t)i * bs;  // column i of L
    double p0 = 0.0, p1 = 0.0, p2 = 0.0, p3 = 0.0;
    int t = i + 1;
    for (; t + 4 <= bs; t += 4) {
      p0 += Ci[t] * xs[t * 64 + lane];
      p1 += Ci[t + 1] * xs[(t + 1) * 64 + lane];
      p2 += Ci[t + 2] * xs[(t + 2) * 64 + lane];
      p3 += Ci[t + 3] * xs[(t + 3) * 64 + lane];
    }
    for (; t < bs; ++t) p0 += Ci[t] * xs[t * 64 + lane];
    const double s = xs[i * 64 + lane] - ((p0 + p1) + (p2 + p3));
    const double lii = Ci[i];
    xs[i * 64 + lane] = lii > 0.0 ? s / lii : 0.0;
  }
  if (ok)
    for (int i = 0; i < bs; ++i) out[(size_t)i * ncols + col] = xs[i * 64 + lane];
}

// ---- Md[c] = sum_i U[c][i] Y[c][i] (one workgroup per component, fixed reduction order)
__global__ void __launch_bounds__(256) rowdot_kernel(const int8_t* Ut, const double* Yt, int m, double* Md) {
  __shared__ double red[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double acc = 0.0;
  for (int i = tid; i < m; i += 256) {
    const int u = Ut[(size_t)c * m + i];
    if (u) acc += (double)u * Yt[(size_t)c * m + i];
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) red[wid] = acc;
  __syncthreads();
  if (tid == 0) Md[c] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ---- one workgroup per component row: T[c] = T_tau(fp32(X[c]); h) -----------------------------
template <bool W>
__global__ void __launch_bounds__(512) select_rows_kernel(const double* X, int L, float tau, const float* h,
                                                          int EHm, int8_t* T, double* PHC, int* flags,
                                                          int flag_empty) {
  __shared__ SelScratch s;
  const int c = blockIdx.x;
  const double* x = X + (size_t)c * L;
  if (flags[0]) {  // residual is zero: nothing to select
    for (int j = threadIdx.x; j < L; j += 512) T[(size_t)c * L + j] = 0;
    return;
  }
  const SelResult r = ternary_select<512, W>(x, h, L, tau, EHm, s);
  for (int j = threadIdx.x; j < L; j += 512) {
    const float xv = (float)x[j];
    T[(size_t)c * L + j] = selected(xv, r) ? (xv > 0.0f ? (int8_t)1 : (int8_t)-1) : (int8_t)0;
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
                                                       const double* PHC, int* flags, int* used) {
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
      for (int i = tid; i < m; i += 512) Ut[(size_t)c * m + i] = (i == r) ? (int8_t)1 : (int8_t)0;
      if (tid == 0) {
        used[r] = 1;
        flags[2] += 1;
      }
    }
    __syncthreads();
  }
}

// ---- scales and energy: one workgroup, thread t owns component t.  The sequential scale of each
// component against the residual left by the earlier ones of the block:
//   p_t = Md_t - sum_{c < t} d_c (u_t . u_c) (v_c^T H v_t),   d_t = fp32(p_t / q_t),
// the subtractions applied in ascending c (as the textbook loop does); the Gram of U is exactly
// symmetric (integer entries), so row c is read for column c.
__global__ void __launch_bounds__(256) scales_kernel(const double* Md, const double* GU, const double* GV, int bs,
                                                     int k0, int T, float* dvec, float* D, double* energy,
                                                     double* st, int* flags, u64* stats) {
#pragma clang fp contract(off)
  __shared__ float ds[256];
  __shared__ double ps[256], qs[256];
  const int tid = threadIdx.x;
  if (tid == 0) {
    if (flags[0]) {
      if (st[1] > 0.0) stats[3] += (u64)bs;  // zero components (none counted when A = 0)
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
    return;
  }
  const bool own = tid < bs;
  double acc = own ? Md[tid] : 0.0;
  const double q = own ? GU[(size_t)tid * bs + tid] * GV[(size_t)tid * bs + tid] : 0.0;
  double gu = own ? GU[tid] : 0.0, gv = own ? GV[tid] : 0.0;  // row 0
  for (int c = 0; c < bs; ++c) {
    if (tid == c) {
      const float d = q > 0.0 ? (float)(acc / q) : 0.0f;
      ds[c] = d;
      ps[c] = acc;
      qs[c] = q;
    }
    // prefetch row c + 1 before waiting
    double gu2 = 0.0, gv2 = 0.0;
    if (own && c + 1 < bs) {
      gu2 = GU[(size_t)(c + 1) * bs + tid];
      gv2 = GV[(size_t)(c + 1) * bs + tid];
    }
    __syncthreads();
    if (own && tid > c) acc -= (double)ds[c] * gu * gv;
    gu = gu2;
    gv = gv2;
  }
  __syncthreads();
  if (own) {
    dvec[tid] = ds[tid];
    D[k0 + tid] = ds[tid];
  }
  if (tid == 0) {
    double E = st[0];
    const double E0 = st[1];
    for (int c = 0; c < bs; ++c) {
      const double dd = (double)ds[c];
      E = E - (2.0 * dd * ps[c] - dd * dd * qs[c]);
      energy[k0 + c] = 1.0 - E / E0;
    }
    st[0] = E;
  }
}

// ---- update: R <- fl32(R - U diag(d) V^T), fp64 MFMA with K = bs ----------------------------
// Tile 64 x 64 of R; wave w owns rows 16w..16w+15 and four 16-column strips.
// A[i][k] = d_k U[k][i], B[k][j] = V[k][j].
__global__ void __launch_bounds__(256) update_kernel(float* R, int ldr, int m, int n, const int8_t* Ut,
                                                     const int8_t* Vt, const float* dvec, int bs, const int* flags) {
  if (flags[0]) return;
  __shared__ int8_t Us[256][64 + 4];
  __shared__ int8_t Vs[256][64 + 4];
  __shared__ float ds[256];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int bs4 = (bs + 3) & ~3;
  for (int x = tid; x < bs4 * 64; x += 256) {
    const int c = x / 64, r = x % 64;
    Us[c][r] = (c < bs && i0 + r < m) ? Ut[(size_t)c * m + i0 + r] : (int8_t)0;
    Vs[c][r] = (c < bs && j0 + r < n) ? Vt[(size_t)c * n + j0 + r] : (int8_t)0;
  }
  for (int c = tid; c < bs4; c += 256) ds[c] = c < bs ? dvec[c] : 0.0f;
  __syncthreads();
  dbl4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (dbl4){0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < bs4; k0 += 4) {
    const int k = k0 + (lane >> 4);
    const double a = (double)ds[k] * (double)Us[k][wid * 16 + (lane & 15)];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double bv = (double)Vs[k][t * 16 + (lane & 15)];
      acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wid * 16 + (lane >> 4) + 4 * r;
      if (i < m && j < n) {
        float* p = R + (size_t)i * ldr + j;
        const double s = acc[t][r];
        if (s != 0.0) *p = (float)((double)*p - s);
      }
    }
  }
}

// ---- emit: pack the block's components into B and C rows ----------------------------------
__global__ void __launch_bounds__(256) emit_kernel(const int8_t* Ut, const int8_t* Vt, int m, int n, int bs, int k0,
                                                   uint32_t* Bp, uint32_t* Cp, const int* flags) {
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  const bool dead = flags[0] != 0;
  const long long totB = (long long)bs * wm, totC = (long long)bs * wn;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < totB + totC; x += (long long)gridDim.x * 256) {
    const bool isB = x < totB;
    const long long y = isB ? x : x - totB;
    const int words = isB ? wm : wn, len = isB ? m : n;
    const int c = (int)(y / words), w = (int)(y - (long long)c * words);
    const int8_t* src = isB ? Ut + (size_t)c * m : Vt + (size_t)c * n;
    unsigned word = 0u;
    if (!dead)
      for (int q = 0; q < 16; ++q) {
        const int i = w * 16 + q;
        if (i < len) word |= tcode(src[i]) << (2 * q);
      }
    (isB ? Bp : Cp)[(size_t)(k0 + c) * words + w] = word;
  }
}

// E0 from the per-row energies (fixed order), dead flag for A = 0
__global__ void block_init_kernel(const double* rowE, int m, double* st, int* flags) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
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

template <int NCT, typename TR>
static void launch_rw(const TR* R, int ldr, int m, int n, const int8_t* T, const float* h, int bs, int nsplit,
                      double* part, hipStream_t st) {
  const int kspan = ((n + nsplit - 1) / nsplit + 31) / 32 * 32;
  hipLaunchKernelGGL((contract_rw_kernel<NCT, TR>), dim3((m + 63) / 64, nsplit), dim3(256), 0, st, R, ldr, m, n,
                     T, h, bs, kspan, part);
}

template <int NCT>
static void launch_utr(const float* R, int ldr, int m, int n, const int8_t* U, int bs, int nsplit, double* part,
                       hipStream_t st) {
  const int kspan = ((m + nsplit - 1) / nsplit + 31) / 32 * 32;
  hipLaunchKernelGGL(contract_utr_kernel<NCT>, dim3((n + 63) / 64, nsplit), dim3(256), 0, st, R, ldr, m, n, U, bs,
                     kspan, part);
}

// split-K factor: about 512 workgroups, at least 256 of K per split, at most cap splits
static int splits_for(int tiles, int K, int cap) {
  int s = (512 + tiles - 1) / tiles;
  const int maxs = (K + 255) / 256;
  s = s > maxs ? maxs : s;
  s = s > cap ? cap : s;
  return s < 1 ? 1 : s;
}

static void reduce_splits(const double* part, int ns, long long cnt, double* out, hipStream_t st) {
  const long long nb = (cnt + 255) / 256;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)(nb < 4096 ? nb : 4096)), dim3(256), 0, st, part, ns, cnt,
                     out);
}

// part[s][c][i] = sum over split s of R[i][j] h_j T[c][j], R rows x K (ld ldr), then out = sum over s
template <typename TR>
static void rw_contract(const TR* R, int ldr, int rows, int K, const int8_t* T, const float* h, int bs, int cap,
                        double* part, double* out, hipStream_t st) {
  const int ns = splits_for((rows + 63) / 64, K, cap);
  const int nct = (bs + 15) / 16;
  if (nct <= 1) launch_rw<1, TR>(R, ldr, rows, K, T, h, bs, ns, part, st);
  else if (nct <= 2) launch_rw<2, TR>(R, ldr, rows, K, T, h, bs, ns, part, st);
  else if (nct <= 4) launch_rw<4, TR>(R, ldr, rows, K, T, h, bs, ns, part, st);
  else if (nct <= 8) launch_rw<8, TR>(R, ldr, rows, K, T, h, bs, ns, part, st);
  else launch_rw<16, TR>(R, ldr, rows, K, T, h, bs, ns, part, st);
  reduce_splits(part, ns, (long long)bs * rows, out, st);
}

// Y^T (bs x m) = (R diag(h) T^T)^T
static void rw_product(const BlockLaunch& L, const BlockWs& w, const int8_t* T, const float* h, int bs,
                       double* outT, hipStream_t st) {
  rw_contract<float>(L.R, L.ldr, L.m, L.n, T, h, bs, kMaxSplit, w.part, outT, st);
}

// G (bs x bs) = T diag(w) T^T for ternary rows T (bs x len); integer-exact without weights
static void gram_product(const BlockLaunch& L, const BlockWs& w, const int8_t* T, int len, const float* wt, int bs,
                         double* G, hipStream_t st) {
  const int mx = L.m > L.n ? L.m : L.n;
  long long cap = (long long)kMaxSplit * mx / bs;  // partials must fit the split buffer
  cap = cap > 64 ? 64 : cap;
  rw_contract<int8_t>(T, len, bs, len, T, wt, bs, (int)cap, w.part, G, st);
}

// X (bs x n) = U^T R
static void utr_product(const BlockLaunch& L, const BlockWs& w, int bs, hipStream_t st) {
  const int ns = splits_for((L.n + 63) / 64, L.m, kMaxSplit);
  const int nct = (bs + 15) / 16;
  if (nct <= 1) launch_utr<1>(L.R, L.ldr, L.m, L.n, w.Ut, bs, ns, w.part, st);
  else if (nct <= 2) launch_utr<2>(L.R, L.ldr, L.m, L.n, w.Ut, bs, ns, w.part, st);
  else if (nct <= 4) launch_utr<4>(L.R, L.ldr, L.m, L.n, w.Ut, bs, ns, w.part, st);
  else if (nct <= 8) launch_utr<8>(L.R, L.ldr, L.m, L.n, w.Ut, bs, ns, w.part, st);
  else launch_utr<16>(L.R, L.ldr, L.m, L.n, w.Ut, bs, ns, w.part, st);
  reduce_splits(w.part, ns, (long long)bs * L.n, w.X, st);
}

// Cholesky of G + eps I into w.Lc / w.LT
static void cholesky(const BlockWs& w, const double* G, int bs, hipStream_t st) {
  if (bs <= 128)
    hipLaunchKernelGGL(chol_kernel<256>, dim3(1), dim3(256), 0, st, G, bs, w.Lc, w.LT);
  else
    hipLaunchKernelGGL(chol_kernel<1024>, dim3(1), dim3(1024), 0, st, G, bs, w.Lc, w.LT);
}

// out (bs x ncols) = (L L^T)^-1 in
static void solve(const BlockWs& w, int bs, const double* in, double* out, int ncols, hipStream_t st) {
  const size_t smem = (size_t)bs * 64 * sizeof(double);
  hipLaunchKernelGGL(solve_kernel, dim3((ncols + 63) / 64), dim3(64), smem, st, w.Lc, w.LT, bs, in, out, ncols);
}

static void select_rows(const double* X, int L, int bs, float tau, const float* h, int EHm, int8_t* T, double* PHC,
                        int* flags, int flag_empty, hipStream_t st) {
  if (h)
    hipLaunchKernelGGL(select_rows_kernel<true>, dim3(bs), dim3(512), 0, st, X, L, tau, h, EHm, T, PHC, flags,
                       flag_empty);
  else
    hipLaunchKernelGGL(select_rows_kernel<false>, dim3(bs), dim3(512), 0, st, X, L, tau, h, EHm, T, PHC, flags,
                       flag_empty);
}

hipError_t block_run(const BlockLaunch& L, hipStream_t st, double* flops) {
  if (L.b > 256) return hipErrorInvalidValue;
  const BlockWs w = carve(L.ws, L.m, L.n, L.b);
  const int m = L.m, n = L.n;
  {
    const hipError_t e = hipFuncSetAttribute((const void*)solve_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)((size_t)L.b * 64 * sizeof(double)));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(block_init_kernel, dim3(1), dim3(256), 0, st, L.rowE, m, w.st, w.flags);
  const int nblocks = (L.k + L.b - 1) / L.b;
  double fl = 0.0;
  for (int s = 0; s < nblocks; ++s) {
    const int bs = (L.k - s * L.b) < L.b ? (L.k - s * L.b) : L.b;
    const int k0 = s * L.b;
    // sketch
    hipLaunchKernelGGL(omega_kernel, dim3(256), dim3(256), 0, st, w.Vt, bs, n, (long long)s, w.flags);
    rw_product(L, w, w.Vt, nullptr, bs, w.Yt, st);
    select_rows(w.Yt, m, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 1, st);
    hipLaunchKernelGGL(zero_check_kernel, dim3(1), dim3(256), 0, st, L.R, L.ldr, m, n, w.flags, w.st);
    hipLaunchKernelGGL(fallback_kernel, dim3(1), dim3(512), 0, st, L.R, L.ldr, m, n, bs, w.Ut, w.PHC, w.flags,
                       w.used);
    fl += 2.0 * m * n * bs;
    for (int t = 0; t < L.T; ++t) {
      // V-step: G = (U^T U + eps I)^-1 U^T R, rows ternarized with weights h
      gram_product(L, w, w.Ut, m, nullptr, bs, w.GU, st);
      cholesky(w, w.GU, bs, st);
      utr_product(L, w, bs, st);
      solve(w, bs, w.X, w.X, n, st);
      select_rows(w.X, n, bs, L.tau, L.h, L.EHm, w.Vt, w.PHC, w.flags, 0, st);
      // U-step: F^T = (V^T H V + eps I)^-1 (R H V)^T, columns ternarized without weights
      gram_product(L, w, w.Vt, n, L.h, bs, w.GV, st);
      cholesky(w, w.GV, bs, st);
      rw_product(L, w, w.Vt, L.h, bs, w.Yt, st);
      solve(w, bs, w.Yt, w.Ft, m, st);
      select_rows(w.Ft, m, bs, L.tau, nullptr, 0, w.Ut, w.PHC, w.flags, 0, st);
      fl += 4.0 * m * n * bs;
    }
    // scales against Q = R H V of the last U-step, then the update and the outputs
    gram_product(L, w, w.Ut, m, nullptr, bs, w.GU, st);
    hipLaunchKernelGGL(rowdot_kernel, dim3(bs), dim3(256), 0, st, w.Ut, w.Yt, m, w.Md);
    hipLaunchKernelGGL(scales_kernel, dim3(1), dim3(256), 0, st, w.Md, w.GU, w.GV, bs, k0, L.T, w.d, L.D, L.energy,
                       w.st, w.flags, L.stats);
    hipLaunchKernelGGL(update_kernel, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, st, L.R, L.ldr, m, n, w.Ut,
                       w.Vt, w.d, bs, w.flags);
    hipLaunchKernelGGL(emit_kernel, dim3(256), dim3(256), 0, st, w.Ut, w.Vt, m, n, bs, k0, L.Bp, L.Cp, w.flags);
    fl += 2.0 * m * n * bs;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  *flops = fl;
  return hipGetLastError();
}

}  // namespace externd
