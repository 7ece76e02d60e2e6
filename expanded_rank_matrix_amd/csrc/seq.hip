// Sequential-deflation ALS as one persistent cooperative kernel (gfx950, wave64).
//
// Method (ExTernD review, Method and Key idea; pith.science, "What carries the argument"):
// component after component, u0 is the ternarized row-sum pattern of the residual; then
// als_iters times v = T_tau(R^T u; h) (V-step, corrected weighted projection) and
// u = T_tau(R H v) (U-step); the scale d = u^T R H v / (|u|^2 v^T H v) is rounded to fp32,
// the energy bookkeeping is E <- E - (2 d p - d^2 q), and the residual is deflated,
// R_ij <- fl32(R_ij - d u_i v_j), before the next component.  An iteration that reproduces the
// previous u (or v) has reached an exact fixed point; the remaining iterations would repeat it,
// so the loop stops there (the result is the same).
//
// MI355X layout.  The residual is kept twice: R (m x n) and its transpose RT (n x m), both
// row-major.  Workgroup g owns a fixed slab of R rows and a fixed slab of RT rows, so both
// matvecs are reduction-free across workgroups: a U-step row dot product z_i = R_i . (h v) and a
// V-step row dot product w_j = RT_j . u are finished inside the owning workgroup.  When it fits,
// the R slab lives in the workgroup's LDS for the whole run (the U-steps and the R half of the
// deflation never touch HBM) and only the RT slab is streamed; one XCD's RT slabs (m n / 8 floats)
// then fit its L2.  The only
// cross-workgroup traffic per half-step is the finished vector (z or w, fp64) plus one grid
// barrier; every workgroup then runs the same deterministic selection redundantly, so all of
// them agree on u or v without a broadcast.  Deflation is applied lazily: the pending component
// is subtracted from RT rows during the next V-step read and from R rows during the next U-step
// read (one read-modify-write pass fused with a matvec).  The tracked row sums rs (fp64
// recurrence rs <- rs - d (sum v) u) are replicated: every workgroup keeps a private copy in
// global memory (it stays in its XCD's L2), so the next u0 is chosen without another exchange.
#include <algorithm>

#include "externd_internal.hpp"
#include "select.hpp"

namespace externd {

struct SeqArgs {
  float* R;    // m x ldr
  float* RT;   // n x ldt
  const float* h;
  const double* rs0;   // m
  const double* rowE;  // m
  double* xz;          // m
  double* xw;          // n
  double* xf;          // 4 * gridDim.x
  double* rsg;         // gridDim.x x m: private row-sum copies
  unsigned* bar;
  uint32_t* Bp;
  uint32_t* Cp;
  float* D;
  double* energy;
  u64* stats;          // [0] passes [1] early exits [2] fallbacks [3] zero components
                       // [4] safeguard activations [5] components fitted before a target stop
                       // [6] refits discarded for the old component
  double* bytes;       // algorithmic bytes
  int m, n, ldr, ldt, k, T, wm, wn, EHm;
  float tau;
  unsigned spin_limit;
  double target;       // > 0: stop once the energy reaches it
  int safeguard;       // 1: Prop. 2 best single-entry safeguard
  int sweeps;          // refinement sweeps after the greedy pass
  int ablation;        // 2: the V-step projection ignores the weights
};

__device__ __forceinline__ int code_at(const uint32_t* pk, int i) {
  const unsigned c = (pk[i >> 4] >> ((i & 15) * 2)) & 3u;
  return c == 0u ? 0 : (c == 1u ? 1 : -1);
}

// Dynamic LDS of the sequential kernel; every region starts on a 16-byte boundary.
struct SeqLds {
  size_t dl, kl, hl, pk, part, slab, total;
};
__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }
// keys: the LDS array of the exchanged vector's fp32 bit patterns, which the unweighted
// selections and the packing read (without it they take the general selection and round the
// fp64 values themselves).
__host__ __device__ inline SeqLds seq_lds_layout(int m, int n, bool weighted, int G, bool rl, bool keys) {
  const size_t L = (size_t)(m > n ? m : n);
  const size_t n4 = (size_t)((n + 3) & ~3), m4 = (size_t)((m + 3) & ~3);
  const size_t wm = (size_t)((m + 15) / 16), wn = (size_t)((n + 15) / 16);
  const size_t parts = 8 * 16;  // matvec segment sums (at least kMvPart)
  SeqLds s;
  s.dl = al16(weighted ? sizeof(SelScratchT<true>) : sizeof(SelScratchT<false>));
  s.kl = al16(s.dl + 8 * L);
  s.hl = al16(s.kl + (keys ? 4 * L : 0));
  s.pk = al16(s.hl + (weighted ? 4 * n4 : 0));
  s.part = al16(s.pk + 4 * (4 * wm + 3 * wn + 4));
  s.slab = al16(s.part + 8 * parts);
  s.total = al16(s.slab + (rl ? 4 * n4 * (((size_t)m + G - 1) / G) : 0));
  return s;
}

struct SeqShared {
  int ivals[8];
  int pk_changed[16];
  int pk_sum[16];
  double pk_p[16];
};

struct PackOut {
  int changed;  // some word differs from the previous contents
  int sum;      // signed sum of the codes
  double p;     // sum of |vals| over the support (when asked for)
};

// Rows [r0, r1) of a row-major matrix (leading dimension ld floats, len4 float4 per row) dotted
// with a packed ternary vector pk_w (times the LDS weights hl when given); the results go to
// out[row] (exchange buffer, device-coherent stores).  Each row is split into S column segments
// (S a power of two, chosen so that the R x S (row, segment) items spread evenly over the waves);
// wave w owns segment w % S of rows w / S, w / S + waves / S, ...  A lane covers float4 columns
// lane, lane + 64, ... of its segment in chunks of kQL, kRW rows at a time; it decodes the weights
// of a chunk once for all of its rows when the segment is one chunk, else once per group of rows.
// A row's sum is fixed-order: lane partials, a DPP wave sum,
// then the segments in order: deterministic, with one barrier only when S > 1.  Pending deflation
// of rows whose own code in pk_own is nonzero is fused in: x <- fl32(x - own * other * d) where
// pk_other is nonzero, written back by the wave that owns the (row, segment).
constexpr int kQMax = 8;    // longest row accepted: len4 <= kQMax * 512 float4 (n <= 16384)
constexpr int kQL = 5;     // float4 columns per lane per chunk
constexpr int kRW = 2;     // rows of one wave handled together (more spills registers)
constexpr int kMvPart = 8 * 16;  // LDS doubles for the segment sums (needs R * S <= 3 * waves)
// The 2-bit code at bit offset off of word (0, 1 or 3 = -1) as -1, 0, 1: a signed bit-field
// extract.
__device__ __forceinline__ int code2(unsigned word, int off) { return __builtin_amdgcn_sbfe(word, off, 2); }
template <int NT>
__device__ __forceinline__ void slab_matvec(float* base, int row_base, int ld, int len4, int r0, int r1,
                                            const uint32_t* pk_w, const float* hl, bool apply,
                                            const uint32_t* pk_own, const uint32_t* pk_other, float d,
                                            double* part, double* out) {
  constexpr int NW = NT / 64;
  static_assert(kMvPart >= 3 * NW, "segment sums need 3 x waves doubles");
  // the wave index as a scalar, so that the item loops below branch per wave instead of masking
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = r1 - r0;
  if (R <= 0) return;
  int S = 1;
  while (S < NW && R * (2 * S) <= 3 * NW) S *= 2;
  const int seg = wid % S, rw0 = wid / S, rstep = NW / S;
  const int segq = (len4 + S - 1) / S;
  const int qb = seg * segq, qe = min(len4, qb + segq);
  const int mine = R > rw0 ? (R - rw0 + rstep - 1) / rstep : 0;  // rows r0 + rw0 + rstep * j
  const float4* h4 = reinterpret_cast<const float4*>(hl);
  // Every load of a chunk (the rows, their weights, the deflation codes) is issued before any is
  // used: indexes past the segment are clamped to its last column and their weights and codes
  // masked to zero, so they add 0 * x and are never written back.
  auto load_rows = [&](int j0, int nr, int q0, float4 (&xr)[kRW][kQL]) {
#pragma unroll
    for (int k = 0; k < kRW; ++k) {
      if (k < nr) {  // uniform within the wave
        const float4* r4 = reinterpret_cast<const float4*>(base + (size_t)(r0 + rw0 + rstep * (j0 + k) - row_base) * ld);
#pragma unroll
        for (int qi = 0; qi < kQL; ++qi) {
          const int q = q0 + lane + 64 * qi;
          xr[k][qi] = r4[q < qe ? q : qe - 1];
        }
      }
    }
  };
  auto decode = [&](int q0, double (&w)[kQL][4], float (&od)[kQL][4]) {
#pragma unroll
    for (int qi = 0; qi < kQL; ++qi) {
      const int q = q0 + lane + 64 * qi;
      const int qc = q < qe ? q : qe - 1;
      const unsigned okm = q < qe ? 0xFFFFFFFFu : 0u;
      const unsigned word = pk_w[qc >> 2] & okm;
      const int off = (q & 3) * 8;
      float4 h = make_float4(1.f, 1.f, 1.f, 1.f);
      if (hl) h = h4[qc];
      const float hh[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const double c = (double)code2(word, off + 2 * t);
        w[qi][t] = hl ? c * (double)hh[t] : c;
      }
      if (apply) {
        const unsigned ow = pk_other[qc >> 2] & okm;
#pragma unroll
        for (int t = 0; t < 4; ++t) od[qi][t] = d * (float)code2(ow, off + 2 * t);
      }
    }
  };
  auto own_codes = [&](int j0, int nr, int (&oc)[kRW]) {
#pragma unroll
    for (int k = 0; k < kRW; ++k) oc[k] = (apply && k < nr) ? code_at(pk_own, r0 + rw0 + rstep * (j0 + k)) : 0;
  };
  auto compute = [&](int j0, int nr, int q0, const float4 (&xr)[kRW][kQL], const double (&w)[kQL][4],
                     const float (&od)[kQL][4], const int (&oc)[kRW], double (&acc)[kRW]) {
#pragma unroll
    for (int k = 0; k < kRW; ++k) {
      if (k >= nr) break;  // uniform within the wave
      const int row = r0 + rw0 + rstep * (j0 + k);
      float4* r4 = reinterpret_cast<float4*>(base + (size_t)(row - row_base) * ld);
      double a0 = 0.0, a1 = 0.0;
#pragma unroll
      for (int qi = 0; qi < kQL; ++qi) {
        float v[4] = {xr[k][qi].x, xr[k][qi].y, xr[k][qi].z, xr[k][qi].w};
        if (oc[k] != 0) {  // uniform within the wave
          const float sg = oc[k] > 0 ? -1.0f : 1.0f;
          bool any = false;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[t] = fmaf(sg, od[qi][t], v[t]);
            any = any || od[qi][t] != 0.0f;
          }
          const int q = q0 + lane + 64 * qi;
          if (q < qe && any) r4[q] = make_float4(v[0], v[1], v[2], v[3]);
        }
        a0 = fma((double)v[0], w[qi][0], a0);
        a1 = fma((double)v[1], w[qi][1], a1);
        a0 = fma((double)v[2], w[qi][2], a0);
        a1 = fma((double)v[3], w[qi][3], a1);
      }
      acc[k] += a0 + a1;
    }
  };
  auto finish = [&](int j0, int nr, const double (&acc)[kRW]) {
#pragma unroll
    for (int k = 0; k < kRW; ++k) {
      if (k >= nr) break;
      const int rl = rw0 + rstep * (j0 + k);
      const double v = wave_sum_f64(acc[k]);
      if (lane == 0) {
        if (S == 1) st_dev(out + r0 + rl, v);
        else part[rl * S + seg] = v;
      }
    }
  };
  if (qe - qb <= 64 * kQL) {
    // the segment is one chunk: its weights are decoded once for all of the wave's rows
    double w[kQL][4];
    float od[kQL][4];
    for (int j0 = 0; j0 < mine; j0 += kRW) {
      const int nr = min(kRW, mine - j0);
      float4 xr[kRW][kQL];
      load_rows(j0, nr, qb, xr);
      if (j0 == 0) decode(qb, w, od);  // overlaps the first rows' loads
      int oc[kRW];
      own_codes(j0, nr, oc);
      double acc[kRW];
#pragma unroll
      for (int k = 0; k < kRW; ++k) acc[k] = 0.0;
      compute(j0, nr, qb, xr, w, od, oc, acc);
      finish(j0, nr, acc);
    }
  } else {
    for (int j0 = 0; j0 < mine; j0 += kRW) {
      const int nr = min(kRW, mine - j0);
      int oc[kRW];
      own_codes(j0, nr, oc);
      double acc[kRW];
#pragma unroll
      for (int k = 0; k < kRW; ++k) acc[k] = 0.0;
      for (int q0 = qb; q0 < qe; q0 += 64 * kQL) {
        float4 xr[kRW][kQL];
        load_rows(j0, nr, q0, xr);
        double w[kQL][4];
        float od[kQL][4];
        decode(q0, w, od);
        compute(j0, nr, q0, xr, w, od, oc, acc);
      }
      finish(j0, nr, acc);
    }
  }
  if (S > 1) {
    __syncthreads();
    if (tid < R) {
      double t = 0.0;
      for (int s2 = 0; s2 < S; ++s2) t += part[tid * S + s2];
      st_dev(out + r0 + tid, t);
    }
  }
}

// Apply the pending deflation to rows [r0, r1) (used where no matvec pass is due).
template <int NT>
__device__ __forceinline__ void slab_deflate(float* base, int row_base, int ld, int len4, int r0, int r1, const uint32_t* pk_own,
                             const uint32_t* pk_other, float d) {
  for (int r = r0; r < r1; ++r) {
    const int oc = code_at(pk_own, r);
    if (oc == 0) continue;
    float4* r4 = reinterpret_cast<float4*>(base + (size_t)(r - row_base) * ld);
    for (int q = threadIdx.x; q < len4; q += NT) {
      const unsigned word = pk_other[q >> 2] >> ((q & 3) * 8);
      if (!(word & 0xFFu)) continue;
      float4 x = r4[q];
      float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const unsigned cd = (word >> (2 * c)) & 3u;
        if (cd != 0u) {
          const int sg = (cd == 1u ? 1 : -1) * oc;
          xv[c] = sg > 0 ? xv[c] - d : xv[c] + d;
        }
      }
      r4[q] = make_float4(xv[0], xv[1], xv[2], xv[3]);
    }
  }
  __syncthreads();
}

// Per-workgroup part of the safeguard's search: the largest h_j R_ij^2 over rows [r0, r1)
// (smallest row-major index on ties); wave w leaves (value, index, R_ij) in part[3w..3w+2].
// Rows are read as float4 (ld is a multiple of 4); a lane visits its entries in increasing index
// order, so a strict comparison keeps the smallest index among its equal maxima.
template <int NW>
__device__ __forceinline__ void best_entry_rows(const float* Rb, int Rrow0, int Rld, int r0, int r1, int n,
                                                const float* hl, double* part) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int q4 = (n + 3) >> 2;
  double best = 0.0;
  int bidx = -1;
  float bval = 0.0f;
  for (int i = r0 + wid; i < r1; i += NW) {
    const float4* row = reinterpret_cast<const float4*>(Rb + (size_t)(i - Rrow0) * Rld);
    for (int q = lane; q < q4; q += 64) {
      const float4 x4 = row[q];
      const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * q + c;
        const double r = (double)xs[c];
        const double sv = (hl ? (double)hl[j < n ? j : 0] * r : r) * r;
        if (j < n && sv > best) {
          best = sv;
          bidx = i * n + j;
          bval = xs[c];
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double b2 = __shfl_xor(best, o);
    const int i2 = __shfl_xor(bidx, o);
    const float v2 = __shfl_xor(bval, o);
    if (b2 > best || (b2 == best && b2 > 0.0 && i2 < bidx)) {
      best = b2;
      bidx = i2;
      bval = v2;
    }
  }
  if (lane == 0) {
    part[3 * wid] = best;
    part[3 * wid + 1] = (double)bidx;
    part[3 * wid + 2] = (double)bval;
  }
  __syncthreads();
}

// Start of a refit in a refinement sweep: the pending deflation of the previous fit is applied to
// this workgroup's rows of both residual copies (where not yet fused), then the component's
// previous codes are read back (device-coherent) into du/dv (its add-back, the new pending
// update) and pu (the ALS's initial u).  Workgroup 0 adds the deflation's bytes to *bytes.
template <int NT>
__device__ __forceinline__ void refit_begin(float* Rb, int Rrow0, int Rld, int len4r, float* RT, int ldt, int len4t,
                                         int r0, int r1, int c0, int c1, bool apply_r, bool apply_rt, float pd,
                                         uint32_t* du, uint32_t* dv, uint32_t* pu, const uint32_t* Bk,
                                         const uint32_t* Ck, int wm, int wn, double* bytes) {
  __shared__ int cnt[2];
  const int tid = threadIdx.x;
  if (tid == 0) {
    cnt[0] = 0;
    cnt[1] = 0;
  }
  __syncthreads();
  if (apply_r) slab_deflate<NT>(Rb, Rrow0, Rld, len4r, r0, r1, du, dv, pd);
  if (apply_rt) slab_deflate<NT>(RT, 0, ldt, len4t, c0, c1, dv, du, pd);
  if (bytes) {
    int pu_n = 0, pv_n = 0;
    if (apply_r)
      for (int w = tid; w < wm; w += NT) pu_n += __popc((du[w] | (du[w] >> 1)) & 0x55555555u);
    if (apply_rt)
      for (int w = tid; w < wn; w += NT) pv_n += __popc((dv[w] | (dv[w] >> 1)) & 0x55555555u);
    if (pu_n) atomicAdd(&cnt[0], pu_n);
    if (pv_n) atomicAdd(&cnt[1], pv_n);
  }
  __syncthreads();
  if (bytes && tid == 0)  // rows of R and of its transpose read and written
    bytes[0] += 8.0 * (double)(len4r * 4) * (double)cnt[0] + 8.0 * (double)(len4t * 4) * (double)cnt[1];
  for (int w = tid; w < wm; w += NT) {
    const unsigned x = ld_dev(Bk + w);
    du[w] = x;
    pu[w] = x;
  }
  for (int w = tid; w < wn; w += NT) dv[w] = ld_dev(Ck + w);
  __syncthreads();
}

// 2 d v^T H w - d^2 |u|^2 |v|^2_H for the exchanged w (dl) and the packed u, v: the change of
// the energy when d u v^T is added back to the residual behind w = (R + d u v^T)^T u.  Sums in
// a fixed order; each thread reads only the dl entries it stored itself.
template <int NT>
__device__ __forceinline__ double addback_energy(const double* dl, const uint32_t* du, const uint32_t* dv,
                                              const float* hl, int n, int wm, double d, double* part) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double pv_acc = 0.0, hv_acc = 0.0, un_acc = 0.0;
  for (int j = tid; j < n; j += NT) {
    const int c = code_at(dv, j);
    if (c != 0) {
      const double hj = hl ? (double)hl[j] : 1.0;
      pv_acc += (double)c * hj * dl[j];
      hv_acc += hj;
    }
  }
  for (int w = tid; w < wm; w += NT) un_acc += (double)__popc((du[w] | (du[w] >> 1)) & 0x55555555u);
  pv_acc = wave_sum_f64(pv_acc);
  hv_acc = wave_sum_f64(hv_acc);
  un_acc = wave_sum_f64(un_acc);
  __syncthreads();
  if (lane == 0) {
    part[3 * wid] = pv_acc;
    part[3 * wid + 1] = hv_acc;
    part[3 * wid + 2] = un_acc;
  }
  __syncthreads();
  double pp = 0.0, hh = 0.0, uu = 0.0;
  for (int w = 0; w < NW; ++w) {
    pp += part[3 * w];
    hh += part[3 * w + 1];
    uu += part[3 * w + 2];
  }
  __syncthreads();
  return 2.0 * d * pp - d * d * (uu * hh);
}

template <int NT, bool WV, bool RL, bool EXT, bool KEYS>
__global__ void __launch_bounds__(NT) seq_kernel(SeqArgs a) {
  constexpr int NW = NT / 64;
  extern __shared__ __align__(16) char smem[];
  SelScratchT<WV>& s = *reinterpret_cast<SelScratchT<WV>*>(smem);
  const int m = a.m, n = a.n;
  const int m4 = (m + 3) & ~3, n4 = (n + 3) & ~3;
  const SeqLds lay = seq_lds_layout(m, n, WV, (int)gridDim.x, RL, KEYS);
  double* dl = reinterpret_cast<double*>(smem + lay.dl);    // exchanged vector (z or w)
  unsigned* kl = reinterpret_cast<unsigned*>(smem + lay.kl);  // its fp32 roundings (bit patterns)
  float* hl = reinterpret_cast<float*>(smem + lay.hl);      // n4 column weights (weighted)
  uint32_t* pk = reinterpret_cast<uint32_t*>(smem + lay.pk);
  double* part = reinterpret_cast<double*>(smem + lay.part);
  const int wm = a.wm, wn = a.wn;
  uint32_t* pu = pk;            // current u
  uint32_t* pv = pu + wm;       // current v
  uint32_t* pu_prev = pv + wn;  // u that produced the current v
  uint32_t* du = pu_prev + wm;  // pending deflation component
  uint32_t* dv = du + wm;
  uint32_t* pu0 = dv + wn;      // u0 of this component (for the byte count)
  __shared__ SeqShared sh;
  __shared__ int bar_flag;
  // workgroup 0's per-component statistics, accumulated here and added to stats / bytes once at
  // the end (no global read-modify-write on the way to the next component)
  __shared__ u64 st_acc[5];  // passes, early exits, fallbacks, safeguard activations, reverts
  __shared__ double bytes_acc;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const int r0 = (int)((long long)g * m / G), r1 = (int)((long long)(g + 1) * m / G);
  const int c0 = (int)((long long)g * n / G), c1 = (int)((long long)(g + 1) * n / G);
  const float* hw = WV ? hl : nullptr;
  unsigned epoch = 0;
  double* rs = a.rsg + (size_t)g * m;  // this workgroup's copy of the row sums
  // the residual rows this workgroup owns: LDS-resident (RL) or in HBM
  float* Rb = RL ? reinterpret_cast<float*>(smem + lay.slab) : a.R;
  const int Rld = RL ? n4 : a.ldr, Rrow0 = RL ? r0 : 0;

  if (tid < 5) st_acc[tid] = 0ull;
  if (tid == 0) bytes_acc = 0.0;
  for (int i = tid; i < m; i += NT) rs[i] = a.rs0[i];
  if (RL) {
    const int q4 = n4 / 4;
    for (int x = tid; x < (r1 - r0) * q4; x += NT) {
      const int r = x / q4, q = x - r * q4;
      reinterpret_cast<float4*>(Rb + (size_t)r * n4)[q] =
          reinterpret_cast<const float4*>(a.R + (size_t)(r0 + r) * a.ldr)[q];
    }
  }
  if (WV)
    for (int j = tid; j < n4; j += NT) hl[j] = j < n ? a.h[j] : 0.0f;
  for (int i = tid; i < 4 * wm + 3 * wn; i += NT) pk[i] = 0u;
  double e0 = 0.0;
  for (int i = tid; i < m; i += NT) e0 += a.rowE[i];
  e0 = wave_sum_f64(e0);
  if (lane == 0) s.f_s[wid] = e0;
  __syncthreads();
  double E0 = 0.0;
  for (int w = 0; w < NW; ++w) E0 += s.f_s[w];
  double E = E0;
  bool dead = !(E0 > 0.0);
  bool have_pending = false, r_applied = true, rt_applied = true;
  float pd = 0.0f;
  __syncthreads();

  // Read the exchanged vector (device-coherent loads) into LDS; its largest key and the cleared
  // histogram are prepared for the selection on the way (one barrier).
  // Loads are issued in groups of kXg per thread before any is used, so their latencies overlap.
  constexpr int kXg = 8;
  auto load_exchange = [&](const double* src, int len) {
    unsigned kx = 0u;
    for (int j0 = tid; j0 < len; j0 += kXg * NT) {
      double v[kXg];
#pragma unroll
      for (int u = 0; u < kXg; ++u) v[u] = j0 + u * NT < len ? ld_dev(src + j0 + u * NT) : 0.0;
#pragma unroll
      for (int u = 0; u < kXg; ++u) {
        const unsigned kb = __float_as_uint((float)v[u]);
        if (j0 + u * NT < len) {
          dl[j0 + u * NT] = v[u];
          if (KEYS) kl[j0 + u * NT] = kb;
        }
        const unsigned k = kb & 0x7FFFFFFFu;
        kx = k > kx ? k : kx;
      }
    }
    select_prepare<NT>(s, kx);
  };
  // Unweighted projection of the vector in dl / kl (select_prepare done): the key-array selection,
  // or, when its candidate window is too wide or there is no key array, the general one (same
  // result either way).
  auto select_unweighted = [&](int len) -> SelResult {
    if (!KEYS) return ternary_select<NT, false, double, WV, true>(dl, nullptr, len, a.tau, 0, s);
    unsigned km = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) km = s.red_u[w] > km ? s.red_u[w] : km;
    bool ok = true;
    const SelResult r = ternary_select_keys<NT>(kl, len, a.tau, km, s, &ok);
    if (ok) return r;
    select_prepare<NT>(s, km);
    return ternary_select<NT, false, double, WV, true>(dl, nullptr, len, a.tau, 0, s);
  };
  // Pack the selection r of vals[0..len) into dst (2-bit codes).  Wave w takes the 256-element
  // groups w, w + NW, ...; lane l reads elements 4l..4l+3 of a group with one 16-byte load,
  // forms their 8 code bits at bit 8 (l % 4) of its word, and an OR over lanes l - 3..l (two DPP
  // row shifts) leaves word l / 4 of the group in lane l when l % 4 == 3, which writes it.  prev,
  // when given, receives the old words.  Block totals are combined in wave order (deterministic).
  auto pack_sel = [&](const double* vals, const unsigned* kv, int len, const SelResult& r, uint32_t* dst,
                      uint32_t* prev, bool want_p) -> PackOut {
    const int words = (len + 15) >> 4;
    const int ng = (len + 255) >> 8;
    int changed = 0, sum = 0;
    double pacc = 0.0;
    // the support is |key| >= kthr; kthr >= 1, so zero entries and the masked tail never enter
    const unsigned kthr = r.count > 0u ? max(max(r.ekey, r.tkey), 1u) : 0xFFFFFFFFu;
    const bool holder = (lane & 3) == 3;
    const int sh8 = 8 * (lane & 3);
    constexpr int kPg = 2;  // groups per wave whose loads are issued together
    for (int g0 = __builtin_amdgcn_readfirstlane(wid); g0 < ng; g0 += kPg * NW) {
      unsigned kq[kPg][4];
      double av[kPg][4];  // |vals| (when want_p)
      unsigned olds[kPg];
#pragma unroll
      for (int u = 0; u < kPg; ++u) {
        const int g = g0 + u * NW, i = g * 256 + 4 * lane, w = g * 16 + (lane >> 2);
        // 16-byte loads at a clamped index (the regions are padded to 16 bytes, so a group's last
        // load stays inside them); elements past len are masked below
        const int ic = (g < ng && i < len) ? i : 0;
        if (KEYS) {
          const uint4 k4 = *reinterpret_cast<const uint4*>(kv + ic);
          kq[u][0] = k4.x;
          kq[u][1] = k4.y;
          kq[u][2] = k4.z;
          kq[u][3] = k4.w;
        }
        if (!KEYS || want_p) {
          const double2 v01 = *reinterpret_cast<const double2*>(vals + ic);
          const double2 v23 = *reinterpret_cast<const double2*>(vals + ic + 2);
          const double vv[4] = {v01.x, v01.y, v23.x, v23.y};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (!KEYS) kq[u][e] = __float_as_uint((float)vv[e]);
            av[u][e] = fabs(vv[e]);
          }
        }
        olds[u] = dst[(g < ng && w < words) ? w : 0];
      }
#pragma unroll
      for (int u = 0; u < kPg; ++u) {
        const int g = g0 + u * NW;
        if (g >= ng) break;  // uniform within the wave
        const int rem = len - (g * 256 + 4 * lane);  // elements of this lane that exist
        unsigned byte = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned kb = e < rem ? kq[u][e] : 0u;
          const bool sel = (kb & 0x7FFFFFFFu) >= kthr;
          const unsigned neg = sel ? kb >> 31 : 0u;
          byte |= ((sel ? 1u : 0u) | (neg << 1)) << (2 * e);
          sum += (sel ? 1 : 0) - 2 * (int)neg;
          if (want_p) pacc += sel ? av[u][e] : 0.0;  // + 0.0 leaves the (nonnegative) sum unchanged
        }
        unsigned x = byte << sh8;
        x |= dpp32<0x111, 0xF>(x);
        x |= dpp32<0x112, 0xF>(x);
        const int w = g * 16 + (lane >> 2);
        if (holder && w < words) {
          const unsigned old = olds[u];
          if (prev) prev[w] = old;
          changed |= x != old ? 1 : 0;
          dst[w] = x;
        }
      }
    }
    sum = (int)wave_sum_u32((unsigned)sum);
    const int wch = __ballot(changed != 0) != 0ull ? 1 : 0;
    if (want_p) pacc = wave_sum_f64(pacc);
    if (lane == 0) {
      sh.pk_changed[wid] = wch;
      sh.pk_sum[wid] = sum;
      sh.pk_p[wid] = pacc;
    }
    __syncthreads();
    PackOut o;
    o.changed = 0;
    o.sum = 0;
    o.p = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      o.changed |= sh.pk_changed[w2];
      o.sum += sh.pk_sum[w2];
      o.p += sh.pk_p[w2];
    }
    return o;
  };
  // Largest |R_ij| over the residual (smallest row-major index on ties), after the pending
  // deflation.  Returns the row, -1 if R == 0, -2 on a barrier failure.
  // Best of the workgroups' candidates (value, index, entry) at xf[4q..4q+2] after a grid
  // barrier: the largest value > 0, the smallest index on ties.  One load per thread and a tree
  // of the same comparison (it is a total order, so the result does not depend on the tree).
  // Leaves (value, index, entry) in part[0..2] for every thread.
  auto global_best = [&]() {
    double v = 0.0, ix = -1.0, ev = 0.0;
    if (tid < G) {
      v = ld_dev(a.xf + 4 * tid);
      ix = ld_dev(a.xf + 4 * tid + 1);
      ev = ld_dev(a.xf + 4 * tid + 2);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double v2 = __shfl_xor(v, o), i2 = __shfl_xor(ix, o), e2 = __shfl_xor(ev, o);
      if (v2 > v || (v2 == v && v2 > 0.0 && i2 < ix)) {
        v = v2;
        ix = i2;
        ev = e2;
      }
    }
    __syncthreads();  // part may still be read by the caller's earlier step
    if (lane == 0) {
      part[3 * wid] = v;
      part[3 * wid + 1] = ix;
      part[3 * wid + 2] = ev;
    }
    __syncthreads();
    if (tid == 0) {
      double bb = 0.0, bi = -1.0, bv = 0.0;
      for (int w = 0; w < NW; ++w) {
        const double v3 = part[3 * w], i3 = part[3 * w + 1];
        if (v3 > bb || (v3 == bb && v3 > 0.0 && i3 < bi)) {
          bb = v3;
          bi = i3;
          bv = part[3 * w + 2];
        }
      }
      part[0] = bb;
      part[1] = bi;
      part[2] = bv;
    }
    __syncthreads();
  };
  auto fallback_row = [&]() -> int {
    if (have_pending && !r_applied) {
      slab_deflate<NT>(Rb, Rrow0, Rld, n4 / 4, r0, r1, du, dv, pd);
      r_applied = true;
    }
    double best = 0.0, bidx = -1.0;
    for (int i = r0 + wid; i < r1; i += NW) {
      const float* row = Rb + (size_t)(i - Rrow0) * Rld;
      for (int j = lane; j < n; j += 64) {
        const double v = fabs((double)row[j]);
        const double idx = (double)i * (double)n + (double)j;
        if (v > best || (v == best && v > 0.0 && idx < bidx)) {
          best = v;
          bidx = idx;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double b2 = __shfl_xor(best, o), i2 = __shfl_xor(bidx, o);
      if (b2 > best || (b2 == best && b2 > 0.0 && i2 < bidx)) {
        best = b2;
        bidx = i2;
      }
    }
    if (lane == 0) {
      part[2 * wid] = best;
      part[2 * wid + 1] = bidx;
    }
    __syncthreads();
    if (tid == 0) {
      double bb = 0.0, bi = -1.0;
      for (int w = 0; w < NW; ++w) {
        const double v = part[2 * w], ix = part[2 * w + 1];
        if (v > bb || (v == bb && v > 0.0 && ix < bi)) {
          bb = v;
          bi = ix;
        }
      }
      st_dev(a.xf + 4 * g, bb);
      st_dev(a.xf + 4 * g + 1, bi);
      st_dev(a.xf + 4 * g + 2, 0.0);
    }
    ++epoch;
    if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return -2;
    global_best();
    const int row = part[0] > 0.0 ? (int)(part[1] / (double)n) : -1;
    __syncthreads();  // part is reused by the next pass
    return row;
  };
  // Prop. 2 safeguard: the single entry whose removal lowers the residual most, i.e. the largest
  // h_j R_ij^2 (fp64, h_j R_ij first), smallest row-major index on ties, over the residual after
  // the pending deflation.  All workgroups return the same (row, col, value); row -1 if R == 0,
  // -2 on a barrier failure.
  auto best_entry = [&](double* sbest, int* col, float* val) -> int {
    if (have_pending && !r_applied) {
      slab_deflate<NT>(Rb, Rrow0, Rld, n4 / 4, r0, r1, du, dv, pd);
      r_applied = true;
    }
    best_entry_rows<NW>(Rb, Rrow0, Rld, r0, r1, n, WV ? hl : nullptr, part);
    if (tid == 0) {
      double bb = 0.0, bi = -1.0, bv = 0.0;
      for (int w = 0; w < NW; ++w) {
        const double v = part[3 * w], ix = part[3 * w + 1];
        if (v > bb || (v == bb && v > 0.0 && ix < bi)) {
          bb = v;
          bi = ix;
          bv = part[3 * w + 2];
        }
      }
      st_dev(a.xf + 4 * g, bb);
      st_dev(a.xf + 4 * g + 1, bi);
      st_dev(a.xf + 4 * g + 2, bv);
    }
    ++epoch;
    if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return -2;
    global_best();
    const double bb = part[0], bi = part[1];
    const int row = bb > 0.0 ? (int)(bi / (double)n) : -1;
    *sbest = bb;
    *col = row >= 0 ? (int)(bi - (double)row * (double)n) : 0;
    *val = (float)part[2];
    __syncthreads();  // part is reused by the next pass
    return row;
  };
  auto set_unit_u = [&](int r) {
    for (int w = tid; w < wm; w += NT) pu[w] = (w == (r >> 4)) ? (1u << (2 * (r & 15))) : 0u;
    __syncthreads();
  };
  // Component outputs are stored device-coherently: a refinement sweep reads them back from
  // every workgroup.  counted = false for a refit that came out zero (energy from E).
  auto emit_zero = [&](int comp, bool counted, double energy) {
    if (g == 0) {
      for (int w = tid; w < wm; w += NT) st_dev(a.Bp + (size_t)comp * wm + w, 0u);
      for (int w = tid; w < wn; w += NT) st_dev(a.Cp + (size_t)comp * wn + w, 0u);
      if (tid == 0) {
        st_dev(reinterpret_cast<unsigned*>(a.D) + comp, 0u);
        a.energy[comp] = energy;
        if (counted) a.stats[3] += 1ull;
      }
    }
  };


  // Pass 0 is the greedy pass over all k components; an energy-target stop leaves it by break
  // with comp at the last fitted component.  Passes 1..sweeps refit the fitted components in
  // order (backfitting): the previous fit's deflation is applied to both residual copies, the
  // component's own contribution becomes the pending update (added back inside the refit's
  // first passes), and the ALS starts from the component's previous u.
  int used = a.k;
  const int nsweeps = EXT ? a.sweeps : 0;  // sweeps and the safeguard exist only in the EXT kernels
  for (int sweep = 0; sweep <= nsweeps; ++sweep) {
  if (EXT && sweep > 0) {
    if (!(E0 > 0.0)) break;
    dead = false;
  }
  const int ncomp = (!EXT || sweep == 0) ? a.k : used;
  int comp = 0;
  for (; comp < ncomp; ++comp) {
    bool fallback = false, refit_plus = false;
    float d_old = 0.0f;
    double E_before = 0.0;  // refit: the energy before the add-back
    if (EXT && sweep > 0) {
      // ---------------- refit: add-back pending, u from the previous fit
      refit_begin<NT>(Rb, Rrow0, Rld, n4 / 4, a.RT, a.ldt, m4 / 4, r0, r1, c0, c1, have_pending && !r_applied,
                      have_pending && !rt_applied, pd, du, dv, pu, a.Bp + (size_t)comp * wm,
                      a.Cp + (size_t)comp * wn, wm, wn, g == 0 ? a.bytes : nullptr);
      d_old = __uint_as_float(ld_dev(reinterpret_cast<const unsigned*>(a.D) + comp));
      pd = -d_old;
      have_pending = d_old != 0.0f;
      r_applied = false;
      rt_applied = false;
      refit_plus = have_pending;
      E_before = E;
      __syncthreads();
    } else {
    if (dead) {
      emit_zero(comp, true, 1.0);
      if (a.target > 0.0) break;
      continue;
    }
    // ---------------- initial u: ternarized fp32 row sums
    {
      unsigned kx = 0u;
      for (int i0 = tid; i0 < m; i0 += kXg * NT) {
        double v[kXg];
#pragma unroll
        for (int u = 0; u < kXg; ++u) v[u] = i0 + u * NT < m ? rs[i0 + u * NT] : 0.0;
#pragma unroll
        for (int u = 0; u < kXg; ++u) {
          const unsigned kb = __float_as_uint((float)v[u]);
          if (i0 + u * NT < m) {
            dl[i0 + u * NT] = v[u];
            if (KEYS) kl[i0 + u * NT] = kb;
          }
          const unsigned k = kb & 0x7FFFFFFFu;
          kx = k > kx ? k : kx;
        }
      }
      select_prepare<NT>(s, kx);
    }
    const SelResult su = select_unweighted(m);
    if (su.count == 0u) {
      const int r = fallback_row();
      if (r == -2) return;
      if (r < 0) {
        dead = true;
        E = 0.0;
        emit_zero(comp, true, 1.0);
        if (a.target > 0.0) break;
        continue;
      }
      set_unit_u(r);
      fallback = true;
    } else {
      pack_sel(dl, kl, m, su, pu, nullptr, false);
    }
    }  // pass 0
    for (int w = tid; w < wm; w += NT) pu0[w] = pu[w];
    __syncthreads();

    // ---------------- ALS
    double p = 0.0, Hv = 0.0;
    unsigned cnt_u = 0;
    int sumv = 0, passes = 0, usteps = 0;
    bool early = false;
    double vbytes = 0.0;
    int t = 0;
    while (t < a.T) {
      // ---- V-step: w_j = RT_j . u on owned RT rows (pending deflation fused)
      slab_matvec<NT>(a.RT, 0, a.ldt, m4 / 4, c0, c1, pu, nullptr, have_pending && !rt_applied, dv, du, pd,
                      part, a.xw);
      rt_applied = true;
      ++passes;
      ++epoch;
      if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return;
      load_exchange(a.xw, n);
      if (EXT && refit_plus) {
        // energy with the contribution restored, from w = (R + X)^T u_old:
        //   |R + X|^2_H = E + 2 d v_old^T H w - d^2 |u_old|^2 |v_old|^2_H
        refit_plus = false;
        const double dd0 = (double)d_old;
        E = E + addback_energy<NT>(dl, du, dv, WV ? hl : nullptr, n, wm, dd0, part);
      }
      // (ablation: the projection may ignore the weights; the scale and energy stay weighted)
      const bool naive_w = EXT && WV && (a.ablation & 2);
      const SelResult sv = (naive_w || !WV) ? select_unweighted(n)
                                            : ternary_select<NT, WV, double, WV, true>(dl, hw, n, a.tau, a.EHm, s);
      if (sv.count == 0u) {
        // R^T u == 0: only possible for the initial u; restart from the largest-entry row
        if (fallback) {
          dead = true;
          break;
        }
        const int r = fallback_row();
        if (r == -2) return;
        if (r < 0) {
          dead = true;
          break;
        }
        set_unit_u(r);
        for (int w = tid; w < wm; w += NT) pu0[w] = pu[w];
        fallback = true;
        __syncthreads();
        continue;
      }
      const PackOut pvo = pack_sel(dl, kl, n, sv, pv, nullptr, false);
      sumv = pvo.sum;
      const int vchanged = pvo.changed;
      Hv = sv.H;
      if (naive_w) {  // sum of h over supp(v), fixed order
        double hs = 0.0;
        for (int j = tid; j < n; j += NT)
          if (code_at(pv, j) != 0) hs += (double)hl[j];
        hs = wave_sum_f64(hs);
        __syncthreads();
        if (lane == 0) part[wid] = hs;
        __syncthreads();
        Hv = 0.0;
        for (int w = 0; w < NW; ++w) Hv += part[w];
        __syncthreads();
      }
      if (t >= 1) vbytes += 4.0 * (double)n * (double)cnt_u;  // rows of the u behind this V-step
      if (t >= 1 && !vchanged) {
        early = true;
        break;
      }
      // ---- U-step: z_i = R_i . (h v) on owned R rows (pending deflation fused)
      slab_matvec<NT>(Rb, Rrow0, Rld, n4 / 4, r0, r1, pv, hw, have_pending && !r_applied, du, dv, pd, part,
                      a.xz);
      r_applied = true;
      ++passes;
      ++usteps;
      ++epoch;
      if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return;
      load_exchange(a.xz, m);
      const SelResult s2 = select_unweighted(m);
      // new u, the previous one kept in pu_prev, and p = sum over supp(u) of u_i z_i with the
      // fp64 z (fixed reduction order)
      const PackOut puo = pack_sel(dl, kl, m, s2, pu, pu_prev, true);
      p = puo.p;
      cnt_u = s2.count;
      const int uchanged = puo.changed;
      ++t;
      if (!uchanged && t < a.T) {
        early = true;
        break;
      }
    }
    if (dead) {
      if (EXT && sweep > 0) {  // the residual with the contribution restored is zero
        emit_zero(comp, false, 1.0 - E / E0);
        dead = false;
        continue;
      }
      E = 0.0;
      emit_zero(comp, true, 1.0);
      if (a.target > 0.0) break;
      continue;
    }
    // ---------------- safeguard, scale, energy, outputs
    double q = (double)cnt_u * Hv;
    bool sg_on = false;
    float d_sg = 0.0f;
    if (EXT && a.safeguard) {
      // keep whichever removes more energy: the ALS component (p^2 / q) or the best entry
      double sbest;
      int col;
      float rv;
      const int row = best_entry(&sbest, &col, &rv);
      if (row == -2) return;
      if (row >= 0 && sbest > p * p / q) {
        sg_on = true;
        set_unit_u(row);
        for (int w = tid; w < wn; w += NT)
          pv[w] = (w == (col >> 4)) ? ((rv > 0.0f ? 1u : 3u) << (2 * (col & 15))) : 0u;
        const double hj = WV ? (double)hl[col] : 1.0;
        d_sg = fabsf(rv);
        p = hj * (double)d_sg;
        q = hj;
        cnt_u = 1;
        sumv = rv > 0.0f ? 1 : -1;
        __syncthreads();
      }
    }
    float d = sg_on ? d_sg : (float)(p / q);
    double dd = (double)d;
    E = E - (2.0 * dd * p - dd * dd * q);
    bool reverted = false;
    if (EXT && sweep > 0 && E > E_before + 1e-9 * E0) {
      // the refit leaves more than the old component did: deflate the old one again (its
      // codes are the pending add-back's, already applied to both copies)
      reverted = true;
      for (int w = tid; w < wm; w += NT) pu[w] = du[w];
      for (int w = tid; w < wn; w += NT) pv[w] = dv[w];
      d = d_old;
      dd = (double)d;
      E = E_before;
      __syncthreads();
    }
    if (g == 0) {
      for (int w = tid; w < wm; w += NT) st_dev(a.Bp + (size_t)comp * wm + w, pu[w]);
      for (int w = tid; w < wn; w += NT) st_dev(a.Cp + (size_t)comp * wn + w, pv[w]);
      // |supp u0 U supp u_prev| (fused deflate + first V-step rows) and |supp u_prev| (writes),
      // counted by wave 0 alone; one barrier keeps du unchanged until it has been read
      if (tid < 64) {
        int un = 0, pn = 0;
        for (int w = tid; w < wm; w += 64) {
          const unsigned dw = have_pending ? du[w] : 0u;
          const unsigned x = pu0[w] | dw;
          un += __popc((x | (x >> 1)) & 0x55555555u);
          pn += __popc((dw | (dw >> 1)) & 0x55555555u);
        }
        un = (int)wave_sum_u32((unsigned)un);
        pn = (int)wave_sum_u32((unsigned)pn);
        if (tid == 0) {
          st_dev(reinterpret_cast<unsigned*>(a.D) + comp, __float_as_uint(d));
          a.energy[comp] = 1.0 - E / E0;
          st_acc[0] += (u64)passes;
          if (early) st_acc[1] += 1ull;
          if (fallback) st_acc[2] += 1ull;
          if (sg_on) st_acc[3] += 1ull;
          if (reverted) st_acc[4] += 1ull;
          bytes_acc += 4.0 * (double)n * (double)un + 4.0 * (double)n * (double)pn +
                       (double)usteps * 4.0 * (double)m * (double)n + vbytes +
                       (EXT && a.safeguard ? 4.0 * (double)m * (double)n : 0.0);
        }
      }
      __syncthreads();
    }
    // row-sum recurrence and pending deflation
    const double dsv = dd * (double)sumv;
    for (int i = tid; i < m; i += NT) {
      const int ui = code_at(pu, i);
      if (ui != 0) rs[i] = rs[i] - (double)ui * dsv;
    }
    for (int w = tid; w < wm; w += NT) du[w] = pu[w];
    for (int w = tid; w < wn; w += NT) dv[w] = pv[w];
    pd = d;
    have_pending = true;
    r_applied = false;
    rt_applied = false;
    __syncthreads();
    if ((!EXT || sweep == 0) && a.target > 0.0 && 1.0 - E / E0 >= a.target) break;
  }
  if (!EXT || sweep == 0) used = comp < a.k ? comp + 1 : a.k;
  }  // passes
  // components after an energy-target stop: zero, the final energy held (1 after a zero
  // component: E was set to 0 there)
  if (used < a.k && g == 0) {
    const double held = E0 > 0.0 ? 1.0 - E / E0 : 1.0;
    for (long long x = tid; x < (long long)(a.k - used) * wm; x += NT) a.Bp[(size_t)used * wm + x] = 0u;
    for (long long x = tid; x < (long long)(a.k - used) * wn; x += NT) a.Cp[(size_t)used * wn + x] = 0u;
    for (int c = used + tid; c < a.k; c += NT) {
      a.D[c] = 0.0f;
      a.energy[c] = held;
    }
  }
  if (g == 0 && tid == 0) {
    a.stats[5] = (u64)used;
    a.stats[0] += st_acc[0];
    a.stats[1] += st_acc[1];
    a.stats[2] += st_acc[2];
    a.stats[4] += st_acc[3];
    a.stats[6] += st_acc[4];
    a.bytes[0] += bytes_acc;
  }
  // apply the last pending deflation to R (the transpose copy is no longer needed)
  if (have_pending && !r_applied) slab_deflate<NT>(Rb, Rrow0, Rld, n4 / 4, r0, r1, du, dv, pd);
  if (RL) {  // the final residual back to HBM
    const int q4 = n4 / 4;
    for (int x = tid; x < (r1 - r0) * q4; x += NT) {
      const int r = x / q4, q = x - r * q4;
      reinterpret_cast<float4*>(a.R + (size_t)(r0 + r) * a.ldr)[q] =
          reinterpret_cast<const float4*>(Rb + (size_t)r * n4)[q];
    }
  }
}

size_t seq_smem_bytes(int m, int n, bool weighted, int G, bool rl, bool keys) {
  return seq_lds_layout(m, n, weighted, G, rl, keys).total;
}

template <bool WV, bool RL, bool EXT, bool KEYS>
static hipError_t launch_one(const SeqArgs& a, int G, size_t smem, hipStream_t st) {
  auto kern = seq_kernel<512, WV, RL, EXT, KEYS>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  SeqArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchCooperativeKernel((const void*)kern, dim3(G), dim3(512), args, (unsigned)smem, st);
}

template <bool WV, bool RL, bool KEYS>
static int coresident_one(size_t smem) {
  int nb = 0, nb2 = 0;
  auto kern = seq_kernel<512, WV, RL, false, KEYS>;
  auto kern2 = seq_kernel<512, WV, RL, true, KEYS>;
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, 512, smem) != hipSuccess) return 0;
  if (hipFuncSetAttribute((const void*)kern2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb2, kern2, 512, smem) != hipSuccess) return 0;
  return nb < nb2 ? nb : nb2;
}

constexpr size_t kLdsBytes = 160 * 1024;

int seq_plan(int m, int n, bool weighted, int ncu, bool allow_rl, int* grid, bool* rl, bool* keys) {
  const int want = (int)std::max<long long>(1, std::min<long long>(ncu, ((long long)std::max(m, n) + 7) / 8));
  // in order of preference: the R slab in LDS (one workgroup per CU, where the caller allows it)
  // with, then without the key array; then R in HBM with, then without it
  for (int c = 0; c < 4; ++c) {
    const bool try_rl = c < 2, kc = (c & 1) == 0;
    if (try_rl && (!allow_rl || weighted)) continue;
    const size_t smem = seq_smem_bytes(m, n, weighted, want, try_rl, kc);
    if (smem > kLdsBytes) continue;
    int per = 0;
    if (weighted) per = kc ? coresident_one<true, false, true>(smem) : coresident_one<true, false, false>(smem);
    else if (try_rl) per = kc ? coresident_one<false, true, true>(smem) : coresident_one<false, true, false>(smem);
    else per = kc ? coresident_one<false, false, true>(smem) : coresident_one<false, false, false>(smem);
    if (per < 1 || want > ncu * per) continue;
    *grid = want;
    *rl = try_rl;
    *keys = kc;
    return 1;
  }
  return 0;
}

hipError_t seq_launch(const SeqLaunch& L, hipStream_t st) {
  SeqArgs a;
  a.R = L.R;
  a.RT = L.RT;
  a.h = L.h;
  a.rs0 = L.rs0;
  a.rowE = L.rowE;
  a.xz = L.xz;
  a.xw = L.xw;
  a.xf = L.xf;
  a.rsg = L.rsg;
  a.bar = L.bar;
  a.Bp = L.Bp;
  a.Cp = L.Cp;
  a.D = L.D;
  a.energy = L.energy;
  a.stats = L.stats;
  a.bytes = L.bytes;
  a.m = L.m;
  a.n = L.n;
  a.ldr = L.ldr;
  a.ldt = L.ldt;
  a.k = L.k;
  a.T = L.T;
  a.wm = (L.m + 15) / 16;
  a.wn = (L.n + 15) / 16;
  a.EHm = L.EHm;
  a.tau = L.tau;
  a.spin_limit = L.spin_limit;
  a.target = L.target;
  a.safeguard = L.safeguard;
  a.sweeps = L.sweeps;
  a.ablation = L.ablation;
  const size_t smem = seq_smem_bytes(L.m, L.n, L.h != nullptr, L.grid, L.rl, L.keys);
  // the weighted kernels never hold the slab in LDS (seq_plan), so they exist only without RL
  const bool ext = L.sweeps > 0 || L.safeguard || (L.h && (L.ablation & 2));
#define EXTERND_SEQ(EXT, KEYS)                                                                         \
  (L.h ? launch_one<true, false, EXT, KEYS>(a, L.grid, smem, st)                                       \
       : (L.rl ? launch_one<false, true, EXT, KEYS>(a, L.grid, smem, st)                               \
               : launch_one<false, false, EXT, KEYS>(a, L.grid, smem, st)))
  if (ext) return L.keys ? EXTERND_SEQ(true, true) : EXTERND_SEQ(true, false);
  return L.keys ? EXTERND_SEQ(false, true) : EXTERND_SEQ(false, false);
#undef EXTERND_SEQ
}

// ---- standalone matvec with the same slab routine (kernel-level parity tests) ----------
// Each workgroup packs the ternary vector into LDS and runs slab_matvec over its rows.
__global__ void __launch_bounds__(512) matvec_rows_kernel(float* Rp, int rows, int len4, int ld, const int8_t* t,
                                                           const float* h, double* out) {
  extern __shared__ __align__(16) char smem[];
  const int words = (len4 * 4 + 15) / 16;
  uint32_t* pk = reinterpret_cast<uint32_t*>(smem);
  float* hl = reinterpret_cast<float*>(smem + al16(4 * (size_t)words));
  double* part = reinterpret_cast<double*>(smem + al16(4 * (size_t)words) + al16(h ? 16 * (size_t)len4 : 0));
  const int len = len4 * 4;  // t and h are padded to len4 * 4 by the caller
  for (int w = threadIdx.x; w < words; w += 512) {
    unsigned word = 0u;
    for (int q = 0; q < 16; ++q) {
      const int i = w * 16 + q;
      if (i < len) word |= tcode(t[i]) << (2 * q);
    }
    pk[w] = word;
  }
  if (h)
    for (int j = threadIdx.x; j < len; j += 512) hl[j] = h[j];
  __syncthreads();
  const int G = gridDim.x, g = blockIdx.x;
  const int r0 = (int)((long long)g * rows / G), r1 = (int)((long long)(g + 1) * rows / G);
  slab_matvec<512>(Rp, 0, ld, len4, r0, r1, pk, h ? hl : nullptr, false, nullptr, nullptr, 0.0f, part, out);
}

hipError_t matvec_rows(float* Rp, int rows, int len4, int ld, const int8_t* t, const float* h, double* out,
                       hipStream_t st) {
  const int words = (len4 * 4 + 15) / 16;
  const int G = rows < 256 ? rows : 256;
  if (len4 > kQMax * 512) return hipErrorInvalidValue;
  const size_t smem = al16(4 * (size_t)words) + al16(h ? 16 * (size_t)len4 : 0) + 8 * (size_t)kMvPart;
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)matvec_rows_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(matvec_rows_kernel, dim3(G), dim3(512), smem, st, Rp, rows, len4, ld, t, h, out);
  return hipGetLastError();
}

}  // namespace externd
