// Sequential-deflation ALS as one persistent cooperative kernel (gfx950, wave64).
//
// Method (ExTernD review, Method and Key idea; pith.science, "What carries the argument"):
// component after component, u0 is the ternarized row-sum pattern of the residual; then
// als_iters times v = T_tau(R^T u; h) (V-step, corrected weighted projection) and
// u = T_tau(R H v) (U-step); the scale d = u^T R H v / (|u|^2 v^T H v) is rounded to fp32,
// the energy bookkeeping is E <- E - (2 d p - d^2 q), and the residual is deflated,
// R_ij <- fl32(R_ij - d u_i v_j), before the next component.
//
// MI355X layout.  The residual lives in HBM twice: R (m x n) and its transpose RT (n x m), both
// row-major.  Workgroup g owns a fixed slab of R rows and a fixed slab of RT rows, so both
// matvecs are reduction-free: a U-step row dot product z_i = R_i . (h v) and a V-step row dot
// product w_j = RT_j . u are finished inside the owning workgroup.  The only cross-workgroup
// traffic per half-step is the finished vector (z or w, fp64) plus one grid barrier; every
// workgroup then runs the same deterministic selection redundantly, so all of them agree on u
// or v without a broadcast.  Deflation is applied lazily: the pending component is subtracted
// from RT rows during the next V-step read and from R rows during the next U-step read (one
// read-modify-write pass fused with a matvec).  The tracked row sums rs (fp64 recurrence
// rs <- rs - d (sum v) u) are replicated in every workgroup's LDS, so the next u0 is chosen
// without another exchange.
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
  double* xf;          // 2 * gridDim.x
  unsigned* bar;
  uint32_t* Bp;
  uint32_t* Cp;
  float* D;
  double* energy;
  u64* stats;          // [0] passes [1] early exits [2] fallbacks [3] zero components
  double* bytes;       // algorithmic bytes
  int m, n, ldr, ldt, k, T, wm, wn, EHm;
  float tau;
  unsigned spin_limit;
};


__device__ __forceinline__ int code_at(const uint32_t* pk, int i) {
  const unsigned c = (pk[i >> 4] >> ((i & 15) * 2)) & 3u;
  return c == 0u ? 0 : (c == 1u ? 1 : -1);
}

// Row dot product with optional fused pending deflation.
//   row: fp32 row of length len (padded to a multiple of 4, padding zero)
//   wt:  LDS weights (len, padded) used as (double)(x * wt) when exact_f32 (ternary weights) or
//        (double)x * (double)wt otherwise
//   dfl: if nonzero, subtract sgn * d on columns whose code in pk_other is nonzero, where
//        sgn = own_code * code(col); the updated row is written back.
// Returns the fp64 dot product of one wave (lane 0 holds the full sum after reduction).
__device__ __forceinline__ double row_dot(float* row, int len4, const float* wt, bool exact_f32,
                                          int own_code, float d, const uint32_t* pk_other,
                                          int lane) {
  double acc = 0.0;
  float4* r4 = reinterpret_cast<float4*>(row);
  const float4* w4 = reinterpret_cast<const float4*>(wt);
  for (int q = lane; q < len4; q += 64) {
    float4 x = r4[q];
    if (own_code != 0) {
      const unsigned word = pk_other[q >> 2] >> ((q & 3) * 8);
      float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const unsigned c = (word >> (2 * t)) & 3u;
        if (c != 0u) {
          const int sg = (c == 1u ? 1 : -1) * own_code;
          xs[t] = sg > 0 ? xs[t] - d : xs[t] + d;
        }
      }
      x = make_float4(xs[0], xs[1], xs[2], xs[3]);
      r4[q] = x;
    }
    const float4 w = w4[q];
    if (exact_f32) {
      acc += (double)(x.x * w.x);
      acc += (double)(x.y * w.y);
      acc += (double)(x.z * w.z);
      acc += (double)(x.w * w.w);
    } else {
      acc += (double)x.x * (double)w.x;
      acc += (double)x.y * (double)w.y;
      acc += (double)x.z * (double)w.z;
      acc += (double)x.w * (double)w.w;
    }
  }
  return wave_sum_f64(acc);
}

// Dynamic LDS of the sequential kernel; every region starts on a 16-byte boundary.
struct SeqLds {
  size_t rs, hv, uf, tmp, pk, total;
};
__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ inline SeqLds seq_lds_layout(int m, int n) {
  const size_t m4 = (size_t)((m + 3) & ~3), n4 = (size_t)((n + 3) & ~3);
  const size_t wm = (size_t)((m + 15) / 16), wn = (size_t)((n + 15) / 16);
  SeqLds L;
  L.rs = al16(sizeof(SelScratch));
  L.hv = al16(L.rs + 8 * (size_t)m);
  L.uf = al16(L.hv + 4 * n4);
  L.tmp = al16(L.uf + 4 * m4);
  L.pk = al16(L.tmp + (m4 > n4 ? m4 : n4));
  L.total = al16(L.pk + 4 * (4 * wm + 3 * wn));
  return L;
}

struct SeqShared {
  int flag;
  int ivals[8];
  double dvals[8];
};

template <int NT, int NE>
__global__ void __launch_bounds__(NT) seq_kernel(SeqArgs a) {
  constexpr int kNT = NT;
  constexpr int kNW = NT / 64;
  extern __shared__ __align__(16) char smem[];
  SelScratch& s = *reinterpret_cast<SelScratch*>(smem);
  const int m = a.m, n = a.n;
  const int m4 = (m + 3) & ~3, n4 = (n + 3) & ~3;
  const SeqLds lay = seq_lds_layout(m, n);
  double* rs = reinterpret_cast<double*>(smem + lay.rs);  // m: replicated row sums
  float* hv = reinterpret_cast<float*>(smem + lay.hv);    // n4: signed weights of v
  float* uf = reinterpret_cast<float*>(smem + lay.uf);    // m4: u as fp32 {-1,0,1}
  int8_t* tmp = reinterpret_cast<int8_t*>(smem + lay.tmp);  // max(m4, n4) staging for packing
  uint32_t* pk = reinterpret_cast<uint32_t*>(smem + lay.pk);
  const int wm = a.wm, wn = a.wn;
  uint32_t* pu = pk;            // current u
  uint32_t* pv = pu + wm;       // current v
  uint32_t* pu_prev = pv + wn;  // u that produced the current v
  uint32_t* pv_prev = pu_prev + wm;
  uint32_t* du = pv_prev + wn;  // pending deflation component
  uint32_t* dv = du + wm;
  uint32_t* pu0 = dv + wn;      // u0 of this component (for the byte count)
  __shared__ SeqShared sh;
  __shared__ int bar_flag;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const int r0 = (int)((long long)g * m / G), r1 = (int)((long long)(g + 1) * m / G);
  const int c0 = (int)((long long)g * n / G), c1 = (int)((long long)(g + 1) * n / G);
  const bool weighted = a.h != nullptr;
  unsigned epoch = 0;

  // ---- set-up: replicated row sums, E0 in a fixed order, padding cleared
  for (int i = tid; i < m; i += kNT) rs[i] = a.rs0[i];
  for (int i = tid; i < m4; i += kNT) uf[i] = 0.0f;
  for (int i = tid; i < n4; i += kNT) hv[i] = 0.0f;
  for (int i = tid; i < 4 * wm + 3 * wn; i += kNT) pk[i] = 0u;
  double e0 = 0.0;
  for (int i = tid; i < m; i += kNT) e0 += a.rowE[i];
  e0 = wave_sum_f64(e0);
  if (lane == 0) s.red_d[wid] = e0;
  __syncthreads();
  double E0 = 0.0;
  for (int w = 0; w < kNW; ++w) E0 += s.red_d[w];
  double E = E0;
  bool dead = !(E0 > 0.0);
  bool have_pending = false, r_applied = true, rt_applied = true;
  float pd = 0.0f;
  __syncthreads();

  // element slots of this thread for selections: index = tid + e * kNT
  float av[NE], hw[NE];
  double zd[NE];
  int sg[NE];

  for (int comp = 0; comp < a.k; ++comp) {
    if (dead) {
      if (g == 0) {
        for (int w = tid; w < wm; w += kNT) a.Bp[(size_t)comp * wm + w] = 0u;
        for (int w = tid; w < wn; w += kNT) a.Cp[(size_t)comp * wn + w] = 0u;
        if (tid == 0) {
          a.D[comp] = 0.0f;
          a.energy[comp] = 1.0;
          a.stats[3] += 1ull;
        }
      }
      continue;
    }
    // ---------------- initial u: ternarized fp32 row sums
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int i = tid + e * kNT;
      const float x = i < m ? (float)rs[i] : 0.0f;
      av[e] = fabsf(x);
      sg[e] = x > 0.0f ? 1 : (x < 0.0f ? -1 : 0);
      hw[e] = 1.0f;
    }
    SelResult su = ternary_select<kNT, NE, false>(av, hw, a.tau, 0, s);
    bool fallback = false;
    auto write_u_from_slots = [&](const SelResult& r) {
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int i = tid + e * kNT;
        if (i < m) {
          const unsigned k = __float_as_uint(av[e]);
          const bool on = r.count > 0u && k != 0u && k >= r.ekey && k >= r.tkey;
          tmp[i] = on ? (int8_t)sg[e] : (int8_t)0;
          uf[i] = on ? (float)sg[e] : 0.0f;
        }
      }
      __syncthreads();
      for (int w = tid; w < wm; w += kNT) {
        unsigned word = 0u;
        for (int t = 0; t < 16; ++t) {
          const int i = w * 16 + t;
          if (i < m) word |= tcode(tmp[i]) << (2 * t);
        }
        pu[w] = word;
      }
      __syncthreads();
    };
    // Largest |R_ij| over the whole residual (smallest row-major index on ties); applies the
    // pending deflation to R rows first.  Returns the row, or -1 if R == 0 (or on error).
    auto fallback_row = [&]() -> int {
      double best = 0.0, bidx = -1.0;
      for (int i = r0 + wid; i < r1; i += kNW) {
        float* row = a.R + (size_t)i * a.ldr;
        const int oc = (have_pending && !r_applied) ? code_at(du, i) : 0;
        if (oc != 0) row_dot(row, n4 / 4, hv, true, oc, pd, dv, lane);  // writes the deflated row
        for (int j = lane; j < n; j += 64) {
          const double v = fabs((double)row[j]);
          const double idx = (double)i * (double)n + (double)j;
          if (v > best || (v == best && v > 0.0 && idx < bidx)) {
            best = v;
            bidx = idx;
          }
        }
      }
      // block argmax (value desc, index asc)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double b2 = __shfl_xor(best, o), i2 = __shfl_xor(bidx, o);
        if (b2 > best || (b2 == best && b2 > 0.0 && i2 < bidx)) {
          best = b2;
          bidx = i2;
        }
      }
      __syncthreads();
      if (lane == 0) {
        s.red_d[wid] = best;
        sh.dvals[0] = 0.0;
      }
      if (lane == 0) s.c_plo[wid] = (u64)__double_as_longlong(bidx);
      __syncthreads();
      if (tid == 0) {
        double bb = 0.0, bi = -1.0;
        for (int w = 0; w < kNW; ++w) {
          const double v = s.red_d[w], ix = __longlong_as_double((long long)s.c_plo[w]);
          if (v > bb || (v == bb && v > 0.0 && ix < bi)) {
            bb = v;
            bi = ix;
          }
        }
        st_dev(a.xf + 2 * g, bb);
        st_dev(a.xf + 2 * g + 1, bi);
      }
      r_applied = true;
      ++epoch;
      if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return -2;
      if (tid == 0) {
        double bb = 0.0, bi = -1.0;
        for (int q = 0; q < G; ++q) {
          const double v = ld_dev(a.xf + 2 * q), ix = ld_dev(a.xf + 2 * q + 1);
          if (v > bb || (v == bb && v > 0.0 && ix < bi)) {
            bb = v;
            bi = ix;
          }
        }
        sh.ivals[0] = bb > 0.0 ? (int)(bi / (double)n) : -1;
      }
      __syncthreads();
      return sh.ivals[0];
    };
    auto set_unit_u = [&](int r) {
      for (int i = tid; i < m; i += kNT) uf[i] = i == r ? 1.0f : 0.0f;
      for (int w = tid; w < wm; w += kNT) pu[w] = (w == (r >> 4)) ? (1u << (2 * (r & 15))) : 0u;
      __syncthreads();
    };
    if (su.count == 0u) {
      const int r = fallback_row();
      if (r == -2) return;
      if (r < 0) {
        dead = true;
        E = 0.0;
        --comp;
        continue;
      }
      set_unit_u(r);
      fallback = true;
    } else {
      write_u_from_slots(su);
    }
    for (int w = tid; w < wm; w += kNT) pu0[w] = pu[w];
    __syncthreads();

    // ---------------- ALS
    double p = 0.0, Hv = 0.0;
    unsigned cnt_u = 0, cnt_v = 0;
    int sumv = 0;
    int passes = 0, usteps = 0;
    bool early = false;
    double vbytes = 0.0;
    int t = 0;
    while (t < a.T) {
      // ---- V-step: w_j = RT_j . u on owned RT rows (pending deflation fused)
      for (int j = c0 + wid; j < c1; j += kNW) {
        float* row = a.RT + (size_t)j * a.ldt;
        const int oc = (have_pending && !rt_applied) ? code_at(dv, j) : 0;
        const double wj = row_dot(row, m4 / 4, uf, true, oc, pd, du, lane);
        if (lane == 0) st_dev(a.xw + j, wj);
      }
      rt_applied = true;
      ++passes;
      ++epoch;
      if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int j = tid + e * kNT;
        const double w = j < n ? ld_dev(a.xw + j) : 0.0;
        const float x = (float)w;
        av[e] = fabsf(x);
        sg[e] = x > 0.0f ? 1 : (x < 0.0f ? -1 : 0);
        hw[e] = (weighted && j < n) ? a.h[j] : 1.0f;
      }
      SelResult sv = (weighted ? ternary_select<kNT, NE, true>(av, hw, a.tau, a.EHm, s) : ternary_select<kNT, NE, false>(av, hw, a.tau, 0, s));
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
        for (int w = tid; w < wm; w += kNT) pu0[w] = pu[w];
        fallback = true;
        __syncthreads();
        continue;
      }
      // build v: signed weights for the U-step and the packed form
      if (tid == 0) sh.ivals[1] = 0;
      __syncthreads();
      int lsum = 0;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int j = tid + e * kNT;
        if (j < n) {
          const unsigned k = __float_as_uint(av[e]);
          const bool on = k != 0u && k >= sv.ekey && k >= sv.tkey;
          const int vj = on ? sg[e] : 0;
          tmp[j] = (int8_t)vj;
          hv[j] = vj == 0 ? 0.0f : (vj > 0 ? hw[e] : -hw[e]);
          lsum += vj;
        }
      }
      if (lsum != 0) atomicAdd(&sh.ivals[1], lsum);
      __syncthreads();
      int changed = 0;
      for (int w = tid; w < wn; w += kNT) {
        unsigned word = 0u;
        for (int q = 0; q < 16; ++q) {
          const int j = w * 16 + q;
          if (j < n) word |= tcode(tmp[j]) << (2 * q);
        }
        if (word != pv[w]) changed = 1;
        pv[w] = word;
      }
      sumv = sh.ivals[1];
      const int vchanged = __syncthreads_or(changed);
      Hv = sv.H;
      cnt_v = sv.count;
      if (t >= 1) {
        // a V-step beyond the first reads the rows of the u that produced it
        vbytes += 4.0 * (double)n * (double)cnt_u;
      }
      if (t >= 1 && !vchanged) {
        early = true;
        break;
      }
      // ---- U-step: z_i = R_i . (h v) on owned R rows (pending deflation fused)
      for (int i = r0 + wid; i < r1; i += kNW) {
        float* row = a.R + (size_t)i * a.ldr;
        const int oc = (have_pending && !r_applied) ? code_at(du, i) : 0;
        const double zi = row_dot(row, n4 / 4, hv, !weighted, oc, pd, dv, lane);
        if (lane == 0) st_dev(a.xz + i, zi);
      }
      r_applied = true;
      ++passes;
      ++usteps;
      ++epoch;
      if (grid_barrier(a.bar, epoch, a.spin_limit, &bar_flag)) return;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int i = tid + e * kNT;
        const double z = i < m ? ld_dev(a.xz + i) : 0.0;
        zd[e] = z;
        const float x = (float)z;
        av[e] = fabsf(x);
        sg[e] = x > 0.0f ? 1 : (x < 0.0f ? -1 : 0);
        hw[e] = 1.0f;
      }
      SelResult s2 = ternary_select<kNT, NE, false>(av, hw, a.tau, 0, s);
      // p = sum over supp(u) of u_i z_i (fp64 z), fixed reduction order
      double lp = 0.0;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const unsigned k = __float_as_uint(av[e]);
        if (s2.count > 0u && k != 0u && k >= s2.ekey && k >= s2.tkey) lp += fabs(zd[e]);
      }
      lp = wave_sum_f64(lp);
      if (lane == 0) s.red_d[wid] = lp;
      __syncthreads();
      p = 0.0;
      for (int w = 0; w < kNW; ++w) p += s.red_d[w];
      cnt_u = s2.count;
      // new u; compare with the u that produced v
      for (int w = tid; w < wm; w += kNT) pu_prev[w] = pu[w];
      __syncthreads();
      write_u_from_slots(s2);
      int uchanged = 0;
      for (int w = tid; w < wm; w += kNT)
        if (pu[w] != pu_prev[w]) uchanged = 1;
      uchanged = __syncthreads_or(uchanged);
      ++t;
      if (!uchanged && t < a.T) {
        early = true;
        break;
      }
    }
    if (dead) {
      E = 0.0;
      --comp;
      continue;
    }
    // ---------------- scale, energy, outputs
    const double q = (double)cnt_u * Hv;
    const float d = (float)(p / q);
    const double dd = (double)d;
    E = E - (2.0 * dd * p - dd * dd * q);
    if (g == 0) {
      for (int w = tid; w < wm; w += kNT) a.Bp[(size_t)comp * wm + w] = pu[w];
      for (int w = tid; w < wn; w += kNT) a.Cp[(size_t)comp * wn + w] = pv[w];
      // |supp u0 U supp u_prev| for the fused deflate + first V-step read
      if (tid == 0) sh.ivals[2] = 0;
      __syncthreads();
      int un = 0;
      for (int w = tid; w < wm; w += kNT) {
        const unsigned x = pu0[w] | (have_pending ? du[w] : 0u);
        un += __popc((x | (x >> 1)) & 0x55555555u);
      }
      if (un) atomicAdd(&sh.ivals[2], un);
      if (tid == 0) sh.ivals[3] = 0;
      __syncthreads();
      int pn = 0;
      if (have_pending)
        for (int w = tid; w < wm; w += kNT) pn += __popc((du[w] | (du[w] >> 1)) & 0x55555555u);
      if (pn) atomicAdd(&sh.ivals[3], pn);
      __syncthreads();
      if (tid == 0) {
        a.D[comp] = d;
        a.energy[comp] = 1.0 - E / E0;
        a.stats[0] += (u64)passes;
        if (early) a.stats[1] += 1ull;
        if (fallback) a.stats[2] += 1ull;
        const double nU = (double)usteps;
        a.bytes[0] += 4.0 * (double)n * (double)sh.ivals[2] + 4.0 * (double)n * (double)sh.ivals[3] +
                      nU * 4.0 * (double)m * (double)n + vbytes;
      }
    }
    // row-sum recurrence and pending deflation
    const double dsv = dd * (double)sumv;
    for (int i = tid; i < m; i += kNT) {
      const float ui = uf[i];
      if (ui != 0.0f) rs[i] = rs[i] - (double)ui * dsv;
    }
    for (int w = tid; w < wm; w += kNT) du[w] = pu[w];
    for (int w = tid; w < wn; w += kNT) dv[w] = pv[w];
    pd = d;
    have_pending = true;
    r_applied = false;
    rt_applied = false;
    __syncthreads();
  }
  // apply the last pending deflation to R (the transpose copy is no longer needed)
  if (have_pending && !r_applied) {
    for (int i = r0 + wid; i < r1; i += kNW) {
      const int oc = code_at(du, i);
      if (oc != 0) row_dot(a.R + (size_t)i * a.ldr, n4 / 4, hv, true, oc, pd, dv, lane);
    }
  }
}

size_t seq_smem_bytes(int m, int n) { return seq_lds_layout(m, n).total; }

// Threads per workgroup: 512 (up to 256 VGPRs per lane) when the longer side fits 16 slots per
// thread, else 1024.
static int seq_threads(int m, int n) { return (m > n ? m : n) <= 512 * 16 ? 512 : 1024; }

int seq_elems_per_thread(int m, int n) {
  const int L = m > n ? m : n;
  const int nt = seq_threads(m, n);
  return (L + nt - 1) / nt;
}

template <int NT, int E>
static hipError_t launch_e(const SeqArgs& a, int G, size_t smem, hipStream_t st) {
  auto kern = seq_kernel<NT, E>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  SeqArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchCooperativeKernel((const void*)kern, dim3(G), dim3(NT), args, (unsigned)smem, st);
}

template <int NT, int E>
static int max_coresident(size_t smem) {
  int nb = 0;
  auto kern = seq_kernel<NT, E>;
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, NT, smem) != hipSuccess) return 0;
  return nb;
}

int seq_max_blocks_per_cu(int m, int n) {
  const size_t smem = seq_smem_bytes(m, n);
  if (smem > 160 * 1024) return 0;
  const int E = seq_elems_per_thread(m, n);
  if (seq_threads(m, n) == 1024) return E <= 16 ? max_coresident<1024, 16>(smem) : 0;
  if (E <= 1) return max_coresident<512, 1>(smem);
  if (E <= 2) return max_coresident<512, 2>(smem);
  if (E <= 4) return max_coresident<512, 4>(smem);
  if (E <= 6) return max_coresident<512, 6>(smem);
  if (E <= 8) return max_coresident<512, 8>(smem);
  if (E <= 12) return max_coresident<512, 12>(smem);
  return max_coresident<512, 16>(smem);
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
  const size_t smem = seq_smem_bytes(L.m, L.n);
  const int E = seq_elems_per_thread(L.m, L.n);
  if (seq_threads(L.m, L.n) == 1024) {
    if (E <= 16) return launch_e<1024, 16>(a, L.grid, smem, st);
    return hipErrorInvalidValue;
  }
  if (E <= 1) return launch_e<512, 1>(a, L.grid, smem, st);
  if (E <= 2) return launch_e<512, 2>(a, L.grid, smem, st);
  if (E <= 4) return launch_e<512, 4>(a, L.grid, smem, st);
  if (E <= 6) return launch_e<512, 6>(a, L.grid, smem, st);
  if (E <= 8) return launch_e<512, 8>(a, L.grid, smem, st);
  if (E <= 12) return launch_e<512, 12>(a, L.grid, smem, st);
  return launch_e<512, 16>(a, L.grid, smem, st);
}

// ---- standalone matvec with the same row routine (kernel-level parity tests) -----------
__global__ void __launch_bounds__(256) matvec_rows_kernel(float* Rp, int rows, int len4, int ld,
                                                           const float* wt, bool exact, double* out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const double v = row_dot(Rp + (size_t)row * ld, len4, wt, exact, 0, 0.0f, nullptr, lane);
  if (lane == 0) out[row] = v;
}

hipError_t matvec_rows(float* Rp, int rows, int len4, int ld, const float* wt, bool exact, double* out,
                       hipStream_t st) {
  hipLaunchKernelGGL(matvec_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, Rp, rows, len4, ld, wt,
                     exact, out);
  return hipGetLastError();
}

}  // namespace externd
