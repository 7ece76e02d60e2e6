// Exact ternary projection T_tau(x; h) computed by one workgroup.
//
// Definition (reading of the adaptive ternarization operator, ExTernD review, Method;
// pith.science free parameters, tau / Eq. 2): among the elements with |x_i| >= tau * max|x|
// (and x_i != 0), the support is the top-j set by |x| whose score S = (sum h|x|)^2 / (sum h)
// is largest, the smallest j on ties; the result carries the signs of x.  With weights this is
// the corrected V-step of the importance-weighted variant (review, Method).
//
// GPU formulation.  The score of a prefix that splits a group of equal |x| is never above both
// ends of the group (S along a tie group is quasi-convex in the weight added), so the optimum is
// a threshold t: support = {eligible i : |x_i| >= t}, t one of the distinct eligible values, and
// "smallest j" means "largest t".  The search therefore needs no sort:
//   1. histogram the eligible values into 256 bins of their fp32 bit pattern (16 per octave
//      below the maximum), with per-bin counts, min/max key and exact 128-bit fixed-point sums
//      of h|x| and h (integer sums are order independent, so every decision is deterministic);
//   2. every bin boundary is a candidate threshold with an exact score; a bin's interior can
//      only win if the bound (P_above + max_bin * H_bin)^2 / (H_above + H_bin) reaches the best
//      boundary score (S along the bin is quasi-convex in the added weight and each added
//      element contributes at most max_bin per unit weight);
//   3. the few surviving elements are scored directly (score of "all elements >= this one");
//      if too many survive, the surviving bin range is re-histogrammed with finer bins.
#pragma once
#include "common.hpp"

namespace externd {

constexpr int kBins = 256;
constexpr int kCandMax = 256;

struct SelRange {
  unsigned key_hi, key_lo;  // keys in (key_lo, key_hi]
  int shift, tail;          // bin = (key_hi - key) >> shift, clamped to the last bin if tail
  u64 ab_plo, ab_phi, ab_hlo, ab_hhi;  // sums over eligible elements above key_hi
  unsigned ab_cnt;
};

// Pending refinement ranges are disjoint and each holds more than kCandMax elements, so for
// L <= 16384 fewer than 64 are ever pending at once.
constexpr int kStack = 72;
constexpr int kMaxLen = 16384;

struct SelScratch {
  unsigned cnt[kBins];
  unsigned kmin[kBins];
  unsigned kmax[kBins];
  u64 p_lo[kBins], p_hi[kBins], h_lo[kBins], h_hi[kBins];
  u64 xp_lo[kBins], xp_hi[kBins], xh_lo[kBins], xh_hi[kBins];  // exclusive prefix per bin
  unsigned xcnt[kBins];
  unsigned char cand[kBins];
  unsigned short chunk_lo[kBins], chunk_hi[kBins];
  unsigned c_key[kCandMax];
  unsigned c_bin[kCandMax];
  u64 c_plo[kCandMax], c_phi[kCandMax], c_hlo[kCandMax], c_hhi[kCandMax];
  u64 r_plo[kCandMax], r_phi[kCandMax], r_hlo[kCandMax], r_hhi[kCandMax];
  unsigned r_cnt[kCandMax];
  unsigned red_u[16];
  double red_d[16];
  unsigned red_k[16];
  SelRange stack[kStack];
  int sp;
  SelRange cur;
  unsigned ncand;
  unsigned ncand_tot;
  int nchunks;
  // best threshold so far
  double best_S;
  unsigned best_key;
  u64 best_plo, best_phi, best_hlo, best_hhi;
  unsigned best_cnt;
};

struct SelResult {
  unsigned tkey;  // support = eligible elements with key >= tkey (nothing if count == 0)
  unsigned ekey;  // eligibility: key >= ekey
  double P, H;    // sum h|x| and sum h over the support (real units)
  unsigned count; // support size
};

__device__ __forceinline__ bool better(double S1, unsigned k1, double S2, unsigned k2) {
  return S1 > S2 || (S1 == S2 && k1 > k2);
}

__device__ __forceinline__ unsigned bin_of(unsigned k, const SelRange& r) {
  unsigned b = (r.key_hi - k) >> r.shift;
  return b > (unsigned)(kBins - 1) ? (unsigned)(kBins - 1) : b;
}

// All NT threads of the workgroup call this with E slots each: a[e] = |x| (0 for padding),
// hw[e] = weight (used only when W), and all receive the same result.  EHm: exponent with
// max(h) < 2^EHm (W only).
template <int NT, int E, bool W>
__device__ SelResult ternary_select(const float (&a)[E], const float (&hw)[E], float tau, int EHm,
                                    SelScratch& s) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int NW = NT / 64;
  SelResult out;
  // ---- max |x|
  unsigned km = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned k = __float_as_uint(a[e]);
    km = k > km ? k : km;
  }
  km = wave_max_u32(km);
  if (lane == 0) s.red_u[wid] = km;
  __syncthreads();
  km = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) km = s.red_u[w] > km ? s.red_u[w] : km;
  out.tkey = 0xFFFFFFFFu;
  out.ekey = 0xFFFFFFFFu;
  out.P = 0.0;
  out.H = 0.0;
  out.count = 0;
  if (km == 0u) {
    __syncthreads();
    return out;
  }
  const float M = __uint_as_float(km);
  const double theta = (double)tau * (double)M;
  // smallest eligible key: the least positive float f with (double)f >= theta
  unsigned ekey;
  {
    unsigned t = __float_as_uint((float)theta);
    if ((double)__uint_as_float(t) < theta) ++t;
    while (t > 1u && (double)__uint_as_float(t - 1u) >= theta) --t;
    ekey = t == 0u ? 1u : t;
  }
  out.ekey = ekey;
  const int EM = exp_bound(M);
  const int scP = W ? (100 - EM - EHm) : (100 - EM);
  const int scH = W ? (100 - EHm) : 0;
  // fixed-point terms of element e: h|x| * 2^scP and h * 2^scH
  auto pterm = [&](int e) -> u128 {
    return W ? fixp((double)hw[e] * (double)a[e], scP) : fixp((double)a[e], scP);
  };
  auto hterm = [&](int e) -> u128 { return W ? fixp((double)hw[e], scH) : mk128(1ull, 0ull); };
  auto keyof = [&](int e) -> unsigned {
    const unsigned k = __float_as_uint(a[e]);
    return k >= ekey ? k : 0u;
  };
  if (tid == 0) {
    SelRange r;
    r.key_hi = km;
    r.key_lo = 0u;
    r.shift = 19;
    r.tail = 1;
    r.ab_plo = r.ab_phi = r.ab_hlo = r.ab_hhi = 0ull;
    r.ab_cnt = 0u;
    s.stack[0] = r;
    s.sp = 1;
    s.best_S = -1.0;
    s.best_key = 0u;
    s.best_plo = s.best_phi = s.best_hlo = s.best_hhi = 0ull;
    s.best_cnt = 0u;
  }
  const double hi_scale = ldexp(1.0, scP - scH);
  __syncthreads();
  while (s.sp > 0) {
    // ---- pop a key range; clear bins
    __syncthreads();
    if (tid == 0) {
      s.sp -= 1;
      s.cur = s.stack[s.sp];
      s.ncand = 0u;
    }
    for (int b = tid; b < kBins; b += NT) {
      s.cnt[b] = 0u;
      s.kmin[b] = 0xFFFFFFFFu;
      s.kmax[b] = 0u;
      s.p_lo[b] = s.p_hi[b] = 0ull;
      if (W) s.h_lo[b] = s.h_hi[b] = 0ull;
      s.cand[b] = 0;
    }
    __syncthreads();
    const SelRange R = s.cur;
    // ---- histogram
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const unsigned k = keyof(e);
      if (k != 0u && k > R.key_lo && k <= R.key_hi) {
        const unsigned b = bin_of(k, R);
        atomicAdd(&s.cnt[b], 1u);
        atomicMin(&s.kmin[b], k);
        atomicMax(&s.kmax[b], k);
        const u128 pe = pterm(e);
        const u64 o = atomicAdd(&s.p_lo[b], pe.lo);
        atomicAdd(&s.p_hi[b], pe.hi + ((o + pe.lo < o) ? 1ull : 0ull));
        if (W) {
          const u128 he = hterm(e);
          const u64 o2 = atomicAdd(&s.h_lo[b], he.lo);
          atomicAdd(&s.h_hi[b], he.hi + ((o2 + he.lo < o2) ? 1ull : 0ull));
        }
      }
    }
    __syncthreads();
    // ---- wave 0: prefix sums, boundary scores, interior bounds (4 bins per lane)
    if (wid == 0) {
      u128 tp = mk128(0, 0), th = mk128(0, 0);
      unsigned tc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = lane * 4 + q;
        tp = add128(tp, mk128(s.p_lo[b], s.p_hi[b]));
        if (W) th = add128(th, mk128(s.h_lo[b], s.h_hi[b]));
        tc += s.cnt[b];
      }
      // inclusive wave scan of lane totals, then exclusive
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u64 a0 = __shfl_up(tp.lo, o), a1 = __shfl_up(tp.hi, o);
        const unsigned c0 = __shfl_up(tc, o);
        u64 b0 = 0, b1 = 0;
        if (W) {
          b0 = __shfl_up(th.lo, o);
          b1 = __shfl_up(th.hi, o);
        }
        if (lane >= o) {
          tp = add128(tp, mk128(a0, a1));
          if (W) th = add128(th, mk128(b0, b1));
          tc += c0;
        }
      }
      u128 run = mk128(__shfl_up(tp.lo, 1), __shfl_up(tp.hi, 1));
      u128 runh = mk128(0, 0);
      if (W) runh = mk128(__shfl_up(th.lo, 1), __shfl_up(th.hi, 1));
      unsigned runc = __shfl_up(tc, 1);
      if (lane == 0) {
        run = mk128(0, 0);
        runh = mk128(0, 0);
        runc = 0;
      }
      run = add128(run, mk128(R.ab_plo, R.ab_phi));
      if (W) runh = add128(runh, mk128(R.ab_hlo, R.ab_hhi));
      runc += R.ab_cnt;
      double bS = s.best_S;
      unsigned bK = s.best_key;
      int bq = -1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = lane * 4 + q;
        s.xp_lo[b] = run.lo;
        s.xp_hi[b] = run.hi;
        if (W) {
          s.xh_lo[b] = runh.lo;
          s.xh_hi[b] = runh.hi;
        }
        s.xcnt[b] = runc;
        const unsigned c = s.cnt[b];
        run = add128(run, mk128(s.p_lo[b], s.p_hi[b]));
        if (W) runh = add128(runh, mk128(s.h_lo[b], s.h_hi[b]));
        runc += c;
        if (c == 0u) continue;
        const double Pd = to_double(run);
        const double Hd = W ? to_double(runh) : (double)runc;
        const double Sb = Pd * Pd / Hd;
        const unsigned kb = s.kmin[b];
        if (better(Sb, kb, bS, bK)) {
          bS = Sb;
          bK = kb;
          bq = q;
        }
      }
      unsigned bl = bq >= 0 ? (unsigned)lane : 64u;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double S2 = __shfl_xor(bS, o);
        const unsigned k2 = __shfl_xor(bK, o);
        const unsigned l2 = __shfl_xor(bl, o);
        if (better(S2, k2, bS, bK) || (S2 == bS && k2 == bK && l2 < bl)) {
          bS = S2;
          bK = k2;
          bl = l2;
        }
      }
      if (bq >= 0 && (unsigned)lane == bl) {
        // recompute the inclusive sums of the winning bin from the stored exclusive prefix
        const int b = lane * 4 + bq;
        const u128 P = add128(mk128(s.xp_lo[b], s.xp_hi[b]), mk128(s.p_lo[b], s.p_hi[b]));
        s.best_S = bS;
        s.best_key = bK;
        s.best_plo = P.lo;
        s.best_phi = P.hi;
        if (W) {
          const u128 H = add128(mk128(s.xh_lo[b], s.xh_hi[b]), mk128(s.h_lo[b], s.h_hi[b]));
          s.best_hlo = H.lo;
          s.best_hhi = H.hi;
        }
        s.best_cnt = s.xcnt[b] + s.cnt[b];
      }
      unsigned nc = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = lane * 4 + q;
        const unsigned c = s.cnt[b];
        if (c < 2u || s.kmin[b] == s.kmax[b]) continue;
        const double Pe = to_double(mk128(s.xp_lo[b], s.xp_hi[b]));
        const double He = W ? to_double(mk128(s.xh_lo[b], s.xh_hi[b])) : (double)s.xcnt[b];
        const double Hb = W ? to_double(mk128(s.h_lo[b], s.h_hi[b])) : (double)c;
        const double hiP = (double)__uint_as_float(s.kmax[b]) * hi_scale;
        const double t1 = Pe + hiP * Hb;
        double ub = t1 * t1 / (He + Hb);
        if (He > 0.0) ub = fmax(ub, Pe * Pe / He);
        if (ub * (1.0 + 1e-9) >= bS) {
          s.cand[b] = 1;
          nc += c;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) nc += __shfl_xor(nc, o);
      if (lane == 0) {
        s.ncand_tot = nc;
        s.nchunks = 0;
        if (nc > 0u && nc <= (unsigned)kCandMax) {
          s.chunk_lo[0] = 0;
          s.chunk_hi[0] = kBins - 1;
          s.nchunks = 1;
        } else if (nc > 0u) {
          // too many survivors: score runs of candidate bins in chunks; refine oversized bins
          int nch = 0;
          unsigned acc = 0u;
          int open = -1;
          for (int b = 0; b < kBins; ++b) {
            if (!s.cand[b]) continue;
            const unsigned c = s.cnt[b];
            if (c > (unsigned)kCandMax) {
              s.cand[b] = 0;
              if (s.sp < kStack) {
                SelRange r;
                const unsigned top = R.key_hi - ((unsigned)b << R.shift);
                const bool last_tail = R.tail && b == kBins - 1;
                const unsigned bot = last_tail ? R.key_lo : R.key_hi - ((unsigned)(b + 1) << R.shift);
                r.key_hi = top;
                r.key_lo = bot;
                int nsh = 0;
                while (((top - bot - 1u) >> nsh) > (unsigned)(kBins - 1)) ++nsh;
                r.shift = nsh;
                r.tail = 0;
                r.ab_plo = s.xp_lo[b];
                r.ab_phi = s.xp_hi[b];
                r.ab_hlo = W ? s.xh_lo[b] : 0ull;
                r.ab_hhi = W ? s.xh_hi[b] : 0ull;
                r.ab_cnt = s.xcnt[b];
                s.stack[s.sp] = r;
                s.sp += 1;
              }
              continue;
            }
            if (open >= 0 && acc + c > (unsigned)kCandMax) {
              s.chunk_hi[nch++] = (unsigned short)(b - 1);
              open = -1;
            }
            if (open < 0) {
              open = b;
              s.chunk_lo[nch] = (unsigned short)b;
              acc = 0u;
            }
            acc += c;
          }
          if (open >= 0) s.chunk_hi[nch++] = (unsigned short)(kBins - 1);
          s.nchunks = nch;
        }
      }
    }
    __syncthreads();
    const int nchunks = s.nchunks;
    for (int ch = 0; ch < nchunks; ++ch) {
      const unsigned clo = s.chunk_lo[ch], chi = s.chunk_hi[ch];
      if (tid == 0) s.ncand = 0u;
      __syncthreads();
      // ---- gather the surviving elements of this chunk
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned k = keyof(e);
        if (k != 0u && k > R.key_lo && k <= R.key_hi) {
          const unsigned b = bin_of(k, R);
          if (b >= clo && b <= chi && s.cand[b]) {
            const unsigned slot = atomicAdd(&s.ncand, 1u);
            if (slot < (unsigned)kCandMax) {
              const u128 pe = pterm(e);
              s.c_key[slot] = k;
              s.c_bin[slot] = b;
              s.c_plo[slot] = pe.lo;
              s.c_phi[slot] = pe.hi;
              if (W) {
                const u128 he = hterm(e);
                s.c_hlo[slot] = he.lo;
                s.c_hhi[slot] = he.hi;
              }
            }
          }
        }
      }
      __syncthreads();
      // ---- score "all eligible elements >= this one" for each survivor
      const unsigned nc = s.ncand < (unsigned)kCandMax ? s.ncand : (unsigned)kCandMax;
      double myS = -1.0;
      unsigned myK = 0u;
      for (unsigned t = tid; t < nc; t += NT) {
        const unsigned kt = s.c_key[t], bt = s.c_bin[t];
        u128 P = mk128(s.xp_lo[bt], s.xp_hi[bt]);
        u128 H = W ? mk128(s.xh_lo[bt], s.xh_hi[bt]) : mk128(0, 0);
        unsigned C = s.xcnt[bt];
        for (unsigned j = 0; j < nc; ++j) {
          if (s.c_bin[j] == bt && s.c_key[j] >= kt) {
            P = add128(P, mk128(s.c_plo[j], s.c_phi[j]));
            if (W) H = add128(H, mk128(s.c_hlo[j], s.c_hhi[j]));
            ++C;
          }
        }
        s.r_plo[t] = P.lo;
        s.r_phi[t] = P.hi;
        if (W) {
          s.r_hlo[t] = H.lo;
          s.r_hhi[t] = H.hi;
        }
        s.r_cnt[t] = C;
        const double Pd = to_double(P);
        const double Hd = W ? to_double(H) : (double)C;
        const double St = Pd * Pd / Hd;
        if (better(St, kt, myS, myK)) {
          myS = St;
          myK = kt;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double S2 = __shfl_xor(myS, o);
        const unsigned k2 = __shfl_xor(myK, o);
        if (better(S2, k2, myS, myK)) {
          myS = S2;
          myK = k2;
        }
      }
      if (lane == 0) {
        s.red_d[wid] = myS;
        s.red_k[wid] = myK;
      }
      __syncthreads();
      if (tid == 0) {
        double S = -1.0;
        unsigned K = 0u;
        for (int w = 0; w < NW; ++w)
          if (better(s.red_d[w], s.red_k[w], S, K)) {
            S = s.red_d[w];
            K = s.red_k[w];
          }
        if (better(S, K, s.best_S, s.best_key)) {
          for (unsigned t = 0; t < nc; ++t)
            if (s.c_key[t] == K) {  // every slot holding this key carries identical sums
              s.best_S = S;
              s.best_key = K;
              s.best_plo = s.r_plo[t];
              s.best_phi = s.r_phi[t];
              if (W) {
                s.best_hlo = s.r_hlo[t];
                s.best_hhi = s.r_hhi[t];
              }
              s.best_cnt = s.r_cnt[t];
              break;
            }
        }
      }
      __syncthreads();
    }
  }
  out.tkey = s.best_key;
  out.count = s.best_cnt;
  out.P = ldexp(to_double(mk128(s.best_plo, s.best_phi)), -scP);
  out.H = W ? ldexp(to_double(mk128(s.best_hlo, s.best_hhi)), -scH) : (double)s.best_cnt;
  __syncthreads();
  return out;
}

}  // namespace externd
