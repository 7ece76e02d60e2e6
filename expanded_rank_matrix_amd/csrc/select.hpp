// Exact ternary projection T_tau(x; h) computed by one workgroup.
//
// Definition (reading of the adaptive ternarization operator, ExTernD review, Method;
// pith.science free parameters, tau / Eq. 2): among the elements with |x_i| >= tau * max|x|
// (and x_i != 0), the support is the top-j set by |x| whose score S = (sum h|x|)^2 / (sum h)
// is largest, the smallest j on ties; the result carries the signs of x.  With weights this is
// the corrected V-step of the importance-weighted variant (review, Method).
//
// GPU formulation.  Along a group of equal |x| the score of a partial prefix is quasi-convex in
// the weight added, so it never beats both ends of the group: the optimum is a threshold t,
// support = {eligible i : |x_i| >= t}, t one of the distinct eligible values, and "smallest j"
// means "largest t".  The search needs no sort:
//   1. histogram the eligible values by their fp32 bit pattern ("key") into 1024 bins (64 per
//      octave below the maximum, the last bin catches the rest), with counts and fp64 sums of
//      h|x| and h (LDS atomics; used for pruning only);
//   2. every bin boundary is a threshold whose score follows from the prefix sums; a bin's
//      interior can only win if (P_above + top_of_bin * H_bin)^2 / (H_above + H_bin) reaches the
//      best boundary score (each added element adds at most top_of_bin per unit weight, and the
//      score is quasi-convex in the added weight).  The bins that can hold the optimum form a
//      narrow window (typically three bins, a few dozen elements).  A window with too many
//      elements is histogrammed again over its own key range at a finer bin width;
//   3. the window's elements are scored exactly: P(t) = P_above + sum over window elements with
//      key >= t, every sum an exact 128-bit fixed-point integer (order independent), so the
//      decision is canonical: it depends neither on the launch shape nor on atomic ordering.
//      Each wave scores 64 window elements against the whole window (LDS broadcast reads).
#pragma once
#include "common.hpp"

namespace externd {

constexpr int kSelBins = 1024;      // bins per histogram level
constexpr int kSelShift0 = 23 - 6;  // first level: fp32 mantissa bits dropped per bin (64/octave)
constexpr int kWinMax = 256;        // window elements scored in one pass (4 waves x 64)
constexpr int kSelLevels = 4;       // histogram levels before the distinct-key walk

// LDS scratch of one selection; the weight sums exist only where weighted selections run.
template <bool HW>
struct SelScratchT {
  unsigned cnt[kSelBins];
  double psum[kSelBins];
  double hsum[HW ? kSelBins : 1];
  unsigned w_key[kWinMax];
  u64 w_plo[kWinMax], w_phi[kWinMax];
  u64 w_hlo[HW ? kWinMax : 1], w_hhi[HW ? kWinMax : 1];
  u64 a_plo[16], a_phi[16], a_hlo[16], a_hhi[16];  // per-wave exact partial sums
  unsigned a_cnt[16];
  u64 f_plo[16], f_phi[16], f_hlo[16], f_hhi[16];  // per-wave best threshold
  unsigned f_cnt[16];
  double f_s[16];
  unsigned f_k[16];
  double d_p[16], d_h[16];  // per-wave fp64 sums above a refined histogram's range
  unsigned red_u[16];
  double w_sp[16], w_sh[16];  // per-wave scan totals
  unsigned w_sc[16];
  double w_bn[16], w_bd[16];  // per-wave best boundary
  int w_lo[16], w_hi[16];     // per-wave candidate bin range
  unsigned w_clo[16], w_chi[16];
  double bn, bd;              // best boundary score so far, as a fraction
  unsigned slot;
};

struct SelResult {
  unsigned tkey;   // support = eligible elements with key >= tkey
  unsigned ekey;   // eligibility: key >= ekey
  double P, H;     // sum h|x| and sum h over the support (real units)
  unsigned count;  // support size (0: empty)
};

__device__ __forceinline__ bool better(double S1, unsigned k1, double S2, unsigned k2) {
  return S1 > S2 || (S1 == S2 && k1 > k2);
}

// Whether a slot holding x is in the support of r.
__device__ __forceinline__ bool selected(float x, const SelResult& r) {
  const unsigned k = __float_as_uint(x) & 0x7FFFFFFFu;
  return r.count > 0u && k != 0u && k >= r.ekey && k >= r.tkey;
}

// Clears the first histogram and publishes each wave's largest key (kx: this thread's largest
// |x| bit pattern) for a following ternary_select<..., PRE = true>; ends with a barrier.  Lets a
// caller that already touches every element fold this pass into its own loop.
template <int NT, bool HW>
__device__ __forceinline__ void select_prepare(SelScratchT<HW>& s, unsigned kx) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  kx = wave_max_u32(kx);
  if (lane == 0) s.red_u[wid] = kx;
  for (int b = tid; b < kSelBins; b += NT) {
    s.cnt[b] = 0u;
    s.psum[b] = 0.0;
    if (HW) s.hsum[b] = 0.0;
  }
  if (tid == 0) {
    s.slot = 0u;
    s.bn = 0.0;
    s.bd = 1.0;
  }
  __syncthreads();
}

// All NT threads of the workgroup call this.  vals[0..L) (LDS or global, fp32 or fp64) holds the
// vector; its fp32 rounding is what is projected.  hl[0..L) holds the weights (read only when W).
// EHm: exponent with max(h) < 2^EHm (W only).  Every thread receives the same result.  PRE: the
// caller already ran select_prepare with the vector's largest key.
template <int NT, bool W, typename T, bool HW, bool PRE = false>
__device__ __forceinline__ SelResult ternary_select(const T* vals, const float* hl, int L, float tau, int EHm,
                                    SelScratchT<HW>& s) {
  static_assert(HW || !W, "a weighted selection needs the weighted scratch");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int NW = NT / 64;
  SelResult out;
  out.tkey = 0xFFFFFFFFu;
  out.ekey = 0xFFFFFFFFu;
  out.P = 0.0;
  out.H = 0.0;
  out.count = 0u;
  if (!PRE) {  // max |x| and the cleared histogram
    unsigned kx = 0;
    for (int i = tid; i < L; i += NT) {
      const unsigned k = __float_as_uint((float)vals[i]) & 0x7FFFFFFFu;
      kx = k > kx ? k : kx;
    }
    select_prepare<NT>(s, kx);
  }
  unsigned km = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) km = s.red_u[w] > km ? s.red_u[w] : km;
  if (km == 0u) {
    __syncthreads();
    return out;
  }
  const float M = __uint_as_float(km);
  const double theta = (double)tau * (double)M;
  unsigned ekey;  // the least positive float f with (double)f >= theta
  {
    unsigned t = __float_as_uint((float)theta);
    if ((double)__uint_as_float(t) < theta) ++t;
    while (t > 1u && (double)__uint_as_float(t - 1u) >= theta) --t;
    ekey = t == 0u ? 1u : t;
  }
  out.ekey = ekey;
  auto keyof = [&](int i) -> unsigned {
    const unsigned k = __float_as_uint((float)vals[i]) & 0x7FFFFFFFu;
    return k >= ekey ? k : 0u;
  };

  // ---- histogram levels.  Level 0 covers keys <= km with bins of 2^17 keys (the last bin
  // catches the rest); a later level covers the previous window (wk_lo, wk_hi] at a finer shift.
  unsigned kt = km, klo = 0u, wk_hi = 0u, wk_lo = 0u;
  int sh = kSelShift0;
  int mode = 0;
  for (int level = 0; level < kSelLevels; ++level) {
    if (level > 0) {
      for (int b = tid; b < kSelBins; b += NT) {
        s.cnt[b] = 0u;
        s.psum[b] = 0.0;
        if (W) s.hsum[b] = 0.0;
      }
      __syncthreads();
    }
    // Bin b is stored at (b % BPL) * NT + b / BPL so that thread t, which owns bins
    // BPL t .. BPL t + BPL - 1 in the scan below, reads consecutive addresses across lanes.
    constexpr int BPL = kSelBins / NT;
    double dp = 0.0, dh = 0.0;  // fp64 sums above the range (level > 0)
    for (int i = tid; i < L; i += NT) {
      const unsigned k = keyof(i);
      if (k == 0u || k <= klo) continue;
      const double av = (double)__uint_as_float(k);
      const double hw = W ? (double)hl[i] : 1.0;
      if (k > kt) {
        dp += hw * av;
        dh += hw;
        continue;
      }
      unsigned b = (kt - k) >> sh;
      b = b > (unsigned)(kSelBins - 1) ? (unsigned)(kSelBins - 1) : b;
      const unsigned hb = (b % BPL) * NT + b / BPL;
      atomicAdd(&s.cnt[hb], 1u);
      atomicAdd(&s.psum[hb], hw * av);
      if (W) atomicAdd(&s.hsum[hb], hw);
    }
    if (level > 0) {
      dp = wave_sum_f64(dp);
      dh = wave_sum_f64(dh);
      if (lane == 0) {
        s.d_p[wid] = dp;
        s.d_h[wid] = dh;
      }
    }
    __syncthreads();
    // ---- all threads: prefix sums, boundary scores, interior bounds -> window of bins.  Scores
    // are compared as fractions (num * den' vs num' * den) to avoid fp64 divisions.  Every thread
    // ends with the same window (the cross-wave steps read the same LDS values in the same order).
    double bp[BPL], bh[BPL];
    unsigned bc[BPL];
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      bc[q] = s.cnt[q * NT + tid];
      bp[q] = s.psum[q * NT + tid];
      bh[q] = W ? s.hsum[q * NT + tid] : (double)bc[q];
    }
    double P0 = 0.0, H0 = 0.0;
    if (level > 0) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        P0 += s.d_p[w];
        H0 += s.d_h[w];
      }
    }
    double tp = 0.0, th = 0.0;
    unsigned tc = 0u;
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      tp += bp[q];
      th += bh[q];
      tc += bc[q];
    }
    const double ip = wave_scan_f64(tp), ih = W ? wave_scan_f64(th) : 0.0;
    const unsigned ic = wave_scan_u32(tc);
    if (lane == 63) {
      s.w_sp[wid] = ip;
      s.w_sh[wid] = W ? ih : (double)ic;
      s.w_sc[wid] = ic;
    }
    __syncthreads();
    double rp0 = P0, rh0 = H0;  // prefix before this thread's first bin
    unsigned rc0 = 0u;
    for (int w = 0; w < wid; ++w) {
      rp0 += s.w_sp[w];
      rh0 += s.w_sh[w];
      rc0 += s.w_sc[w];
    }
    rp0 += ip - tp;
    rh0 += W ? ih - th : (double)(ic - tc);
    rc0 += ic - tc;
    // best boundary score as a fraction bn / bd (carried over from earlier levels)
    double bn = s.bn, bd = s.bd;
    {
      double rp = rp0, rh = rh0;
#pragma unroll
      for (int q = 0; q < BPL; ++q) {
        rp += bp[q];
        rh += bh[q];
        if (bc[q] != 0u && rp * rp * bd > bn * rh) {
          bn = rp * rp;
          bd = rh;
        }
      }
    }
    // wave maximum (lane 63); a zero-filled operand (0, 0) never wins
#define EXTERND_STEP(C, R)                                  \
  {                                                         \
    const double n2 = dppf64<C, R>(bn), d2 = dppf64<C, R>(bd); \
    if (n2 * bd > bn * d2) {                                \
      bn = n2;                                              \
      bd = d2;                                              \
    }                                                       \
  }
    EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
    if (lane == 63) {
      s.w_bn[wid] = bn;
      s.w_bd[wid] = bd;
    }
    __syncthreads();
    bn = s.w_bn[0];
    bd = s.w_bd[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
      if (s.w_bn[w] * bd > bn * s.w_bd[w]) {
        bn = s.w_bn[w];
        bd = s.w_bd[w];
      }
    const double cutn = bn * (1.0 - 1e-9);  // candidate if score * bd >= cutn
    int lo = kSelBins, hi = -1;
    unsigned clo = 0u, chi = 0u;  // element counts before bin lo / through bin hi
    {
      double rp = rp0, rh = rh0;
      unsigned rc = rc0;
#pragma unroll
      for (int q = 0; q < BPL; ++q) {
        const int b = tid * BPL + q;
        const unsigned c = bc[q];
        const double Pi = rp + bp[q], Hi = rh + bh[q];
        bool cand = c != 0u && Pi * Pi * bd >= cutn * Hi;
        if (!cand && c >= 2u) {
          const unsigned off = (unsigned)b << sh;
          const unsigned top = kt > off ? kt - off : 0u;  // largest key the bin can hold
          const double t1 = rp + (double)__uint_as_float(top) * bh[q];
          cand = t1 * t1 * bd >= cutn * Hi || (rh > 0.0 && rp * rp * bd >= cutn * rh);
        }
        if (cand) {
          if (b < lo) {
            lo = b;
            clo = rc;
          }
          if (b > hi) {
            hi = b;
            chi = rc + c;
          }
        }
        rp = Pi;
        rh = Hi;
        rc += c;
      }
    }
    // wave minimum of lo and maximum of hi (lane 63), with their counts; encoded so that a
    // zero-filled operand is neutral: xlo = kSelBins - lo, xhi = hi + 1
    {
      unsigned xlo = (unsigned)(kSelBins - lo), xhi = (unsigned)(hi + 1);
#define EXTERND_STEP(C, R)                                                  \
  {                                                                         \
    const unsigned l2 = dpp32<C, R>(xlo), c2 = dpp32<C, R>(clo);              \
    const unsigned h2 = dpp32<C, R>(xhi), d2 = dpp32<C, R>(chi);              \
    if (l2 > xlo) {                                                         \
      xlo = l2;                                                             \
      clo = c2;                                                             \
    }                                                                       \
    if (h2 > xhi) {                                                         \
      xhi = h2;                                                             \
      chi = d2;                                                             \
    }                                                                       \
  }
      EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
      if (lane == 63) {
        s.w_lo[wid] = kSelBins - (int)xlo;
        s.w_hi[wid] = (int)xhi - 1;
        s.w_clo[wid] = clo;
        s.w_chi[wid] = chi;
      }
    }
    __syncthreads();
    lo = kSelBins;
    hi = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (s.w_lo[w] < lo) {
        lo = s.w_lo[w];
        clo = s.w_clo[w];
      }
      if (s.w_hi[w] > hi) {
        hi = s.w_hi[w];
        chi = s.w_chi[w];
      }
    }
    const unsigned nw = chi - clo;
    {
      const unsigned offlo = (unsigned)lo << sh;
      const unsigned whi = kt > offlo ? kt - offlo : 0u;
      const long long wlo = (long long)kt - ((long long)(hi + 1) << sh);
      // the last bin of the first level also holds every smaller key
      const bool tail = level == 0 && hi == kSelBins - 1;
      const unsigned wlo_u = (tail || wlo < (long long)klo) ? klo : (unsigned)wlo;
      int md = 1, nsh = 0;
      if (nw > (unsigned)kWinMax) {
        md = 2;
        const unsigned range = whi - wlo_u;  // keys in (wlo_u, whi]
        if (sh > 0 && range > 1u) {
          while (((range - 1u) >> nsh) > (unsigned)(kSelBins - 1)) ++nsh;
          if (nsh < sh || tail) md = 3;  // a finer (or tail-resolving) level exists
        }
      }
      wk_hi = whi;
      wk_lo = wlo_u;
      mode = md;
      if (tid == 0) {
        s.bn = bn;
        s.bd = bd;
      }
      if (mode != 3 || level == kSelLevels - 1) {
        if (mode == 3) mode = 2;
        break;
      }
      kt = whi;
      klo = wlo_u;
      sh = nsh;
    }
  }
  const int EM = exp_bound(M);
  const int scP = W ? (100 - EM - EHm) : (100 - EM);
  const int scH = W ? (100 - EHm) : 0;
  auto pterm = [&](int i, unsigned k) -> u128 {
    const double av = (double)__uint_as_float(k);
    return W ? fixp((double)hl[i] * av, scP) : fixp(av, scP);
  };
  auto hterm = [&](int i) -> u128 { return W ? fixp((double)hl[i], scH) : mk128(1ull, 0ull); };
  // per-wave exact partials -> LDS -> every thread sums them in wave order
  auto block_sum128 = [&](u128 p, u128 h, unsigned c, u128& P, u128& H, unsigned& C) {
    p = wave_sum128(p);
    if (W) h = wave_sum128(h);
    c = wave_sum_u32(c);
    __syncthreads();
    if (lane == 0) {
      s.a_plo[wid] = p.lo;
      s.a_phi[wid] = p.hi;
      s.a_hlo[wid] = h.lo;
      s.a_hhi[wid] = h.hi;
      s.a_cnt[wid] = c;
    }
    __syncthreads();
    P = mk128(0, 0);
    H = mk128(0, 0);
    C = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      P = add128(P, mk128(s.a_plo[w], s.a_phi[w]));
      if (W) H = add128(H, mk128(s.a_hlo[w], s.a_hhi[w]));
      C += s.a_cnt[w];
    }
  };
  // ---- one pass: exact sums above the window and, to be scored, the window's elements
  u128 AP, AH;
  unsigned AC;
  {
    u128 p = mk128(0, 0), h = mk128(0, 0);
    unsigned c = 0u;
    for (int i = tid; i < L; i += NT) {
      const unsigned k = keyof(i);
      if (k == 0u || k <= wk_lo) continue;
      if (k > wk_hi) {
        p = add128(p, pterm(i, k));
        if (W) h = add128(h, hterm(i));
        ++c;
      } else if (mode == 1) {
        const unsigned slot = atomicAdd(&s.slot, 1u);
        if (slot < (unsigned)kWinMax) {
          const u128 pe = pterm(i, k);
          s.w_key[slot] = k;
          s.w_plo[slot] = pe.lo;
          s.w_phi[slot] = pe.hi;
          if (W) {
            const u128 he = hterm(i);
            s.w_hlo[slot] = he.lo;
            s.w_hhi[slot] = he.hi;
          }
        }
      }
    }
    block_sum128(p, h, c, AP, AH, AC);  // its barriers also publish the window
  }
  double myS = -1.0;
  unsigned myK = 0u;
  u128 myP = mk128(0, 0), myH = mk128(0, 0);
  unsigned myC = 0u;
  if (mode == 1) {
    // wave w scores window elements 64 w .. 64 w + 63 against every window element
    const unsigned ns = s.slot;
    const int nwin = ns < (unsigned)kWinMax ? (int)ns : kWinMax;
    const int e = wid * 64 + lane;
    if (wid * 64 < nwin) {
      const unsigned ke = e < nwin ? s.w_key[e] : 0xFFFFFFFFu;
      u128 P = AP, H = AH;
      unsigned C = AC;
#pragma unroll 4
      for (int j = 0; j < nwin; ++j) {
        const unsigned kj = s.w_key[j];
        const u64 plo = s.w_plo[j], phi = s.w_phi[j];
        const bool in = kj >= ke;
        P = add128(P, mk128(in ? plo : 0ull, in ? phi : 0ull));
        if (W) {
          const u64 hlo = s.w_hlo[j], hhi = s.w_hhi[j];
          H = add128(H, mk128(in ? hlo : 0ull, in ? hhi : 0ull));
        }
        C += in ? 1u : 0u;
      }
      if (e < nwin) {
        const double Pd = to_double(P);
        const double Hd = W ? to_double(H) : (double)C;
        myS = Pd * Pd / Hd;
        myK = ke;
        myP = P;
        myH = H;
        myC = C;
      }
    }
  } else {
    // Many window elements with few distinct keys (heavy ties): walk the distinct keys
    // downwards and score each with an exact block reduction.
    unsigned prev = wk_hi + 1u;
    for (;;) {
      unsigned best = 0u;
      for (int i = tid; i < L; i += NT) {
        const unsigned k = keyof(i);
        if (k > wk_lo && k < prev) best = k > best ? k : best;
      }
      best = wave_max_u32(best);
      __syncthreads();
      if (lane == 0) s.red_u[wid] = best;
      __syncthreads();
      best = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) best = s.red_u[w] > best ? s.red_u[w] : best;
      if (best == 0u) break;
      u128 p = mk128(0, 0), h = mk128(0, 0);
      unsigned c = 0u;
      for (int i = tid; i < L; i += NT) {
        const unsigned k = keyof(i);
        if (k >= best && k <= wk_hi) {
          p = add128(p, pterm(i, k));
          if (W) h = add128(h, hterm(i));
          ++c;
        }
      }
      u128 P, H;
      unsigned C;
      block_sum128(p, h, c, P, H, C);
      P = add128(P, AP);
      if (W) H = add128(H, AH);
      C += AC;
      const double Pd = to_double(P);
      const double Hd = W ? to_double(H) : (double)C;
      const double St = Pd * Pd / Hd;
      if (tid == 0 && better(St, best, myS, myK)) {  // tracked by thread 0 only
        myS = St;
        myK = best;
        myP = P;
        myH = H;
        myC = C;
      }
      prev = best;
    }
  }
  // ---- argmax over (score desc, key desc): within the wave (toward lane 63; a zero-filled
  // operand, score 0, loses to every real threshold), then across waves.  Lanes with equal
  // (score, key) hold equal sums.
  int src = lane;
#define EXTERND_STEP(C, R)                                                               \
  {                                                                                      \
    const double S2 = dppf64<C, R>(myS);                                                 \
    const unsigned k2 = dpp32<C, R>(myK), s2 = dpp32<C, R>((unsigned)src);                \
    if (better(S2, k2, myS, myK)) {                                                      \
      myS = S2;                                                                          \
      myK = k2;                                                                          \
      src = (int)s2;                                                                     \
    }                                                                                    \
  }
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  myS = readlane_f64(myS, 63);
  myK = readlane32(myK, 63);
  src = (int)readlane32((unsigned)src, 63);
  {
    const u64 plo = readlane64(myP.lo, src), phi = readlane64(myP.hi, src);
    const u64 hlo = readlane64(myH.lo, src), hhi = readlane64(myH.hi, src);
    const unsigned cc = __builtin_amdgcn_readlane(myC, src);
    if (lane == 0) {
      s.f_s[wid] = myS;
      s.f_k[wid] = myK;
      s.f_plo[wid] = plo;
      s.f_phi[wid] = phi;
      s.f_hlo[wid] = hlo;
      s.f_hhi[wid] = hhi;
      s.f_cnt[wid] = cc;
    }
  }
  __syncthreads();
  double S = -1.0;
  unsigned K = 0u;
  int bw = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (better(s.f_s[w], s.f_k[w], S, K)) {
      S = s.f_s[w];
      K = s.f_k[w];
      bw = w;
    }
  out.tkey = K;
  out.count = s.f_cnt[bw];
  out.P = ldexp(to_double(mk128(s.f_plo[bw], s.f_phi[bw])), -scP);
  out.H = W ? ldexp(to_double(mk128(s.f_hlo[bw], s.f_hhi[bw])), -scH) : (double)out.count;
  __syncthreads();
  return out;
}

}  // namespace externd
