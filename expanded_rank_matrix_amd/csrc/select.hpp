// Ternary projection T_tau(x; h) computed by one workgroup.
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
//      octave below the maximum, the last bin catches the rest): counts and sums of h|x| and h as
//      64-bit fixed-point integers (LDS integer atomics: exact, so the sums do not depend on the
//      order in which threads add them);
//   2. every bin boundary is a threshold whose score follows from the prefix sums; a bin's
//      interior can only win if (P_above + top_of_bin * H_bin)^2 / (H_above + H_bin) reaches the
//      best boundary score (each added element adds at most top_of_bin per unit weight, and the
//      score is quasi-convex in the added weight).  The bins that can hold the optimum form a
//      narrow window (typically three bins, a few dozen elements); the prefix sums also give the
//      sums over everything above it.  A window with too many elements is histogrammed again over
//      its own key range at a finer bin width;
//   3. the window's elements are scored: P(t) = P_above + sum over window elements with key >= t,
//      all in the same fixed point, so every workgroup that runs the selection on the same vector
//      reaches the same decision whatever its thread count or atomic ordering.
// Fixed-point scales: one unit of P is 2^-sP with sP = 62 - EM - EHm - LB (|x| < 2^EM, h < 2^EHm,
// L < 2^LB), so no sum can overflow, and each element is truncated by less than 2^-47 of the
// largest |x|.
#pragma once
#include "common.hpp"

namespace externd {

constexpr int kSelBins = 1024;      // bins per histogram level
constexpr int kSelShift0 = 23 - 6;  // first level: fp32 mantissa bits dropped per bin (64/octave)
constexpr int kWinMax = 256;        // window elements scored in one pass (4 waves x 64)
static_assert(kWinMax % 16 == 0, "the key selection pads its window to a multiple of 16");
constexpr int kSelLevels = 4;       // histogram levels before the distinct-key walk

// LDS scratch of one selection; the weight sums exist only where weighted selections run.
template <bool HW>
struct SelScratchT {
  unsigned cnt[kSelBins];
  u64 psum[kSelBins];
  u64 hsum[HW ? kSelBins : 1];
  alignas(16) unsigned w_key[kWinMax];
  alignas(16) u64 w_p[kWinMax];
  u64 w_h[HW ? kWinMax : 1];
  u64 a_p[16], a_h[16];  // per-wave sums (above a refined range; the distinct-key walk)
  unsigned a_c[16];
  u64 w_sp[16], w_sh[16];  // per-wave scan totals
  unsigned w_sc[16];
  double w_bn[16], w_bd[16];  // per-wave best boundary
  int w_lo[16], w_hi[16];     // per-wave candidate bin range
  unsigned w_clo[16], w_chi[16];
  u64 w_plo[16], w_hlo[16];   // sums over everything above bin lo
  double f_s[16];             // per-wave best threshold
  unsigned f_k[16], f_c[16];
  u64 f_p[16], f_h[16];
  unsigned red_u[16];
  double bn, bd;  // best boundary score so far, as a fraction
  unsigned slot;
  // window of the key-array selection: keys [win_klo, win_khi], sums above it, element count
  unsigned win_klo, win_khi, win_ac, win_nw;
  u64 win_ap;
};

struct SelResult {
  unsigned tkey;   // support = eligible elements with key >= tkey
  unsigned ekey;   // eligibility: key >= ekey
  double P, H;     // sum h|x| and sum h over the support (real units, from the fixed point)
  unsigned count;  // support size (0: empty)
};

__device__ __forceinline__ bool better(double S1, unsigned k1, double S2, unsigned k2) {
  return S1 > S2 || (S1 == S2 && k1 > k2);
}

// floor(x * 2^sc) for finite x >= 0 whose result is below 2^63.
__device__ __forceinline__ u64 fix64(double x, int sc) {
  const u64 bits = (u64)__double_as_longlong(x);
  const int ef = (int)((bits >> 52) & 0x7FF);
  if (ef == 0) return 0ull;  // zero or subnormal: far below one unit
  const u64 mant = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int sh = ef - 1075 + sc;
  if (sh >= 0) return mant << sh;
  return sh > -64 ? mant >> (-sh) : 0ull;
}

// floor(value * 2^sc) for the positive finite fp32 bit pattern k, whose result is below 2^63
// (the same value as fix64 of its exact double).
__device__ __forceinline__ u64 fixkey(unsigned k, int sc) {
  const unsigned ex = k >> 23;
  const u64 mant = (u64)((k & 0x7FFFFFu) | (ex != 0u ? 0x800000u : 0u));
  const int sh = (int)(ex != 0u ? ex : 1u) - 150 + sc;
  const u64 up = mant << (sh & 63), dn = mant >> ((-sh) & 63);
  return sh >= 0 ? up : (sh > -64 ? dn : 0ull);
}

__device__ __forceinline__ u64 wave_scan_u64(u64 v) {
#define EXTERND_STEP(C, R) v += dpp64<C, R>(v);
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  return v;
}
__device__ __forceinline__ u64 wave_sum_u64(u64 v) { return readlane64(wave_scan_u64(v), 63); }

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
    s.psum[b] = 0ull;
    if (HW) s.hsum[b] = 0ull;
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
  // fixed-point scales (see the header)
  const int LB = 32 - __clz((unsigned)L);
  const int EM = exp_bound(M);
  const int sP = 62 - EM - (W ? EHm : 0) - LB;
  const int sH = 62 - EHm - LB;
  auto pterm = [&](int i, unsigned k) -> u64 {
    if (!W) return fixkey(k, sP);
    return fix64((double)hl[i] * (double)__uint_as_float(k), sP);
  };
  auto hterm = [&](int i) -> u64 { return W ? fix64((double)hl[i], sH) : 1ull; };
  // Passes over the vector take kGrp elements per thread at a time, loading them all first so
  // that their latencies overlap.
  constexpr int kGrp = 4;
  // a key's value per unit of H, in P units: converts top * H_bin into P units
  const double tconv = W ? ldexp(1.0, sP - sH) : ldexp(1.0, sP);

  // ---- histogram levels.  Level 0 covers keys <= km with bins of 2^17 keys (the last bin
  // catches the rest); a later level covers the previous window (wk_lo, wk_hi] at a finer shift.
  unsigned kt = km, klo = 0u, wk_hi = 0u, wk_lo = 0u;
  int sh = kSelShift0;
  int mode = 0;
  u64 AP = 0ull, AH = 0ull;  // sums over everything above the window
  unsigned AC = 0u;
  for (int level = 0; level < kSelLevels; ++level) {
    if (level > 0) {
      for (int b = tid; b < kSelBins; b += NT) {
        s.cnt[b] = 0u;
        s.psum[b] = 0ull;
        if (W) s.hsum[b] = 0ull;
      }
      __syncthreads();
    }
    // Bin b is stored at (b % BPL) * NT + b / BPL so that thread t, which owns bins
    // BPL t .. BPL t + BPL - 1 in the scan below, reads consecutive addresses across lanes.
    constexpr int BPL = kSelBins / NT;
    u64 dp = 0ull, dh = 0ull;  // sums above the range (level > 0)
    unsigned dc = 0u;
    for (int i0 = tid; i0 < L; i0 += kGrp * NT) {
      unsigned kk[kGrp];
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {  // clamped index: every load is issued before any is used
        const int i = i0 + u * NT;
        const unsigned k = keyof(i < L ? i : L - 1);
        kk[u] = i < L ? k : 0u;
      }
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const unsigned k = kk[u];
        const int i = i0 + u * NT;
        if (k == 0u || k <= klo) continue;
        const u64 pt = pterm(i, k), ht = hterm(i);
        if (k > kt) {
          dp += pt;
          dh += ht;
          ++dc;
          continue;
        }
        unsigned b = (kt - k) >> sh;
        b = b > (unsigned)(kSelBins - 1) ? (unsigned)(kSelBins - 1) : b;
        const unsigned hb = (b % BPL) * NT + b / BPL;
        atomicAdd(&s.cnt[hb], 1u);
        atomicAdd(&s.psum[hb], pt);
        if (W) atomicAdd(&s.hsum[hb], ht);
      }
    }
    if (level > 0) {
      dp = wave_sum_u64(dp);
      dh = W ? wave_sum_u64(dh) : 0ull;
      dc = wave_sum_u32(dc);
      if (lane == 0) {
        s.a_p[wid] = dp;
        s.a_h[wid] = dh;
        s.a_c[wid] = dc;
      }
    }
    __syncthreads();
    // ---- all threads: prefix sums, boundary scores, interior bounds -> window of bins.  Scores
    // are compared as fractions (num * den' vs num' * den) to avoid divisions.  Every thread ends
    // with the same window (the cross-wave steps read the same LDS values in the same order).
    u64 bp[BPL], bh[BPL];
    unsigned bc[BPL];
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      bc[q] = s.cnt[q * NT + tid];
      bp[q] = s.psum[q * NT + tid];
      bh[q] = W ? s.hsum[q * NT + tid] : (u64)bc[q];
    }
    u64 P0 = 0ull, H0 = 0ull;
    unsigned C0 = 0u;
    if (level > 0) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        P0 += s.a_p[w];
        H0 += s.a_h[w];
        C0 += s.a_c[w];
      }
      if (!W) H0 = C0;
    }
    u64 tp = 0ull, th = 0ull;
    unsigned tc = 0u;
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      tp += bp[q];
      th += bh[q];
      tc += bc[q];
    }
    const u64 ip = wave_scan_u64(tp);
    const unsigned ic = wave_scan_u32(tc);
    const u64 ih = W ? wave_scan_u64(th) : (u64)ic;
    if (lane == 63) {
      s.w_sp[wid] = ip;
      s.w_sh[wid] = ih;
      s.w_sc[wid] = ic;
    }
    __syncthreads();
    u64 rp0 = P0, rh0 = H0;  // sums before this thread's first bin
    unsigned rc0 = C0;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) {  // all loads issued together, then masked
      const u64 p = s.w_sp[w], h = s.w_sh[w];
      const unsigned c = s.w_sc[w];
      rp0 += w < wid ? p : 0ull;
      rh0 += w < wid ? h : 0ull;
      rc0 += w < wid ? c : 0u;
    }
    rp0 += ip - tp;
    rh0 += ih - th;
    rc0 += ic - tc;
    // best boundary score as a fraction bn / bd (carried over from earlier levels)
    double bn = s.bn, bd = s.bd;
    {
      u64 rp = rp0, rh = rh0;
#pragma unroll
      for (int q = 0; q < BPL; ++q) {
        rp += bp[q];
        rh += bh[q];
        const double pd = (double)rp, hd = (double)rh;
        if (bc[q] != 0u && pd * pd * bd > bn * hd) {
          bn = pd * pd;
          bd = hd;
        }
      }
    }
    // wave maximum (lane 63); a zero-filled operand (0, 0) never wins
#define EXTERND_STEP(C, R)                                     \
  {                                                            \
    const double n2 = dppf64<C, R>(bn), d2 = dppf64<C, R>(bd); \
    if (n2 * bd > bn * d2) {                                   \
      bn = n2;                                                 \
      bd = d2;                                                 \
    }                                                          \
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
    unsigned clo = 0u, chi = 0u;  // element counts above bin lo / through bin hi
    u64 plo = 0ull, hlo = 0ull;   // sums above bin lo
    {
      u64 rp = rp0, rh = rh0;
      unsigned rc = rc0;
#pragma unroll
      for (int q = 0; q < BPL; ++q) {
        const int b = tid * BPL + q;
        const unsigned c = bc[q];
        const u64 Pi = rp + bp[q], Hi = rh + bh[q];
        const double pid = (double)Pi, hid = (double)Hi, rpd = (double)rp, rhd = (double)rh;
        bool cand = c != 0u && pid * pid * bd >= cutn * hid;
        if (!cand && c >= 2u) {
          const unsigned off = (unsigned)b << sh;
          const unsigned top = kt > off ? kt - off : 0u;  // largest key the bin can hold
          const double t1 = rpd + (double)__uint_as_float(top) * tconv * (double)bh[q];
          cand = t1 * t1 * bd >= cutn * hid || (rh > 0ull && rpd * rpd * bd >= cutn * rhd);
        }
        if (cand) {
          if (b < lo) {
            lo = b;
            clo = rc;
            plo = rp;
            hlo = rh;
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
    // wave minimum of lo and maximum of hi, then their prefix sums from the lanes that hold them
    // (thread t holds bins BPL t .. BPL t + BPL - 1)
    {
      const int wlo = kSelBins - (int)wave_max_u32((unsigned)(kSelBins - lo));
      const int whi = (int)wave_max_u32((unsigned)(hi + 1)) - 1;
      const int llo = wlo < kSelBins ? wlo / BPL - wid * 64 : 0;
      const int lhi = whi >= 0 ? whi / BPL - wid * 64 : 0;
      const unsigned c_lo = readlane32(clo, llo), c_hi = readlane32(chi, lhi);
      const u64 p_lo = readlane64(plo, llo), h_lo = readlane64(hlo, llo);
      if (lane == 0) {
        s.w_lo[wid] = wlo;
        s.w_hi[wid] = whi;
        s.w_clo[wid] = c_lo;
        s.w_chi[wid] = c_hi;
        s.w_plo[wid] = p_lo;
        s.w_hlo[wid] = h_lo;
      }
    }
    __syncthreads();
    lo = kSelBins;
    hi = -1;
    int low = 0, hiw = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int l = s.w_lo[w], h = s.w_hi[w];
      low = l < lo ? w : low;
      lo = l < lo ? l : lo;
      hiw = h > hi ? w : hiw;
      hi = h > hi ? h : hi;
    }
    clo = s.w_clo[low];
    plo = s.w_plo[low];
    hlo = s.w_hlo[low];
    chi = s.w_chi[hiw];
    const unsigned nw = chi - clo;
    AP = plo;
    AH = hlo;
    AC = clo;
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
  // ---- the window's elements into LDS
  if (mode == 1) {
    for (int i0 = tid; i0 < L; i0 += kGrp * NT) {
      unsigned kk[kGrp];
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {  // clamped index: every load is issued before any is used
        const int i = i0 + u * NT;
        const unsigned k = keyof(i < L ? i : L - 1);
        kk[u] = i < L ? k : 0u;
      }
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const unsigned k = kk[u];
        if (k != 0u && k > wk_lo && k <= wk_hi) {
          const int i = i0 + u * NT;
          const unsigned slot = atomicAdd(&s.slot, 1u);
          if (slot < (unsigned)kWinMax) {
            s.w_key[slot] = k;
            s.w_p[slot] = pterm(i, k);
            if (W) s.w_h[slot] = hterm(i);
          }
        }
      }
    }
    __syncthreads();
  }
  double myS = -1.0;
  unsigned myK = 0u, myC = 0u;
  u64 myP = 0ull, myH = 0ull;
  int nact = 1;  // waves that hold candidate thresholds (uniform)
  if (mode == 1) {
    // Element e's threshold sums P_e = AP + sum of w_p[j] over window elements j with
    // w_key[j] >= w_key[e].  The window's elements come in nch chunks of 64 (one per lane); each
    // chunk's j range is split into NW / nch parts, one wave per (chunk, part), whose partial sums
    // go to the (now free) bin arrays.  The waves of the first nch then add the parts in order.
    const unsigned ns = s.slot;
    const int nwin = ns < (unsigned)kWinMax ? (int)ns : kWinMax;
    const int nch = nwin > 64 ? (nwin + 63) >> 6 : 1;
    nact = nch;
    const int parts = NW / nch;
    const int span = (nwin + parts - 1) / parts;
    const int ch = wid % nch, part = wid / nch;
    const int e = ch * 64 + lane;
    if (part < parts) {
      const unsigned ke = e < nwin ? s.w_key[e] : 0xFFFFFFFFu;
      const int j0 = part * span, j1 = j0 + span < nwin ? j0 + span : nwin;
      u64 P = 0ull, H = 0ull;
      unsigned C = 0u;
#pragma unroll 4
      for (int j = j0; j < j1; ++j) {  // unconditional loads, masked sums
        const unsigned kj = s.w_key[j];
        const u64 pj = s.w_p[j], hj = W ? s.w_h[j] : 0ull;
        const u64 msk = kj >= ke ? ~0ull : 0ull;
        P += pj & msk;
        if (W) H += hj & msk;
        C += kj >= ke ? 1u : 0u;
      }
      const int slot = part * (nch * 64) + e;
      s.psum[slot] = P;
      if (W) s.hsum[slot] = H;
      s.cnt[slot] = C;
    }
    __syncthreads();
    if (wid < nch && e < nwin) {
      u64 P = AP, H = AH;
      unsigned C = AC;
#pragma unroll
      for (int q = 0; q < NW; ++q) {  // all loads issued together, then masked
        const int slot = (q < parts ? q : 0) * (nch * 64) + e;
        const u64 pq = s.psum[slot], hq = W ? s.hsum[slot] : 0ull;
        const unsigned cq = s.cnt[slot];
        P += q < parts ? pq : 0ull;
        if (W) H += q < parts ? hq : 0ull;
        C += q < parts ? cq : 0u;
      }
      const double Pd = (double)P;
      const double Hd = W ? (double)H : (double)C;
      myS = Pd * Pd / Hd;
      myK = s.w_key[e];
      myP = P;
      myH = W ? H : (u64)C;
      myC = C;
    }
  } else {
    // Many window elements with few distinct keys (heavy ties): walk the distinct keys
    // downwards and score each with a block reduction.
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
      u64 p = 0ull, h = 0ull;
      unsigned c = 0u;
      for (int i = tid; i < L; i += NT) {
        const unsigned k = keyof(i);
        if (k >= best && k <= wk_hi) {
          p += pterm(i, k);
          if (W) h += hterm(i);
          ++c;
        }
      }
      p = wave_sum_u64(p);
      h = W ? wave_sum_u64(h) : 0ull;
      c = wave_sum_u32(c);
      __syncthreads();
      if (lane == 0) {
        s.a_p[wid] = p;
        s.a_h[wid] = h;
        s.a_c[wid] = c;
      }
      __syncthreads();
      u64 P = AP, H = AH;
      unsigned C = AC;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        P += s.a_p[w];
        H += s.a_h[w];
        C += s.a_c[w];
      }
      if (!W) H = C;
      const double Pd = (double)P;
      const double St = Pd * Pd / (double)H;
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
  // ---- argmax over (score desc, key desc) among the candidate waves: within the wave (toward
  // lane 63; a zero-filled operand, score 0, loses to every real threshold), then across them.
  // Lanes with equal (score, key) hold equal sums.
  if (wid < nact) {
    int src = lane;
#define EXTERND_STEP(C, R)                                                 \
  {                                                                        \
    const double S2 = dppf64<C, R>(myS);                                   \
    const unsigned k2 = dpp32<C, R>(myK), s2 = dpp32<C, R>((unsigned)src); \
    if (better(S2, k2, myS, myK)) {                                        \
      myS = S2;                                                            \
      myK = k2;                                                            \
      src = (int)s2;                                                       \
    }                                                                      \
  }
    EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
    myS = readlane_f64(myS, 63);
    myK = readlane32(myK, 63);
    src = (int)readlane32((unsigned)src, 63);
    const u64 pp = readlane64(myP, src), hh = readlane64(myH, src);
    const unsigned cc = readlane32(myC, src);
    if (lane == 0) {
      s.f_s[wid] = myS;
      s.f_k[wid] = myK;
      s.f_p[wid] = pp;
      s.f_h[wid] = hh;
      s.f_c[wid] = cc;
    }
  }
  __syncthreads();
  double S = -1.0;
  unsigned K = 0u;
  int bw = 0;
  for (int w = 0; w < nact; ++w)
    if (better(s.f_s[w], s.f_k[w], S, K)) {
      S = s.f_s[w];
      K = s.f_k[w];
      bw = w;
    }
  out.tkey = K;
  out.count = s.f_c[bw];
  out.P = ldexp((double)s.f_p[bw], -sP);
  out.H = W ? ldexp((double)s.f_h[bw], -sH) : (double)out.count;
  __syncthreads();
  return out;
}

// ---- the same selection for unweighted vectors held as fp32 bit patterns in LDS ---------------
// keys[0..L): the fp32 roundings of the vector (sign bit included), km: the largest |key|, the
// histogram cleared beforehand (select_prepare).  The result equals ternary_select<NT, false>'s on
// the same values: the same candidate rule and the same exact scoring, with less work per element
// and fewer workgroup barriers, which is what bounds a selection of a few thousand values:
//  * bins are aligned to the fp32 exponent (64 per octave, bin b holds the keys with
//    key >> 17 == (km >> 17) - b, the last bin the rest), so every element of a bin but the last has
//    the same exponent and the bin's sum of P is an integer sum of 24-bit mantissas, shifted into
//    the fixed-point scale once per bin instead of once per element;
//  * thread t owns bins 2t and 2t + 1 (a wave: 128 contiguous bins), so the prefix sums, the best
//    boundary and the candidate window take one wave scan and one eight-value exchange each, and
//    every thread learns the window without a further round;
//  * the window's elements are scored by one wave, reading them four at a time.
// The window holds at most kWinMax elements; `ok` comes back false (result unset, every thread
// alike) when it would hold more, and the caller runs ternary_select instead after clearing the
// histogram again.
template <int NT, bool HW>
__device__ __forceinline__ SelResult ternary_select_keys(const unsigned* keys, int L, float tau, unsigned km,
                                                         SelScratchT<HW>& s, bool* ok) {
  static_assert(NT == 512, "two bins per thread");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int kLast = kSelBins - 1;
  SelResult out;
  out.tkey = 0xFFFFFFFFu;
  out.ekey = 0xFFFFFFFFu;
  out.P = 0.0;
  out.H = 0.0;
  out.count = 0u;
  *ok = true;
  if (km == 0u) return out;
  const float M = __uint_as_float(km);
  const double theta = (double)tau * (double)M;
  unsigned ekey;
  {
    unsigned t = __float_as_uint((float)theta);
    if ((double)__uint_as_float(t) < theta) ++t;
    while (t > 1u && (double)__uint_as_float(t - 1u) >= theta) --t;
    ekey = t == 0u ? 1u : t;
  }
  out.ekey = ekey;
  const int LB = 32 - __clz((unsigned)L);
  const int sP = 62 - exp_bound(M) - LB;
  const unsigned top = km >> 17;
  // ---- histogram
  constexpr int kGrp = 8;
  for (int i0 = tid; i0 < L; i0 += kGrp * NT) {
    unsigned kk[kGrp];
#pragma unroll
    for (int u = 0; u < kGrp; ++u) {  // clamped index: every load is issued before any is used
      const int i = i0 + u * NT;
      kk[u] = keys[i < L ? i : L - 1] & (i < L ? 0x7FFFFFFFu : 0u);
    }
#pragma unroll
    for (int u = 0; u < kGrp; ++u) {
      const unsigned k = kk[u];
      if (k == 0u || k < ekey) continue;
      const unsigned d = top - (k >> 17);
      if (d < (unsigned)kLast) {  // one atomic: the count in bits 40.., the mantissa sum below
        atomicAdd(&s.psum[d], (1ull << 40) | (u64)((k & 0x7FFFFFu) | ((k >> 23) != 0u ? 0x800000u : 0u)));
      } else {
        atomicAdd(&s.cnt[kLast], 1u);
        atomicAdd(&s.psum[kLast], fixkey(k, sP));
      }
    }
  }
  __syncthreads();
  // ---- A1: own two bins, wave scan, wave totals
  const int b0 = 2 * tid;
  auto conv = [&](int b, u64 v, unsigned cb) -> u64 {
    if (b == kLast || cb == 0u) return v;
    const int ex = (int)((top - (unsigned)b) >> 6);
    const int sh = (ex > 0 ? ex : 1) - 150 + sP;
    return sh >= 0 ? (v << (sh & 63)) : (sh > -64 ? (v >> ((-sh) & 63)) : 0ull);
  };
  // bins below the last hold count << 40 | mantissa sum (at most 2^24 L < 2^40); the last bin's
  // count is in cnt
  const ulonglong2 pp2 = *reinterpret_cast<const ulonglong2*>(&s.psum[b0]);
  constexpr u64 kM40 = (1ull << 40) - 1ull;
  const unsigned c0 = (unsigned)(pp2.x >> 40);
  const unsigned c1 = b0 + 1 == kLast ? s.cnt[kLast] : (unsigned)(pp2.y >> 40);
  const u64 p0 = conv(b0, pp2.x & kM40, c0), p1 = conv(b0 + 1, b0 + 1 == kLast ? pp2.y : (pp2.y & kM40), c1);
  const u64 tp = p0 + p1;
  const unsigned tc = c0 + c1;
  const u64 ip = wave_scan_u64(tp);
  const unsigned ic = wave_scan_u32(tc);
  if (lane == 63) {
    s.w_sp[wid] = ip;
    s.w_sc[wid] = ic;
  }
  __syncthreads();
  // ---- A2: prefix at the own bins, boundary scores, wave best
  u64 P0 = ip - tp;
  unsigned C0 = ic - tc;
#pragma unroll
  for (int w = 0; w < NW - 1; ++w) {
    const u64 pw = s.w_sp[w];
    const unsigned cw = s.w_sc[w];
    P0 += w < wid ? pw : 0ull;
    C0 += w < wid ? cw : 0u;
  }
  const u64 P1 = P0 + p0, P2 = P1 + p1;  // prefix through bin b0, b0 + 1
  const unsigned C1 = C0 + c0, C2 = C1 + c1;
  double bn = 0.0, bd = 1.0;
  {
    const double d1 = (double)P1, d2 = (double)P2;
    if (c0 != 0u) {
      bn = d1 * d1;
      bd = (double)C1;
    }
    if (c1 != 0u && d2 * d2 * bd > bn * (double)C2) {
      bn = d2 * d2;
      bd = (double)C2;
    }
  }
#define EXTERND_STEP(C, R)                                     \
  {                                                            \
    const double n2 = dppf64<C, R>(bn), d2 = dppf64<C, R>(bd); \
    if (n2 * bd > bn * d2) {                                   \
      bn = n2;                                                 \
      bd = d2;                                                 \
    }                                                          \
  }
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  if (lane == 63) {
    s.w_bn[wid] = bn;
    s.w_bd[wid] = bd;
  }
  __syncthreads();
  // ---- A3: global best, candidate bins, per-wave window
  bn = s.w_bn[0];
  bd = s.w_bd[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const double n2 = s.w_bn[w], d2 = s.w_bd[w];
    if (n2 * bd > bn * d2) {
      bn = n2;
      bd = d2;
    }
  }
  const double cutn = bn * (1.0 - 1e-9);
  const double tconv = ldexp(1.0, sP);
  auto cand_of = [&](int b, unsigned cb, u64 Pa, u64 Pb, unsigned Ca, unsigned Cb) -> bool {
    if (cb == 0u) return false;
    const double pbd = (double)Pb, pad = (double)Pa;
    bool cand = pbd * pbd * bd >= cutn * (double)Cb;
    if (!cand && cb >= 2u) {
      unsigned tk = b < kLast ? (((top - (unsigned)b) << 17) | 0x1FFFFu) : (((top - (unsigned)(kLast - 1)) << 17) - 1u);
      tk = tk < km ? tk : km;
      const double t1 = pad + (double)__uint_as_float(tk) * tconv * (double)cb;
      cand = t1 * t1 * bd >= cutn * (double)Cb || (Ca > 0u && pad * pad * bd >= cutn * (double)Ca);
    }
    return cand;
  };
  const bool k0 = cand_of(b0, c0, P0, P1, C0, C1);
  const bool k1 = cand_of(b0 + 1, c1, P1, P2, C1, C2);
  // this thread's lowest / highest candidate bin with the sums above it / the count through it
  const int tlo = k0 ? b0 : (k1 ? b0 + 1 : kSelBins);
  const int thi = k1 ? b0 + 1 : (k0 ? b0 : -1);
  const u64 tap = k0 ? P0 : P1;
  const unsigned tac = k0 ? C0 : C1, tch = k1 ? C2 : C1;
  const int wlo = kSelBins - (int)wave_max_u32((unsigned)(kSelBins - tlo));
  const int whi = (int)wave_max_u32((unsigned)(thi + 1)) - 1;
  if (lane == 0) {
    s.w_lo[wid] = wlo;
    s.w_hi[wid] = whi;
  }
  {
    const int llo = wlo < kSelBins ? (wlo >> 1) - wid * 64 : 0;
    const int lhi = whi >= 0 ? (whi >> 1) - wid * 64 : 0;
    const u64 ap_lo = readlane64(tap, llo);
    const unsigned ac_lo = readlane32(tac, llo), ac_hi = readlane32(tch, lhi);
    if (lane == 0) {
      s.w_plo[wid] = ap_lo;
      s.w_clo[wid] = ac_lo;
      s.w_chi[wid] = ac_hi;
    }
  }
  __syncthreads();
  // ---- A4: the window (every thread), then the gather
  int lo = kSelBins, hi = -1, wl = 0, wh = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int l = s.w_lo[w], h = s.w_hi[w];
    wl = l < lo ? w : wl;
    lo = l < lo ? l : lo;
    wh = h > hi ? w : wh;
    hi = h > hi ? h : hi;
  }
  const u64 AP = s.w_plo[wl];
  const unsigned AC = s.w_clo[wl];
  const unsigned nw = hi >= lo ? s.w_chi[wh] - AC : 0u;
  if (nw == 0u || nw > (unsigned)kWinMax) {
    *ok = false;
    __syncthreads();
    return out;
  }
  const unsigned khi = lo == 0 ? km : ((((top - (unsigned)lo) << 17) | 0x1FFFFu) < km ? (((top - (unsigned)lo) << 17) | 0x1FFFFu) : km);
  unsigned klo = hi < kLast ? ((top - (unsigned)hi) << 17) : ekey;
  klo = klo > ekey ? klo : ekey;
  for (int i0 = tid; i0 < L; i0 += kGrp * NT) {
    unsigned kk[kGrp];
#pragma unroll
    for (int u = 0; u < kGrp; ++u) {  // clamped index: every load is issued before any is used
      const int i = i0 + u * NT;
      kk[u] = keys[i < L ? i : L - 1] & (i < L ? 0x7FFFFFFFu : 0u);
    }
#pragma unroll
    for (int u = 0; u < kGrp; ++u) {
      const unsigned k = kk[u];
      if (k != 0u && k >= klo && k <= khi) {
        const unsigned slot = atomicAdd(&s.slot, 1u);
        s.w_key[slot] = k;
        s.w_p[slot] = fixkey(k, sP);
      }
    }
  }
  __syncthreads();
  // ---- scoring by wave 0: lane e holds window elements e, e + 64, ...; P(t) = AP + sum of the
  // window values with key >= t, read four at a time
  const int ns = (int)nw;
  if (wid == 0) {
    double myS = -1.0;
    unsigned myK = 0u, myC = 0u;
    u64 myP = 0ull;
    // pad the window to a multiple of 16 with key 0, which no element's threshold admits
    // (kWinMax is a multiple of 16)
    const int ns16 = (ns + 15) & ~15;
    for (int e = ns + lane; e < ns16; e += 64) {
      s.w_key[e] = 0u;
      s.w_p[e] = 0ull;
    }
    for (int e = lane; e < ((ns + 63) & ~63); e += 64) {
      const unsigned ke = s.w_key[e < ns ? e : 0] | (e < ns ? 0u : 0xFFFFFFFFu);
      u64 P = AP;
      unsigned C = AC;
      for (int j = 0; j < ns16; j += 16) {  // sixteen elements: twelve loads in flight
        uint4 kq[4];
        ulonglong2 pq[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) kq[q] = *reinterpret_cast<const uint4*>(&s.w_key[j + 4 * q]);
#pragma unroll
        for (int q = 0; q < 8; ++q) pq[q] = *reinterpret_cast<const ulonglong2*>(&s.w_p[j + 2 * q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool i0 = kq[q].x >= ke, i1 = kq[q].y >= ke, i2 = kq[q].z >= ke, i3 = kq[q].w >= ke;
          P += (i0 ? pq[2 * q].x : 0ull) + (i1 ? pq[2 * q].y : 0ull) + (i2 ? pq[2 * q + 1].x : 0ull) +
               (i3 ? pq[2 * q + 1].y : 0ull);
          C += (unsigned)i0 + (unsigned)i1 + (unsigned)i2 + (unsigned)i3;
        }
      }
      if (e < ns) {
        const double Pd = (double)P;
        const double S = Pd * Pd / (double)C;
        if (better(S, ke, myS, myK)) {
          myS = S;
          myK = ke;
          myP = P;
          myC = C;
        }
      }
    }
    int src = lane;
#define EXTERND_STEP(C, R)                                                 \
  {                                                                        \
    const double S2 = dppf64<C, R>(myS);                                   \
    const unsigned k2 = dpp32<C, R>(myK), s2 = dpp32<C, R>((unsigned)src); \
    if (better(S2, k2, myS, myK)) {                                        \
      myS = S2;                                                            \
      myK = k2;                                                            \
      src = (int)s2;                                                       \
    }                                                                      \
  }
    EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
    myK = readlane32(myK, 63);
    src = (int)readlane32((unsigned)src, 63);
    const u64 pp = readlane64(myP, src);
    const unsigned cc2 = readlane32(myC, src);
    if (lane == 0) {
      s.f_k[0] = myK;
      s.f_c[0] = cc2;
      s.f_p[0] = pp;
    }
  }
  __syncthreads();
  out.tkey = s.f_k[0];
  out.count = s.f_c[0];
  out.P = ldexp((double)s.f_p[0], -sP);
  out.H = (double)out.count;
  return out;
}

}  // namespace externd
