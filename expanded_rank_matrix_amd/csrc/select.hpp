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
//   1. histogram the eligible values by their fp32 bit pattern into 1024 bins (64 per octave
//      below the maximum, the last bin catches the rest), with counts and fp64 sums of h|x|
//      and h (LDS atomics; used for pruning only);
//   2. every bin boundary is a threshold whose score follows from the prefix sums; a bin's
//      interior can only win if (P_above + top_of_bin * H_bin)^2 / (H_above + H_bin) reaches the
//      best boundary score (each added element adds at most top_of_bin per unit weight, and the
//      score is quasi-convex in the added weight).  The bins that can hold the optimum form a
//      narrow window (typically three bins);
//   3. the window's elements are scored exactly: P(t) = P_above + sum over window elements
//      >= t, every sum an exact 128-bit fixed-point integer (order independent), so the decision
//      is canonical: it depends neither on the launch shape nor on atomic ordering.
#pragma once
#include "common.hpp"

namespace externd {

constexpr int kSelBins = 1024;     // 64 per octave
constexpr int kSelShift = 23 - 6;  // fp32 mantissa bits dropped per bin
constexpr int kWinMax = 256;       // window elements scored in one pass

struct SelScratch {
  unsigned cnt[kSelBins];
  double psum[kSelBins];
  double hsum[kSelBins];
  unsigned w_key[kWinMax];
  u64 w_plo[kWinMax], w_phi[kWinMax], w_hlo[kWinMax], w_hhi[kWinMax];
  u64 a_plo[16], a_phi[16], a_hlo[16], a_hhi[16];
  unsigned a_cnt[16];
  unsigned red_u[16];
  double red_d[16];
  unsigned red_k[16];
  unsigned wk_hi, wk_lo;  // window keys in (wk_lo, wk_hi]
  unsigned slot;
  unsigned walk;
  int mode;  // 1: window scored in one pass, 2: window scored by exact block reductions
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

__device__ __forceinline__ u128 shfl_xor128(u128 v, int o) {
  return mk128(__shfl_xor(v.lo, o), __shfl_xor(v.hi, o));
}

// Whether a slot holding x is in the support of r.
__device__ __forceinline__ bool selected(float x, const SelResult& r) {
  const unsigned k = __float_as_uint(x) & 0x7FFFFFFFu;
  return r.count > 0u && k != 0u && k >= r.ekey && k >= r.tkey;
}

// All NT threads of the workgroup call this.  vals[0..L) (LDS or global, fp32 or fp64) holds the
// vector; its fp32 rounding is what is projected.  hl[0..L) holds the weights (read only when W).
// EHm: exponent with max(h) < 2^EHm (W only).  Every thread receives the same result.
template <int NT, bool W, typename T>
__device__ SelResult ternary_select(const T* vals, const float* hl, int L, float tau, int EHm,
                                    SelScratch& s) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int NW = NT / 64;
  SelResult out;
  out.tkey = 0xFFFFFFFFu;
  out.ekey = 0xFFFFFFFFu;
  out.P = 0.0;
  out.H = 0.0;
  out.count = 0u;
  // ---- max |x|; clear the histogram meanwhile
  unsigned km = 0;
  for (int i = tid; i < L; i += NT) {
    const unsigned k = __float_as_uint((float)vals[i]) & 0x7FFFFFFFu;
    km = k > km ? k : km;
  }
  km = wave_max_u32(km);
  if (lane == 0) s.red_u[wid] = km;
  for (int b = tid; b < kSelBins; b += NT) {
    s.cnt[b] = 0u;
    s.psum[b] = 0.0;
    if (W) s.hsum[b] = 0.0;
  }
  if (tid == 0) s.slot = 0u;
  __syncthreads();
  km = 0;
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
  // ---- approximate histogram.  Bin b is stored at (b % 16) * 64 + b / 16 so that the scan
  // below (lane l owns bins 16 l .. 16 l + 15) reads consecutive addresses across lanes.
  for (int i = tid; i < L; i += NT) {
    const unsigned k = keyof(i);
    if (k != 0u) {
      unsigned b = (km - k) >> kSelShift;
      b = b > (unsigned)(kSelBins - 1) ? (unsigned)(kSelBins - 1) : b;
      const unsigned hb = (b & 15u) * 64u + (b >> 4);
      const double av = (double)__uint_as_float(k);
      atomicAdd(&s.cnt[hb], 1u);
      atomicAdd(&s.psum[hb], W ? (double)hl[i] * av : av);
      if (W) atomicAdd(&s.hsum[hb], (double)hl[i]);
    }
  }
  __syncthreads();
  // ---- wave 0: prefix sums, boundary scores, interior bounds -> window of bins.  Scores are
  // compared as fractions (num * den' vs num' * den) to avoid fp64 divisions.
  if (wid == 0) {
    constexpr int BPL = kSelBins / 64;  // contiguous bins per lane
    auto binp = [&](int q) -> double { return s.psum[q * 64 + lane]; };
    auto binh = [&](int q) -> double { return W ? s.hsum[q * 64 + lane] : (double)s.cnt[q * 64 + lane]; };
    double tp = 0.0, th = 0.0;
    _Pragma("unroll 2") for (int q = 0; q < BPL; ++q) {
      tp += binp(q);
      th += binh(q);
    }
    double ip = tp, ih = th;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double a0 = __shfl_up(ip, o), a1 = __shfl_up(ih, o);
      if (lane >= o) {
        ip += a0;
        ih += a1;
      }
    }
    // best boundary score as a fraction bn / bd
    double bn = 0.0, bd = 1.0;
    {
      double rp = ip - tp, rh = ih - th;
      _Pragma("unroll 2") for (int q = 0; q < BPL; ++q) {
        rp += binp(q);
        rh += binh(q);
        if (s.cnt[q * 64 + lane] != 0u && rp * rp * bd > bn * rh) {
          bn = rp * rp;
          bd = rh;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double n2 = __shfl_xor(bn, o), d2 = __shfl_xor(bd, o);
      if (n2 * bd > bn * d2) {
        bn = n2;
        bd = d2;
      }
    }
    const double cutn = bn * (1.0 - 1e-9);  // candidate if score * bd >= cutn
    int lo = kSelBins, hi = -1;
    {
      double rp = ip - tp, rh = ih - th;
      _Pragma("unroll 2") for (int q = 0; q < BPL; ++q) {
        const int b = lane * BPL + q;
        const unsigned c = s.cnt[q * 64 + lane];
        const double hbq = binh(q);
        const double Pi = rp + binp(q), Hi = rh + hbq;
        bool cand = c != 0u && Pi * Pi * bd >= cutn * Hi;
        if (!cand && c >= 2u) {
          const unsigned top = km - ((unsigned)b << kSelShift);  // largest key the bin can hold
          const double t1 = rp + (double)__uint_as_float(top) * hbq;
          cand = t1 * t1 * bd >= cutn * Hi || (rh > 0.0 && rp * rp * bd >= cutn * rh);
        }
        if (cand) {
          lo = b < lo ? b : lo;
          hi = b > hi ? b : hi;
        }
        rp = Pi;
        rh = Hi;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    unsigned nw = 0u;
    _Pragma("unroll 2") for (int q = 0; q < BPL; ++q) {
      const int b = lane * BPL + q;
      if (b >= lo && b <= hi) nw += s.cnt[q * 64 + lane];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nw += __shfl_xor(nw, o);
    if (lane == 0) {
      s.wk_hi = km - ((unsigned)lo << kSelShift);
      const long long klo = (long long)km - ((long long)(hi + 1) << kSelShift);
      s.wk_lo = (hi == kSelBins - 1 || klo < 0) ? 0u : (unsigned)klo;
      s.mode = nw <= (unsigned)kWinMax ? 1 : 2;
    }
  }
  __syncthreads();
  const unsigned wk_hi = s.wk_hi, wk_lo = s.wk_lo;
  const int mode = s.mode;
  const int EM = exp_bound(M);
  const int scP = W ? (100 - EM - EHm) : (100 - EM);
  const int scH = W ? (100 - EHm) : 0;
  auto pterm = [&](int i, unsigned k) -> u128 {
    const double av = (double)__uint_as_float(k);
    return W ? fixp((double)hl[i] * av, scP) : fixp(av, scP);
  };
  auto hterm = [&](int i) -> u128 { return W ? fixp((double)hl[i], scH) : mk128(1ull, 0ull); };
  // Exact block sum over eligible slots with key >= kmin (and key <= kmax); all threads call.
  auto exact_sum = [&](unsigned kmin, unsigned kmax, u128& P, u128& H, unsigned& C) {
    u128 p = mk128(0, 0), h = mk128(0, 0);
    unsigned c = 0u;
    for (int i = tid; i < L; i += NT) {
      const unsigned k = keyof(i);
      if (k != 0u && k >= kmin && k <= kmax) {
        p = add128(p, pterm(i, k));
        if (W) h = add128(h, hterm(i));
        ++c;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      p = add128(p, shfl_xor128(p, o));
      if (W) h = add128(h, shfl_xor128(h, o));
      c += __shfl_xor(c, o);
    }
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
  // ---- gather the window (one-pass mode)
  if (mode == 1) {
    for (int i = tid; i < L; i += NT) {
      const unsigned k = keyof(i);
      if (k != 0u && k > wk_lo && k <= wk_hi) {
        const unsigned slot = atomicAdd(&s.slot, 1u);
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
  // exact sums of the elements above the window
  u128 AP, AH;
  unsigned AC;
  exact_sum(wk_hi + 1u, 0xFFFFFFFFu, AP, AH, AC);
  double myS = -1.0;
  unsigned myK = 0u;
  if (mode == 1) {
    const unsigned nwin = s.slot;
    for (unsigned t = tid; t < nwin; t += NT) {
      const unsigned kt = s.w_key[t];
      u128 P = AP, H = AH;
      unsigned C = AC;
      _Pragma("unroll 2") for (unsigned j = 0; j < nwin; ++j) {
        if (s.w_key[j] >= kt) {
          P = add128(P, mk128(s.w_plo[j], s.w_phi[j]));
          if (W) H = add128(H, mk128(s.w_hlo[j], s.w_hhi[j]));
          ++C;
        }
      }
      const double Pd = to_double(P);
      const double Hd = W ? to_double(H) : (double)C;
      const double St = Pd * Pd / Hd;
      if (better(St, kt, myS, myK)) {
        myS = St;
        myK = kt;
      }
    }
  } else {
    // Large window (heavy ties or an unusually flat score): walk its distinct keys downwards
    // and score each with an exact block reduction.  Slow, and only reached by unusual inputs.
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
      u128 P, H;
      unsigned C;
      exact_sum(best, wk_hi, P, H, C);
      P = add128(P, AP);
      if (W) H = add128(H, AH);
      C += AC;
      const double Pd = to_double(P);
      const double Hd = W ? to_double(H) : (double)C;
      const double St = Pd * Pd / Hd;
      if (better(St, best, myS, myK)) {
        myS = St;
        myK = best;
      }
      prev = best;
    }
  }
  // ---- block argmax over (score desc, key desc)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double S2 = __shfl_xor(myS, o);
    const unsigned k2 = __shfl_xor(myK, o);
    if (better(S2, k2, myS, myK)) {
      myS = S2;
      myK = k2;
    }
  }
  __syncthreads();
  if (lane == 0) {
    s.red_d[wid] = myS;
    s.red_k[wid] = myK;
  }
  __syncthreads();
  double S = -1.0;
  unsigned K = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (better(s.red_d[w], s.red_k[w], S, K)) {
      S = s.red_d[w];
      K = s.red_k[w];
    }
  // ---- exact support sums at the chosen threshold
  u128 P, H;
  unsigned C;
  exact_sum(K, 0xFFFFFFFFu, P, H, C);
  out.tkey = K;
  out.count = C;
  out.P = ldexp(to_double(P), -scP);
  out.H = W ? ldexp(to_double(H), -scH) : (double)C;
  __syncthreads();
  return out;
}

}  // namespace externd
