// Device helpers shared by the decomposition kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace externd {

typedef unsigned long long u64;

// ---- cross-workgroup communication ---------------------------------------------------
// Data exchanged between workgroups is written and read with agent-scope relaxed atomics
// (global_store/global_load with the device-coherence bit), so that no L2 writeback or
// invalidate is needed and each workgroup's residual rows stay cached in its XCD's L2.
__device__ __forceinline__ void st_dev(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_dev(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_dev(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_dev(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier words (unsigned): [0] error flag, [64] release epoch, [128 + 64*l] leaf counters,
// [2048] root counter.  Leaves are 16 groups of workgroups (blockIdx % 16).
constexpr int kBarWords = 4096;
constexpr int kBarLeaves = 16;

// Grid barrier for a cooperative launch.  Every thread must have finished its exchange stores
// (they are waited for here).  Returns nonzero if the wait exceeded spin_limit polls or the
// error flag is set; the caller then stops.  `epoch` increases by one per barrier.
__device__ __forceinline__ int grid_barrier(unsigned* bar, unsigned epoch, unsigned spin_limit,
                                            int* flag_lds) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int G = gridDim.x;
    const int nleaf = G < kBarLeaves ? G : kBarLeaves;
    const int leaf = blockIdx.x % nleaf;
    const unsigned members = G / nleaf + ((int)(G % nleaf) > leaf ? 1u : 0u);
    int bad = 0;
    const unsigned old = add_dev(bar + 128 + 64 * leaf, 1u);
    if (old == members * epoch - 1u) {
      const unsigned o2 = add_dev(bar + 2048, 1u);
      if (o2 == (unsigned)nleaf * epoch - 1u) st_dev(bar + 64, epoch);
    }
    unsigned polls = 0;
    while ((int)(ld_dev(bar + 64) - epoch) < 0) {
      if (ld_dev(bar) != 0u || ++polls > spin_limit) {
        st_dev(bar, 1u);
        bad = 1;
        break;
      }
    }
    *flag_lds = bad;
  }
  __syncthreads();
  return *flag_lds;
}

// ---- 128-bit unsigned fixed point ----------------------------------------------------
// Sums of fixed-point values are exact and independent of summation order, which makes every
// selection decision deterministic regardless of how the work was split.
struct u128 {
  u64 lo, hi;
};
__device__ __forceinline__ u128 mk128(u64 lo, u64 hi) {
  u128 r;
  r.lo = lo;
  r.hi = hi;
  return r;
}
__device__ __forceinline__ u128 add128(u128 a, u128 b) {
  u128 r;
  r.lo = a.lo + b.lo;
  r.hi = a.hi + b.hi + (r.lo < a.lo ? 1ull : 0ull);
  return r;
}
__device__ __forceinline__ double to_double(u128 a) {
  return (double)a.hi * 18446744073709551616.0 + (double)a.lo;
}
// floor(x * 2^scale) for finite x >= 0 whose result is below 2^101.
__device__ __forceinline__ u128 fixp(double x, int scale) {
  const u64 bits = (u64)__double_as_longlong(x);
  const int ef = (int)((bits >> 52) & 0x7FF);
  u64 mant = bits & 0xFFFFFFFFFFFFFull;
  int e;
  if (ef == 0) {
    e = -1074;
  } else {
    mant |= (1ull << 52);
    e = ef - 1075;
  }
  const int sh = e + scale;
  u128 r = mk128(0ull, 0ull);
  if (mant == 0ull) return r;
  if (sh >= 0) {
    if (sh < 64) {
      r.lo = mant << sh;
      r.hi = sh == 0 ? 0ull : (mant >> (64 - sh));
    } else {
      r.hi = mant << (sh - 64);
    }
  } else if (sh > -64) {
    r.lo = mant >> (-sh);
  }
  return r;
}

// Exponent E with |x| < 2^E (x finite, nonzero), via frexp.
__device__ __forceinline__ int exp_bound(float x) {
  int e;
  frexpf(x, &e);
  return e;
}

// ---- wave / block reductions --------------------------------------------------------
// Wave-wide scans and reductions move data with DPP (no LDS round trip).  Encodings (gfx9):
// row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.  The six steps
//   row_shr 1, 2, 4, 8 (inclusive scan inside each row of 16 lanes; lanes that would read
//   outside their row read zero), row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3
// leave the inclusive scan of the wave in every lane, so lane 63 holds the total.  Every op
// below must therefore treat a zero operand as neutral.  Reductions broadcast lane 63's value
// with readlane, so all lanes receive bitwise the same result.
template <int CTRL, int RM>
__device__ __forceinline__ unsigned dpp32(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, RM, 0xF, true);
}
template <int CTRL, int RM>
__device__ __forceinline__ u64 dpp64(u64 v) {
  const unsigned lo = dpp32<CTRL, RM>((unsigned)v);
  const unsigned hi = dpp32<CTRL, RM>((unsigned)(v >> 32));
  return ((u64)hi << 32) | lo;
}
template <int CTRL, int RM>
__device__ __forceinline__ double dppf64(double v) {
  return __longlong_as_double((long long)dpp64<CTRL, RM>((u64)__double_as_longlong(v)));
}
__device__ __forceinline__ unsigned readlane32(unsigned v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ u64 readlane64(u64 v, int l) {
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)v, l);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(v >> 32), l);
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  return __longlong_as_double((long long)readlane64((u64)__double_as_longlong(v), l));
}

#define EXTERND_WAVE_STEPS(STEP) \
  STEP(0x111, 0xF)               \
  STEP(0x112, 0xF)               \
  STEP(0x114, 0xF)               \
  STEP(0x118, 0xF)               \
  STEP(0x142, 0xA)               \
  STEP(0x143, 0xC)

__device__ __forceinline__ double wave_scan_f64(double v) {
#define EXTERND_STEP(C, R) v += dppf64<C, R>(v);
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  return v;
}
__device__ __forceinline__ unsigned wave_scan_u32(unsigned v) {
#define EXTERND_STEP(C, R) v += dpp32<C, R>(v);
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) { return readlane_f64(wave_scan_f64(v), 63); }
__device__ __forceinline__ unsigned wave_sum_u32(unsigned v) { return readlane32(wave_scan_u32(v), 63); }
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#define EXTERND_STEP(C, R)              \
  {                                     \
    const unsigned t = dpp32<C, R>(v);  \
    v = t > v ? t : v;                  \
  }
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  return readlane32(v, 63);
}

// Wave sum of 128-bit values (exact, any order), same result in every lane.
__device__ __forceinline__ u128 wave_sum128(u128 v) {
#define EXTERND_STEP(C, R) v = add128(v, mk128(dpp64<C, R>(v.lo), dpp64<C, R>(v.hi)));
  EXTERND_WAVE_STEPS(EXTERND_STEP)
#undef EXTERND_STEP
  return mk128(readlane64(v.lo, 63), readlane64(v.hi, 63));
}

// Ternary packing: element t in bits 2(t%16)..2(t%16)+1 of word t/16; 00 = 0, 01 = +1, 11 = -1.
__device__ __forceinline__ unsigned tcode(int s) { return s == 0 ? 0u : (s > 0 ? 1u : 3u); }

}  // namespace externd
