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
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned t = __shfl_xor(v, o);
    v = t > v ? t : v;
  }
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Ternary packing: element t in bits 2(t%16)..2(t%16)+1 of word t/16; 00 = 0, 01 = +1, 11 = -1.
__device__ __forceinline__ unsigned tcode(int s) { return s == 0 ? 0u : (s > 0 ? 1u : 3u); }

}  // namespace externd
