// C ABI of libexternd: argument validation, workspace, launch sequence, status codes.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>

#include "externd.h"
#include "externd_internal.hpp"

using namespace externd;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

#define HIP_OR_FAIL(expr)                                                                          \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return fail(EXTERND_EDEVICE, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

int64_t rank_of(int64_t m, int64_t n, float mu) {
  if (m < 1 || n < 1 || !std::isfinite(mu) || !(mu > 0.0f)) return -1;
  const double k = std::floor((double)mu * (double)(m < n ? m : n) + 1e-9);
  if (!(k >= 1.0) || k > 2147483647.0) return -1;
  return (int64_t)k;
}

// Stream-ordered workspace that is always released.
struct Workspace {
  hipStream_t st;
  void* p = nullptr;
  explicit Workspace(hipStream_t s) : st(s) {}
  ~Workspace() {
    if (p) (void)hipFreeAsync(p, st);
  }
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

unsigned spin_limit_from_env() {
  const char* s = std::getenv("EXTERND_SPIN_LIMIT");
  if (s && *s) {
    const long long v = std::atoll(s);
    if (v > 0) return (unsigned)v;
  }
  return 1u << 24;
}

int exp_bound_host(float x) {
  int e;
  std::frexp(x, &e);
  return e;
}

}  // namespace

extern "C" {

int64_t externd_rank(int64_t m, int64_t n, float mu) { return rank_of(m, n, mu); }

int64_t externd_packed_words(int64_t len) { return len < 0 ? -1 : (len + 15) / 16; }

const char* externd_status_string(int status) {
  switch (status) {
    case EXTERND_OK: return "EXTERND_OK";
    case EXTERND_EINVAL: return "EXTERND_EINVAL";
    case EXTERND_ENOMEM: return "EXTERND_ENOMEM";
    case EXTERND_EDEVICE: return "EXTERND_EDEVICE";
    case EXTERND_ENONFINITE: return "EXTERND_ENONFINITE";
    default: return "EXTERND_UNKNOWN";
  }
}

const char* externd_last_error(void) { return g_last_error.c_str(); }

int externd_decompose(const float* A, int64_t m, int64_t n, float mu, float tau, const float* h, int als_iters,
                      int block, uint32_t* B_packed, uint32_t* C_packed, float* D, double* energy, void* stream,
                      externd_stats* stats) {
  return externd_decompose_ex(A, m, n, mu, tau, h, als_iters, block, B_packed, C_packed, D, energy, nullptr, stream,
                              stats);
}

int externd_decompose_ex(const float* A, int64_t m, int64_t n, float mu, float tau, const float* h, int als_iters,
                         int block, uint32_t* B_packed, uint32_t* C_packed, float* D, double* energy,
                         const externd_options* options, void* stream, externd_stats* stats) {
  const auto t0 = std::chrono::steady_clock::now();
  g_last_error.clear();
  const double target = options ? options->energy_target : 0.0;
  const int safeguard = options ? options->safeguard : 0;
  const int sweeps = options ? options->sweeps : 0;
  const int ablation = options ? options->ablation : 0;
  const int residual_hbm = options ? options->residual_hbm : 0;
  if (ablation & ~3) return fail(EXTERND_EINVAL, "ablation must be a combination of 1 and 2");
  if (residual_hbm != 0 && residual_hbm != 1) return fail(EXTERND_EINVAL, "residual_hbm must be 0 or 1");
  if (sweeps < 0 || sweeps > 64) return fail(EXTERND_EINVAL, "sweeps must be in [0, 64]");
  if (!(target == 0.0 || (target > 0.0 && target <= 1.0)))
    return fail(EXTERND_EINVAL, "energy_target must be 0 (off) or in (0, 1]");
  if (safeguard != 0 && safeguard != 1) return fail(EXTERND_EINVAL, "safeguard must be 0 or 1");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!A || !B_packed || !C_packed || !D || !energy) return fail(EXTERND_EINVAL, "null pointer argument");
  if (m < 1 || n < 1) return fail(EXTERND_EINVAL, "m and n must be >= 1 (got %lld x %lld)", (long long)m, (long long)n);
  if (m > 16384 || n > 16384)
    return fail(EXTERND_EINVAL, "max(m, n) must be <= 16384 (got %lld x %lld)", (long long)m, (long long)n);
  if (!std::isfinite(tau) || tau < 0.0f || tau > 1.0f) return fail(EXTERND_EINVAL, "tau must be in [0, 1]");
  if (als_iters < 1) return fail(EXTERND_EINVAL, "als_iters must be >= 1");
  if (block < -1) return fail(EXTERND_EINVAL, "block must be >= -1");
  const int64_t k = rank_of(m, n, mu);
  if (k < 1) return fail(EXTERND_EINVAL, "mu must be finite and > 0 with k = floor(mu min(m,n)) >= 1");
  int64_t b = block == -1 ? std::max<int64_t>(1, std::min<int64_t>(256, std::min(m, n) / 8)) : (block <= 1 ? 1 : block);
  if (b > k) b = k;
  if (safeguard && b > 1) return fail(EXTERND_EINVAL, "the safeguard applies to the sequential path only (block resolved to %lld)", (long long)b);
  if ((ablation & 1) && b == 1)
    return fail(EXTERND_EINVAL, "ablation 1 (targets without decorrelation) applies to the block path only");
  const int mi = (int)m, ni = (int)n, ki = (int)k, bi = (int)b;
  const int ldr = (ni + 3) & ~3, ldt = (mi + 3) & ~3;

  // ---- workspace layout
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  const size_t o_flags = take(64);
  const size_t o_bar = take(sizeof(unsigned) * kBarWords);
  const size_t o_stats = take(8 * sizeof(u64));
  const size_t o_bytes = take(sizeof(double));
  const size_t o_R = take((size_t)mi * ldr * sizeof(float));
  const size_t o_rs = take((size_t)mi * sizeof(double));
  const size_t o_rowE = take((size_t)mi * sizeof(double));
  size_t o_RT = 0, o_xz = 0, o_xw = 0, o_xf = 0, o_rsg = 0, o_blk = 0;
  int grid = 0;
  bool rl = false, keys = true;
  if (b == 1) {
    o_RT = take((size_t)ni * ldt * sizeof(float));
    o_xz = take((size_t)mi * sizeof(double));
    o_xw = take((size_t)ni * sizeof(double));
    int dev = 0;
    HIP_OR_FAIL(hipGetDevice(&dev));
    int ncu = 0;
    HIP_OR_FAIL(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    if (!seq_plan(mi, ni, h != nullptr, ncu, residual_hbm == 0, &grid, &rl, &keys))
      return fail(EXTERND_EINVAL, "problem too large for the sequential kernel's on-chip state (%d x %d)", mi, ni);
    o_xf = take((size_t)4 * grid * sizeof(double));
    o_rsg = take((size_t)grid * mi * sizeof(double));
  } else {
    o_RT = take((size_t)ni * ldt * sizeof(float));
    o_blk = take(block_workspace_bytes(mi, ni, bi, h != nullptr));
  }
  Workspace ws(st);
  if (hipMallocAsync(&ws.p, off, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(EXTERND_ENOMEM, "workspace allocation of %zu bytes failed", off);
  }
  char* base = static_cast<char*>(ws.p);
  unsigned* flags = reinterpret_cast<unsigned*>(base + o_flags);
  unsigned* bar = reinterpret_cast<unsigned*>(base + o_bar);
  u64* dstats = reinterpret_cast<u64*>(base + o_stats);
  double* dbytes = reinterpret_cast<double*>(base + o_bytes);
  float* R = reinterpret_cast<float*>(base + o_R);
  double* rs = reinterpret_cast<double*>(base + o_rs);
  double* rowE = reinterpret_cast<double*>(base + o_rowE);
  HIP_OR_FAIL(hipMemsetAsync(base, 0, o_R, st));  // flags, barrier words, counters

  // ---- input checks (one host round trip)
  HIP_OR_FAIL(check_inputs(A, mi, ni, h, flags, st));
  unsigned hflags[2] = {0u, 0u};
  HIP_OR_FAIL(hipMemcpyAsync(hflags, flags, sizeof(hflags), hipMemcpyDeviceToHost, st));
  HIP_OR_FAIL(hipStreamSynchronize(st));
  if (hflags[0] & 1u) return fail(EXTERND_ENONFINITE, "A contains NaN or Inf");
  if (hflags[0] & 2u) return fail(EXTERND_ENONFINITE, "importance_weights contain NaN or Inf");
  if (hflags[0] & 4u) return fail(EXTERND_EINVAL, "importance_weights must be > 0");
  int EHm = 0;
  if (h) {
    float hmax;
    std::memcpy(&hmax, &hflags[1], sizeof(float));
    EHm = exp_bound_host(hmax);
  }

  // ---- staging
  HIP_OR_FAIL(stage_rows(A, mi, ni, h, R, ldr, rs, rowE, st));
  hipEvent_t e0, e1;
  HIP_OR_FAIL(hipEventCreate(&e0));
  HIP_OR_FAIL(hipEventCreate(&e1));
  struct EvGuard {
    hipEvent_t a, b;
    ~EvGuard() {
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
    }
  } evg{e0, e1};
  double flops = 0.0, blk_bytes = -1.0;
  if (b == 1) {
    float* RT = reinterpret_cast<float*>(base + o_RT);
    HIP_OR_FAIL(stage_transpose(A, mi, ni, RT, ldt, st));
    SeqLaunch L;
    L.R = R;
    L.RT = RT;
    L.h = h;
    L.rs0 = rs;
    L.rowE = rowE;
    L.xz = reinterpret_cast<double*>(base + o_xz);
    L.xw = reinterpret_cast<double*>(base + o_xw);
    L.xf = reinterpret_cast<double*>(base + o_xf);
    L.rsg = reinterpret_cast<double*>(base + o_rsg);
    L.rl = rl;
    L.keys = keys;
    L.bar = bar;
    L.Bp = B_packed;
    L.Cp = C_packed;
    L.D = D;
    L.energy = energy;
    L.stats = dstats;
    L.bytes = dbytes;
    L.m = mi;
    L.n = ni;
    L.ldr = ldr;
    L.ldt = ldt;
    L.k = ki;
    L.T = als_iters;
    L.EHm = EHm;
    L.grid = grid;
    L.tau = tau;
    L.spin_limit = spin_limit_from_env();
    L.target = target;
    L.safeguard = safeguard;
    L.sweeps = sweeps;
    L.ablation = ablation;
    HIP_OR_FAIL(hipEventRecord(e0, st));
    HIP_OR_FAIL(seq_launch(L, st));
    HIP_OR_FAIL(hipEventRecord(e1, st));
  } else {
    float* RT = reinterpret_cast<float*>(base + o_RT);
    HIP_OR_FAIL(stage_transpose(A, mi, ni, RT, ldt, st));
    BlockLaunch L;
    L.R = R;
    L.RT = RT;
    L.m = mi;
    L.n = ni;
    L.ldr = ldr;
    L.ldt = ldt;
    L.k = ki;
    L.b = bi;
    L.T = als_iters;
    L.EHm = EHm;
    L.tau = tau;
    L.h = h;
    L.rowE = rowE;
    L.Bp = B_packed;
    L.Cp = C_packed;
    L.D = D;
    L.energy = energy;
    L.stats = dstats;
    L.ws = base + o_blk;
    L.target = target;
    L.sweeps = sweeps;
    L.ablation = ablation;
    HIP_OR_FAIL(hipEventRecord(e0, st));
    HIP_OR_FAIL(block_run(L, st, &flops, &blk_bytes));
    HIP_OR_FAIL(hipEventRecord(e1, st));
  }
  // final explicit energy from the residual
  HIP_OR_FAIL(row_energy(R, mi, ni, ldr, h, rs, st));
  u64 hst[8];
  unsigned hbar = 0;
  double hbytes = 0.0;
  HIP_OR_FAIL(hipMemcpyAsync(hst, dstats, sizeof(hst), hipMemcpyDeviceToHost, st));
  HIP_OR_FAIL(hipMemcpyAsync(&hbar, bar, sizeof(unsigned), hipMemcpyDeviceToHost, st));
  HIP_OR_FAIL(hipMemcpyAsync(&hbytes, dbytes, sizeof(double), hipMemcpyDeviceToHost, st));
  double* hrow = nullptr;
  if (stats) {
    hrow = static_cast<double*>(std::malloc(2 * sizeof(double) * (size_t)mi));
    if (!hrow) return fail(EXTERND_ENOMEM, "host allocation failed");
    HIP_OR_FAIL(hipMemcpyAsync(hrow, rs, sizeof(double) * mi, hipMemcpyDeviceToHost, st));
    HIP_OR_FAIL(hipMemcpyAsync(hrow + mi, rowE, sizeof(double) * mi, hipMemcpyDeviceToHost, st));
  }
  const hipError_t se = hipStreamSynchronize(st);
  if (se != hipSuccess) {
    std::free(hrow);
    return fail(EXTERND_EDEVICE, "decomposition failed on the device: %s", hipGetErrorString(se));
  }
  if (hbar != 0u) {
    std::free(hrow);
    return fail(EXTERND_EDEVICE, "grid barrier wait exceeded its limit (device-side failure)");
  }
  if (stats) {
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    double er = 0.0, e0s = 0.0;
    for (int i = 0; i < mi; ++i) er += hrow[i];
    for (int i = 0; i < mi; ++i) e0s += hrow[mi + i];
    std::free(hrow);
    stats->k = k;
    stats->passes = (int64_t)hst[0];
    stats->early_exits = (int64_t)hst[1];
    stats->fallback_inits = (int64_t)hst[2];
    stats->zero_components = (int64_t)hst[3];
    stats->block = b;
    stats->energy_final_explicit = e0s > 0.0 ? 1.0 - er / e0s : 1.0;
    stats->kernel_ms = ms;
    stats->bytes_algorithmic = blk_bytes >= 0.0 ? blk_bytes : hbytes;
    stats->flops_algorithmic = flops;
    stats->components_used = hst[5] > 0 ? (int64_t)hst[5] : k;
    stats->safeguard_activations = (int64_t)hst[4];
    stats->sweep_reverts = (int64_t)hst[6];
    stats->residual_lds = rl ? 1 : 0;
    stats->seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  }
  return EXTERND_OK;
}

int externd_project(const float* X, int64_t count, int64_t L, float tau, const float* h, int8_t* V, double* PHC,
                    void* stream) {
  g_last_error.clear();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!X || !V || !PHC) return fail(EXTERND_EINVAL, "null pointer argument");
  if (count < 1 || count > 2147483647 || L < 1 || L > 16384) return fail(EXTERND_EINVAL, "need count >= 1 and 1 <= L <= 16384");
  if (!std::isfinite(tau) || tau < 0.0f || tau > 1.0f) return fail(EXTERND_EINVAL, "tau must be in [0, 1]");
  int EHm = 0;
  unsigned* flags = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&flags), 64, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(EXTERND_ENOMEM, "workspace allocation failed");
  }
  struct F {
    unsigned* p;
    hipStream_t s;
    ~F() { (void)hipFreeAsync(p, s); }
  } fg{flags, st};
  HIP_OR_FAIL(hipMemsetAsync(flags, 0, 64, st));
  HIP_OR_FAIL(check_inputs(X, (int)count, (int)L, h, flags, st));
  unsigned hflags[2];
  HIP_OR_FAIL(hipMemcpyAsync(hflags, flags, sizeof(hflags), hipMemcpyDeviceToHost, st));
  HIP_OR_FAIL(hipStreamSynchronize(st));
  if (hflags[0] & 1u) return fail(EXTERND_ENONFINITE, "X contains NaN or Inf");
  if (hflags[0] & 2u) return fail(EXTERND_ENONFINITE, "h contains NaN or Inf");
  if (hflags[0] & 4u) return fail(EXTERND_EINVAL, "h must be > 0");
  if (h) {
    float hmax;
    std::memcpy(&hmax, &hflags[1], sizeof(float));
    EHm = exp_bound_host(hmax);
  }
  HIP_OR_FAIL(project_rows(X, (int)count, (int)L, tau, h, EHm, V, PHC, st));
  HIP_OR_FAIL(hipStreamSynchronize(st));
  return EXTERND_OK;
}

// Workspace of externd_apply_factors: one buffer per (device, stream), grown on demand and held
// until the process ends, so that a call after the first is its kernels alone.  Calls on one
// stream use its buffer in stream order; the lock keeps two threads from enqueueing on one stream
// at once.
struct InferBuffer {
  std::mutex mu;
  void* p = nullptr;
  size_t bytes = 0;
};

static InferBuffer& infer_buffer(int dev, hipStream_t st) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, std::unique_ptr<InferBuffer>> buffers;
  std::lock_guard<std::mutex> g(mu);
  std::unique_ptr<InferBuffer>& b = buffers[std::make_pair(dev, st)];
  if (!b) b.reset(new InferBuffer);
  return *b;
}

int externd_apply_factors(const uint32_t* B_packed, const uint32_t* C_packed, const float* D, int64_t k, int64_t m,
                          int64_t n, const float* X, int64_t batch, float* Y, void* stream) {
  g_last_error.clear();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!B_packed || !C_packed || !D || !X || !Y) return fail(EXTERND_EINVAL, "null pointer argument");
  if (k < 1 || k > 2147483647 || m < 1 || n < 1 || m > 2147483647 - 15 || n > 2147483647 - 15)
    return fail(EXTERND_EINVAL, "need k, m, n >= 1 (and below 2^31)");
  if (batch < 1 || batch > 65535) return fail(EXTERND_EINVAL, "need 1 <= batch <= 65535");
  const size_t wsb = infer_workspace_bytes((int)k, (int)m, (int)batch);
  int dev = 0;
  HIP_OR_FAIL(hipGetDevice(&dev));
  InferBuffer& buf = infer_buffer(dev, st);
  std::lock_guard<std::mutex> lock(buf.mu);
  if (buf.bytes < wsb) {
    if (buf.p) {  // earlier calls on this stream may still use the buffer
      HIP_OR_FAIL(hipStreamSynchronize(st));
      (void)hipFree(buf.p);
      buf.p = nullptr;
      buf.bytes = 0;
    }
    if (hipMalloc(&buf.p, wsb) != hipSuccess) {
      (void)hipGetLastError();
      buf.p = nullptr;
      return fail(EXTERND_ENOMEM, "workspace allocation failed");
    }
    buf.bytes = wsb;
  }
  HIP_OR_FAIL(infer_run(B_packed, C_packed, D, (int)k, (int)m, (int)n, X, (int)batch, Y, buf.p, st));
  return EXTERND_OK;
}

int externd_apply_factors_static(const uint32_t* B_packed, const uint32_t* C_packed, const float* D, int64_t k,
                                 int64_t m, int64_t n, const float* X, int64_t batch, float* Y, void* stream) {
  g_last_error.clear();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!B_packed || !C_packed || !D || !X || !Y) return fail(EXTERND_EINVAL, "null pointer argument");
  if (k < 1 || k > 2147483647 || m < 1 || n < 1 || m > 2147483647 - 15 || n > 2147483647 - 15)
    return fail(EXTERND_EINVAL, "need k, m, n >= 1 (and below 2^31)");
  if (batch < 1 || batch > 65535) return fail(EXTERND_EINVAL, "need 1 <= batch <= 65535");
  const size_t need = infer_workspace_bytes((int)k, (int)m, (int)batch);
  if (need > kInferStaticBytes)
    return fail(EXTERND_EINVAL,
                "batch x (k + m) too large for the fixed workspace: needs %zu bytes, the limit is %zu "
                "(8 batch (k + m) + 4 batch ceil(k / 32) + 4 ceil(batch / 2) ceil(m / 256) bytes, each part "
                "rounded up to 256)", need,
                kInferStaticBytes);
  void* ws = nullptr;
  HIP_OR_FAIL(infer_static_scratch(&ws));
  HIP_OR_FAIL(infer_run(B_packed, C_packed, D, (int)k, (int)m, (int)n, X, (int)batch, Y, ws, st));
  return EXTERND_OK;
}

int externd_matvec(const float* R, int64_t m, int64_t n, const int8_t* t, const float* h, int transpose, double* out,
                   void* stream) {
  g_last_error.clear();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!R || !t || !out) return fail(EXTERND_EINVAL, "null pointer argument");
  if (m < 1 || n < 1 || m > 16384 || n > 16384) return fail(EXTERND_EINVAL, "need 1 <= m, n <= 16384");
  const int mi = (int)m, ni = (int)n;
  // stage the operand the way the decomposition kernel holds it: padded rows (R or R^T), the
  // ternary vector and the weights padded with zeros
  const int rows = transpose ? ni : mi, len = transpose ? mi : ni;
  const int ld = (len + 3) & ~3;
  const bool weighted = h && !transpose;
  void* p = nullptr;
  const size_t b_R = al256((size_t)rows * ld * 4), b_t = al256((size_t)ld), b_h = al256((size_t)ld * 4);
  const size_t b_s = al256((size_t)mi * 16);
  if (hipMallocAsync(&p, b_R + b_t + b_h + b_s, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(EXTERND_ENOMEM, "workspace allocation failed");
  }
  struct F {
    void* p;
    hipStream_t s;
    ~F() { (void)hipFreeAsync(p, s); }
  } fg{p, st};
  char* base = static_cast<char*>(p);
  float* Rs = reinterpret_cast<float*>(base);
  int8_t* tp = reinterpret_cast<int8_t*>(base + b_R);
  float* hp = reinterpret_cast<float*>(base + b_R + b_t);
  double* scratch = reinterpret_cast<double*>(base + b_R + b_t + b_h);
  if (transpose) HIP_OR_FAIL(stage_transpose(R, mi, ni, Rs, ld, st));
  else HIP_OR_FAIL(stage_rows(R, mi, ni, nullptr, Rs, ld, scratch, scratch + mi, st));
  HIP_OR_FAIL(hipMemsetAsync(tp, 0, (size_t)ld, st));
  HIP_OR_FAIL(hipMemcpyAsync(tp, t, (size_t)len, hipMemcpyDeviceToDevice, st));
  if (weighted) {
    HIP_OR_FAIL(hipMemsetAsync(hp, 0, (size_t)ld * 4, st));
    HIP_OR_FAIL(hipMemcpyAsync(hp, h, (size_t)len * 4, hipMemcpyDeviceToDevice, st));
  }
  HIP_OR_FAIL(matvec_rows(Rs, rows, ld / 4, ld, tp, weighted ? hp : nullptr, out, st));
  HIP_OR_FAIL(hipStreamSynchronize(st));
  return EXTERND_OK;
}

}  // extern "C"
