// C ABI of the fused diagonal-GMM EM library (declared in include/flashgmm.h):
// argument validation, the context and its workspace, and the order of
// kernel launches for each entry point.  All device work goes through the
// launchers in gmm_kernels.hip; nothing here computes on the host.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "flashgmm.h"
#include "gmm_internal.h"

// default limit of the soft assignment's own buffers (the selections of all
// rows and the radix-sort buffer that builds the lists from them)
constexpr int64_t kAssignLimitDefault = (int64_t)20 << 30;

struct gmm_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  gmm::Plan plan{};
  gmm::Workspace ws{};
  void* base = nullptr;
  size_t bytes = 0;
  int path = GMM_PATH_AUTO;
  std::string err;
  double logits_since = 0.0;  // N*K summed over E-steps since gmm_refine_stats
  // kernel timing (gmm_profile)
  bool prof = false;
  std::vector<hipEvent_t> ev_free;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_pending[2];
  hipEvent_t ev_open[2] = {nullptr, nullptr};
  // out-of-core E-step: a copy stream, two device staging buffers of
  // stage_rows x D floats (grown on demand) and their events
  hipStream_t copy_stream = nullptr;
  float* stage[2] = {nullptr, nullptr};
  int64_t stage_rows = 0;
  hipEvent_t ev_copied[2] = {nullptr, nullptr};
  hipEvent_t ev_used[2] = {nullptr, nullptr};
  // soft assignment over several chunks: every row's selections, kept from
  // the counting sweep for the scatter (grown on demand, at most
  // kSelKeepBytes)
  int32_t* selkeep = nullptr;
  size_t selkeep_bytes = 0;
  void* sortbuf = nullptr;  // list sort (grown on demand)
  size_t sortbuf_bytes = 0;
  int64_t assign_limit = kAssignLimitDefault;  // bytes of selkeep + sortbuf (gmm_set_assign_limit)
};

namespace {

thread_local std::string g_create_err;

gmm_status fail(gmm_ctx* c, gmm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c)
    c->err = buf;
  else
    g_create_err = buf;
  return st;
}

gmm_status hip_fail(gmm_ctx* c, hipError_t e, const char* what) {
  return fail(c, GMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

gmm_status check_x(gmm_ctx* c, const float* X, int64_t N, int64_t ldx) {
  if (!X) return fail(c, GMM_ERR_INVALID_ARG, "X is NULL");
  if (!aligned16(X)) return fail(c, GMM_ERR_INVALID_ARG, "X must be 16-byte aligned");
  if (N < 1) return fail(c, GMM_ERR_INVALID_ARG, "N must be >= 1 (got %lld)", (long long)N);
  if (ldx < c->plan.D || (ldx & 3))
    return fail(c, GMM_ERR_INVALID_ARG, "ldx must be >= D and a multiple of 4 (got %lld, D=%d)",
                (long long)ldx, c->plan.D);
  if (N > ((int64_t)1 << 40)) return fail(c, GMM_ERR_INVALID_ARG, "N too large");
  return GMM_OK;
}

gmm_status check_params(gmm_ctx* c, const void* w, const void* mu, const void* var) {
  if (!w || !mu || !var) return fail(c, GMM_ERR_INVALID_ARG, "weights/means/vars must be non-NULL");
  if (!aligned16(w) || !aligned16(mu) || !aligned16(var))
    return fail(c, GMM_ERR_INVALID_ARG, "weights/means/vars must be 16-byte aligned");
  return GMM_OK;
}

template <class T>
T* carve(char*& p, size_t count) {
  T* r = reinterpret_cast<T*>(p);
  size_t b = (count * sizeof(T) + 255) / 256 * 256;
  p += b;
  return r;
}

hipEvent_t take_event(gmm_ctx* c) {
  if (!c->ev_free.empty()) {
    hipEvent_t e = c->ev_free.back();
    c->ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void hook_before(void* user, int which, hipStream_t s) {
  gmm_ctx* c = (gmm_ctx*)user;
  hipEvent_t e = take_event(c);
  if (e && hipEventRecord(e, s) == hipSuccess) c->ev_open[which] = e;
}

void hook_after(void* user, int which, hipStream_t s) {
  gmm_ctx* c = (gmm_ctx*)user;
  hipEvent_t b = c->ev_open[which];
  c->ev_open[which] = nullptr;
  if (!b) return;
  hipEvent_t e = take_event(c);
  if (e && hipEventRecord(e, s) == hipSuccess)
    c->ev_pending[which].push_back({b, e});
  else
    c->ev_free.push_back(b);
}

bool want_fused(const gmm_ctx* c) {
  if (c->path == GMM_PATH_TWO_SWEEP) return false;
  // float64 logits: one sweep wherever the fused kernel fits (measured 566 against 710 ms per 1e6 rows at
  // D=768, K=4096, whose 128 component groups exceed the refined kernels' AUTO limit)
  if (c->ws.f64) return c->plan.fused64OK != 0;
  if (c->path == GMM_PATH_FUSED) return c->plan.fusedOK != 0;
  return c->plan.fusedOK != 0 && c->plan.P <= 64;
}

// var_iso (isotropic model): var is its broadcast, and the fused isotropic
// kernel runs where it applies (else the diagonal kernels on the broadcast)
gmm_status estep_into(gmm_ctx* c, const float* X, int64_t N, int64_t ldx, const float* w, const float* mu,
                      const float* var, double* Nk, double* S1, double* S2, double* ll, int accumulate,
                      const float* var_iso = nullptr, bool hard = false) {
  hipStream_t s = c->stream;
  hipError_t e = gmm::launch_precompute(c->plan, c->ws, w, mu, var, s);
  if (e != hipSuccess) return hip_fail(c, e, "precompute launch");
  const bool fused = want_fused(c);
  const char* envi = getenv("FLASHGMM_ISO_KERNEL");  // 0: diagonal kernels on the broadcast (measurements)
  const bool iso = var_iso && fused && gmm::iso_kernel_ok(c->plan, c->ws, hard) && !(envi && atoi(envi) == 0);
  if (hard && !iso) return fail(c, GMM_ERR_UNSUPPORTED, "no fused k-means kernel for this shape");
  if (iso) {
    e = gmm::launch_precompute_iso(c->plan, c->ws, mu, var_iso, s);
    if (e != hipSuccess) return hip_fail(c, e, "precompute launch");
  }
  gmm::LaunchHooks hk;
  hk.before = hook_before;
  hk.after = hook_after;
  hk.user = c;
  int nslots = 0;
  e = gmm::launch_estep(c->plan, c->ws, X, N, ldx, fused, s, c->prof ? &hk : nullptr, &nslots,
                        iso ? (hard ? 2 : 1) : 0);
  if (e != hipSuccess) return hip_fail(c, e, fused ? "fused E-step launch" : "two-sweep E-step launch");
  e = gmm::launch_reduce(c->plan, c->ws, Nk, S1, S2, ll, accumulate, nslots, fused ? nslots : c->plan.Glogz, N,
                         s);
  c->logits_since += (double)N * (double)c->plan.K * (fused ? 1.0 : 2.0);
  if (e != hipSuccess) return hip_fail(c, e, "reduce launch");
  return GMM_OK;
}

gmm_status soft_assign_run(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* weights,
                           const float* means, const float* vars, float threshold, int32_t max_extra,
                           int64_t* list_offsets, int32_t* list_ids, int64_t ids_capacity, int64_t* nnz);

}  // namespace

extern "C" {

size_t gmm_workspace_bytes(int32_t K, int32_t D) {
  if (K < 1 || K > 65536 || D < 1 || D > 1024) return 0;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  gmm::Plan p0 = gmm::make_plan(K, D, prop.multiProcessorCount, 1, 1);
  int o1 = 1, o2 = 1;
  if (gmm::occupancy(p0, &o1, &o2) != hipSuccess) return 0;
  gmm::Plan p = gmm::make_plan(K, D, prop.multiProcessorCount, o1, o2);
  return gmm::workspace_bytes(p);
}

gmm_status gmm_create(gmm_ctx** out, int32_t K, int32_t D, void* hip_stream) {
  g_create_err.clear();
  if (!out) return fail(nullptr, GMM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (K < 1 || K > 65536) return fail(nullptr, GMM_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  if (D < 1 || D > 1024) return fail(nullptr, GMM_ERR_INVALID_ARG, "D must be in [1, 1024] (got %d)", D);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, GMM_ERR_UNSUPPORTED, "built for gfx950, device is %s", prop.gcnArchName);
  gmm::Plan p0 = gmm::make_plan(K, D, prop.multiProcessorCount, 1, 1);
  if (!gmm::plan_shape_ok(p0)) return fail(nullptr, GMM_ERR_UNSUPPORTED, "no kernel for K=%d D=%d", K, D);
  int o1 = 1, o2 = 1;
  e = gmm::occupancy(p0, &o1, &o2);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  if (o1 < 1 || o2 < 1) return fail(nullptr, GMM_ERR_UNSUPPORTED, "E-step kernel does not fit a CU");

  gmm_ctx* c = new (std::nothrow) gmm_ctx();
  if (!c) return fail(nullptr, GMM_ERR_OOM, "host allocation failed");
  c->device = dev;
  c->stream = (hipStream_t)hip_stream;
  c->plan = gmm::make_plan(K, D, prop.multiProcessorCount, o1, o2);
  int oa = 0;
  e = gmm::assign_occupancy(c->plan, &oa);
  if (e != hipSuccess) {
    delete c;
    return fail(nullptr, GMM_ERR_HIP, "assignment kernel occupancy: %s", hipGetErrorString(e));
  }
  c->plan.occAssign = oa;
  e = gmm::fused64_fits(c->plan, &c->plan.fused64OK);
  if (e != hipSuccess) {
    delete c;
    return fail(nullptr, GMM_ERR_HIP, "float64 fused kernel occupancy: %s", hipGetErrorString(e));
  }
  c->bytes = gmm::workspace_bytes(c->plan);
  e = hipMalloc(&c->base, c->bytes);
  if (e != hipSuccess) {
    const size_t bytes = c->bytes;
    delete c;
    return fail(nullptr, GMM_ERR_OOM, "workspace hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
  }
  const gmm::Plan& p = c->plan;
  char* q = (char*)c->base;
  c->ws.wop = carve<float>(q, (size_t)p.Kpad * 2 * p.Dp);
  c->ws.cvec = carve<float>(q, p.Kpad);
  c->ws.cfull = carve<double>(q, p.Kpad);
  c->ws.cpeak = carve<double>(q, p.Kpad);
  c->ws.cshift = carve<double>(q, 1);
  c->ws.w64 = carve<double2>(q, (size_t)p.Kpad * p.Dp);
  c->ws.vexp = carve<float>(q, (size_t)p.K * p.D);
  c->ws.qiso = carve<double>(q, p.K);
  c->ws.wuni = carve<float>(q, p.K);
  c->ws.vhalf = carve<float>(q, p.K);
  c->ws.wiso = carve<float>(q, (size_t)p.Kpad * p.Dp);
  c->ws.ivec = carve<float>(q, p.Kpad);
  c->ws.wsplit = carve<__bf16>(q, (size_t)p.Kpad * 2 * p.Dp * 2);
  c->ws.wsplit_iso = carve<__bf16>(q, (size_t)p.Kpad * p.Dp * 2);
  c->ws.split = 2;
  c->ws.wop64 = carve<double>(q, (size_t)p.Kpad * 2 * p.Dp);
  c->ws.cvec64 = carve<double>(q, p.Kpad);
  c->ws.f64 = 0;
  c->ws.abmax = carve<float2>(q, p.Kpad);
  c->ws.refine = 1;
  c->ws.nrefined = carve<unsigned long long>(q, 1);
  c->ws.slots = carve<double>(q, (size_t)p.R * p.Kpad * p.SR);
  c->ws.llslots = carve<double>(q, p.R > p.Glogz ? p.R : p.Glogz);
  c->ws.logz = carve<float>(q, (size_t)p.chunk);
  c->ws.xbuf = carve<unsigned long long>(q, (size_t)p.R * 4 * p.P * p.BN);
  c->ws.stats = carve<double>(q, (size_t)p.K + 2 * (size_t)p.K * p.D + 1);
  c->ws.colpart = carve<double>(q, (size_t)1024 * p.D);
  c->ws.colmean = carve<double>(q, p.D);
  c->ws.rows = carve<int64_t>(q, p.K);
  c->ws.flags = carve<int>(q, 4);
  c->ws.colG = 1024;
  c->ws.asel = carve<int32_t>(q, (size_t)p.assignChunk * 9);
  c->ws.agco = carve<float4>(q, (size_t)p.Kpad / 32);
  c->ws.acounts = carve<unsigned long long>(q, p.Kpad);
  c->ws.acnt = carve<unsigned>(q, (size_t)p.assignBlocks * p.Kpad);
  c->ws.atot = carve<unsigned>(q, p.Kpad);
  c->ws.acursor = carve<int64_t>(q, p.Kpad);
  c->ws.annz = carve<int64_t>(q, 1);
  e = hipMemsetAsync(c->ws.flags, 0, 16, c->stream);
  if (e == hipSuccess) e = hipMemsetAsync(c->ws.nrefined, 0, 8, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    hipFree(c->base);
    delete c;
    return fail(nullptr, GMM_ERR_HIP, "workspace clear: %s", hipGetErrorString(e));
  }
  *out = c;
  return GMM_OK;
}

static void drop_events(gmm_ctx* ctx) {
  for (int w = 0; w < 2; ++w) {
    for (auto& pr : ctx->ev_pending[w]) {
      ctx->ev_free.push_back(pr.first);
      ctx->ev_free.push_back(pr.second);
    }
    ctx->ev_pending[w].clear();
  }
}

void gmm_destroy(gmm_ctx* ctx) {
  if (!ctx) return;
  hipStreamSynchronize(ctx->stream);
  drop_events(ctx);
  for (hipEvent_t e : ctx->ev_free) hipEventDestroy(e);
  if (ctx->base) hipFree(ctx->base);
  for (int b = 0; b < 2; ++b) {
    if (ctx->stage[b]) hipFree(ctx->stage[b]);
    if (ctx->ev_copied[b]) hipEventDestroy(ctx->ev_copied[b]);
    if (ctx->ev_used[b]) hipEventDestroy(ctx->ev_used[b]);
  }
  if (ctx->copy_stream) hipStreamDestroy(ctx->copy_stream);
  if (ctx->selkeep) hipFree(ctx->selkeep);
  if (ctx->sortbuf) hipFree(ctx->sortbuf);
  delete ctx;
}

gmm_status gmm_profile(gmm_ctx* ctx, int32_t enable) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (enable != 0 && enable != 1) return fail(ctx, GMM_ERR_INVALID_ARG, "enable must be 0 or 1");
  if (!enable) {
    hipError_t e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "stream synchronize");
    drop_events(ctx);
  }
  ctx->prof = enable != 0;
  return GMM_OK;
}

gmm_status gmm_profile_read(gmm_ctx* ctx, double* stats_ms, int64_t* stats_launches, double* logz_ms,
                            int64_t* logz_launches) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "stream synchronize");
  double ms[2] = {0.0, 0.0};
  int64_t n[2] = {0, 0};
  for (int w = 0; w < 2; ++w) {
    for (auto& pr : ctx->ev_pending[w]) {
      float t = 0.f;
      e = hipEventElapsedTime(&t, pr.first, pr.second);
      if (e != hipSuccess) return hip_fail(ctx, e, "hipEventElapsedTime");
      ms[w] += t;
      n[w] += 1;
    }
  }
  drop_events(ctx);
  if (stats_ms) *stats_ms = ms[0];
  if (stats_launches) *stats_launches = n[0];
  if (logz_ms) *logz_ms = ms[1];
  if (logz_launches) *logz_launches = n[1];
  return GMM_OK;
}

const char* gmm_last_error(const gmm_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_err.c_str(); }

gmm_status gmm_set_path(gmm_ctx* ctx, int32_t path) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (path < GMM_PATH_AUTO || path > GMM_PATH_FUSED) return fail(ctx, GMM_ERR_INVALID_ARG, "unknown path %d", path);
  if (path == GMM_PATH_FUSED && !ctx->plan.fusedOK)
    return fail(ctx, GMM_ERR_UNSUPPORTED, "fused path needs %d co-resident workgroups per row tile", ctx->plan.P);
  ctx->path = path;
  return GMM_OK;
}

gmm_status gmm_set_precision(gmm_ctx* ctx, int32_t mode) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (mode != GMM_PREC_REFINED && mode != GMM_PREC_FP32 && mode != GMM_PREC_FP64)
    return fail(ctx, GMM_ERR_INVALID_ARG, "unknown precision mode %d", mode);
  ctx->ws.refine = (mode == GMM_PREC_REFINED) ? 1 : 0;
  ctx->ws.f64 = (mode == GMM_PREC_FP64) ? 1 : 0;
  return GMM_OK;
}

gmm_status gmm_set_mfma(gmm_ctx* ctx, int32_t kind) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (kind != GMM_MFMA_SPLIT_BF16 && kind != GMM_MFMA_SPLIT_LOGITS && kind != GMM_MFMA_FP32)
    return fail(ctx, GMM_ERR_INVALID_ARG, "unknown matrix instruction kind %d", kind);
  ctx->ws.split = (kind == GMM_MFMA_SPLIT_BF16) ? 2 : (kind == GMM_MFMA_SPLIT_LOGITS) ? 1 : 0;
  return GMM_OK;
}

gmm_status gmm_set_assign_limit(gmm_ctx* ctx, int64_t bytes) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (bytes < 0) return fail(ctx, GMM_ERR_INVALID_ARG, "bytes must be >= 0");
  hipError_t e = hipStreamSynchronize(ctx->stream);  // the buffers may still be read
  if (e != hipSuccess) return hip_fail(ctx, e, "stream synchronize");
  ctx->assign_limit = bytes;
  if (ctx->selkeep && (int64_t)ctx->selkeep_bytes > bytes) {
    hipFree(ctx->selkeep);
    ctx->selkeep = nullptr;
    ctx->selkeep_bytes = 0;
  }
  if (ctx->sortbuf && (int64_t)ctx->sortbuf_bytes > bytes) {
    hipFree(ctx->sortbuf);
    ctx->sortbuf = nullptr;
    ctx->sortbuf_bytes = 0;
  }
  return GMM_OK;
}

int32_t gmm_split_level(const gmm_ctx* ctx, int32_t model) {
  if (!ctx || model < 0 || model > 2) return -1;
  if (!want_fused(ctx) || !ctx->ws.split || !ctx->ws.refine || ctx->ws.f64) return 0;
  if (model > 0 && !gmm::iso_kernel_ok(ctx->plan, ctx->ws, model == 2)) return 0;
  if (!gmm::split_kernel_ok(ctx->plan, model)) return 0;
  return (ctx->ws.split == 2 && gmm::split_kernel_ok(ctx->plan, model + 3)) ? 2 : 1;
}

gmm_status gmm_init(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const int64_t* init_rows,
                    float var_floor, float* weights, float* means, float* vars) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (!init_rows) return fail(ctx, GMM_ERR_INVALID_ARG, "init_rows is NULL");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  const int K = ctx->plan.K;
  for (int k = 0; k < K; ++k)
    if (init_rows[k] < 0 || init_rows[k] >= N)
      return fail(ctx, GMM_ERR_INVALID_ARG, "init_rows[%d]=%lld out of [0, N)", k, (long long)init_rows[k]);
  hipError_t e = hipMemcpyAsync(ctx->ws.rows, init_rows, (size_t)K * 8, hipMemcpyHostToDevice, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init rows copy");
  e = gmm::launch_init(ctx->plan, ctx->ws, X, N, ldx, var_floor, weights, means, vars, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init launch");
  // init_rows is a host array the caller may reuse as soon as we return
  e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init");
  return GMM_OK;
}

gmm_status gmm_estep_stats(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* weights,
                           const float* means, const float* vars, double* Nk, double* S1, double* S2,
                           double* loglik, int32_t accumulate) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (!Nk || !S1 || !S2 || !loglik) return fail(ctx, GMM_ERR_INVALID_ARG, "statistics outputs must be non-NULL");
  if (accumulate != 0 && accumulate != 1) return fail(ctx, GMM_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  return estep_into(ctx, X, N, ldx, weights, means, vars, Nk, S1, S2, loglik, accumulate);
}

gmm_status gmm_mstep(gmm_ctx* ctx, const double* Nk, const double* S1, const double* S2, double n_total,
                     float var_floor, float* weights, float* means, float* vars) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (!Nk || !S1 || !S2) return fail(ctx, GMM_ERR_INVALID_ARG, "statistics inputs must be non-NULL");
  gmm_status st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (!(n_total > 0.0) || !isfinite(n_total)) return fail(ctx, GMM_ERR_INVALID_ARG, "n_total must be > 0");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  hipError_t e = gmm::launch_mstep(ctx->plan, ctx->ws, Nk, S1, S2, n_total, var_floor, weights, means, vars,
                                   ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "mstep launch");
  return GMM_OK;
}

gmm_status gmm_fit(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, int32_t T, float var_floor,
                   float* weights, float* means, float* vars, double* loglik_hist) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (T < 1) return fail(ctx, GMM_ERR_INVALID_ARG, "T must be >= 1");
  if (!loglik_hist) return fail(ctx, GMM_ERR_INVALID_ARG, "loglik_hist is NULL");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  const int K = ctx->plan.K, D = ctx->plan.D;
  double* Nk = ctx->ws.stats;
  double* S1 = Nk + K;
  double* S2 = S1 + (size_t)K * D;
  for (int t = 0; t < T; ++t) {
    st = estep_into(ctx, X, N, ldx, weights, means, vars, Nk, S1, S2, loglik_hist + t, 0);
    if (st) return st;
    hipError_t e = gmm::launch_mstep(ctx->plan, ctx->ws, Nk, S1, S2, (double)N, var_floor, weights, means, vars,
                                     ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "mstep launch");
  }
  return GMM_OK;
}

gmm_status gmm_init_iso(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const int64_t* init_rows,
                        float var_floor, float* weights, float* means, float* var_iso) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, var_iso);
  if (st) return st;
  if (!init_rows) return fail(ctx, GMM_ERR_INVALID_ARG, "init_rows is NULL");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  const int K = ctx->plan.K;
  for (int k = 0; k < K; ++k)
    if (init_rows[k] < 0 || init_rows[k] >= N)
      return fail(ctx, GMM_ERR_INVALID_ARG, "init_rows[%d]=%lld out of [0, N)", k, (long long)init_rows[k]);
  hipError_t e = hipMemcpyAsync(ctx->ws.rows, init_rows, (size_t)K * 8, hipMemcpyHostToDevice, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init rows copy");
  e = gmm::launch_init_iso(ctx->plan, ctx->ws, X, N, ldx, var_floor, weights, means, var_iso, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init launch");
  e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init");
  return GMM_OK;
}

gmm_status gmm_estep_stats_iso(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* weights,
                               const float* means, const float* var_iso, double* Nk, double* S1, double* Q,
                               double* loglik, int32_t accumulate) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, var_iso);
  if (st) return st;
  if (!Nk || !S1 || !Q || !loglik) return fail(ctx, GMM_ERR_INVALID_ARG, "statistics outputs must be non-NULL");
  if (accumulate != 0 && accumulate != 1) return fail(ctx, GMM_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  const gmm::Plan& p = ctx->plan;
  hipError_t e = gmm::launch_iso_expand(p, ctx->ws, var_iso, ctx->stream);
  // S2 goes to the statistics scratch; cleared first when the reduction adds
  double* S2 = ctx->ws.stats + p.K + (size_t)p.K * p.D;
  if (e == hipSuccess && accumulate) e = gmm::launch_fill_zero(S2, (size_t)p.K * p.D, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "isotropic set-up");
  st = estep_into(ctx, X, N, ldx, weights, means, ctx->ws.vexp, Nk, S1, S2, loglik, accumulate, var_iso);
  if (st) return st;
  e = gmm::launch_iso_q(p, S2, Q, accumulate, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "isotropic Q");
  return GMM_OK;
}

gmm_status gmm_mstep_iso(gmm_ctx* ctx, const double* Nk, const double* S1, const double* Q, double n_total,
                         float var_floor, float* weights, float* means, float* var_iso) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  if (!Nk || !S1 || !Q) return fail(ctx, GMM_ERR_INVALID_ARG, "statistics inputs must be non-NULL");
  gmm_status st = check_params(ctx, weights, means, var_iso);
  if (st) return st;
  if (!(n_total > 0.0) || !isfinite(n_total)) return fail(ctx, GMM_ERR_INVALID_ARG, "n_total must be > 0");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  hipError_t e = gmm::launch_mstep_iso(ctx->plan, ctx->ws, Nk, S1, Q, n_total, var_floor, weights, means, var_iso,
                                       ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "mstep launch");
  return GMM_OK;
}

gmm_status gmm_fit_iso(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, int32_t T, float var_floor,
                       float* weights, float* means, float* var_iso, double* loglik_hist) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, var_iso);
  if (st) return st;
  if (T < 1) return fail(ctx, GMM_ERR_INVALID_ARG, "T must be >= 1");
  if (!loglik_hist) return fail(ctx, GMM_ERR_INVALID_ARG, "loglik_hist is NULL");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  const gmm::Plan& p = ctx->plan;
  const int K = p.K, D = p.D;
  double* Nk = ctx->ws.stats;
  double* S1 = Nk + K;
  double* S2 = S1 + (size_t)K * D;
  for (int t = 0; t < T; ++t) {
    hipError_t e = gmm::launch_iso_expand(p, ctx->ws, var_iso, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "isotropic set-up");
    st = estep_into(ctx, X, N, ldx, weights, means, ctx->ws.vexp, Nk, S1, S2, loglik_hist + t, 0, var_iso);
    if (st) return st;
    e = gmm::launch_iso_q(p, S2, ctx->ws.qiso, 0, ctx->stream);
    if (e == hipSuccess)
      e = gmm::launch_mstep_iso(p, ctx->ws, Nk, S1, ctx->ws.qiso, (double)N, var_floor, weights, means, var_iso,
                                ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "isotropic mstep launch");
  }
  return GMM_OK;
}

gmm_status gmm_soft_assign(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* weights,
                           const float* means, const float* vars, float threshold, int32_t max_extra,
                           int64_t* list_offsets, int32_t* list_ids, int64_t ids_capacity, int64_t* nnz) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (!(threshold > 0.f && threshold <= 1.f)) return fail(ctx, GMM_ERR_INVALID_ARG, "threshold must be in (0, 1]");
  if (max_extra < 0 || max_extra > 8) return fail(ctx, GMM_ERR_INVALID_ARG, "max_extra must be in [0, 8]");
  if (!list_offsets || !nnz) return fail(ctx, GMM_ERR_INVALID_ARG, "list_offsets and nnz must be non-NULL");
  if (ids_capacity < 0) return fail(ctx, GMM_ERR_INVALID_ARG, "ids_capacity must be >= 0");
  if (ids_capacity > 0 && !list_ids) return fail(ctx, GMM_ERR_INVALID_ARG, "list_ids is NULL");
  if (N >= ((int64_t)1 << 31)) return fail(ctx, GMM_ERR_INVALID_ARG, "N must be < 2^31 for int32 ids");
  return soft_assign_run(ctx, X, N, ldx, weights, means, vars, threshold, max_extra, list_offsets, list_ids,
                         ids_capacity, nnz);
}

}  // extern "C"

namespace {

// the soft assignment after argument checks (also the k-means assignment)
gmm_status soft_assign_run(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* weights,
                           const float* means, const float* vars, float threshold, int32_t max_extra,
                           int64_t* list_offsets, int32_t* list_ids, int64_t ids_capacity, int64_t* nnz) {
  const gmm::Plan& p = ctx->plan;
  if (p.occAssign < 1) return fail(ctx, GMM_ERR_UNSUPPORTED, "no soft-assignment kernel for this context's shape");
  hipStream_t s = ctx->stream;
  hipError_t e = gmm::launch_precompute(p, ctx->ws, weights, means, vars, s);
  if (e == hipSuccess) e = gmm::launch_assign_begin(p, ctx->ws, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "soft assignment set-up");
  const int64_t CH = p.assignChunk;
  // Where the input spans several chunks, the selections of all rows are
  // kept from the counting sweep (N x (1 + max_extra) ints, within the
  // context's assignment limit) so that the lists need no second logit sweep;
  // if that buffer cannot be had, every chunk is selected again before its
  // scatter.
  const size_t keep_bytes = (size_t)N * (size_t)(1 + max_extra) * sizeof(int32_t);
  const size_t limit = (size_t)ctx->assign_limit;
  bool keep = N <= CH;
  if (!keep && keep_bytes <= limit) {
    if (ctx->selkeep_bytes < keep_bytes) {
      e = hipStreamSynchronize(s);  // the old buffer may still be read
      if (e != hipSuccess) return hip_fail(ctx, e, "soft assignment set-up");
      if (ctx->selkeep) hipFree(ctx->selkeep);
      ctx->selkeep = nullptr;
      ctx->selkeep_bytes = 0;
      void* q = nullptr;
      if (hipMalloc(&q, keep_bytes) == hipSuccess) {
        ctx->selkeep = static_cast<int32_t*>(q);
        ctx->selkeep_bytes = keep_bytes;
      } else {
        (void)hipGetLastError();  // not fatal: fall back to selecting twice
      }
    }
    keep = ctx->selkeep != nullptr && ctx->selkeep_bytes >= keep_bytes;
  }
  const int stride = 1 + max_extra;
  auto chunk_sel = [&](int64_t r0) -> int32_t* {
    return (N <= CH || !keep) ? ctx->ws.asel : ctx->selkeep + r0 * stride;
  };
  // pass A: select every row and count list sizes
  for (int64_t r0 = 0; r0 < N; r0 += CH) {
    const int64_t rows = (N - r0 < CH) ? N - r0 : CH;
    e = gmm::launch_assign_select(p, ctx->ws, X, r0, rows, ldx, threshold, max_extra, true, chunk_sel(r0), s);
    if (e != hipSuccess) return hip_fail(ctx, e, "assignment selection");
  }
  e = gmm::launch_assign_offsets(p, ctx->ws, list_offsets, s);
  int64_t total = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&total, ctx->ws.annz, sizeof total, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "list offsets");
  *nnz = total;
  gmm_status chk = gmm_check(ctx);
  if (chk != GMM_OK) return chk;
  if (total > ids_capacity)
    return fail(ctx, GMM_ERR_CAPACITY, "ids_capacity %lld < nnz %lld", (long long)ids_capacity, (long long)total);
  // pass B: place rows into the lists in row order.  With every row's
  // selections at hand, one stable sort of (list, row) pairs does it;
  // otherwise (or without the sort buffer) chunk by chunk
  const size_t held = (N <= CH) ? 0 : keep_bytes;  // the kept selections count against the limit
  if (keep) {
    const size_t need = gmm::sort_lists_bytes(N * stride, p.K);
    const bool fits = need > 0 && held + need <= limit;
    if (fits && ctx->sortbuf_bytes < need) {
      e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(ctx, e, "soft assignment");
      if (ctx->sortbuf) hipFree(ctx->sortbuf);
      ctx->sortbuf = nullptr;
      ctx->sortbuf_bytes = 0;
      if (hipMalloc(&ctx->sortbuf, need) == hipSuccess)
        ctx->sortbuf_bytes = need;
      else
        (void)hipGetLastError();  // not fatal: the chunked scatter runs
    }
    if (fits && ctx->sortbuf && ctx->sortbuf_bytes >= need) {
      e = gmm::sort_lists(chunk_sel(0), N, stride, p.K, list_ids, total, ctx->sortbuf, ctx->sortbuf_bytes, s);
      if (e != hipSuccess) return hip_fail(ctx, e, "list sort");
      e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(ctx, e, "soft assignment");
      return gmm_check(ctx);
    }
  }
  for (int64_t r0 = 0; r0 < N; r0 += CH) {
    const int64_t rows = (N - r0 < CH) ? N - r0 : CH;
    if (!keep) {
      e = gmm::launch_assign_select(p, ctx->ws, X, r0, rows, ldx, threshold, max_extra, false, chunk_sel(r0), s);
      if (e != hipSuccess) return hip_fail(ctx, e, "assignment selection");
    }
    e = gmm::launch_assign_scatter(p, ctx->ws, chunk_sel(r0), r0, rows, max_extra, list_offsets, list_ids, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "list scatter");
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "soft assignment");
  return gmm_check(ctx);
}

// k-means helpers: assignment of every row to its nearest centre (CSR)
gmm_status kmeans_assign(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* centres,
                         int64_t* offsets, int32_t* ids) {
  hipError_t e = gmm::launch_kmeans_params(ctx->plan, ctx->ws, centres, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "k-means set-up");
  int64_t nnz = 0;
  return soft_assign_run(ctx, X, N, ldx, ctx->ws.wuni, centres, ctx->ws.vexp, 1.0f, 0, offsets, ids, N, &nnz);
}

// Out-of-core E-step: rows [r0, r0 + rows) of a host X are copied into
// alternating device staging buffers on the copy stream while the E-step of
// the previous chunk runs on the context's stream; an event per buffer,
// recorded after every E-step that reads the buffer and kept across calls,
// keeps a copy from overwriting a chunk whose E-step has not finished, also
// that of the previous call or fit iteration.  The
// statistics accumulate over the chunks exactly as gmm_estep_stats with
// accumulate = 1 on the same row ranges.  Staging rows have a stride of D
// rounded up to 4 floats; the padding floats are never read as data.
gmm_status stage_setup(gmm_ctx* c, int64_t chunk) {
  if (!c->copy_stream) {
    hipError_t e = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking);
    for (int b = 0; b < 2 && e == hipSuccess; ++b) {
      e = hipEventCreateWithFlags(&c->ev_copied[b], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_used[b], hipEventDisableTiming);
    }
    if (e != hipSuccess) return hip_fail(c, e, "copy stream set-up");
  }
  if (chunk > c->stage_rows) {
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->copy_stream);
    if (e != hipSuccess) return hip_fail(c, e, "stream synchronize");
    for (int b = 0; b < 2; ++b) {
      if (c->stage[b]) hipFree(c->stage[b]);
      c->stage[b] = nullptr;
    }
    c->stage_rows = 0;
    const size_t bytes = (size_t)chunk * ((c->plan.D + 3) & ~3) * sizeof(float);
    for (int b = 0; b < 2; ++b) {
      e = hipMalloc(&c->stage[b], bytes);
      if (e != hipSuccess) return fail(c, GMM_ERR_OOM, "staging hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    c->stage_rows = chunk;
  }
  return GMM_OK;
}

gmm_status estep_host(gmm_ctx* c, const float* Xh, int64_t N, int64_t ldx, const float* w, const float* mu,
                      const float* var, double* Nk, double* S1, double* S2, double* ll, int accumulate,
                      int64_t chunk) {
  gmm_status st = stage_setup(c, chunk);
  if (st) return st;
  const int D = c->plan.D;
  const int ld = (D + 3) & ~3;  // staging row stride (the kernels' float4 rows)
  int i = 0;
  for (int64_t r0 = 0; r0 < N; r0 += chunk, ++i) {
    const int64_t rows = (N - r0 < chunk) ? N - r0 : chunk;
    const int b = i & 1;
    // the last E-step that read buffer b, in this call or an earlier one
    // (waiting on an event never recorded returns at once)
    hipError_t e = hipStreamWaitEvent(c->copy_stream, c->ev_used[b], 0);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(c->stage[b], (size_t)ld * sizeof(float), Xh + r0 * ldx, (size_t)ldx * sizeof(float),
                           (size_t)D * sizeof(float), (size_t)rows, hipMemcpyHostToDevice, c->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(c->ev_copied[b], c->copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(c->stream, c->ev_copied[b], 0);
    if (e != hipSuccess) return hip_fail(c, e, "chunk copy");
    st = estep_into(c, c->stage[b], rows, ld, w, mu, var, Nk, S1, S2, ll, (i > 0) ? 1 : accumulate);
    if (st) return st;
    e = hipEventRecord(c->ev_used[b], c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "chunk event");
  }
  return GMM_OK;
}

gmm_status check_host_x(gmm_ctx* c, const float* Xh, int64_t N, int64_t ldx, int64_t chunk) {
  if (!Xh) return fail(c, GMM_ERR_INVALID_ARG, "X is NULL");
  if (N < 1) return fail(c, GMM_ERR_INVALID_ARG, "N must be >= 1 (got %lld)", (long long)N);
  if (ldx < c->plan.D) return fail(c, GMM_ERR_INVALID_ARG, "ldx must be >= D (got %lld, D=%d)", (long long)ldx, c->plan.D);
  if (chunk < 1 || chunk > ((int64_t)1 << 30)) return fail(c, GMM_ERR_INVALID_ARG, "chunk_rows must be in [1, 2^30]");
  return GMM_OK;
}

gmm_status kmeans_check(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* centres,
                        const int64_t* offsets, const int32_t* ids, bool lists_required = true) {
  gmm_status st = check_x(ctx, X, N, ldx);
  if (st) return st;
  if (!centres || !aligned16(centres)) return fail(ctx, GMM_ERR_INVALID_ARG, "centres must be non-NULL, 16-byte aligned");
  if (lists_required && (!offsets || !ids)) return fail(ctx, GMM_ERR_INVALID_ARG, "list scratch must be non-NULL");
  if (N >= ((int64_t)1 << 31)) return fail(ctx, GMM_ERR_INVALID_ARG, "N must be < 2^31 for int32 ids");
  return GMM_OK;
}

}  // namespace

extern "C" {

gmm_status gmm_estep_stats_host(gmm_ctx* ctx, const float* X_host, int64_t N, int64_t ldx, const float* weights,
                                const float* means, const float* vars, double* Nk, double* S1, double* S2,
                                double* loglik, int32_t accumulate, int64_t chunk_rows) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_host_x(ctx, X_host, N, ldx, chunk_rows);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (!Nk || !S1 || !S2 || !loglik) return fail(ctx, GMM_ERR_INVALID_ARG, "statistics outputs must be non-NULL");
  if (accumulate != 0 && accumulate != 1) return fail(ctx, GMM_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  return estep_host(ctx, X_host, N, ldx, weights, means, vars, Nk, S1, S2, loglik, accumulate, chunk_rows);
}

gmm_status gmm_fit_host(gmm_ctx* ctx, const float* X_host, int64_t N, int64_t ldx, int32_t T, float var_floor,
                        float* weights, float* means, float* vars, double* loglik_hist, int64_t chunk_rows) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = check_host_x(ctx, X_host, N, ldx, chunk_rows);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (T < 1) return fail(ctx, GMM_ERR_INVALID_ARG, "T must be >= 1");
  if (!loglik_hist) return fail(ctx, GMM_ERR_INVALID_ARG, "loglik_hist is NULL");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  const int K = ctx->plan.K, D = ctx->plan.D;
  double* Nk = ctx->ws.stats;
  double* S1 = Nk + K;
  double* S2 = S1 + (size_t)K * D;
  for (int t = 0; t < T; ++t) {
    st = estep_host(ctx, X_host, N, ldx, weights, means, vars, Nk, S1, S2, loglik_hist + t, 0, chunk_rows);
    if (st) return st;
    hipError_t e = gmm::launch_mstep(ctx->plan, ctx->ws, Nk, S1, S2, (double)N, var_floor, weights, means, vars,
                                     ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "mstep launch");
  }
  return GMM_OK;
}

gmm_status gmm_kmeans(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, int32_t iters, float* centres,
                      double* counts, int64_t* list_offsets, int32_t* list_ids) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = kmeans_check(ctx, X, N, ldx, centres, list_offsets, list_ids, false);
  if (st) return st;
  if (iters < 1) return fail(ctx, GMM_ERR_INVALID_ARG, "iters must be >= 1");
  if (!counts) return fail(ctx, GMM_ERR_INVALID_ARG, "counts is NULL");
  const gmm::Plan& p = ctx->plan;
  const char* envk = getenv("FLASHGMM_KMEANS_FUSED");  // 0: the list path (measurements)
  if (want_fused(ctx) && gmm::iso_kernel_ok(p, ctx->ws, true) && !(envk && atoi(envk) == 0)) {
    // one fused sweep per iteration: nearest centre (exchanged argmax),
    // one-hot statistics, then centres = S1 / n
    double* Nk = ctx->ws.stats;
    double* S1 = Nk + p.K;
    double* S2 = S1 + (size_t)p.K * p.D;
    double* ll = S2 + (size_t)p.K * p.D;
    for (int it = 0; it < iters; ++it) {
      hipError_t e = gmm::launch_kmeans_params(p, ctx->ws, centres, ctx->stream);
      if (e != hipSuccess) return hip_fail(ctx, e, "k-means set-up");
      st = estep_into(ctx, X, N, ldx, ctx->ws.wuni, centres, ctx->ws.vexp, Nk, S1, S2, ll, 0, ctx->ws.vhalf, true);
      if (st) return st;
      e = gmm::launch_kmeans_update(p, Nk, S1, centres, counts, ctx->stream);
      if (e != hipSuccess) return hip_fail(ctx, e, "centroid update");
    }
    if (list_offsets && list_ids) {  // the rows' lists for the returned centres
      st = kmeans_assign(ctx, X, N, ldx, centres, list_offsets, list_ids);
      if (st) return st;
    }
    hipError_t e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "k-means");
    return gmm_check(ctx);
  }
  if (!list_offsets || !list_ids)
    return fail(ctx, GMM_ERR_INVALID_ARG, "this shape runs k-means through the lists: list scratch is required");
  for (int it = 0; it < iters; ++it) {
    st = kmeans_assign(ctx, X, N, ldx, centres, list_offsets, list_ids);
    if (st) return st;
    hipError_t e = gmm::launch_centroids(ctx->plan, ctx->ws, X, N, ldx, list_offsets, list_ids, centres, counts, 0,
                                         1.f, 0, nullptr, nullptr, nullptr, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "centroid update");
  }
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "k-means");
  return GMM_OK;
}

gmm_status gmm_init_kmeans(gmm_ctx* ctx, const float* X, int64_t N, int64_t ldx, const float* centres,
                           float var_floor, int32_t isotropic, float* weights, float* means, float* vars,
                           int64_t* list_offsets, int32_t* list_ids) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  gmm_status st = kmeans_check(ctx, X, N, ldx, centres, list_offsets, list_ids);
  if (st) return st;
  st = check_params(ctx, weights, means, vars);
  if (st) return st;
  if (isotropic != 0 && isotropic != 1) return fail(ctx, GMM_ERR_INVALID_ARG, "isotropic must be 0 or 1");
  if (!(var_floor > 0.f) || !isfinite(var_floor)) return fail(ctx, GMM_ERR_INVALID_ARG, "var_floor must be > 0");
  hipError_t e = gmm::launch_colvar(ctx->plan, ctx->ws, X, N, ldx, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "column variances");
  st = kmeans_assign(ctx, X, N, ldx, centres, list_offsets, list_ids);
  if (st) return st;
  e = gmm::launch_centroids(ctx->plan, ctx->ws, X, N, ldx, list_offsets, list_ids, const_cast<float*>(centres),
                            nullptr, 1, var_floor, isotropic, weights, means, vars, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "mixture from clusters");
  e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "init from k-means");
  return GMM_OK;
}

gmm_status gmm_refine_stats(gmm_ctx* ctx, int64_t* refined, double* logits) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "stream synchronize");
  unsigned long long n = 0;
  e = hipMemcpy(&n, ctx->ws.nrefined, sizeof n, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(ctx->ws.nrefined, 0, sizeof n);
  if (e != hipSuccess) return hip_fail(ctx, e, "refine counter");
  if (refined) *refined = (int64_t)n;
  if (logits) *logits = ctx->logits_since;
  ctx->logits_since = 0.0;
  return GMM_OK;
}

gmm_status gmm_check(gmm_ctx* ctx) {
  if (!ctx) return GMM_ERR_INVALID_ARG;
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "stream synchronize");
  int flags[4] = {0, 0, 0, 0};
  e = hipMemcpy(flags, ctx->ws.flags, sizeof flags, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(ctx, e, "flag read");
  if (flags[0] || flags[1] || flags[2]) {
    hipMemset(ctx->ws.flags, 0, sizeof flags);
    if (flags[1]) return fail(ctx, GMM_ERR_HIP, "fused E-step exchange timed out");
    if (flags[2]) return fail(ctx, GMM_ERR_HIP, "inverted lists: second selection pass disagreed with the first");
    return fail(ctx, GMM_ERR_NUMERIC, "non-finite log-likelihood, statistics or logits");
  }
  return GMM_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Entry point that allocates nothing (gmm_estep_stats_noalloc).  Its
// workspace is carved from `scratch`, a file-scope device array of
// GMM_NOALLOC_SCRATCH_BYTES that each device holds from the first call on
// it until the process ends.  In host code the array's name is only a
// host-side stand-in, so the device address is taken once per device with
// hipGetSymbolAddress and only that address is used afterwards.
static __device__ __align__(256) unsigned char scratch[GMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};

// Workspace of the E-step alone (precomputed operands, statistics slots,
// exchange words, flags), carved in order from base; returns the bytes used.
size_t carve_estep(const gmm::Plan& p, char* base, gmm::Workspace& ws) {
  char* q = base;
  ws = gmm::Workspace{};
  ws.wop = carve<float>(q, (size_t)p.Kpad * 2 * p.Dp);
  ws.cvec = carve<float>(q, p.Kpad);
  ws.cfull = carve<double>(q, p.Kpad);
  ws.cpeak = carve<double>(q, p.Kpad);
  ws.cshift = carve<double>(q, 1);
  ws.w64 = carve<double2>(q, (size_t)p.Kpad * p.Dp);
  ws.abmax = carve<float2>(q, p.Kpad);
  ws.wsplit = carve<__bf16>(q, (size_t)p.Kpad * 2 * p.Dp * 2);
  ws.cvec64 = carve<double>(q, p.Kpad);  // written by the shift kernel whatever the precision
  // flags (4 ints) and the refined-logit counter share one cleared block
  ws.flags = carve<int>(q, 16);
  ws.nrefined = reinterpret_cast<unsigned long long*>(ws.flags + 8);
  ws.llslots = carve<double>(q, p.R > p.Glogz ? p.R : p.Glogz);
  ws.logz = carve<float>(q, (size_t)p.chunk);
  ws.xbuf = carve<unsigned long long>(q, (size_t)p.R * 4 * p.P * p.BN);
  ws.slots = carve<double>(q, (size_t)p.R * p.Kpad * p.SR);
  ws.refine = 1;
  ws.f64 = 0;
  ws.split = 2;
  return (size_t)(q - base);
}

}  // namespace

extern "C" gmm_status gmm_estep_stats_noalloc(int32_t K, int32_t D, const float* X, int64_t N, int64_t ldx,
                                              const float* weights, const float* means, const float* vars,
                                              double* Nk, double* S1, double* S2, double* loglik,
                                              int32_t accumulate, void* hip_stream) {
  g_create_err.clear();
  if (K < 1 || K > 65536) return fail(nullptr, GMM_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  if (D < 1 || D > 1024) return fail(nullptr, GMM_ERR_INVALID_ARG, "D must be in [1, 1024] (got %d)", D);
  if (!X || !aligned16(X)) return fail(nullptr, GMM_ERR_INVALID_ARG, "X must be non-NULL and 16-byte aligned");
  if (N < 1 || N > ((int64_t)1 << 40)) return fail(nullptr, GMM_ERR_INVALID_ARG, "N out of range (got %lld)", (long long)N);
  if (ldx < D || (ldx & 3))
    return fail(nullptr, GMM_ERR_INVALID_ARG, "ldx must be >= D and a multiple of 4 (got %lld)", (long long)ldx);
  if (!weights || !means || !vars || !aligned16(weights) || !aligned16(means) || !aligned16(vars))
    return fail(nullptr, GMM_ERR_INVALID_ARG, "weights/means/vars must be non-NULL and 16-byte aligned");
  if (!Nk || !S1 || !S2 || !loglik) return fail(nullptr, GMM_ERR_INVALID_ARG, "statistics outputs must be non-NULL");
  if (accumulate != 0 && accumulate != 1) return fail(nullptr, GMM_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(nullptr, GMM_ERR_UNSUPPORTED, "device index %d", dev);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, GMM_ERR_UNSUPPORTED, "built for gfx950, device is %s", prop.gcnArchName);
  if (!g_scratch[dev]) {  // once per device, with that device current
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(nullptr, GMM_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  gmm::Plan p0 = gmm::make_plan(K, D, prop.multiProcessorCount, 1, 1);
  if (!gmm::plan_shape_ok(p0)) return fail(nullptr, GMM_ERR_UNSUPPORTED, "no kernel for K=%d D=%d", K, D);
  int o1 = 1, o2 = 1;
  e = gmm::occupancy(p0, &o1, &o2);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  gmm::Plan p = gmm::make_plan(K, D, prop.multiProcessorCount, o1, o2);
  p.chunk = (int64_t)1 << 18;  // two-sweep log Z chunk
  // as many row groups (statistics slots) as the scratch holds, up to the plan's
  char* base = (char*)g_scratch[dev];
  gmm::Workspace ws;
  const int Rmax = p.R;
  for (; p.R >= 1; --p.R) {
    p.G = p.R * p.P;
    if (carve_estep(p, base, ws) <= (size_t)GMM_NOALLOC_SCRATCH_BYTES) break;
  }
  if (p.R < 1) {
    p.R = 1;
    p.G = p.P;
    return fail(nullptr, GMM_ERR_CAPACITY, "K=%d D=%d needs %zu bytes of scratch, the maximum is %zu", K, D,
                carve_estep(p, base, ws), (size_t)GMM_NOALLOC_SCRATCH_BYTES);
  }
  (void)Rmax;
  if (!ws.wop || !ws.cvec || !ws.cfull || !ws.cpeak || !ws.cshift || !ws.w64 || !ws.abmax || !ws.wsplit ||
      !ws.cvec64 || !ws.flags || !ws.llslots || !ws.logz || !ws.xbuf || !ws.slots)
    return fail(nullptr, GMM_ERR_HIP, "scratch workspace incomplete");
  hipStream_t s = (hipStream_t)hip_stream;
  // the array keeps the last call's contents: flags and counter start at zero
  e = gmm::launch_fill_zero(reinterpret_cast<double*>(ws.flags), 8, s);
  if (e == hipSuccess) e = gmm::launch_precompute(p, ws, weights, means, vars, s);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "precompute launch: %s", hipGetErrorString(e));
  const bool fused = p.fusedOK != 0 && p.P <= 64;
  int nslots = 0;
  e = gmm::launch_estep(p, ws, X, N, ldx, fused, s, nullptr, &nslots, 0);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "E-step launch: %s", hipGetErrorString(e));
  e = gmm::launch_reduce(p, ws, Nk, S1, S2, loglik, accumulate, nslots, fused ? nslots : p.Glogz, N, s);
  if (e != hipSuccess) return fail(nullptr, GMM_ERR_HIP, "reduce launch: %s", hipGetErrorString(e));
  return GMM_OK;
}
