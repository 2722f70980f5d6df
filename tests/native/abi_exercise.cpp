// Exercises every entry point of the C ABI (include/flashgmm.h) from plain host
// code: valid calls on a small seeded problem and the argument errors the
// header documents.  Built with the library's host code under AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/native/build_sanitized.sh), so that
// the validation, workspace carving, host-memory staging and list building on
// the host side run under the sanitizers on a real device.  The device code is
// compiled as usual (device sanitizers are not used).  Prints one line per
// stage and "abi_exercise: ok" at the end; exits non-zero on the first
// unexpected status.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "flashgmm.h"

namespace {

int g_fail = 0;

void expect(gmm_status got, gmm_status want, const char* what, gmm_ctx* ctx = nullptr) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want,
                 gmm_last_error(ctx) ? gmm_last_error(ctx) : "");
    g_fail = 1;
  }
}

void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "FAIL %s: %s\n", what, hipGetErrorString(e));
    std::fflush(nullptr);
    std::_Exit(2);  // no exit handlers: see the end of main
  }
}

template <class T>
T* dev(size_t n) {
  void* p = nullptr;
  hip_ok(hipMalloc(&p, n * sizeof(T) + 16), "hipMalloc");
  return static_cast<T*>(p);
}

// splitmix64: the rows of a small mixture (K well-separated centres)
uint64_t g_state = 0x5EEDull;
double uniform() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
double normal() {
  const double u = uniform() + 1e-300, v = uniform();
  return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
}

}  // namespace

int main() {
  std::setvbuf(stdout, nullptr, _IONBF, 0);  // stage lines survive an abort
  const int32_t K = 40, D = 24;
  // more than one 2^19-row selection chunk, so that the kept-selection and
  // list-sort buffers are used
  const int64_t N = 600013, ldx = D;
  std::vector<float> centres((size_t)K * D), X((size_t)N * ldx);
  for (auto& c : centres) c = (float)(8.0 * (2.0 * uniform() - 1.0));
  for (int64_t n = 0; n < N; ++n) {
    const int k = (int)(n % K);
    for (int d = 0; d < D; ++d) X[(size_t)n * ldx + d] = centres[(size_t)k * D + d] + (float)normal();
  }
  std::vector<int64_t> rows(K);
  for (int k = 0; k < K; ++k) rows[k] = 7 + 149 * k;  // distinct, in range

  float* dX = dev<float>(X.size());
  hip_ok(hipMemcpy(dX, X.data(), X.size() * 4, hipMemcpyHostToDevice), "copy X");
  float *w = dev<float>(K), *mu = dev<float>((size_t)K * D), *var = dev<float>((size_t)K * D);
  double *Nk = dev<double>(K), *S1 = dev<double>((size_t)K * D), *S2 = dev<double>((size_t)K * D);
  double *ll = dev<double>(1), *hist = dev<double>(8);

  // ---- context-free calls and their errors
  std::printf("stage: context-free\n");
  gmm_ctx* bad = nullptr;
  expect(gmm_create(&bad, 0, D, nullptr), GMM_ERR_INVALID_ARG, "create K=0");
  expect(gmm_create(nullptr, K, D, nullptr), GMM_ERR_INVALID_ARG, "create out=NULL");
  if (std::strlen(gmm_last_error(nullptr)) == 0) {
    std::fprintf(stderr, "FAIL last_error(NULL) empty after a failed create\n");
    g_fail = 1;
  }
  if (gmm_workspace_bytes(K, D) == 0) {
    std::fprintf(stderr, "FAIL workspace_bytes\n");
    g_fail = 1;
  }
  gmm_destroy(nullptr);

  gmm_ctx* ctx = nullptr;
  expect(gmm_create(&ctx, K, D, nullptr), GMM_OK, "create");
  if (!ctx) return 1;

  // ---- settings
  std::printf("stage: settings\n");
  expect(gmm_set_path(ctx, 99), GMM_ERR_INVALID_ARG, "set_path bad", ctx);
  expect(gmm_set_precision(ctx, 99), GMM_ERR_INVALID_ARG, "set_precision bad", ctx);
  expect(gmm_set_mfma(ctx, 99), GMM_ERR_INVALID_ARG, "set_mfma bad", ctx);
  expect(gmm_set_assign_limit(ctx, -1), GMM_ERR_INVALID_ARG, "set_assign_limit bad", ctx);
  expect(gmm_set_path(ctx, GMM_PATH_AUTO), GMM_OK, "set_path", ctx);
  expect(gmm_set_precision(ctx, GMM_PREC_REFINED), GMM_OK, "set_precision", ctx);
  expect(gmm_set_mfma(ctx, GMM_MFMA_SPLIT_BF16), GMM_OK, "set_mfma", ctx);
  (void)gmm_split_level(ctx, 0);

  // ---- init, E-step, M-step, fit
  std::printf("stage: init / estep / mstep / fit\n");
  expect(gmm_init(ctx, dX, N, ldx, rows.data(), 1e-6f, w, mu, var), GMM_OK, "init", ctx);
  expect(gmm_init(ctx, nullptr, N, ldx, rows.data(), 1e-6f, w, mu, var), GMM_ERR_INVALID_ARG, "init X=NULL", ctx);
  expect(gmm_init(ctx, dX, N, D - 1, rows.data(), 1e-6f, w, mu, var), GMM_ERR_INVALID_ARG, "init ldx<D", ctx);
  expect(gmm_estep_stats(ctx, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 0), GMM_OK, "estep", ctx);
  expect(gmm_estep_stats(ctx, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 1), GMM_OK, "estep accumulate", ctx);
  expect(gmm_estep_stats(ctx, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 2), GMM_ERR_INVALID_ARG, "estep acc=2", ctx);
  expect(gmm_estep_stats(ctx, dX, 0, ldx, w, mu, var, Nk, S1, S2, ll, 0), GMM_ERR_INVALID_ARG, "estep N=0", ctx);
  expect(gmm_estep_stats(ctx, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 0), GMM_OK, "estep again", ctx);
  expect(gmm_mstep(ctx, Nk, S1, S2, (double)N, 1e-6f, w, mu, var), GMM_OK, "mstep", ctx);
  expect(gmm_mstep(ctx, Nk, S1, S2, 0.0, 1e-6f, w, mu, var), GMM_ERR_INVALID_ARG, "mstep n_total=0", ctx);
  expect(gmm_profile(ctx, 1), GMM_OK, "profile on", ctx);
  expect(gmm_fit(ctx, dX, N, ldx, 4, 1e-6f, w, mu, var, hist), GMM_OK, "fit", ctx);
  double sms = 0, lms = 0;
  int64_t sl = 0, ln = 0, nref = 0;
  double nlog = 0;
  expect(gmm_profile_read(ctx, &sms, &sl, &lms, &ln), GMM_OK, "profile_read", ctx);
  expect(gmm_profile(ctx, 0), GMM_OK, "profile off", ctx);
  expect(gmm_refine_stats(ctx, &nref, &nlog), GMM_OK, "refine_stats", ctx);
  expect(gmm_set_path(ctx, GMM_PATH_TWO_SWEEP), GMM_OK, "two-sweep", ctx);
  expect(gmm_fit(ctx, dX, N, ldx, 2, 1e-6f, w, mu, var, hist), GMM_OK, "fit two-sweep", ctx);
  expect(gmm_set_precision(ctx, GMM_PREC_FP64), GMM_OK, "fp64", ctx);
  expect(gmm_estep_stats(ctx, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 0), GMM_OK, "estep fp64", ctx);
  expect(gmm_set_precision(ctx, GMM_PREC_REFINED), GMM_OK, "refined", ctx);
  expect(gmm_set_path(ctx, GMM_PATH_AUTO), GMM_OK, "auto", ctx);
  expect(gmm_check(ctx), GMM_OK, "check", ctx);

  // ---- out-of-core: pageable and pinned host rows, two chunk sizes
  std::printf("stage: host-memory E-step\n");
  expect(gmm_estep_stats_host(ctx, X.data(), N, ldx, w, mu, var, Nk, S1, S2, ll, 0, 70000), GMM_OK, "estep_host", ctx);
  float* pinned = nullptr;
  hip_ok(hipHostMalloc((void**)&pinned, X.size() * 4, hipHostMallocDefault), "hipHostMalloc");
  std::memcpy(pinned, X.data(), X.size() * 4);
  expect(gmm_fit_host(ctx, pinned, N, ldx, 2, 1e-6f, w, mu, var, hist, 250000), GMM_OK, "fit_host", ctx);
  expect(gmm_estep_stats_host(ctx, pinned, N, ldx, w, mu, var, Nk, S1, S2, ll, 0, 0), GMM_ERR_INVALID_ARG,
         "estep_host chunk=0", ctx);
  expect(gmm_check(ctx), GMM_OK, "check host", ctx);

  // ---- soft assignment: capacity error, then the lists, then the chunked builder
  std::printf("stage: soft assignment\n");
  int64_t* off = dev<int64_t>(K + 1);
  int32_t* ids = dev<int32_t>((size_t)N * 4);
  int64_t nnz = 0;
  expect(gmm_soft_assign(ctx, dX, N, ldx, w, mu, var, 0.1f, 3, off, ids, 0, &nnz), GMM_ERR_CAPACITY,
         "soft_assign capacity", ctx);
  expect(gmm_soft_assign(ctx, dX, N, ldx, w, mu, var, 0.1f, 3, off, ids, N * 4, &nnz), GMM_OK, "soft_assign", ctx);
  const int64_t nnz_sorted = nnz;
  expect(gmm_set_assign_limit(ctx, 0), GMM_OK, "assign limit 0", ctx);
  expect(gmm_soft_assign(ctx, dX, N, ldx, w, mu, var, 0.1f, 3, off, ids, N * 4, &nnz), GMM_OK, "soft_assign chunked",
         ctx);
  if (nnz != nnz_sorted) {
    std::fprintf(stderr, "FAIL soft_assign nnz %lld vs %lld\n", (long long)nnz, (long long)nnz_sorted);
    g_fail = 1;
  }
  expect(gmm_soft_assign(ctx, dX, N, ldx, w, mu, var, 0.f, 3, off, ids, N * 4, &nnz), GMM_ERR_INVALID_ARG,
         "soft_assign threshold 0", ctx);
  expect(gmm_soft_assign(ctx, dX, N, ldx, w, mu, var, 0.1f, 9, off, ids, N * 4, &nnz), GMM_ERR_INVALID_ARG,
         "soft_assign m=9", ctx);

  // ---- isotropic model and k-means
  std::printf("stage: isotropic / k-means\n");
  float* viso = dev<float>(K);
  double* Q = dev<double>(K);
  expect(gmm_init_iso(ctx, dX, N, ldx, rows.data(), 1e-6f, w, mu, viso), GMM_OK, "init_iso", ctx);
  expect(gmm_estep_stats_iso(ctx, dX, N, ldx, w, mu, viso, Nk, S1, Q, ll, 0), GMM_OK, "estep_iso", ctx);
  expect(gmm_mstep_iso(ctx, Nk, S1, Q, (double)N, 1e-6f, w, mu, viso), GMM_OK, "mstep_iso", ctx);
  expect(gmm_fit_iso(ctx, dX, N, ldx, 2, 1e-6f, w, mu, viso, hist), GMM_OK, "fit_iso", ctx);
  float* cen = dev<float>((size_t)K * D);
  double* cnt = dev<double>(K);
  hip_ok(hipMemcpy(cen, mu, (size_t)K * D * 4, hipMemcpyDeviceToDevice), "copy centres");
  expect(gmm_kmeans(ctx, dX, N, ldx, 3, cen, cnt, off, ids), GMM_OK, "kmeans", ctx);
  expect(gmm_init_kmeans(ctx, dX, N, ldx, cen, 1e-6f, 0, w, mu, var, off, ids), GMM_OK, "init_kmeans", ctx);
  expect(gmm_check(ctx), GMM_OK, "check iso", ctx);

  // ---- the entry point that allocates nothing
  std::printf("stage: no-alloc E-step\n");
  expect(gmm_estep_stats_noalloc(K, D, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 0, nullptr), GMM_OK, "noalloc");
  expect(gmm_estep_stats_noalloc(K, D, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 1, nullptr), GMM_OK,
         "noalloc accumulate");
  expect(gmm_estep_stats_noalloc(0, D, dX, N, ldx, w, mu, var, Nk, S1, S2, ll, 0, nullptr), GMM_ERR_INVALID_ARG,
         "noalloc K=0");
  hip_ok(hipDeviceSynchronize(), "synchronize");

  gmm_destroy(ctx);
  for (void* p : {(void*)dX, (void*)w, (void*)mu, (void*)var, (void*)Nk, (void*)S1, (void*)S2, (void*)ll, (void*)hist,
                  (void*)off, (void*)ids, (void*)viso, (void*)Q, (void*)cen, (void*)cnt})
    hip_ok(hipFree(p), "hipFree");
  hip_ok(hipHostFree(pinned), "hipHostFree");
  std::printf(g_fail ? "abi_exercise: FAILED\n" : "abi_exercise: ok\n");
  // End without the exit handlers: under AddressSanitizer the HIP runtime's
  // own teardown (its static destructors, after main) frees memory whose
  // quarantine recycling reaches device allocations after the runtime has
  // unloaded, which trips an internal sanitizer check.  Everything this
  // program allocated has been released above.
  std::fflush(nullptr);
  std::_Exit(g_fail);
}
