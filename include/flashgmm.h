/*
 * flashgmm.h - C ABI of the fused diagonal-covariance Gaussian-mixture EM step
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "Flash-GMM: A Memory-Efficient Kernel for Scalable
 * Soft Clustering" (Bloch et al., arXiv 2606.10896): one pass over the data
 * computes each point's K log-densities, normalises them with a per-point
 * log-sum-exp into responsibilities, and folds those straight into the
 * M-step sufficient statistics, so the N x K responsibility matrix is never
 * stored (Section 3.1 and Algorithm 1 of that paper; Section 3.2 for the
 * memory claim).  Here the covariance is diagonal (sigma^2_kd) rather than
 * the paper's isotropic sigma^2_k I.
 *
 * Conventions for every entry point:
 *   - Pointers marked [dev] are device pointers on the context's device; [host]
 *     are host pointers.  All arrays are dense row-major.  The caller owns
 *     every array it passes; the library never frees or keeps them.
 *   - X has N rows of D float32 values with a row stride of ldx floats
 *     (ldx >= D, ldx % 4 == 0) and a 16-byte aligned base.
 *   - Parameters: weights float32[K], means float32[K*D], vars float32[K*D]
 *     (variances, not standard deviations), 16-byte aligned.
 *   - Work is enqueued on the context's HIP stream and is complete when that
 *     stream is synchronised.  Entry points that return values to the host
 *     (gmm_soft_assign, gmm_check) synchronise the stream themselves.
 *   - No entry point aborts or throws.  Arguments are checked before anything
 *     is launched; a failure returns a status and leaves a message for
 *     gmm_last_error().  A failed call leaves caller arrays unspecified only
 *     when the status is GMM_ERR_HIP or GMM_ERR_NUMERIC.
 *   - The same inputs on the same device and build give bit-identical
 *     outputs: fixed reduction trees, and floating-point atomic adds only
 *     into words that a single lane of a single workgroup writes (their
 *     order is that lane's program order), never a contended one.
 *   - A context is not thread-safe; distinct contexts are independent.
 */
#ifndef FLASHGMM_H
#define FLASHGMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gmm_ctx gmm_ctx;

typedef enum {
    GMM_OK = 0,
    GMM_ERR_INVALID_ARG = 1, /* a pointer, size or option is out of range */
    GMM_ERR_UNSUPPORTED = 2, /* valid request that the library or device cannot run */
    GMM_ERR_OOM = 3,         /* workspace allocation failed */
    GMM_ERR_HIP = 4,         /* a HIP runtime call or kernel failed */
    GMM_ERR_NUMERIC = 5,     /* non-finite log-likelihood or statistics */
    GMM_ERR_CAPACITY = 6     /* ids_capacity smaller than the lists need */
} gmm_status;

/* Execution path of the E-step (gmm_set_path).  AUTO picks FUSED when the
 * component groups of one row tile fit the cooperative grid (at most 64 of
 * them; under GMM_PREC_FP64 as many as fit), else TWO_SWEEP. */
typedef enum {
    GMM_PATH_AUTO = 0,
    GMM_PATH_TWO_SWEEP = 1, /* Algorithm 1's two sweeps: log Z first, then
                               responsibilities and statistics with the
                               logits recomputed (Section 3.1) */
    GMM_PATH_FUSED = 2      /* one sweep: the workgroups that share a row tile
                               exchange per-row log-sum-exp partials, so each
                               logit is computed once */
} gmm_path;

/* Precision of the logits (gmm_set_precision).
 * REFINED (default): the K logits of every point come from a first-pass
 *   MFMA contraction (split-bfloat16 or fp32, gmm_set_mfma), and each logit
 *   that can carry a responsibility above e^-16 of the point's largest one
 *   (judged with a rigorous bound on the first pass's error) is recomputed
 *   in float64 before the log-sum-exp, so responsibilities, statistics and
 *   log-likelihood carry float64-grade logits wherever they matter.
 * FP32: no refinement; fp32 expanded-quadratic logits throughout (errors of
 *   1e-4..1e-2 nats on data spread over many cluster widths).
 * FP64: every logit from a float64 MFMA contraction (v_mfma_f64, half the
 *   fp32 matrix rate), rounded once to fp32; for data whose responsibilities
 *   are diffuse, where REFINED would recompute a large share of the logits. */
typedef enum {
    GMM_PREC_REFINED = 0,
    GMM_PREC_FP32 = 1,
    GMM_PREC_FP64 = 2
} gmm_precision;

/* Matrix instructions of the fused E-step contractions (gmm_set_mfma).
 * Under REFINED precision the first-pass logits may be split-bfloat16:
 *   every float of the contraction is split into two bfloat16 (x = x_hi +
 *   x_lo, within 2^-16 |x|) and the contraction is three bfloat16 MFMA
 *   passes (hi.hi + hi.lo + lo.hi), about 5x the fp32 MFMA throughput; these
 *   logits only decide which logits are recomputed in float64 (the error
 *   bound includes the split error), never the values of those that matter.
 * The statistics contraction may be split-bfloat16 in three parts: a
 *   float32 value is exactly hi + mid + lo, and the six products of order up
 *   to two (hi.hi, hi.mid, mid.hi, hi.lo, lo.hi, mid.mid) give float32-level
 *   accuracy at about 2.7x the fp32 MFMA throughput.
 * SPLIT_BF16 (default): split logits and split statistics where built (the
 *   diagonal kernel); split logits alone elsewhere they are built.
 * SPLIT_LOGITS: split logits, fp32 statistics.
 * FP32: fp32 MFMA for both.
 * Split logits are built for the fused E-steps with D <= 128 (diagonal;
 * isotropic and the k-means hard assignment for D > 16) and for the soft
 * assignment (gmm_soft_assign, D <= 128); split statistics for the fused
 * E-steps; elsewhere FP32 runs. */
typedef enum {
    GMM_MFMA_SPLIT_BF16 = 0,
    GMM_MFMA_SPLIT_LOGITS = 1,
    GMM_MFMA_FP32 = 2
} gmm_mfma_kind;

/* Create a context for K components of dimension D on the current HIP device.
 * hip_stream is a hipStream_t (NULL = the null stream).  Allocates the
 * workspace, whose size depends on K, D and the device but not on N (see
 * gmm_workspace_bytes).  The only later allocations are those of the
 * out-of-core calls (gmm_estep_stats_host, gmm_fit_host): a copy stream and
 * two device staging buffers, made on their first use and grown when a call
 * asks for larger chunks; and of gmm_soft_assign: its own buffers (see
 * there), within the limit gmm_set_assign_limit sets.  Every other entry
 * point allocates nothing; all of it is freed by gmm_destroy.
 * 1 <= K <= 65536, 1 <= D <= 1024. */
gmm_status gmm_create(gmm_ctx **out /*[host]*/, int32_t K, int32_t D, void *hip_stream);

/* Release the context and its workspace.  NULL-safe. */
void gmm_destroy(gmm_ctx *ctx);

/* Message of the last failed call on ctx (a context-owned string), or of the
 * last failed context-free call (gmm_create, gmm_estep_stats_noalloc) when
 * ctx is NULL. */
const char *gmm_last_error(const gmm_ctx *ctx);

/* Workspace bytes a context for (K, D) allocates on the current device. */
size_t gmm_workspace_bytes(int32_t K, int32_t D);

/* Select the E-step path (gmm_path).  Both paths compute the same statistics
 * up to float rounding order. */
gmm_status gmm_set_path(gmm_ctx *ctx, int32_t path);

/* Select the logit precision (gmm_precision) of later E-steps. */
gmm_status gmm_set_precision(gmm_ctx *ctx, int32_t mode);

/* Select the matrix instructions (gmm_mfma_kind) of later E-steps. */
gmm_status gmm_set_mfma(gmm_ctx *ctx, int32_t kind);

/* Limit, in bytes, of the device memory gmm_soft_assign may hold in the
 * context beyond its workspace (the kept selections and the list-sort
 * buffer); default 20 GiB.  0 keeps no selections and sorts nothing: every
 * chunk is selected twice and the lists are built block by block.  Buffers
 * already held beyond a new, smaller limit are freed.  bytes >= 0.
 * Synchronises the stream. */
gmm_status gmm_set_assign_limit(gmm_ctx *ctx, int64_t bytes);

/* What the E-step of ctx for model (0 diagonal, 1 isotropic, 2 the k-means
 * hard assignment) runs with the context's current path, precision and
 * instruction setting: 0 fp32 MFMA, 1 split-bfloat16 logits, 2 split-bfloat16
 * logits and statistics; -1 for NULL or an unknown model. */
int32_t gmm_split_level(const gmm_ctx *ctx, int32_t model);

/* Initialisation (not on the pages, which warm-start from k-means):
 * means_k = X[init_rows[k]] for K distinct rows; every component gets the
 * population (ddof 0) variance of each dimension over all N rows, floored at
 * var_floor; weights 1/K.  init_rows [host] int64[K], each in [0, N). */
gmm_status gmm_init(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                    const int64_t *init_rows /*[host]*/, float var_floor,
                    float *weights /*[dev] K*/, float *means /*[dev] K*D*/,
                    float *vars /*[dev] K*D*/);

/* E-step sufficient statistics (Section 2; Algorithm 1 steps 4-17):
 *   Nk[k]   = sum_n r_nk,
 *   S1[k,d] = sum_n r_nk x_nd,   S2[k,d] = sum_n r_nk x_nd^2,
 *   loglik  = sum_n log sum_k pi_k N(x_n | mu_k, diag vars_k),
 * with r_nk the responsibilities of the given parameters.  Outputs are
 * float64 device arrays; accumulate = 0 overwrites them, 1 adds into them
 * (for row chunks of one data set). */
gmm_status gmm_estep_stats(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                           const float *weights, const float *means, const float *vars /*[dev]*/,
                           double *Nk /*[dev] K*/, double *S1 /*[dev] K*D*/,
                           double *S2 /*[dev] K*D*/, double *loglik /*[dev] 1*/,
                           int32_t accumulate);

/* M-step, Eqs. (1)-(3) of Section 2 with a diagonal covariance, in place:
 *   weights_k = Nk_k / n_total,  means_k = S1_k / Nk_k,
 *   vars_kd   = max(S2_kd / Nk_k - means_kd^2, var_floor)   (Eq. (3), new mean).
 * A component with Nk_k < 1e-6 keeps its mean and variances.  float64
 * arithmetic, float32 results.  n_total > 0, var_floor > 0. */
gmm_status gmm_mstep(gmm_ctx *ctx, const double *Nk, const double *S1, const double *S2 /*[dev]*/,
                     double n_total, float var_floor,
                     float *weights, float *means, float *vars /*[dev], in/out*/);

/* T EM iterations from the parameters passed in (updated in place): each is
 * the E-step above followed by the M-step above (Section 2: the E-step's
 * responsibilities, then Eqs. (1)-(3)), the loop of Algorithm 1 run for a
 * fixed number of iterations (Section 3.4 times 30 of them).
 * loglik_hist [dev] float64[T]: entry t is the log-likelihood of the
 * parameters entering iteration t.  No host synchronisation inside. */
gmm_status gmm_fit(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx, int32_t T,
                   float var_floor, float *weights, float *means, float *vars /*[dev] in/out*/,
                   double *loglik_hist /*[dev] T*/);

/* Isotropic model: Sigma_k = sigma^2_k I, the covariance of the pages'
 * Section 2 and Algorithm 1, with Eq. (3) averaged over the D dimensions:
 *   sigma^2_k = sum_n r_nk ||x_n - mu_k||^2 / (D N_k) = (Q_k / N_k - ||mu_k||^2) / D,
 *   Q_k = sum_n r_nk ||x_n||^2.
 * var_iso is a float32 device array of K variances (16-byte aligned); the
 * other arguments, the floor, the empty-component rule, errors and
 * determinism are as in the diagonal calls above.  The E-step runs the
 * diagonal kernels on the variances broadcast over the dimensions (the
 * logits are identical); the workspace holds the K x D broadcast.
 *
 * gmm_init_iso: means are the rows init_rows, every variance is the mean over
 * the dimensions of the population per-dimension variance of X, floored;
 * weights 1/K.  Synchronises the stream (init_rows is a host array). */
gmm_status gmm_init_iso(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                        const int64_t *init_rows /*[host]*/, float var_floor,
                        float *weights /*[dev] K*/, float *means /*[dev] K*D*/, float *var_iso /*[dev] K*/);

/* E-step statistics of the isotropic model: Nk, S1 as gmm_estep_stats, and
 * Q[k] = sum_n r_nk ||x_n||^2 (float64); accumulate as gmm_estep_stats. */
gmm_status gmm_estep_stats_iso(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                               const float *weights, const float *means, const float *var_iso /*[dev]*/,
                               double *Nk /*[dev] K*/, double *S1 /*[dev] K*D*/, double *Q /*[dev] K*/,
                               double *loglik /*[dev] 1*/, int32_t accumulate);

/* M-step of the isotropic model, in place: weights_k = Nk_k / n_total,
 * means_k = S1_k / Nk_k, var_iso_k = max((Q_k / Nk_k - ||means_k||^2) / D,
 * var_floor), all in float64 with float32 results; Nk_k < 1e-6 keeps the
 * component's mean and variance. */
gmm_status gmm_mstep_iso(gmm_ctx *ctx, const double *Nk, const double *S1, const double *Q /*[dev]*/,
                         double n_total, float var_floor,
                         float *weights, float *means, float *var_iso /*[dev], in/out*/);

/* T EM iterations of the isotropic model, as gmm_fit. */
gmm_status gmm_fit_iso(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx, int32_t T,
                       float var_floor, float *weights, float *means, float *var_iso /*[dev] in/out*/,
                       double *loglik_hist /*[dev] T*/);

/* Out-of-core E-step and fit: X_host is a HOST array of N rows (row stride
 * ldx floats), pinned (hipHostMalloc) for the copies to overlap the compute,
 * pageable also accepted.  Rows go to the device in chunks of chunk_rows
 * through two device staging buffers that the context allocates on first use
 * (2 x chunk_rows x D floats, kept until gmm_destroy): the copy of chunk i+1
 * runs on a copy stream of the context while the E-step of chunk i runs on
 * the context's stream.  The statistics are those of gmm_estep_stats with
 * accumulate = 1 over the same row ranges (bit-identical), and gmm_fit_host
 * is gmm_fit on them.  Everything else (outputs, errors, no host
 * synchronisation) as gmm_estep_stats / gmm_fit; X_host must stay valid until
 * the context's stream has synchronised.  This is the pages' route to data
 * sets larger than device memory (N >= 1e9). */
gmm_status gmm_estep_stats_host(gmm_ctx *ctx, const float *X_host /*[host]*/, int64_t N, int64_t ldx,
                                const float *weights, const float *means, const float *vars /*[dev]*/,
                                double *Nk /*[dev] K*/, double *S1 /*[dev] K*D*/, double *S2 /*[dev] K*D*/,
                                double *loglik /*[dev] 1*/, int32_t accumulate, int64_t chunk_rows);
gmm_status gmm_fit_host(gmm_ctx *ctx, const float *X_host /*[host]*/, int64_t N, int64_t ldx, int32_t T,
                        float var_floor, float *weights, float *means, float *vars /*[dev] in/out*/,
                        double *loglik_hist /*[dev] T*/, int64_t chunk_rows);

/* k-means warm start.  The pages seed their mixtures with k-means (the set-up
 * of the IVF experiments); the algorithm is Lloyd's: every row goes to its
 * nearest centre in squared Euclidean distance (lowest index on ties; every
 * candidate that can be nearest is recomputed in float64 and compared after
 * rounding to float32, so the float64 order holds except between distances
 * within about one float32 ulp), then every centre moves to the
 * mean of its rows; a centre with no rows keeps its position.  Centres are
 * float32 [dev] K x D, updated in place over iters iterations; counts [dev]
 * float64[K] receives the cluster sizes of the last assignment.
 * Where the fused path applies (D <= 128, float32 or refined logits) an
 * iteration is one sweep of the fused isotropic E-step kernel with one-hot
 * responsibilities (the row's argmax exchanged like the log-sum-exp) and the
 * centre sums accumulate like the E-step statistics (float32 within 2048-row
 * windows, float64 across); list_offsets [dev] int64[K+1] and list_ids [dev]
 * int32[N] may then be NULL, and if given receive the CSR lists of the rows'
 * nearest returned centres (row ids ascending).  Elsewhere the iterations run
 * through those lists (required then) with float64 sums in list order.
 * Deterministic either way.  N < 2^31.  Synchronises. */
gmm_status gmm_kmeans(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx, int32_t iters,
                      float *centres /*[dev] K*D in/out*/, double *counts /*[dev] K*/,
                      int64_t *list_offsets /*[dev] K+1*/, int32_t *list_ids /*[dev] N*/);

/* Mixture seeded from a clustering: one assignment of the rows to the given
 * centres, then weights_k = n_k / N, means_k = centres_k and the variances of
 * each cluster's rows about its centre, per dimension (vars K x D) or
 * averaged over the dimensions when isotropic = 1 (vars K); an empty cluster
 * gets the variance of all rows; variances floored by var_floor.  Scratch and
 * synchronisation as gmm_kmeans. */
gmm_status gmm_init_kmeans(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                           const float *centres /*[dev] K*D*/, float var_floor, int32_t isotropic,
                           float *weights /*[dev] K*/, float *means /*[dev] K*D*/, float *vars /*[dev]*/,
                           int64_t *list_offsets /*[dev] K+1*/, int32_t *list_ids /*[dev] N*/);

/* Inverted lists of a soft assignment (Section 4.2 argmax assignment and the
 * Section 4.3 multi-assignment, with the threshold and count rule below):
 * each row goes to its highest-responsibility component (lowest index on
 * ties) and to up to max_extra further components whose responsibility is
 * >= threshold, those ranked by responsibility descending, then index
 * ascending.  Output is CSR: list_offsets [dev] int64[K+1], list_ids [dev]
 * int32[nnz] with row ids ascending within each list.  *nnz [host] receives
 * the total.  If ids_capacity < nnz the ids are not written, list_offsets
 * and *nnz are set and GMM_ERR_CAPACITY is returned.  A row whose logits are
 * all -inf or NaN gives GMM_ERR_NUMERIC.  Logits within max(16, 1 - log
 * threshold) nats of a row's largest are evaluated in float64 (under
 * GMM_PREC_REFINED), so ranks and the threshold test are float64-accurate.
 * The result is deterministic.  0 < threshold <= 1, 0 <= max_extra <= 8,
 * N < 2^31.  Rows are selected in chunks of 2^19 by one counting sweep.
 * Over more than one chunk the selections are kept in a context buffer of
 * N * (1 + max_extra) int32; with every row's selections at hand the lists
 * come from one stable radix sort of (list, row) pairs in a second context
 * buffer (about 16 bytes per selection slot).  Both buffers are allocated on
 * first need, grown on demand and held until gmm_destroy, within the
 * context's assignment limit (gmm_set_assign_limit, default 20 GiB); where
 * they do not fit or cannot be allocated, each chunk is selected again and
 * its rows placed block by block.  The lists are the same either way.
 * Synchronises the stream. */
gmm_status gmm_soft_assign(gmm_ctx *ctx, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                           const float *weights, const float *means, const float *vars /*[dev]*/,
                           float threshold, int32_t max_extra,
                           int64_t *list_offsets /*[dev] K+1*/, int32_t *list_ids /*[dev]*/,
                           int64_t ids_capacity, int64_t *nnz /*[host]*/);

/* Synchronise the stream and report device-side faults recorded since the
 * last check: GMM_ERR_NUMERIC if a log-likelihood or statistic came out
 * non-finite, GMM_ERR_HIP if a fused-path exchange timed out. */
gmm_status gmm_check(gmm_ctx *ctx);

/* Kernel timing for measurement tools.  While enabled (enable = 1), every
 * launch of the E-step's dominant kernel (the statistics sweep; for the
 * two-sweep path also the log Z sweep, counted separately) is bracketed by
 * HIP events on the context's stream.  gmm_profile_read synchronises the
 * stream, adds up the elapsed times since the last read (milliseconds) and
 * returns the launch counts; any pointer may be NULL.  enable = 0 stops
 * recording and drops pending events. */
gmm_status gmm_profile(gmm_ctx *ctx, int32_t enable);
gmm_status gmm_profile_read(gmm_ctx *ctx, double *stats_ms, int64_t *stats_launches,
                            double *logz_ms, int64_t *logz_launches);

/* Refinement statistics: synchronises the stream and returns the number of
 * logits recomputed in float64 and the number of logits the E-step sweeps
 * evaluated (N*K per sweep) since the previous call, then resets both. */
gmm_status gmm_refine_stats(gmm_ctx *ctx, int64_t *refined, double *logits);

/* Scratch of gmm_estep_stats_noalloc: 160 MiB of device memory, one array per
 * device, held from the first call on a device until the process ends. */
#define GMM_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * E-step statistics of gmm_estep_stats (same definition, same arguments
 * from X on, same kernels and default settings: refined logits, split
 * bfloat16 contractions, the fused path where it applies) without a
 * context, on the given HIP stream (NULL = the null stream) of the current
 * device.  It calls no allocating routine: its workspace lives in a
 * fixed-size file-scope device array of GMM_NOALLOC_SCRATCH_BYTES.  With as
 * many statistics slots as the context's workspace has (true for K=1024,
 * D=128) the results equal gmm_estep_stats's bit for bit; shapes whose
 * workspace is larger get fewer slots (the same statistics up to the
 * rounding order of the partial sums), and shapes whose smallest workspace
 * does not fit return GMM_ERR_CAPACITY.  Every call on a device shares that
 * device's array: calls that overlap on one device (two streams, two host
 * threads) race and must be serialised by the caller.  Errors: as
 * gmm_estep_stats (launch errors only; device-side faults are not reported);
 * gmm_last_error(NULL) returns the message of a failed call. */
gmm_status gmm_estep_stats_noalloc(int32_t K, int32_t D, const float *X /*[dev]*/, int64_t N, int64_t ldx,
                                   const float *weights, const float *means, const float *vars /*[dev]*/,
                                   double *Nk /*[dev] K*/, double *S1 /*[dev] K*D*/, double *S2 /*[dev] K*D*/,
                                   double *loglik /*[dev] 1*/, int32_t accumulate, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHGMM_H */
