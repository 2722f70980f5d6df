// Internal interface between the C ABI (gmm_api.hip) and the kernels
// (gmm_kernels.hip).  Not installed; no torch types anywhere.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmm {

constexpr int kWave = 64;
constexpr int kWavesPerWG = 8;     // waves of the E-step workgroups
constexpr int kCompsPerWave = 32;  // two 16-wide MFMA component blocks
constexpr int kNumXCD = 8;         // MI355X: 8 accelerator complex dies

// Rows per tile: 64 while a row's features fit one 128-dim wave segment set,
// 16 for wide rows (their tiles would not fit LDS).
// D > 128 (eight dim-segment waves): 32 rows up to D = 768, two 16-row MFMA
// blocks per wave, so each W operand a wave loads serves 32 rows; wider rows
// take 16-row tiles (a 32-row tile of 1024 dims would not fit LDS)
constexpr int bn_for(int WD, int DPW) { return WD * DPW <= 128 ? 64 : WD * DPW <= 768 ? 32 : 16; }

// Shape of the E-step kernels, chosen once per context from (K, D).
//   WC comp groups x WD dim segments = waves per workgroup.
//   DPW dims per wave segment (multiple of 16); Dp = DPW * WD >= D.
//   BN rows per tile.
struct Plan {
  int K, D;
  int WC, WD, DPW, Dp, BN;
  int Kpad;          // multiple of 32 * WC
  int P;             // workgroups sharing one row tile (component groups)
  int R;             // row groups (stats partial slots)
  int G;             // stats grid = R * P
  int Glogz;         // persistent grid of the log Z sweep
  int SR;            // doubles per (slot, component): 2*Dp features + N_k
  int RS;            // LDS floats per tile row
  int fusedOK;       // cooperative grid can hold R*P workgroups
  int fused64OK;     // ... and so can the float64-logit fused kernel
  int64_t chunk;     // rows per two-sweep chunk (log Z buffer length)
  size_t ldsStats, ldsLogz;
  int numCU;
  int occAssign;       // workgroups per CU of the soft-assignment kernel
  int64_t assignChunk; // rows per soft-assignment chunk
  int assignBlocks;    // row blocks per chunk for the ordered list scatter
};

struct Workspace {
  float* wop;        // Kpad * 2*Dp  MFMA-operand-ordered [a | b] per dim
  float* cvec;       // Kpad         per-component constant minus the global offset C (-inf: padding)
  double* cfull;     // Kpad         per-component constant, float64
  double* cpeak;     // Kpad         component log-density at its mean
  double* cshift;    // 1            global logit offset C
  double2* w64;      // Kpad * Dp    float64 (a, b) for the logit refinement
  float2* abmax;     // Kpad         per-component max |a|, max |b|
  int refine;        // 1: float64 refinement of the logits that matter
  int f64;           // 1: float64 MFMA logits (two-sweep path)
  double* wop64;     // Kpad * 2*Dp  as wop, float64
  double* cvec64;    // Kpad         cfull - C, float64 (-inf: padding)
  unsigned long long* nrefined;  // refined-logit counter (gmm_refine_stats)
  double* slots;     // R * Kpad * SR
  double* llslots;   // max(R, Glogz)
  float* logz;       // chunk
  unsigned long long* xbuf;  // R * 2 * P * BN  tagged log-sum-exp exchange
  double* stats;     // K + 2*K*D + 1  (fit's own statistics: Nk, S1, S2, LL)
  double* colpart;   // colG * D  column partial sums (init)
  double* colmean;   // D
  int64_t* rows;     // K  init rows
  int* flags;        // [0] numeric fault, [1] exchange timeout, [2] list overflow
  float* vexp;       // K * D  isotropic variances broadcast over the dimensions
  double* qiso;      // K      isotropic Q_k of gmm_fit_iso
  float* wuni;       // K      k-means: equal weights
  float* vhalf;      // K      k-means: isotropic variances 1/2
  float* wiso;       // Kpad * Dp  isotropic kernel: mu / s^2 in MFMA-operand order
  float* ivec;       // Kpad       isotropic kernel: 1 / (2 s^2)
  __bf16* wsplit;    // Kpad * 2*Dp * 2  split-bf16 [a | b] (hi, lo), WD = 1
  __bf16* wsplit_iso;  // Kpad * Dp * 2  split-bf16 mu / s^2 (hi, lo), isotropic kernel
  int split;         // fused refined E-steps: 0 fp32 MFMA, 1 split-bf16 logits, 2 logits and statistics
  int colG;
  // soft assignment
  int32_t* asel;                 // assignChunk * 9  per-row selections
  float4* agco;                  // Kpad / 32  per-group error-bound coefficients
  unsigned long long* acounts;   // Kpad  list sizes
  unsigned* acnt;                // assignBlocks * Kpad  per-(block, list) counts / ranks
  unsigned* atot;                // Kpad  per-chunk list totals
  int64_t* acursor;              // Kpad  next free position of each list
  int64_t* annz;                 // 1
};

Plan make_plan(int K, int D, int numCU, int occStats, int occLogz);
// Whether the float64-logit fused kernel fits the plan's cooperative grid.
hipError_t fused64_fits(const Plan& p, int* ok);
bool plan_shape_ok(const Plan& p);
size_t workspace_bytes(const Plan& p);

hipError_t occupancy(const Plan& p, int* occStats, int* occLogz);

// Launchers (enqueue on stream; return the first launch error).
hipError_t launch_precompute(const Plan& p, const Workspace& w, const float* weights,
                             const float* means, const float* vars, hipStream_t s);
// Optional per-launch timing hooks: called around the two E-step sweeps.
struct LaunchHooks {
  void (*before)(void* user, int which, hipStream_t s) = nullptr;  // which: 0 stats, 1 log Z
  void (*after)(void* user, int which, hipStream_t s) = nullptr;
  void* user = nullptr;
};
// *nslots receives the number of statistics slots (row groups) written.
// variant (fused path): 0 diagonal, 1 isotropic, 2 isotropic with hard
// (k-means) assignment; 1 and 2 need iso_kernel_ok and launch_precompute_iso
hipError_t launch_estep(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                        bool fused, hipStream_t s, const LaunchHooks* hooks, int* nslots, int variant = 0);
bool iso_kernel_ok(const Plan& p, const Workspace& w, bool hard);
// split-bf16 kernel built for this shape: variant as launch_estep (split
// logits), or 3 + variant (split logits and statistics)
bool split_kernel_ok(const Plan& p, int variant);
hipError_t launch_kmeans_update(const Plan& p, const double* Nk, const double* S1, float* centres, double* counts,
                                hipStream_t s);
hipError_t launch_precompute_iso(const Plan& p, const Workspace& w, const float* means, const float* var_iso,
                                 hipStream_t s);
hipError_t launch_reduce(const Plan& p, const Workspace& w, double* Nk, double* S1, double* S2,
                         double* ll, int accumulate, int nslots, int nllslots, int64_t nrows,
                         hipStream_t s);

hipError_t launch_iso_expand(const Plan& p, const Workspace& w, const float* var_iso, hipStream_t s);
hipError_t launch_iso_q(const Plan& p, const double* S2, double* Q, int accumulate, hipStream_t s);
hipError_t launch_mstep_iso(const Plan& p, const Workspace& w, const double* Nk, const double* S1, const double* Q,
                            double n_total, float var_floor, float* weights, float* means, float* var_iso,
                            hipStream_t s);
hipError_t launch_init_iso(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                           float var_floor, float* weights, float* means, float* var_iso, hipStream_t s);
hipError_t launch_fill_zero(double* p, size_t n, hipStream_t s);
hipError_t launch_kmeans_params(const Plan& p, const Workspace& w, const float* centres, hipStream_t s);
hipError_t launch_centroids(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                            const int64_t* offsets, const int32_t* ids, float* centres, double* counts, int mode,
                            float var_floor, int iso, float* weights, float* means, float* vars, hipStream_t s);
hipError_t launch_colvar(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx, hipStream_t s);
hipError_t launch_mstep(const Plan& p, const Workspace& w, const double* Nk, const double* S1,
                        const double* S2, double n_total, float var_floor, float* weights,
                        float* means, float* vars, hipStream_t s);
hipError_t launch_init(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                       float var_floor, float* weights, float* means, float* vars, hipStream_t s);
// Soft assignment (gmm_assign.hip).  Pass A: select + count each chunk, then
// offsets; pass B: scatter each chunk's selections, selected again unless
// they were kept.  sel receives rows x (1 + max_extra) selections.
hipError_t assign_occupancy(const Plan& p, int* occ);
hipError_t launch_assign_begin(const Plan& p, const Workspace& w, hipStream_t s);
hipError_t launch_assign_select(const Plan& p, const Workspace& w, const float* X, int64_t row0, int64_t rows,
                                int64_t ldx, float threshold, int max_extra, bool count, int32_t* sel,
                                hipStream_t s);
hipError_t launch_assign_offsets(const Plan& p, const Workspace& w, int64_t* offsets, hipStream_t s);
hipError_t launch_assign_scatter(const Plan& p, const Workspace& w, const int32_t* sel, int64_t row0, int64_t rows,
                                 int max_extra, const int64_t* offsets, int32_t* ids, hipStream_t s);
// The lists from the selections of all rows at once (gmm_lists.hip): a stable
// radix sort of (list, row) pairs.  sort_lists_bytes: the buffer it needs for
// n = rows * stride selection slots (0 if the size query fails).
size_t sort_lists_bytes(int64_t n, int K);
hipError_t sort_lists(const int32_t* sel, int64_t rows, int stride, int K, int32_t* ids, int64_t nnz, void* buf,
                      size_t bytes, hipStream_t s);

}  // namespace gmm
