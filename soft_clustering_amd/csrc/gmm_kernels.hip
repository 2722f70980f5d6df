// HIP kernels for gfx950 (MI355X) of the fused diagonal-covariance GMM EM step.
//
// Method: "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
// Section 3.1 and Algorithm 1 (tile the rows, per-row online log-sum-exp over
// component blocks, responsibilities folded into sufficient statistics without
// storing the N x K responsibility matrix), Section 2 for the model and the
// M-step Eqs. (1)-(3).  The covariance here is diagonal.
//
// Design for CDNA4, not a port of the paper's Triton kernel:
//  * The logit contraction L[pt][comp] = sum_f A[pt][f] W[f][comp] + c[comp]
//    uses features A = [x^2 | x] and weights W = [-1/(2 s^2) | mu/s^2] (the
//    expanded quadratic).  By default it runs on the bfloat16 matrix units as
//    a split product (x = x_hi + x_lo, W likewise; three passes of
//    v_mfma_f32_16x16x32_bf16), and every logit that can carry
//    responsibility is recomputed in float64; v_mfma_f32_16x16x4_f32 and
//    v_mfma_f64_16x16x4_f64 variants exist for the other settings.  The
//    accumulator layout (lane = component, register = point) is exactly the
//    A-operand layout of the statistics contraction
//    S[comp][phi] += sum_pt r[comp][pt] F[pt][phi], F = [x^2 | x], so
//    responsibilities go from registers straight into the second MFMA
//    (three-part split bfloat16, six passes, or fp32).
//  * A workgroup owns 32*WC components and a strided set of row tiles; its
//    statistics stay in registers (fp32) and are flushed into a private
//    float64 slot every few tiles; a fixed-order pairwise tree over the slots
//    replaces the paper's atomic adds (Algorithm 1 step 17), so results are
//    bit-reproducible.
//  * The per-row normaliser log Z comes either from a first sweep over all
//    components (two-sweep, as Algorithm 1) or, in the fused path, from the P
//    workgroups that share a row tile exchanging their per-row partial
//    log-sum-exp through tagged 64-bit words in device memory (cooperative
//    launch guarantees they are co-resident), so each logit is computed once.
//  * X tiles are staged in LDS as raw float32 rows (a 4-float pad per row
//    keeps the 16 rows of an MFMA operand load on distinct banks), by LDS DMA
//    where rows need no padding; the split-bfloat16 operand tiles are built
//    from them in LDS once per tile and shared by every wave.
#include "gmm_device.h"

#include <math.h>
#include <stdlib.h>

namespace gmm {

// ---------------------------------------------------------------------------
// Cross-workgroup exchange of one per-row value among the P workgroups of a
// row group (fused path).  Each workgroup publishes its value of row pt as a
// 64-bit word (tile tag in the high half, the float in the low half) with an
// agent-scope atomic store, then gathers the P words of each row, spinning
// (bounded) until their tags match, and combines them in a fixed order: the
// maximum (LSE = false) or the log-sum-exp (LSE = true).  Two rounds per tile
// use separate slots, and slots alternate by tile parity.  A member publishes
// round rd of tile j only after it has gathered round rd of tile j-1 from
// every peer, and each peer publishes that word only after it has read its
// round rd words of tile j-2, so no member overwrites a word a slower member
// has not read yet.
template <int BN>
__device__ __forceinline__ void xpost(const EArgs& a, int rg, int p, int j, int rd, float v) {
  const int tid = threadIdx.x;  // < BN: row
  const unsigned tag = (unsigned)(j + 1);
  unsigned long long* xb = a.xbuf + ((size_t)((rg * 2 + rd) * 2 + (j & 1)) * a.P) * BN;
  const unsigned long long word = ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v);
  __hip_atomic_store(xb + (size_t)p * BN + tid, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BN, int QP, bool LSE>
__device__ __forceinline__ void xgather(const EArgs& a, int rg, int j, int rd, float (*exm)[BN], float (*exs)[BN],
                                        float* vout) {
  const int tid = threadIdx.x;
  const unsigned tag = (unsigned)(j + 1);
  const unsigned long long* xb = a.xbuf + ((size_t)((rg * 2 + rd) * 2 + (j & 1)) * a.P) * BN;
  // The 32-row tiles of the eight-wave (D > 128) kernels have many peers per
  // gathering lane: their words are loaded QB at a time, so the round trips
  // overlap; the 64-row kernels (few peers per lane, no registers to spare)
  // load one at a time.  Either way the words merge in ascending peer order.
  constexpr int QB = (BN <= 32) ? 8 : 1;
  if (tid < QP * BN) {
    const int pt = tid % BN, qp = tid / BN;
    float M = kNegInf, S = 0.f;
    // Bounded wait: a peer that never publishes (impossible while all
    // workgroups are co-resident) ends in flags[1] and a drained grid.
    auto settle = [&](const unsigned long long* src, unsigned long long word) {
      for (int spins = 0; (unsigned)(word >> 32) != tag; ++spins) {
        if ((spins & 255) == 0 && __hip_atomic_load(&a.flags[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
          break;
        if (spins > (1 << 20)) {
          __hip_atomic_store(&a.flags[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const float val = __uint_as_float((unsigned)(word & 0xffffffffu));
      if constexpr (LSE)
        lse_merge(M, S, val, 1.f);
      else
        M = fmaxf(M, val);
    };
    if constexpr (QB == 1) {
      for (int q = qp; q < a.P; q += QP) {
        const unsigned long long* src = xb + (size_t)q * BN + pt;
        settle(src, __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
    } else {
      for (int q0 = qp; q0 < a.P; q0 += QB * QP) {
        unsigned long long wv[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) {
          const int q = q0 + i * QP;
          wv[i] = (q < a.P) ? __hip_atomic_load(xb + (size_t)q * BN + pt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : ((unsigned long long)tag << 32);
        }
        // late words are polled again together (one round trip per poll for
        // the whole batch), with the bounded wait of settle
        for (int spins = 0;; ++spins) {
          unsigned miss = 0;
#pragma unroll
          for (int i = 0; i < QB; ++i) miss |= ((unsigned)(wv[i] >> 32) != tag ? 1u : 0u) << i;
          if (miss == 0) break;
          if ((spins & 255) == 0 && __hip_atomic_load(&a.flags[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
            break;
          if (spins > (1 << 20)) {
            __hip_atomic_store(&a.flags[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
#pragma unroll
          for (int i = 0; i < QB; ++i)
            if ((miss >> i) & 1u)
              wv[i] = __hip_atomic_load(xb + (size_t)(q0 + i * QP) * BN + pt, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < QB; ++i) {
          const int q = q0 + i * QP;
          if (q < a.P) settle(xb + (size_t)q * BN + pt, wv[i]);
        }
      }
    }
    exm[qp][pt] = M;
    exs[qp][pt] = S;
  }
  __syncthreads();
  if (tid < BN) {
    float M = kNegInf, S = 0.f;
#pragma unroll
    for (int k = 0; k < QP; ++k) {
      if constexpr (LSE)
        lse_merge(M, S, exm[k][tid], exs[k][tid]);
      else
        M = fmaxf(M, exm[k][tid]);
    }
    vout[tid] = LSE ? lse_of(M, S) : M;
  }
}

// Exchange of one (value, component) pair per row for the hard (argmax)
// mode: the word holds a 16-bit tile tag (tiles mod 65535, plus 1, so the
// tile two back on the same slot differs), the 16-bit component and the
// float; the gather keeps the largest value, the lowest component on ties.
template <int BN, int QP>
__device__ __forceinline__ void row_exchange_arg(const EArgs& a, int rg, int p, int j, const float* vin,
                                                 const int* kin, float (*exm)[BN], int (*exk)[BN], float* vout,
                                                 int* kout) {
  const int tid = threadIdx.x;
  const unsigned long long tag = (unsigned long long)((unsigned)j % 65535u + 1u);
  unsigned long long* xb = a.xbuf + ((size_t)((rg * 2 + 1) * 2 + (j & 1)) * a.P) * BN;
  if (tid < BN) {
    const unsigned long long word = (tag << 48) | ((unsigned long long)(kin[tid] & 0xFFFF) << 32) |
                                    (unsigned long long)__float_as_uint(vin[tid]);
    __hip_atomic_store(xb + (size_t)p * BN + tid, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < QP * BN) {
    const int pt = tid % BN, qp = tid / BN;
    float M = kNegInf;
    int Kb = 0x7fffffff;
    for (int q = qp; q < a.P; q += QP) {
      const unsigned long long* src = xb + (size_t)q * BN + pt;
      unsigned long long word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int spins = 0; (word >> 48) != tag; ++spins) {  // bounded wait, as in xgather
        if ((spins & 255) == 0 && __hip_atomic_load(&a.flags[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
          break;
        if (spins > (1 << 20)) {
          __hip_atomic_store(&a.flags[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const float val = __uint_as_float((unsigned)(word & 0xffffffffu));
      const int kk = (int)((word >> 32) & 0xFFFF);
      if (val > M || (val == M && kk < Kb)) {
        M = val;
        Kb = kk;
      }
    }
    exm[qp][pt] = M;
    exk[qp][pt] = Kb;
  }
  __syncthreads();
  if (tid < BN) {
    float M = kNegInf;
    int Kb = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < QP; ++k)
      if (exm[k][tid] > M || (exm[k][tid] == M && exk[k][tid] < Kb)) {
        M = exm[k][tid];
        Kb = exk[k][tid];
      }
    vout[tid] = M;
    kout[tid] = Kb;
  }
}

template <int BN, int QP, bool LSE>
__device__ __forceinline__ void row_exchange(const EArgs& a, int rg, int p, int j, int rd, const float* vin,
                                             float (*exm)[BN], float (*exs)[BN], float* vout) {
  if (threadIdx.x < BN) xpost<BN>(a, rg, p, j, rd, vin[threadIdx.x]);
  xgather<BN, QP, LSE>(a, rg, j, rd, exm, exs, vout);
}

// ---------------------------------------------------------------------------
// E-step statistics sweep.  FUSED: per-row log Z by exchange; else from a.logz.
// ISO: the isotropic model (Sigma_k = s_k^2 I) with its own contractions:
// logits x . mu_k / s_k^2 over D features (minus ||x||^2 / (2 s_k^2) added per
// row and component), statistics r^T x over D features, Q_k = sum r ||x||^2
// accumulated like N_k; S1 lands in the slots' x positions, Q in the x^2
// position of dim 0 and zeros in the other x^2 positions, so the diagonal
// reduction yields N_k, S1 and Q = sum_d S2_kd.
//
// HARD (with ISO): the k-means step.  Responsibilities are one-hot at the
// row's largest logit (lowest component on ties) instead of the softmax: the
// refinement threshold is the row's largest lower bound itself (every
// component that can be the argmax is recomputed in float64, then compared
// as float32: the float64 order except within one float32 ulp), the second
// exchange round carries (max, argmax) pairs, and no log-likelihood is
// accumulated.  With equal weights and variances 1/2 the largest logit is the
// nearest centre.
template <int WC, int WD, int DPW, int BN, bool FUSED, int MODE, bool ISO = false, bool HARD = false,
          int SPLIT = 0>
__global__ void __launch_bounds__(kWave* WC* WD, (WC * WD == 4) ? 2 : 1) k_stats(EArgs a) {
  using SH = Shape<WC, WD, DPW, BN>;
  constexpr bool REFINE = MODE == MODE_REFINE, F64 = MODE == MODE_FP64;
  static_assert(!ISO || (FUSED && WD == 1 && !F64), "isotropic kernel: fused path, WD = 1, float32 logits");
  static_assert(!HARD || ISO, "hard assignment: isotropic kernel");
  static_assert(!SPLIT || (FUSED && REFINE && WD == 1), "split-bf16 logits: fused refined kernels, WD = 1");
  static_assert(!SPLIT || !ISO || DPW >= 32, "isotropic split logits: 8 dims per lane group and step");
  using SPR = SplitRow<DPW, ISO>;
  // SPLIT 2: the statistics contraction split too (three-part bf16 operands
  // in LDS); its operands share the region of the logit operands, and the
  // raw tile is single-buffered to make room (the next tile streams in
  // behind the statistics phase instead of behind the whole tile)
  static_assert(SPLIT < 2 || BN % 32 == 0, "split statistics: 32-row pairs");
  using SST = StatSplit<SH, DPW, ISO>;
  // SEG: the float64-logit fused kernel with dim-segment waves keeps the tile
  // segment-major (wave wd's dims of all rows in a block of its own, rows SRS
  // floats apart), since in that kernel a wave reads only its own dims: each
  // wave stages its next block right after its own statistics, with no
  // workgroup barrier between tiles
  constexpr bool SEG = F64 && FUSED && WD > 1;
  constexpr int SRS = SEG ? DPW + 4 : SH::RS;  // LDS floats between a wave's rows
  constexpr int TILEX = SEG ? WD * BN * SRS : SH::TILE;
  constexpr int NB = (SPLIT == 2 || SEG) ? 1 : SH::NBUF;
  constexpr int XSB = (SPLIT == 0) ? 8
                      : (SPLIT == 2 && SST::SIZE > BN * SPR::XSR) ? SST::SIZE : BN * SPR::XSR;
  static_assert(!SPLIT || SH::CPR <= kWave, "split rows follow the one-instruction-per-row DMA assignment");
  constexpr int NPB = SH::NPB;
  constexpr int NFB = ISO ? DPW / 16 : SH::NFB;  // statistics feature blocks
  // row reductions on integer keys except in the soft isotropic kernel
  // (measured faster there with float maxima)
  constexpr bool IK = !ISO || HARD;
  constexpr int FLUSH = 2048 / BN;  // tiles between fp64 flushes (2048 rows)
  // row groups flush at staggered tiles, so the float64 atomics of the grid
  // do not all reach L2 at once; the members of a row group flush together
  // (a flush delays the member's next exchange word, so staggering within a
  // row group would hold the whole group up once per member)
  constexpr int QP = (SH::NT / BN) > 0 ? (SH::NT / BN) : 1;

  __shared__ __attribute__((aligned(16))) float xt[NB][TILEX];
  __shared__ __attribute__((aligned(16))) float red[F64 ? 1 : SH::RED];
  __shared__ double red64[F64 ? SH::RED : 1];
  __shared__ __attribute__((aligned(16))) float lzt[BN];
  __shared__ float lpart[WC][BN];
  __shared__ float exm[QP][BN], exs[QP][BN];
  __shared__ double llred[BN];
  __shared__ float2 nrm[BN];
  __shared__ __attribute__((aligned(16))) float thrs[BN];
  __shared__ float vtmp[BN];
  __shared__ float rlist[SH::COOP ? WC : WC * WD][kRefineCap];  // refinement lists (per group or wave)
  __shared__ unsigned short elist[SH::COOP ? WC : WC * WD][kRefineCap];
  // the diagonal split-statistics kernel pools the refinement lists of its
  // waves into one (rlist / elist as one array of WC * kRefineCap entries)
  constexpr bool POOL = SPLIT == 2 && !ISO && REFINE && FUSED && WD == 1;
  __shared__ int wtot[POOL ? WC + 1 : 1];
  __shared__ __attribute__((aligned(16))) float xn2[ISO ? BN : 4];  // ISO: ||x||^2 of the tile's rows
  __shared__ int lidx[HARD ? WC : 1][BN];                             // HARD: per-wave argmax
  __shared__ int exk[HARD ? QP : 1][BN];
  __shared__ int garg[HARD ? BN : 1];                                 // HARD: the row's argmax
  __shared__ __attribute__((aligned(16))) __bf16 xsb[XSB];  // split operands

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wc = w % WC, wd = w / WC;
  const int g = lane >> 4, r16 = lane & 15;
  const int G = a.R * a.P;
  int rg, p;
  rg_member(G, a.P, rg, p);
  const int fphase = rg % FLUSH;  // flush stagger, by row group
  const int compbase = p * 32 * WC + wc * 32;  // first component of this wave
  const int cb16 = compbase >> 4;
  const float* w0 = ISO ? a.wiso + (size_t)cb16 * DPW * 16 : wop_block(a.wop, cb16, WD, wd, DPW);
  const float* w1 = ISO ? a.wiso + (size_t)(cb16 + 1) * DPW * 16 : wop_block(a.wop, cb16 + 1, WD, wd, DPW);
  const __bf16* ws0 = SPLIT ? a.wsp + (size_t)cb16 * SPR::WBLK : nullptr;
  const __bf16* ws1 = SPLIT ? a.wsp + (size_t)(cb16 + 1) * SPR::WBLK : nullptr;
  const float iv0 = ISO ? a.ivec[compbase + r16] : 0.f;  // 1 / (2 s^2) of the lane's components
  const float iv1 = ISO ? a.ivec[compbase + 16 + r16] : 0.f;
  float q0 = 0.f, q1 = 0.f;                              // ISO: Q partials
  const float c0 = (wd == 0) ? a.cvec[compbase + r16] : 0.f;
  const float c1 = (wd == 0) ? a.cvec[compbase + 16 + r16] : 0.f;
  const double C = *a.cshift;
  float co[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const double* w0d = F64 ? wop_block(a.wop64, cb16, WD, wd, DPW) : nullptr;
  const double* w1d = F64 ? wop_block(a.wop64, cb16 + 1, WD, wd, DPW) : nullptr;
  const double c0d = (F64 && wd == 0) ? a.cvec64[compbase + r16] : 0.0;
  const double c1d = (F64 && wd == 0) ? a.cvec64[compbase + 16 + r16] : 0.0;
  if constexpr (REFINE) lane_coefs(a, compbase, r16, co);
  unsigned nsel = 0;  // refined logits of this wave (counted once at the end)

  const int nt = (int)((a.nrows + BN - 1) / BN);
  f4 sacc[2][NFB];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) sacc[cb][fb] = f4{0.f, 0.f, 0.f, 0.f};
  float nk0 = 0.f, nk1 = 0.f;
  double ll = 0.0;
  bool fresh = (a.slot_acc == 0);
  double* sbase = a.slots + ((size_t)rg * a.Kpad + compbase) * (2 * a.Dp + 1);
  const int SR = 2 * a.Dp + 1;

  // fp32 tile partials -> this workgroup's float64 slot.  Every slot word is
  // written by exactly one lane of one workgroup, so fire-and-forget float64
  // atomic adds (performed in program order per address) stay deterministic.
  auto put = [&](double* ptr, double val) {
    if (fresh)
      __hip_atomic_store(ptr, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_fetch_add(ptr, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto flush = [&]() {
    // slot feature index of x (sq = false) or x^2 (sq = true) of dim d of the
    // wave's segment: quarters of HALF dims alternate x^2, x
    auto fpos = [&](int d, bool sq) { return (2 * (d / SH::HALF) + (sq ? 0 : 1)) * SH::HALF + d % SH::HALF; };
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          double* row = sbase + (size_t)(cb * 16 + 4 * g + v) * SR + wd * 2 * DPW;
          if constexpr (ISO) {
            const int d = fb * 16 + r16;
            put(row + fpos(d, false), (double)sacc[cb][fb][v]);
            if (fresh && d > 0) put(row + fpos(d, true), 0.0);
          } else {
            put(row + fb * 16 + r16, (double)sacc[cb][fb][v]);
          }
        }
        sacc[cb][fb] = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float t0 = nk0 + __shfl_xor(nk0, 16);
    t0 += __shfl_xor(t0, 32);
    float t1 = nk1 + __shfl_xor(nk1, 16);
    t1 += __shfl_xor(t1, 32);
    if (wd == 0 && g == 0) {
      put(sbase + (size_t)r16 * SR + 2 * a.Dp, (double)t0);
      put(sbase + (size_t)(16 + r16) * SR + 2 * a.Dp, (double)t1);
    }
    if constexpr (ISO) {
      float u0 = q0 + __shfl_xor(q0, 16);
      u0 += __shfl_xor(u0, 32);
      float u1 = q1 + __shfl_xor(q1, 16);
      u1 += __shfl_xor(u1, 32);
      if (g == 0) {
        put(sbase + (size_t)r16 * SR + fpos(0, true), (double)u0);
        put(sbase + (size_t)(16 + r16) * SR + fpos(0, true), (double)u1);
      }
      q0 = q1 = 0.f;
    }
    nk0 = nk1 = 0.f;
    fresh = false;
  };

  // X tiles: by LDS DMA where rows need no zero padding (the next tile then
  // streams in behind this tile's work), else through registers between
  // tiles (holding a prefetch across the statistics would cost registers)
  auto stage_now = [&](float* buf, int tile) {
    const int64_t r0 = (int64_t)tile * BN;
    const int rws = (int)min((int64_t)BN, a.nrows - r0);
    if constexpr (SEG) {
      stage_seg<DPW, BN>(buf + wd * BN * SRS, a.X, a.ldx, a.row0 + r0, rws, a.D, wd, a.dma != 0);
      if (a.dma) dma_wait();
    } else if (a.dma) {
      stage_dma<SH>(buf, a.X, a.ldx, a.row0 + r0, rws);
      dma_wait();
    } else {
      Stage<SH, DPW> stg;
      stg.load(a.X, a.ldx, a.row0 + r0, rws, a.D);
      stg.store(buf);
    }
  };
  // split operands of a freshly staged tile: each wave converts the rows its
  // own DMA brought in (register staging: after a barrier, the same rows)
  // the diagonal split-statistics kernel forms the rows' norms there too
  constexpr bool NORMS_IN_SPLIT = SPLIT == 2 && !ISO && REFINE && DPW == 128;
  auto split_now = [&](const float* buf) {
    if constexpr (SPLIT) {
      if (!a.dma) __syncthreads();
      split_rows<SH, DPW, ISO>(buf, xsb, w, NORMS_IN_SPLIT ? nrm : nullptr);
    }
  };
  int j = 0;
  int t = rg;
  if (t < nt) {
    stage_now(xt[0], t);
    split_now(xt[0]);
  }
  __syncthreads();
  for (; t < nt; t += a.R, ++j) {
    const int cur = (NB == 2) ? (j & 1) : 0;
    const int64_t trow = (int64_t)t * BN;
    const int rows = (int)min((int64_t)BN, a.nrows - trow);
    const int tn = t + a.R;
    const bool has_next = tn < nt;
    const bool async_next = (NB == 2) && has_next && a.dma;
    if (async_next)  // the other buffer was released by the last end-of-tile barrier
      stage_dma<SH>(xt[cur ^ 1], a.X, a.ldx, a.row0 + (int64_t)tn * BN,
                    (int)min((int64_t)BN, a.nrows - (int64_t)tn * BN));
    // ---- logits
    f4 acc[NPB][2];
    if constexpr (F64) {
      logits_f64<SH, WC, WD, DPW, SRS>(xt[cur] + (SEG ? wd * BN * SRS : wd * DPW), w0d, w1d, c0d, c1d, acc, red64,
                                       lane, wc, wd);
    } else {
      // diagonal kernel with split statistics: the per-lane constants are
      // reloaded each tile (through an index the compiler cannot hoist), so
      // they are not live across the whole tile; that takes 10 VGPRs off its
      // spills (4.5 % faster; the isotropic kernel is better without)
      constexpr bool RELOAD = SPLIT == 2 && !ISO;
      float c0t = c0, c1t = c1;
      if constexpr (RELOAD) {
        int kk = compbase + r16;
        asm volatile("" : "+v"(kk));
        c0t = (wd == 0) ? a.cvec[kk] : 0.f;
        c1t = (wd == 0) ? a.cvec[kk + 16] : 0.f;
      }
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        acc[pb][0] = f4{c0t, c0t, c0t, c0t};
        acc[pb][1] = f4{c1t, c1t, c1t, c1t};
      }
      if constexpr (ISO) {
        row_norms_iso<SH, DPW>(xt[cur], nrm, xn2);
        if constexpr (SPLIT) logit_tile_split<SH, DPW, true>(xsb, ws0, ws1, acc, lane);
        else logit_tile_iso<SH, DPW>(xt[cur], w0, w1, acc, lane);
        __syncthreads();  // xn2
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
          const f4 n4 = *reinterpret_cast<const f4*>(xn2 + pb * 16 + 4 * g);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[pb][0][v] = fmaf(-iv0, n4[v], acc[pb][0][v]);
            acc[pb][1][v] = fmaf(-iv1, n4[v], acc[pb][1][v]);
          }
        }
      } else if constexpr (SPLIT) {
        logit_tile_split<SH, DPW, false>(xsb, ws0, ws1, acc, lane);
      } else {
        logit_tile<SH, DPW>(xt[cur], w0, w1, acc, lane, wd);
        reduce_partial_logits<SH, WC, WD>(red, acc, lane, wc, wd);
      }
    }

    // ---- float64 refinement of the logits that can matter
    if constexpr (REFINE && SPLIT == 2 && !ISO) {  // per-tile reload, as c0 / c1 above
      int cbo = compbase;
      asm volatile("" : "+v"(cbo));
      lane_coefs(a, cbo, r16, co);
    }
    if constexpr (REFINE) {
      if constexpr (!ISO && !NORMS_IN_SPLIT) {
        row_norms2<SH, DPW>(xt[cur], nrm, a.Dp);
        __syncthreads();
      }
      if constexpr (FUSED) {
        // round 1 of the exchange: each workgroup's largest lower bound
        // L - E of the row's logits; their maximum bounds the row's largest
        // true logit from below, for every workgroup of the row group alike
        if (wd == 0) {
#pragma unroll
          for (int pb = 0; pb < NPB; ++pb) {
            float m4[4];  // four rows, stored together
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float2 nn = nrm[pb * 16 + 4 * g + v];
              const float lb = max2(acc[pb][0][v] - err_bound(a.kappa, co[0], co[1], co[2], nn),
                                    acc[pb][1][v] - err_bound(a.kappa, co[3], co[4], co[5], nn));
              m4[v] = row16_max<IK, false>(lb);
            }
            if (r16 == 0)
#pragma unroll
              for (int v = 0; v < 4; ++v) lpart[wc][pb * 16 + 4 * g + v] = m4[v];
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __syncthreads();
        if (tid < BN) {
          float m = kNegInf;
#pragma unroll
          for (int k = 0; k < WC; ++k) m = fmaxf(m, lpart[k][tid]);
          vtmp[tid] = m;
        }
        if constexpr (SPLIT == 2) {
          // the statistics operands are built while the peers' words travel
          // (every wave is past the logits, so the region is free)
          if (tid < BN) xpost<BN>(a, rg, p, j, 0, vtmp[tid]);
          split_stats<SH, DPW, ISO>(xt[cur], xsb);
          xgather<BN, QP, false>(a, rg, j, 0, exm, exs, thrs);
        } else {
          row_exchange<BN, QP, false>(a, rg, p, j, 0, vtmp, exm, exs, thrs);
        }
        if (tid < BN) thrs[tid] = (tid < rows) ? thrs[tid] - (HARD ? 0.f : kDelta) : kPosInf;
      } else {
        // reference: the row's final log Z from the first sweep
        if (tid < BN) thrs[tid] = ((tid < rows) ? a.logz[trow + tid] : kPosInf) - kDelta;
      }
      __syncthreads();
      if constexpr (POOL)
        refine_pooled<SH, DPW>(acc, thrs, nrm, co, xt[cur], rows, a, C, p * 32 * WC, compbase, &rlist[0][0],
                               &elist[0][0], wtot, WC * WD * kRefineCap, lane, w, nsel);
      else
        refine_tile<SH, WD, DPW>(acc, thrs, nrm, co, xt[cur], rows, a, C, compbase, rlist[SH::COOP ? wc : w],
                                 elist[SH::COOP ? wc : w], lane, wd, nsel);
    }

    // ---- per-row log Z (HARD: the row's argmax)
    if constexpr (HARD) {
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float m = row16_max<IK>(max2(acc[pb][0][v], acc[pb][1][v]));
          // lowest lane of the DPP row holding m, block 0 before block 1
          const float i0 = row16_min<IK>((acc[pb][0][v] == m) ? (float)r16 : 64.f);
          const float i1 = row16_min<IK>((acc[pb][1][v] == m) ? (float)r16 : 64.f);
          if (r16 == 0) {
            lpart[wc][pb * 16 + 4 * g + v] = m;
            lidx[wc][pb * 16 + 4 * g + v] = compbase + (i0 < 16.f ? (int)i0 : (i1 < 16.f ? 16 + (int)i1 : 0));
          }
        }
      __syncthreads();
      if (tid < BN) {
        float M = lpart[0][tid];
        int Kb = lidx[0][tid];
#pragma unroll
        for (int k = 1; k < WC; ++k)
          if (lpart[k][tid] > M) {
            M = lpart[k][tid];
            Kb = lidx[k][tid];
          }
        vtmp[tid] = M;
        garg[tid] = Kb;
      }
      row_exchange_arg<BN, QP>(a, rg, p, j, vtmp, garg, exm, exk, lzt, garg);
      if (tid < BN && tid >= rows) garg[tid] = -1;
    } else if constexpr (FUSED) {
      if (wd == 0) {
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
          // four rows at a time, stored together (one branch per four rows,
          // and the four reductions can interleave)
          float l4[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float m = row16_max<IK, false>(max2(acc[pb][0][v], acc[pb][1][v]));
            // m = -inf (a row of -inf logits) gives ms = -FLT_MAX, e = 0 and -inf
            const float ms = max2(m, -3.40282347e38f);
            float e = __expf(acc[pb][0][v] - ms) + __expf(acc[pb][1][v] - ms);
            e = row16_sum(e);
            l4[v] = ms + ln_rowsum(e);  // e >= 1, or 0 for a row of -inf
          }
          if (r16 == 0)
#pragma unroll
            for (int v = 0; v < 4; ++v) lpart[wc][pb * 16 + 4 * g + v] = l4[v];
        }
      }
      __syncthreads();
      if (tid < BN) {
        float M = kNegInf, S = 0.f;
#pragma unroll
        for (int k = 0; k < WC; ++k) lse_merge(M, S, lpart[k][tid], 1.f);
        vtmp[tid] = lse_of(M, S);
      }
      row_exchange<BN, QP, true>(a, rg, p, j, 1, vtmp, exm, exs, lzt);
      if (tid < BN) {
        const float lz = lzt[tid];
        if (p == 0 && tid < rows) ll += (double)lz;
        if (tid >= rows) lzt[tid] = kPosInf;
      }
    } else {
      if (tid < BN) lzt[tid] = (tid < rows) ? a.logz[trow + tid] : kPosInf;
    }
    __syncthreads();
    if constexpr (SPLIT == 2) {
      // nothing reads the raw tile any more: the next one streams in behind
      // the statistics
      if (has_next && a.dma)
        stage_dma<SH>(xt[0], a.X, a.ldx, a.row0 + (int64_t)tn * BN, (int)min((int64_t)BN, a.nrows - (int64_t)tn * BN));
    }

    // ---- responsibilities and statistics: r goes from the logit
    // accumulators straight into the A operand; B operands are this lane's
    // feature of the step's point (x^2 formed here), loaded one step ahead.
    // Feature f of the segment: quarter q = f / HALF holds x^2 (q even) or x
    // of dims (q / 2) * HALF + f % HALF.
    // lane (g, r16) feeds feature f = fb * 16 + r16 of its segment for point
    // 4g + v of each 16-point block: offsets from xs are compile-time except
    // for DPW = 16, whose 8-dim halves split a 16-lane block
    constexpr bool NARROW = !ISO && SH::HALF < 16;
    const float* xs = xt[cur] + (SEG ? wd * BN * SRS : wd * DPW) + (NARROW ? (r16 & 7) : r16) + 4 * g * SRS;
    auto fdim = [&](int fb) {  // dim offset of feature block fb (minus the lane part)
      if constexpr (ISO) return fb * 16;
      else if constexpr (NARROW) return fb * 8;
      else return ((fb * 16 / SH::HALF) >> 1) * SH::HALF + (fb * 16) % SH::HALF;
    };
    auto fsq = [&](int fb) {  // x^2 feature?
      if constexpr (ISO) return false;
      else if constexpr (NARROW) return r16 < 8;
      else return ((fb * 16 / SH::HALF) & 1) == 0;
    };
    auto bload = [&](int fb, int pt) {
      const float x = xs[pt * SRS + fdim(fb)];
      return fsq(fb) ? x * x : x;
    };
    // responsibilities in place (the logits are not needed afterwards), so
    // the MFMA loop below issues no transcendental work
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      const f4 lz = *reinterpret_cast<const f4*>(lzt + pb * 16 + 4 * g);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if constexpr (HARD) {
          const int k = garg[pb * 16 + 4 * g + v];
          acc[pb][0][v] = (compbase + r16 == k) ? 1.f : 0.f;
          acc[pb][1][v] = (compbase + 16 + r16 == k) ? 1.f : 0.f;
        } else {
          acc[pb][0][v] = __expf(acc[pb][0][v] - lz[v]);
          acc[pb][1][v] = __expf(acc[pb][1][v] - lz[v]);
        }
        nk0 += acc[pb][0][v];
        nk1 += acc[pb][1][v];
      }
      if constexpr (ISO) {
        const f4 n4 = *reinterpret_cast<const f4*>(xn2 + pb * 16 + 4 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          q0 = fmaf(acc[pb][0][v], n4[v], q0);
          q1 = fmaf(acc[pb][1][v], n4[v], q1);
        }
      }
    }
    if constexpr (SPLIT == 2) {
      stats_tile_split<SH, DPW, ISO, HARD>(acc, xsb, sacc, lane);
    } else {
    // one B operand per feature block: each is reloaded for the next point
    // step right after its two MFMAs have read it
    float bx[NFB];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) bx[fb] = bload(fb, 0);
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int step = pb * 4 + v;
        const int np = (step + 1) >> 2, nv = (step + 1) & 3;
        const int ptn = np * 16 + nv;  // relative to the lane's 4g
        const float r0 = acc[pb][0][v];
        const float r1 = acc[pb][1][v];
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
          sacc[0][fb] = mfma(r0, bx[fb], sacc[0][fb]);
          sacc[1][fb] = mfma(r1, bx[fb], sacc[1][fb]);
          if (step + 1 < NPB * 4) bx[fb] = bload(fb, ptn);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    }
    if constexpr (SPLIT == 2) {
      if (has_next) {
        if (a.dma) dma_wait();
        else stage_now(xt[0], tn);  // every read of the raw tile preceded the statistics
      }
      if ((j + 1 + fphase) % FLUSH == 0) flush();
      __syncthreads();  // statistics operands released, next rows visible
      if (has_next) {
        split_rows<SH, DPW, ISO>(xt[0], xsb, w, NORMS_IN_SPLIT ? nrm : nullptr);
        __syncthreads();
      }
      continue;
    }
    if constexpr (SEG) {
      // the wave's own block is free once its own statistics are issued (their
      // operand reads have returned); no other wave reads it.  Every LDS word
      // other waves share is next written behind a barrier of the next tile
      // that this wave only reaches after its statistics.
      if (has_next) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block's reads have returned
        __builtin_amdgcn_sched_barrier(0);
        stage_now(xt[0], tn);
      }
      if ((j + 1 + fphase) % FLUSH == 0) flush();
      continue;
    }
    if (has_next) {
      if (async_next) {
        dma_wait();  // this wave's share of the next tile has landed
      } else {
        if constexpr (NB == 1) __syncthreads();  // every wave is done with the buffer
        stage_now(xt[(NB == 2) ? (cur ^ 1) : 0], tn);
      }
      // every wave finished this tile's logits (barriers since), so the
      // split operands can be overwritten
      split_now(xt[(NB == 2) ? (cur ^ 1) : 0]);
    }
    if ((j + 1 + fphase) % FLUSH == 0) flush();
    __syncthreads();
  }
  if (j == 0 || ((j + fphase) % FLUSH) != 0) flush();
  if constexpr (REFINE) count_refined(a, nsel);

  if constexpr (FUSED) {
    if (p == 0) {
      if (tid < BN) llred[tid] = ll;
      __syncthreads();
      for (int s = BN / 2; s > 0; s >>= 1) {
        if (tid < s) llred[tid] += llred[tid + s];
        __syncthreads();
      }
      if (tid == 0) a.llslots[rg] = a.slot_acc ? a.llslots[rg] + llred[0] : llred[0];
    }
  }
}

// ---------------------------------------------------------------------------
// First sweep of the two-sweep path: log Z of every row of the chunk, over all
// components (Algorithm 1 steps 6-10), plus a float64 log-likelihood partial
// per workgroup.
template <int WC, int WD, int DPW, int BN, int MODE>
__global__ void __launch_bounds__(kWave* WC* WD, (WC * WD == 4) ? 2 : 1) k_logz(EArgs a) {
  using SH = Shape<WC, WD, DPW, BN>;
  constexpr bool REFINE = MODE == MODE_REFINE, F64 = MODE == MODE_FP64;
  constexpr int NPB = SH::NPB;
  __shared__ __attribute__((aligned(16))) float xt[SH::TILE];
  __shared__ __attribute__((aligned(16))) float red[F64 ? 1 : SH::RED];
  __shared__ double red64[F64 ? SH::RED : 1];
  __shared__ float lpart[WC][BN];
  __shared__ double llred[BN];
  __shared__ float2 nrm[BN];
  __shared__ __attribute__((aligned(16))) float thrw[WC][BN];
  __shared__ float rlist[SH::COOP ? WC : WC * WD][kRefineCap];  // refinement lists (per group or wave)
  __shared__ unsigned short elist[SH::COOP ? WC : WC * WD][kRefineCap];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wc = w % WC, wd = w / WC;
  const int g = lane >> 4, r16 = lane & 15;
  const int ncg = a.Kpad / 32;
  const double C = *a.cshift;
  const int nt = (int)((a.nrows + BN - 1) / BN);
  double ll = 0.0;
  unsigned nsel = 0;  // refined logits of this wave (counted once at the end)

  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const int64_t trow = (int64_t)t * BN;
    const int rows = (int)min((int64_t)BN, a.nrows - trow);
    if (a.dma) {
      stage_dma<SH>(xt, a.X, a.ldx, a.row0 + trow, rows);
      dma_wait();
    } else {
      Stage<SH, DPW> stg;
      stg.load(a.X, a.ldx, a.row0 + trow, rows, a.D);
      stg.store(xt);
    }
    __syncthreads();
    if constexpr (REFINE) {
      row_norms2<SH, DPW>(xt, nrm, a.Dp);
      __syncthreads();
    }
    float M[NPB][4], S[NPB][4], Rlb[NPB][4];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        M[pb][v] = kNegInf;
        S[pb][v] = 0.f;
        Rlb[pb][v] = kNegInf;
      }
    for (int cg = wc; cg < ncg; cg += WC) {
      const int compbase = cg * 32;
      f4 acc[NPB][2];
      if constexpr (F64) {
        logits_f64<SH, WC, WD, DPW>(xt + wd * DPW, wop_block(a.wop64, compbase >> 4, WD, wd, DPW),
                                    wop_block(a.wop64, (compbase >> 4) + 1, WD, wd, DPW),
                                    wd == 0 ? a.cvec64[compbase + r16] : 0.0,
                                    wd == 0 ? a.cvec64[compbase + 16 + r16] : 0.0, acc, red64, lane, wc, wd);
      } else {
        const float c0 = (wd == 0) ? a.cvec[compbase + r16] : 0.f;
        const float c1 = (wd == 0) ? a.cvec[compbase + 16 + r16] : 0.f;
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
          acc[pb][0] = f4{c0, c0, c0, c0};
          acc[pb][1] = f4{c1, c1, c1, c1};
        }
        logit_tile<SH, DPW>(xt, wop_block(a.wop, compbase >> 4, WD, wd, DPW),
                            wop_block(a.wop, (compbase >> 4) + 1, WD, wd, DPW), acc, lane, wd);
        reduce_partial_logits<SH, WC, WD>(red, acc, lane, wc, wd);
      }
      if constexpr (REFINE) {
        // reference: running max over the components seen so far of the
        // guaranteed lower bounds L - E (it only grows, so a logit left
        // unrefined stays more than kDelta below the row's final maximum)
        float co[6];
        lane_coefs(a, compbase, r16, co);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float2 nn = nrm[pb * 16 + 4 * g + v];
            const float lb = max2(acc[pb][0][v] - err_bound(a.kappa, co[0], co[1], co[2], nn),
                                  acc[pb][1][v] - err_bound(a.kappa, co[3], co[4], co[5], nn));
            Rlb[pb][v] = fmaxf(Rlb[pb][v], row16_max(lb));
            if (r16 == 0 && wd == 0) thrw[wc][pb * 16 + 4 * g + v] = Rlb[pb][v] - kDelta;
          }
        if constexpr (WD > 1) __syncthreads();
        else { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); __builtin_amdgcn_wave_barrier(); }
        refine_tile<SH, WD, DPW>(acc, thrw[wc], nrm, co, xt, rows, a, C, compbase, rlist[SH::COOP ? wc : w], elist[SH::COOP ? wc : w], lane,
                                 wd, nsel);
      }
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float mn = max2(M[pb][v], max2(acc[pb][0][v], acc[pb][1][v]));
          const float ms = (mn == kNegInf) ? 0.f : mn;
          S[pb][v] = S[pb][v] * __expf(M[pb][v] - ms) + __expf(acc[pb][0][v] - ms) +
                     __expf(acc[pb][1][v] - ms);
          M[pb][v] = mn;
        }
    }
    if (wd == 0) {
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float mr = row16_max(M[pb][v]);
          const float ms = (mr == kNegInf) ? 0.f : mr;
          const float s = row16_sum(S[pb][v] * __expf(M[pb][v] - ms));
          if (r16 == 0) lpart[wc][pb * 16 + 4 * g + v] = ms + ln_rowsum(s);  // s >= 1, or 0
        }
    }
    __syncthreads();
    if (tid < rows) {
      float Mx = kNegInf, Sx = 0.f;
#pragma unroll
      for (int k = 0; k < WC; ++k) lse_merge(Mx, Sx, lpart[k][tid], 1.f);
      const float lz = lse_of(Mx, Sx);
      a.logz[trow + tid] = lz;
      ll += (double)lz;
    }
    __syncthreads();
  }
  if constexpr (REFINE) count_refined(a, nsel);
  if (tid < BN) llred[tid] = ll;
  __syncthreads();
  for (int s = BN / 2; s > 0; s >>= 1) {
    if (tid < s) llred[tid] += llred[tid + s];
    __syncthreads();
  }
  if (tid == 0) a.llslots[blockIdx.x] = a.slot_acc ? a.llslots[blockIdx.x] + llred[0] : llred[0];
}

// ---------------------------------------------------------------------------
// Parameters -> MFMA operands (Algorithm 1 step 8's log z, expanded).
//   a_kd = -1/(2 s^2_kd), b_kd = mu_kd / s^2_kd,
//   c_k  = log pi_k - 1/2 sum_d mu^2/s^2 - 1/2 sum_d log s^2 - D/2 log 2pi,
// computed in float64, stored float32; padding components get c = -inf.
template <class T>
__global__ void k_precompute_w(const float* __restrict__ mu, const float* __restrict__ var, T* wop,
                               int K, int D, int Kpad, int WD, int DPW) {
  const size_t total = (size_t)Kpad * 2 * WD * DPW;
  const int per_cb = WD * (DPW / 8) * 256;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int cb = (int)(idx / per_cb);
    int rem = (int)(idx - (size_t)cb * per_cb);
    const int wd = rem / ((DPW / 8) * 256);
    rem -= wd * (DPW / 8) * 256;
    const int s4 = rem / 256;
    rem -= s4 * 256;
    const int lane = rem >> 2, i = rem & 3;
    const int gg = lane >> 4;
    const int comp = cb * 16 + (lane & 15);
    const int dim = wd * DPW + (gg >> 1) * (DPW / 2) + s4 * 4 + i;
    double val = 0.0;
    if (comp < K && dim < D) {
      const double s2 = (double)var[(size_t)comp * D + dim];
      val = (gg & 1) ? (double)mu[(size_t)comp * D + dim] / s2 : -0.5 / s2;
    }
    wop[idx] = (T)val;
  }
}

// The same [a | b] as split bfloat16 pairs (WD = 1) for logit_tile_split:
// per 16-component block, [step][hi, lo][lane][8]; lane (g, r16) of step st
// holds component r16's a (g even) or b (g odd) of dims
// (g / 2) * DPW / 2 + 8 st .. + 7.  hi = bf16(w), lo = bf16(w - hi) of the
// float32 value w.
__global__ void k_precompute_wsplit(const float* __restrict__ mu, const float* __restrict__ var, __bf16* wsp,
                                    int K, int D, int Kpad, int DPW) {
  const int S = DPW / 16;
  const size_t total = (size_t)Kpad * 2 * DPW;  // (hi, lo) pairs
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int cb = (int)(idx / ((size_t)S * 512));
    int rem = (int)(idx - (size_t)cb * S * 512);
    const int st = rem / 512;
    rem -= st * 512;
    const int lane = rem >> 3, jj = rem & 7;
    const int gg = lane >> 4;
    const int comp = cb * 16 + (lane & 15);
    const int dim = (gg >> 1) * (DPW / 2) + st * 8 + jj;
    double val = 0.0;
    if (comp < K && dim < D) {
      const double s2 = (double)var[(size_t)comp * D + dim];
      val = (gg & 1) ? (double)mu[(size_t)comp * D + dim] / s2 : -0.5 / s2;
    }
    const float vf = (float)val;
    const __bf16 hi = (__bf16)vf;
    const size_t base = ((size_t)(cb * S + st) * 2) * 512 + (size_t)lane * 8 + jj;
    wsp[base] = hi;
    wsp[base + 512] = (__bf16)(vf - (float)hi);
  }
}

// The isotropic W = mu / s^2 as split bfloat16 pairs for the isotropic kernel
// with split logits: per 16-component block, [step][hi, lo][lane][8]; lane
// (g, r16) of step st holds component r16's value for dims
// g * DPW / 4 + 8 st .. + 7.
__global__ void k_precompute_wsplit_iso(const float* __restrict__ mu, const float* __restrict__ var_iso,
                                        __bf16* wsp, int K, int D, int Kpad, int DPW) {
  const int S = DPW / 32, Q = DPW / 4;
  const size_t total = (size_t)Kpad * DPW;  // (hi, lo) pairs
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int cb = (int)(idx / ((size_t)S * 512));
    int rem = (int)(idx - (size_t)cb * S * 512);
    const int st = rem / 512;
    rem -= st * 512;
    const int lane = rem >> 3, jj = rem & 7;
    const int comp = cb * 16 + (lane & 15);
    const int d = (lane >> 4) * Q + st * 8 + jj;
    float vf = 0.f;
    if (comp < K && d < D) vf = (float)((double)mu[(size_t)comp * D + d] / (double)var_iso[comp]);
    const __bf16 hi = (__bf16)vf;
    const size_t base = ((size_t)(cb * S + st) * 2) * 512 + (size_t)lane * 8 + jj;
    wsp[base] = hi;
    wsp[base + 512] = (__bf16)(vf - (float)hi);
  }
}

__global__ void k_precompute_c(const float* __restrict__ w, const float* __restrict__ mu,
                               const float* __restrict__ var, double* cfull, double* cpeak, int K, int D,
                               int Kpad) {
  const int comp = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & 63;
  if (comp >= Kpad) return;
  if (comp >= K) {
    if (lane == 0) {
      cfull[comp] = -__builtin_huge_val();
      cpeak[comp] = -__builtin_huge_val();
    }
    return;
  }
  double q = 0.0, ld = 0.0;
  for (int d = lane; d < D; d += kWave) {
    const double s2 = (double)var[(size_t)comp * D + d];
    const double m = (double)mu[(size_t)comp * D + d];
    q += m * m / s2;
    ld += log(s2);
  }
  for (int o = 32; o > 0; o >>= 1) {
    q += __shfl_xor(q, o);
    ld += __shfl_xor(ld, o);
  }
  if (lane == 0) {
    const double wk = (double)w[comp];
    const double lw = (wk > 0.0) ? log(wk) : ((wk == 0.0) ? -__builtin_huge_val() : __builtin_nan(""));
    // log-density of the component at its own mean, and the full constant
    cpeak[comp] = lw - 0.5 * ld - 0.5 * D * kLog2Pi;
    cfull[comp] = cpeak[comp] - 0.5 * q;
  }
}

// Isotropic kernel operands: W = mu_k / s_k^2 in the order logit_tile_iso
// reads it ([comp block][group of four k-steps][lane][4]: lane (g, r16) holds
// component r16's dims g*Q + 4 s4 .. +3, Q = DPW / 4) and 1 / (2 s_k^2).
__global__ void k_precompute_wiso(const float* __restrict__ mu, const float* __restrict__ var_iso, float* wiso,
                                  float* ivec, int K, int D, int Kpad, int DPW) {
  const int S4 = DPW / 16, Q = DPW / 4;
  const size_t total = (size_t)Kpad * DPW;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const size_t rest = idx >> 8;
    const int s4 = (int)(rest % S4);
    const int cb16 = (int)(rest / S4);
    const int comp = cb16 * 16 + (lane & 15);
    const int d = (lane >> 4) * Q + s4 * 4 + i;
    float val = 0.f;
    if (comp < K && d < D) val = (float)((double)mu[(size_t)comp * D + d] / (double)var_iso[comp]);
    wiso[idx] = val;
    if (idx < (size_t)Kpad) ivec[idx] = (idx < (size_t)K) ? (float)(0.5 / (double)var_iso[idx]) : 0.f;
  }
}

// Float64 (a, b) per component and dimension for the refinement, and the
// per-component maxima of |a| and |b| used in its error bound.
__global__ void k_precompute_w64(const float* __restrict__ mu, const float* __restrict__ var, double2* w64,
                                 float2* abmax, int K, int D, int Kpad, int Dp) {
  const int comp = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & 63;
  if (comp >= Kpad) return;
  double ma = 0.0, mb = 0.0;
  for (int d = lane; d < Dp; d += kWave) {
    double2 ab = make_double2(0.0, 0.0);
    if (comp < K && d < D) {
      const double s2 = (double)var[(size_t)comp * D + d];
      ab = make_double2(-0.5 / s2, (double)mu[(size_t)comp * D + d] / s2);
    }
    w64[(size_t)comp * Dp + d] = ab;
    ma = fmax(ma, fabs(ab.x));
    mb = fmax(mb, fabs(ab.y));
  }
  for (int o = 32; o > 0; o >>= 1) {
    ma = fmax(ma, __shfl_xor(ma, o));
    mb = fmax(mb, __shfl_xor(mb, o));
  }
  if (lane == 0) abmax[comp] = make_float2((float)(ma * (1.0 + 1e-6)), (float)(mb * (1.0 + 1e-6)));
}

// Global logit offset C = max_k (peak log-density) - D/2: a typical logit of
// a point near its component.  c_k - C is rounded to float32, so the fp32
// logits (and log Z) are centred near 0 instead of carrying magnitudes of
// hundreds to thousands of nats; the log-likelihood adds N*C back in fp64.
__global__ void k_precompute_shift(const double* __restrict__ cfull, const double* __restrict__ cpeak,
                                   float* cvec, double* cvec64, double* cshift, int Kpad, int D) {
  __shared__ double red[1024];
  double m = -__builtin_huge_val();
  for (int k = threadIdx.x; k < Kpad; k += blockDim.x) m = fmax(m, cpeak[k]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + st]);
    __syncthreads();
  }
  double C = red[0] - 0.5 * D;
  if (!isfinite(C)) C = 0.0;
  for (int k = threadIdx.x; k < Kpad; k += blockDim.x) {
    cvec[k] = (float)(cfull[k] - C);
    if (cvec64) cvec64[k] = cfull[k] - C;  // only the float64-logit mode reads it
  }
  if (threadIdx.x == 0) *cshift = C;
}

// ---------------------------------------------------------------------------
// Deterministic pairwise sum of n values at a stride (blocks of 4, then a
// binary-counter merge: a fixed tree that depends only on n).
__device__ __forceinline__ double pairwise_sum(const double* p, size_t stride, int n) {
  double st[24];
  int sz[24];
  int top = 0;
  for (int i = 0; i < n; i += 4) {
    double s = 0.0;
    const int e = min(i + 4, n);
    for (int k = i; k < e; ++k) s += p[(size_t)k * stride];
    int c = 1;
    while (top > 0 && sz[top - 1] == c) {
      s = st[top - 1] + s;
      c <<= 1;
      --top;
    }
    st[top] = s;
    sz[top] = c;
    ++top;
  }
  double r = 0.0;
  while (top > 0) r = st[--top] + r;
  return r;
}

// Slots -> caller statistics (the tree that replaces Algorithm 1 step 17).
__global__ void k_reduce(const double* __restrict__ slots, int R, int Kpad, int K, int D, int Dp, int DPW,
                         double* Nk, double* S1, double* S2, int accumulate) {
  const int SR = 2 * Dp + 1;
  const size_t total = (size_t)K * SR;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(idx / SR);
    const int phi = (int)(idx - (size_t)k * SR);
    double* out;
    if (phi == 2 * Dp) {
      out = Nk + k;
    } else {
      const int seg = phi / (2 * DPW);
      const int e = phi - seg * 2 * DPW;
      const int sg = e / (DPW / 2);
      const int dim = seg * DPW + (sg >> 1) * (DPW / 2) + (e - sg * (DPW / 2));
      if (dim >= D) continue;
      out = ((sg & 1) ? S1 : S2) + (size_t)k * D + dim;
    }
    const double v = pairwise_sum(slots + (size_t)k * SR + phi, (size_t)Kpad * SR, R);
    *out = accumulate ? *out + v : v;
  }
}

__global__ void k_reduce_ll(const double* __restrict__ llslots, int n, double* ll, int accumulate,
                            int* flags, const double* __restrict__ cshift, double nrows) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const double v = pairwise_sum(llslots, 1, n) + nrows * (*cshift);
    const double out = accumulate ? *ll + v : v;
    *ll = out;
    if (!isfinite(out)) flags[0] = 1;
  }
}

// ---------------------------------------------------------------------------
// M-step, Eqs. (1)-(3) with a diagonal covariance and a floor; float64.
__global__ void k_mstep(const double* __restrict__ Nk, const double* __restrict__ S1,
                        const double* __restrict__ S2, double n_total, float floor_, float* w,
                        float* mu, float* var, int K, int D, int* flags) {
  const size_t total = (size_t)K * D;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(idx / D);
    const int d = (int)(idx - (size_t)k * D);
    const double nk = Nk[k];
    if (d == 0) w[k] = (float)(nk / n_total);
    if (!isfinite(nk)) flags[0] = 1;
    if (nk >= 1e-6) {
      const double m = S1[idx] / nk;
      double v = S2[idx] / nk - m * m;
      v = fmax(v, (double)floor_);
      mu[idx] = (float)m;
      var[idx] = (float)v;
    }
  }
}

// ---------------------------------------------------------------------------
// Isotropic model, Sigma_k = sigma^2_k I ("Flash-GMM", Section 2, the pages'
// own covariance; Eq. (3) averaged over the D dimensions).  Its E-step is the
// diagonal one with sigma^2_kd = sigma^2_k for every d, so the E-step kernels
// above run on the broadcast variances; Q_k = sum_n r_nk ||x_n||^2 is the sum
// over d of the diagonal S2_kd.  Every reduction over d is a fixed-order
// float64 tree (one wave per component), so results are deterministic.
__device__ __forceinline__ double wave_sum64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ void k_iso_expand(const float* __restrict__ var_iso, float* __restrict__ vexp, int K, int D) {
  const size_t total = (size_t)K * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x)
    vexp[i] = var_iso[i / D];
}

// Q_k (+)= sum_d S2_kd
__global__ void k_iso_q(const double* __restrict__ S2, double* Q, int K, int D, int accumulate) {
  const int k = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & 63;
  if (k >= K) return;
  double t = 0.0;
  for (int d = lane; d < D; d += kWave) t += S2[(size_t)k * D + d];
  t = wave_sum64(t);
  if (lane == 0) Q[k] = accumulate ? Q[k] + t : t;
}

// pi_k = N_k / N; mu_k = S1_k / N_k; sigma^2_k = max((Q_k / N_k - ||mu_k||^2) / D, floor);
// components with N_k < 1e-6 keep mean and variance
__global__ void k_mstep_iso(const double* __restrict__ Nk, const double* __restrict__ S1,
                            const double* __restrict__ Q, double n_total, float floor_, float* w, float* mu,
                            float* var_iso, int K, int D, int* flags) {
  const int k = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & 63;
  if (k >= K) return;
  const double nk = Nk[k];
  if (lane == 0) {
    w[k] = (float)(nk / n_total);
    if (!isfinite(nk)) flags[0] = 1;
  }
  if (!(nk >= 1e-6)) return;
  double mm = 0.0;
  for (int d = lane; d < D; d += kWave) {
    const double m = S1[(size_t)k * D + d] / nk;
    mu[(size_t)k * D + d] = (float)m;
    mm += m * m;
  }
  mm = wave_sum64(mm);
  if (lane == 0) var_iso[k] = (float)fmax((Q[k] / nk - mm) / D, (double)floor_);
}

// init: every component's variance is the mean over d of the per-dimension
// population variances, floored
__global__ void k_iso_init_var(const double* __restrict__ colvar, int D, float floor_, float* var_iso, int K) {
  __shared__ double tot;
  if (threadIdx.x < kWave) {
    double t = 0.0;
    for (int d = threadIdx.x; d < D; d += kWave) t += colvar[d];
    t = wave_sum64(t);
    if (threadIdx.x == 0) tot = t;
  }
  __syncthreads();
  const float v = (float)fmax(tot / D, (double)floor_);
  for (int k = threadIdx.x; k < K; k += blockDim.x) var_iso[k] = v;
}

// ---------------------------------------------------------------------------
// k-means warm start (Lloyd's algorithm; the pages seed their mixtures with
// k-means).  Rows are assigned to their nearest centre by the soft-assignment
// kernels (argmax of the logits with equal weights and variances 1/2, which
// is the argmin of the squared distance, float64-exact near ties, lowest
// index on ties) into CSR lists; one workgroup per centre then sums its
// list's rows in list order (row ids ascending), so the result is
// deterministic.
//   mode 0: centres_k = mean of its rows (an empty list keeps its centre),
//           counts_k = its size;
//   mode 1: the mixture seeded from the clustering: weights_k = n_k / N,
//           means_k = centres_k, vars = population variance of the rows
//           about the centre (colvar, the variance of all rows, for an empty
//           list), averaged over the dimensions when iso, floored.
// centres_k = S1_k / n_k (n_k, exact counts of the one-hot responsibilities)
// for every centre with rows; the others keep their position
__global__ void k_kmeans_update(const double* __restrict__ Nk, const double* __restrict__ S1, float* centres,
                                double* counts, int K, int D) {
  const size_t total = (size_t)K * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(i / D);
    const double n = Nk[k];
    if (n >= 0.5) centres[i] = (float)(S1[i] / n);
    if (i - (size_t)k * D == 0) counts[k] = n;
  }
}

__global__ void k_fill_f32(float* __restrict__ p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void __launch_bounds__(256) k_centroids(const float* __restrict__ X, int64_t ldx,
                                                   const int64_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ ids, int D, float* centres,
                                                   double* counts, int mode, const double* __restrict__ colvar,
                                                   float floor_, int64_t N, int iso, float* weights, float* means,
                                                   float* vars) {
  __shared__ double red[256];
  const int k = blockIdx.x;
  const int64_t b = offsets[k], e = offsets[k + 1];
  const int64_t n = e - b;
  double tsum = 0.0;  // iso: this thread's dims' variances
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const double c = (double)centres[(size_t)k * D + d];
    double acc = 0.0;
    int64_t i = b;
    // eight rows' loads in flight, added in list order
    for (; i + 8 <= e; i += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = X[(int64_t)ids[i + u] * ldx + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double x = (double)v[u];
        acc += (mode == 0) ? x : (x - c) * (x - c);
      }
    }
    for (; i < e; ++i) {
      const double x = (double)X[(int64_t)ids[i] * ldx + d];
      acc += (mode == 0) ? x : (x - c) * (x - c);
    }
    if (mode == 0) {
      if (n > 0) centres[(size_t)k * D + d] = (float)(acc / (double)n);
    } else {
      const double var = (n > 0) ? acc / (double)n : colvar[d];
      means[(size_t)k * D + d] = (float)c;
      if (!iso) vars[(size_t)k * D + d] = (float)fmax(var, (double)floor_);
      tsum += var;
    }
  }
  if (threadIdx.x == 0) {
    if (mode == 0) counts[k] = (double)n;
    else weights[k] = (float)((double)n / (double)N);
  }
  if (mode == 1 && iso) {
    red[threadIdx.x] = tsum;
    __syncthreads();
    for (int st = blockDim.x / 2; st > 0; st >>= 1) {
      if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
      __syncthreads();
    }
    if (threadIdx.x == 0) vars[k] = (float)fmax(red[0] / D, (double)floor_);
  }
}

// ---------------------------------------------------------------------------
// Initialisation: column sums (pass 0) or squared deviations (pass 1) of row
// blocks in float64, then a pairwise tree over blocks.
// Column sums of X over a row range per workgroup (init: the global
// per-dimension variance): pass 0 sums x, pass 1 sums (x - mean)^2.  256 threads:
// CG float4 column groups x RL row lanes; each thread keeps two independent
// float64 accumulators per column (rows alternate), so the float4 loads
// stream; the RL row lanes are then combined in a fixed order through LDS.
// Deterministic: the row range and summation order depend only on N and the
// grid.
__global__ void __launch_bounds__(256) k_colpart(const float* __restrict__ X, int64_t N, int64_t ldx, int D,
                                                 const double* __restrict__ mean, double* part, int pass) {
  __shared__ double red[256 * 4];
  const int D4 = (D + 3) >> 2;
  int CG = 1;
  while (CG < D4 && CG < 256) CG <<= 1;
  const int RL = 256 / CG;
  const int tid = threadIdx.x, cg0 = tid % CG, rl = tid / CG;
  const int64_t per = (N + gridDim.x - 1) / gridDim.x;
  const int64_t r0 = (int64_t)blockIdx.x * per;
  const int64_t r1 = min(N, r0 + per);
  for (int c4 = cg0; c4 < D4 + (CG - D4 % CG) % CG; c4 += CG) {  // uniform trip count
    const bool live = c4 < D4;
    const int d0 = c4 * 4;
    double m[4] = {0.0, 0.0, 0.0, 0.0};
    if (pass && live)
      for (int e = 0; e < 4; ++e) m[e] = (d0 + e < D) ? mean[d0 + e] : 0.0;
    double sa[4] = {0.0, 0.0, 0.0, 0.0}, sb[4] = {0.0, 0.0, 0.0, 0.0};
    if (live) {
      int64_t r = r0 + rl;
      for (; r + RL < r1; r += 2 * RL) {
        const f4 xa = __builtin_nontemporal_load(reinterpret_cast<const f4*>(X + r * ldx + d0));
        const f4 xb = __builtin_nontemporal_load(reinterpret_cast<const f4*>(X + (r + RL) * ldx + d0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double a = (double)xa[e] - m[e], b = (double)xb[e] - m[e];
          sa[e] += pass ? a * a : a;
          sb[e] += pass ? b * b : b;
        }
      }
      if (r < r1) {
        const f4 xa = __builtin_nontemporal_load(reinterpret_cast<const f4*>(X + r * ldx + d0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double a = (double)xa[e] - m[e];
          sa[e] += pass ? a * a : a;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(rl * CG + cg0) * 4 + e] = sa[e] + sb[e];
    __syncthreads();
    if (rl == 0 && live) {
      for (int e = 0; e < 4; ++e) {
        double t = 0.0;
        for (int q = 0; q < RL; ++q) t += red[(q * CG + cg0) * 4 + e];
        if (d0 + e < D) part[(size_t)blockIdx.x * D + d0 + e] = t;
      }
    }
    __syncthreads();
  }
}

__global__ void k_colfinal(const double* __restrict__ part, int nb, int D, double N, double* out) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d < D) out[d] = pairwise_sum(part + d, (size_t)D, nb) / N;
}

__global__ void k_init_params(const float* __restrict__ X, int64_t ldx, const int64_t* __restrict__ rows,
                              const double* __restrict__ colvar, float floor_, float* w, float* mu,
                              float* var, int K, int D) {
  const size_t total = (size_t)K * D;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(idx / D);
    const int d = (int)(idx - (size_t)k * D);
    mu[idx] = X[rows[k] * ldx + d];
    var[idx] = (float)fmax(colvar[d], (double)floor_);
    if (d == 0) w[k] = (float)(1.0 / (double)K);
  }
}

// ---------------------------------------------------------------------------
// Host-side plan, instantiation table and launchers.
template <int WC, int WD, int DPW>
struct Kern {
  static constexpr int BN = bn_for(WD, DPW);
  template <int M>
  static void* stats_fused() { return (void*)&k_stats<WC, WD, DPW, BN, true, M>; }
  template <int M>
  static void* stats_two() { return (void*)&k_stats<WC, WD, DPW, BN, false, M>; }
  template <int M>
  static void* logz() { return (void*)&k_logz<WC, WD, DPW, BN, M>; }
  template <int M>
  static void* stats_iso() {
    if constexpr (WD == 1) return (void*)&k_stats<WC, WD, DPW, BN, true, M, true>;
    else return nullptr;
  }
  template <int M>
  static void* stats_hard() {
    if constexpr (WD == 1) return (void*)&k_stats<WC, WD, DPW, BN, true, M, true, true>;
    else return nullptr;
  }
  static void* stats_split() {
    if constexpr (WD == 1) return (void*)&k_stats<WC, WD, DPW, BN, true, MODE_REFINE, false, false, 1>;
    else return nullptr;
  }
  static void* stats_split2() {
    if constexpr (WD == 1 && BN % 32 == 0) return (void*)&k_stats<WC, WD, DPW, BN, true, MODE_REFINE, false, false, 2>;
    else return nullptr;
  }
  static void* stats_iso_split2() {
    if constexpr (WD == 1 && DPW >= 32 && BN % 32 == 0)
      return (void*)&k_stats<WC, WD, DPW, BN, true, MODE_REFINE, true, false, 2>;
    else return nullptr;
  }
  static void* stats_hard_split2() {
    if constexpr (WD == 1 && DPW >= 32 && BN % 32 == 0)
      return (void*)&k_stats<WC, WD, DPW, BN, true, MODE_REFINE, true, true, 2>;
    else return nullptr;
  }
  static void* stats_iso_split() {
    if constexpr (WD == 1 && DPW >= 32) return (void*)&k_stats<WC, WD, DPW, BN, true, MODE_REFINE, true, false, 1>;
    else return nullptr;
  }
  static void* stats_hard_split() {
    if constexpr (WD == 1 && DPW >= 32) return (void*)&k_stats<WC, WD, DPW, BN, true, MODE_REFINE, true, true, 1>;
    else return nullptr;
  }
};

// Kernel variants of one shape, indexed by logit precision mode (the
// isotropic and hard-assignment kernels have no float64-logit variant).
struct KTab {
  void* fused[3];
  void* iso[2];   // fused isotropic kernels (nullptr where not built)
  void* hard[2];  // fused k-means (hard assignment) kernels
  void* split;    // fused diagonal refined kernel with split-bf16 logits (nullptr where not built)
  void* iso_split;   // the same for the isotropic kernel
  void* hard_split;  // and its hard-assignment mode
  void* split2;      // diagonal kernel with split-bf16 logits and statistics
  void* iso_split2;  // the same for the isotropic kernel
  void* hard_split2; // and its hard-assignment mode
  void* two[3];
  void* logz[3];
};

static bool lookup(int WC, int WD, int DPW, KTab& t) {
#define GMM_K(wc, wd, dpw)                                                                            \
  if (WC == wc && WD == wd && DPW == dpw) {                                                           \
    using KK = Kern<wc, wd, dpw>;                                                                     \
    t = KTab{{KK::stats_fused<0>(), KK::stats_fused<1>(), KK::stats_fused<2>()},                       \
             {KK::stats_iso<0>(), KK::stats_iso<1>()},                                                 \
             {KK::stats_hard<0>(), KK::stats_hard<1>()},                                               \
             KK::stats_split(), KK::stats_iso_split(), KK::stats_hard_split(), KK::stats_split2(),    \
             KK::stats_iso_split2(), KK::stats_hard_split2(),                                          \
             {KK::stats_two<0>(), KK::stats_two<1>(), KK::stats_two<2>()},                                \
             {KK::logz<0>(), KK::logz<1>(), KK::logz<2>()}};                                              \
    return true;                                                                                      \
  }
  GMM_K(1, 1, 16) GMM_K(1, 1, 32) GMM_K(1, 1, 64) GMM_K(1, 1, 128)
  GMM_K(2, 1, 16) GMM_K(2, 1, 32) GMM_K(2, 1, 64) GMM_K(2, 1, 128)
  GMM_K(4, 1, 16) GMM_K(4, 1, 32) GMM_K(4, 1, 64) GMM_K(4, 1, 128)
  GMM_K(8, 1, 16) GMM_K(8, 1, 32) GMM_K(8, 1, 64) GMM_K(8, 1, 128)
  GMM_K(1, 8, 32) GMM_K(1, 8, 64) GMM_K(1, 8, 96) GMM_K(1, 8, 128)
#undef GMM_K
  return false;
}

static size_t lds_stats_bytes(int WC, int WD, int DPW) {
  const int BN = bn_for(WD, DPW);
  const int RS = WD * DPW + 4;  // mirrors Shape
  const int per_cu = (WC * WD == 4) ? 2 : 1;
  const size_t red = WD > 1 ? (size_t)(WD + BN / 16) * WC * 8 * 64 * 4 : 4;
  const int NBUF = ((size_t)BN * RS * 8 + red <= (size_t)(per_cu == 1 ? 140 : 68) * 1024) ? 2 : 1;
  const int QP = (64 * WC * WD) / BN;
  size_t b = (size_t)NBUF * BN * RS * 4 + red;
  b += BN * 4 + (size_t)WC * BN * 4 + 2 * (size_t)QP * BN * 4 + BN * 8 + 4;
  b += BN * 8 + BN * 8 + (size_t)((WD > 1 && WC == 1) ? WC : WC * WD) * 256 * 6;
  return b;
}

Plan make_plan(int K, int D, int numCU, int occStats, int occLogz) {
  Plan p{};
  p.K = K;
  p.D = D;
  if (D <= 128) {
    p.WD = 1;
    p.DPW = D <= 16 ? 16 : D <= 32 ? 32 : D <= 64 ? 64 : 128;
    const int groups = (K + 31) / 32;
    // one 8-wave workgroup per CU (256 components); FLASHGMM_WC=4 selects
    // 4-wave workgroups, two per CU (a tuning knob for measurements)
    const char* env = getenv("FLASHGMM_WC");
    int wmax = (env && atoi(env) == 4) ? 4 : 8;
    // ... unless padding K to 256 wastes much more than padding it to 128
    const int pad8 = (K + 255) / 256 * 256 - K, pad4 = (K + 127) / 128 * 128 - K;
    if (pad8 > pad4 + K / 8) wmax = 4;
    p.WC = groups >= wmax ? wmax : groups >= 4 ? 4 : groups >= 2 ? 2 : 1;
  } else {
    p.WD = 8;
    const int per = (D + 7) / 8;
    p.DPW = per <= 32 ? 32 : per <= 64 ? 64 : per <= 96 ? 96 : 128;
    p.WC = 1;
  }
  p.Dp = p.DPW * p.WD;
  p.BN = bn_for(p.WD, p.DPW);
  const int cw = 32 * p.WC;
  p.Kpad = (K + cw - 1) / cw * cw;
  p.P = p.Kpad / cw;
  p.SR = 2 * p.Dp + 1;
  p.RS = p.WD * (2 * p.DPW + 4);
  p.ldsStats = lds_stats_bytes(p.WC, p.WD, p.DPW);
  const int capS = numCU * (occStats > 0 ? occStats : 1);
  p.fusedOK = (p.P <= capS) ? 1 : 0;
  p.R = capS / p.P;
  if (p.R < 1) p.R = 1;
  p.G = p.R * p.P;
  p.Glogz = numCU * (occLogz > 0 ? occLogz : 1);
  p.chunk = (int64_t)1 << 21;
  p.numCU = numCU;
  p.occAssign = 1;
  p.assignChunk = (int64_t)1 << 19;
  p.assignBlocks = 256;
  return p;
}

bool plan_shape_ok(const Plan& p) {
  KTab t;
  return lookup(p.WC, p.WD, p.DPW, t);
}

size_t workspace_bytes(const Plan& p) {
  const size_t a = 256;
  auto up = [&](size_t b) { return (b + a - 1) / a * a; };
  size_t b = 0;
  b += up((size_t)p.Kpad * 2 * p.Dp * 4);
  b += up((size_t)p.Kpad * 4);
  b += 2 * up((size_t)p.Kpad * 8) + up(8);
  b += up((size_t)p.Kpad * p.Dp * 16) + up((size_t)p.Kpad * 8) + up(8);
  b += up((size_t)p.Kpad * 2 * p.Dp * 8) + up((size_t)p.Kpad * 8);  // wop64, cvec64
  b += up((size_t)p.K * p.D * 4) + up((size_t)p.K * 8);  // isotropic: broadcast variances, Q
  b += 2 * up((size_t)p.K * 4);  // k-means: equal weights, variances 1/2
  b += up((size_t)p.Kpad * p.Dp * 4) + up((size_t)p.Kpad * 4);  // isotropic kernel: W, 1/(2 s^2)
  b += up((size_t)p.Kpad * 2 * p.Dp * 2 * 2);                     // split-bf16 W (hi, lo)
  b += up((size_t)p.Kpad * p.Dp * 2 * 2);                         // the same, isotropic
  b += up((size_t)p.R * p.Kpad * p.SR * 8);
  b += up((size_t)(p.R > p.Glogz ? p.R : p.Glogz) * 8);
  b += up((size_t)p.chunk * 4);
  b += up((size_t)p.R * 4 * p.P * p.BN * 8);
  b += up(((size_t)p.K + 2 * (size_t)p.K * p.D + 1) * 8);
  b += up((size_t)1024 * p.D * 8);
  b += up((size_t)p.D * 8);
  b += up((size_t)p.K * 8);
  b += up(16);
  b += up((size_t)p.assignChunk * 9 * 4);
  b += up((size_t)p.Kpad / 32 * 16);
  b += up((size_t)p.Kpad * 8);
  b += up((size_t)p.assignBlocks * p.Kpad * 4);
  b += up((size_t)p.Kpad * 4);
  b += up((size_t)p.Kpad * 8);
  b += up(8);
  return b;
}

hipError_t occupancy(const Plan& p, int* occStats, int* occLogz) {
  KTab t;
  if (!lookup(p.WC, p.WD, p.DPW, t)) return hipErrorInvalidValue;
  const int nt = 64 * p.WC * p.WD;
  int o1 = 0, o2 = 0;
  // the smaller occupancy of the two precision variants sizes the grids
  int o1b = 0, o2b = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o1, (const void*)t.fused[0], nt, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o1b, (const void*)t.fused[1], nt, 0);
  void* extra[6] = {t.split, t.iso_split, t.hard_split, t.split2, t.iso_split2, t.hard_split2};
  for (int m = 0; m < 10 && e == hipSuccess; ++m) {
    void* kk = (m < 2) ? t.iso[m] : (m < 4) ? t.hard[m - 2] : extra[m - 4];
    if (!kk) continue;
    int oi = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&oi, (const void*)kk, nt, 0);
    if (oi < o1b) o1b = oi;
  }
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o2, (const void*)t.logz[0], nt, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o2b, (const void*)t.logz[1], nt, 0);
  if (e != hipSuccess) return e;
  *occStats = o1 < o1b ? o1 : o1b;
  *occLogz = o2 < o2b ? o2 : o2b;
  return hipSuccess;
}

hipError_t fused64_fits(const Plan& p, int* ok) {
  *ok = 0;
  KTab t;
  if (!lookup(p.WC, p.WD, p.DPW, t)) return hipErrorInvalidValue;
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)t.fused[2], 64 * p.WC * p.WD, 0);
  if (e != hipSuccess) return e;
  *ok = (p.fusedOK && (int64_t)occ * p.numCU >= (int64_t)p.G) ? 1 : 0;
  return hipSuccess;
}

static int grid_for(size_t total, int block) {
  size_t g = (total + block - 1) / block;
  if (g > 65535 * 4) g = 65535 * 4;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_precompute(const Plan& p, const Workspace& w, const float* weights, const float* means,
                             const float* vars, hipStream_t s) {
  const size_t total = (size_t)p.Kpad * 2 * p.Dp;
  hipLaunchKernelGGL(k_precompute_w<float>, dim3(grid_for(total, 256)), dim3(256), 0, s, means, vars, w.wop, p.K,
                     p.D, p.Kpad, p.WD, p.DPW);
  if (w.f64)
    hipLaunchKernelGGL(k_precompute_w<double>, dim3(grid_for(total, 256)), dim3(256), 0, s, means, vars, w.wop64,
                       p.K, p.D, p.Kpad, p.WD, p.DPW);
  hipLaunchKernelGGL(k_precompute_c, dim3((p.Kpad + 3) / 4), dim3(256), 0, s, weights, means, vars, w.cfull,
                     w.cpeak, p.K, p.D, p.Kpad);
  hipLaunchKernelGGL(k_precompute_shift, dim3(1), dim3(1024), 0, s, w.cfull, w.cpeak, w.cvec, w.cvec64, w.cshift, p.Kpad,
                     p.D);
  hipLaunchKernelGGL(k_precompute_w64, dim3((p.Kpad + 3) / 4), dim3(256), 0, s, means, vars, w.w64, w.abmax,
                     p.K, p.D, p.Kpad, p.Dp);
  if (p.WD == 1)
    hipLaunchKernelGGL(k_precompute_wsplit, dim3(grid_for(total, 256)), dim3(256), 0, s, means, vars, w.wsplit,
                       p.K, p.D, p.Kpad, p.DPW);
  return hipGetLastError();
}

static EArgs make_args(const Plan& p, const Workspace& w, const float* X, int64_t ldx) {
  EArgs a{};
  a.X = X;
  a.ldx = ldx;
  a.wop = w.wop;
  a.cvec = w.cvec;
  a.logz = w.logz;
  a.slots = w.slots;
  a.llslots = w.llslots;
  a.xbuf = w.xbuf;
  a.flags = w.flags;
  a.K = p.K;
  a.D = p.D;
  a.Kpad = p.Kpad;
  a.P = p.P;
  a.R = p.R;
  a.Dp = p.Dp;
  a.refine = w.refine;
  a.kappa = (float)((2.0 * p.Dp + 8.0) * 5.9604644775390625e-08);
  a.w64 = w.w64;
  a.cfull = w.cfull;
  a.cshift = w.cshift;
  a.abmax = w.abmax;
  a.nrefined = w.nrefined;
  // LDS DMA staging needs every row's Dp floats to be data (no dims to zero);
  // FLASHGMM_DMA=0 forces the register path (for measurements)
  const char* env = getenv("FLASHGMM_DMA");
  a.dma = (p.D == p.Dp && !(env && atoi(env) == 0)) ? 1 : 0;
  a.wop64 = w.wop64;
  a.cvec64 = w.cvec64;
  a.wiso = w.wiso;
  a.ivec = w.ivec;
  a.wsp = w.wsplit;
  return a;
}

__global__ void k_fill_u64(unsigned long long* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

bool split_kernel_ok(const Plan& p, int variant) {
  KTab t;
  if (!lookup(p.WC, p.WD, p.DPW, t)) return false;
  void* k[6] = {t.split, t.iso_split, t.hard_split, t.split2, t.iso_split2, t.hard_split2};
  return variant >= 0 && variant < 6 && k[variant] != nullptr;
}

bool iso_kernel_ok(const Plan& p, const Workspace& w, bool hard) {
  KTab t;
  if (w.f64 || !lookup(p.WC, p.WD, p.DPW, t)) return false;
  return (hard ? t.hard[w.refine ? 1 : 0] : t.iso[w.refine ? 1 : 0]) != nullptr;
}

hipError_t launch_precompute_iso(const Plan& p, const Workspace& w, const float* means, const float* var_iso,
                                 hipStream_t s) {
  const size_t total = (size_t)p.Kpad * p.DPW;
  hipLaunchKernelGGL(k_precompute_wiso, dim3(grid_for(total, 256)), dim3(256), 0, s, means, var_iso, w.wiso,
                     w.ivec, p.K, p.D, p.Kpad, p.DPW);
  if (p.WD == 1 && p.DPW >= 32)
    hipLaunchKernelGGL(k_precompute_wsplit_iso, dim3(grid_for(total, 256)), dim3(256), 0, s, means, var_iso,
                       w.wsplit_iso, p.K, p.D, p.Kpad, p.DPW);
  return hipGetLastError();
}

hipError_t launch_estep(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx, bool fused,
                        hipStream_t s, const LaunchHooks* hk, int* nslots, int variant) {
  auto pre = [&](int which) {
    if (hk && hk->before) hk->before(hk->user, which, s);
  };
  auto post = [&](int which) {
    if (hk && hk->after) hk->after(hk->user, which, s);
  };
  KTab t;
  if (!lookup(p.WC, p.WD, p.DPW, t)) return hipErrorInvalidValue;
  const int nt = 64 * p.WC * p.WD;
  EArgs a = make_args(p, w, X, ldx);
  const int mode = w.f64 ? 2 : (w.refine ? 1 : 0);
  if (fused && mode == 2 && variant != 0) return hipErrorInvalidValue;  // diagonal kernel only
  if (fused) {
    a.row0 = 0;
    a.nrows = N;
    a.slot_acc = 0;
    const int R = p.R;
    const size_t nx = (size_t)R * 4 * p.P * p.BN;
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(nx, 256)), dim3(256), 0, s, w.xbuf, nx);
    void* args[] = {&a};
    pre(0);
    void* kern = (variant == 2) ? t.hard[mode] : (variant == 1) ? t.iso[mode] : t.fused[mode];
    void* ksplit = (variant == 2) ? t.hard_split : (variant == 1) ? t.iso_split : t.split;
    void* ksplit2 = (variant == 2) ? t.hard_split2 : (variant == 1) ? t.iso_split2 : t.split2;
    if (w.split == 2 && ksplit2) ksplit = ksplit2;  // statistics split too
    if (mode == 1 && w.split && ksplit) {
      // split-bf16 logits: at most 6 Dp exact partial products summed in
      // float32, plus the split's own 3 * 2^-16 relative error per feature
      kern = ksplit;
      a.wsp = variant ? w.wsplit_iso : w.wsplit;
      a.kappa = (float)((6.0 * p.Dp + 8.0) * 5.9604644775390625e-08 * (1.0 + 1.0 / 64.0) + 3.1 * 1.52587890625e-05);
    }
    if (!kern) return hipErrorInvalidValue;
    hipError_t e = hipLaunchCooperativeKernel(kern, dim3(p.G), dim3(nt), args, 0, s);
    if (e != hipSuccess) return e;
    post(0);
    *nslots = R;
    return hipGetLastError();
  }
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    a.row0 = r0;
    a.nrows = (N - r0 < p.chunk) ? (N - r0) : p.chunk;
    a.slot_acc = (r0 > 0) ? 1 : 0;
    void* args[] = {&a};
    pre(1);
    hipError_t e = hipLaunchKernel(t.logz[mode], dim3(p.Glogz), dim3(nt), args, 0, s);
    if (e != hipSuccess) return e;
    post(1);
    pre(0);
    e = hipLaunchKernel(t.two[mode], dim3(p.G), dim3(nt), args, 0, s);
    if (e != hipSuccess) return e;
    post(0);
  }
  *nslots = p.R;
  return hipGetLastError();
}

hipError_t launch_reduce(const Plan& p, const Workspace& w, double* Nk, double* S1, double* S2, double* ll,
                         int accumulate, int nslots, int nllslots, int64_t nrows, hipStream_t s) {
  const size_t total = (size_t)p.K * p.SR;
  hipLaunchKernelGGL(k_reduce, dim3(grid_for(total, 256)), dim3(256), 0, s, w.slots, nslots, p.Kpad, p.K, p.D,
                     p.Dp, p.DPW, Nk, S1, S2, accumulate);
  hipLaunchKernelGGL(k_reduce_ll, dim3(1), dim3(64), 0, s, w.llslots, nllslots, ll, accumulate, w.flags, w.cshift,
                     (double)nrows);
  return hipGetLastError();
}

hipError_t launch_mstep(const Plan& p, const Workspace& w, const double* Nk, const double* S1,
                        const double* S2, double n_total, float var_floor, float* weights, float* means,
                        float* vars, hipStream_t s) {
  const size_t total = (size_t)p.K * p.D;
  hipLaunchKernelGGL(k_mstep, dim3(grid_for(total, 256)), dim3(256), 0, s, Nk, S1, S2, n_total, var_floor,
                     weights, means, vars, p.K, p.D, w.flags);
  return hipGetLastError();
}

hipError_t launch_iso_expand(const Plan& p, const Workspace& w, const float* var_iso, hipStream_t s) {
  const size_t total = (size_t)p.K * p.D;
  hipLaunchKernelGGL(k_iso_expand, dim3(grid_for(total, 256)), dim3(256), 0, s, var_iso, w.vexp, p.K, p.D);
  return hipGetLastError();
}

hipError_t launch_iso_q(const Plan& p, const double* S2, double* Q, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(k_iso_q, dim3((p.K + 3) / 4), dim3(256), 0, s, S2, Q, p.K, p.D, accumulate);
  return hipGetLastError();
}

hipError_t launch_mstep_iso(const Plan& p, const Workspace& w, const double* Nk, const double* S1, const double* Q,
                            double n_total, float var_floor, float* weights, float* means, float* var_iso,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_mstep_iso, dim3((p.K + 3) / 4), dim3(256), 0, s, Nk, S1, Q, n_total, var_floor, weights,
                     means, var_iso, p.K, p.D, w.flags);
  return hipGetLastError();
}

hipError_t launch_init_iso(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                           float var_floor, float* weights, float* means, float* var_iso, hipStream_t s) {
  // the diagonal initialisation leaves the per-dimension variances (before
  // the floor) in the statistics scratch; its K x D variances go to vexp
  hipError_t e = launch_init(p, w, X, N, ldx, var_floor, weights, means, w.vexp, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_iso_init_var, dim3(1), dim3(256), 0, s, (const double*)w.stats, p.D, var_floor, var_iso,
                     p.K);
  return hipGetLastError();
}

hipError_t launch_fill_zero(double* p, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(n, 256)), dim3(256), 0, s, (unsigned long long*)p, n);
  return hipGetLastError();
}

hipError_t launch_kmeans_update(const Plan& p, const double* Nk, const double* S1, float* centres, double* counts,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_kmeans_update, dim3(grid_for((size_t)p.K * p.D, 256)), dim3(256), 0, s, Nk, S1, centres,
                     counts, p.K, p.D);
  return hipGetLastError();
}

hipError_t launch_kmeans_params(const Plan& p, const Workspace& w, const float* centres, hipStream_t s) {
  // equal weights and variances 1/2: the logit of centre k is a constant
  // minus the squared distance to it
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for((size_t)p.K, 256)), dim3(256), 0, s, w.wuni, (size_t)p.K,
                     1.0f / (float)p.K);
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for((size_t)p.K * p.D, 256)), dim3(256), 0, s, w.vexp,
                     (size_t)p.K * p.D, 0.5f);
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for((size_t)p.K, 256)), dim3(256), 0, s, w.vhalf, (size_t)p.K, 0.5f);
  return hipGetLastError();
}

hipError_t launch_centroids(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                            const int64_t* offsets, const int32_t* ids, float* centres, double* counts, int mode,
                            float var_floor, int iso, float* weights, float* means, float* vars, hipStream_t s) {
  hipLaunchKernelGGL(k_centroids, dim3(p.K), dim3(256), 0, s, X, ldx, offsets, ids, p.D, centres, counts, mode,
                     (const double*)w.stats, var_floor, N, iso, weights, means, vars);
  return hipGetLastError();
}

hipError_t launch_colvar(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx, hipStream_t s) {
  const int nb = (int)((N < (int64_t)w.colG) ? N : (int64_t)w.colG);
  hipLaunchKernelGGL(k_colpart, dim3(nb), dim3(256), 0, s, X, N, ldx, p.D, (const double*)nullptr, w.colpart, 0);
  hipLaunchKernelGGL(k_colfinal, dim3((p.D + 255) / 256), dim3(256), 0, s, w.colpart, nb, p.D, (double)N,
                     w.colmean);
  hipLaunchKernelGGL(k_colpart, dim3(nb), dim3(256), 0, s, X, N, ldx, p.D, (const double*)w.colmean, w.colpart,
                     1);
  hipLaunchKernelGGL(k_colfinal, dim3((p.D + 255) / 256), dim3(256), 0, s, w.colpart, nb, p.D, (double)N,
                     w.stats);
  return hipGetLastError();
}

hipError_t launch_init(const Plan& p, const Workspace& w, const float* X, int64_t N, int64_t ldx,
                       float var_floor, float* weights, float* means, float* vars, hipStream_t s) {
  const int nb = (int)((N < (int64_t)w.colG) ? N : (int64_t)w.colG);
  const int bt = 256;
  hipLaunchKernelGGL(k_colpart, dim3(nb), dim3(bt), 0, s, X, N, ldx, p.D, (const double*)nullptr, w.colpart,
                     0);
  hipLaunchKernelGGL(k_colfinal, dim3((p.D + 255) / 256), dim3(256), 0, s, w.colpart, nb, p.D, (double)N,
                     w.colmean);
  // pass 1 writes variances into colpart's partials, final into stats scratch
  hipLaunchKernelGGL(k_colpart, dim3(nb), dim3(bt), 0, s, X, N, ldx, p.D, (const double*)w.colmean,
                     w.colpart, 1);
  double* colvar = w.stats;  // K + 2KD + 1 >= D doubles
  hipLaunchKernelGGL(k_colfinal, dim3((p.D + 255) / 256), dim3(256), 0, s, w.colpart, nb, p.D, (double)N,
                     colvar);
  const size_t total = (size_t)p.K * p.D;
  hipLaunchKernelGGL(k_init_params, dim3(grid_for(total, 256)), dim3(256), 0, s, X, ldx, w.rows, colvar,
                     var_floor, weights, means, vars, p.K, p.D);
  return hipGetLastError();
}

}  // namespace gmm
