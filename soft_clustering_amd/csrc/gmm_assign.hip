// Soft assignment of rows to components and inverted lists (gfx950).
//
// Method: "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
// Section 4.2 (each vector goes to its highest-responsibility component) and
// Section 4.3 (multi-assignment: a vector also goes to further components whose
// responsibility clears a threshold; the lists then serve an IVF index).  The
// responsibilities are r_nk = exp(l_nk - log Z_n) of Section 2.
//
// Rule implemented: per row, the argmax component (lowest index on ties) plus
// up to m further components with r >= threshold, ranked by r descending then
// index ascending.  Output: CSR inverted lists, offsets int64[K+1] and row ids
// int32, ids ascending within each list.
//
// GPU design:
//  * k_assign walks all component groups of a row tile with the same MFMA
//    logit contraction, float64 refinement and online log-sum-exp as the
//    E-step's first sweep.  After each 16-component block the wave transposes
//    its logits through LDS so that lane p holds row p's 16 values, and keeps
//    a sorted top-9 list (value descending, index ascending) per row in
//    registers.  Because r is increasing in l, the extras are the list's
//    entries 2..m+1 that clear log(threshold) against the row's log Z.
//  * Every logit that can be the argmax or clear the threshold lies within
//    delta = max(16, 1 - log threshold) nats of the row's largest logit, and
//    exactly those are recomputed in float64, so ranking and threshold tests
//    use float64-accurate values.
//  * Lists are built deterministically without sorting: pass A counts list
//    sizes (integer atomics), a scan gives the offsets; pass B re-selects each
//    chunk of rows, counts per (row block, list), scans those counts per list
//    and lets one thread per row block place its rows in row order.
#include "gmm_device.h"

#include <limits.h>

namespace gmm {

constexpr int kTopN = 9;  // 1 + the largest max_extra

struct AArgs {
  int32_t* sel;                  // chunk rows x (1 + m) component ids, -1 = none
  unsigned long long* counts;    // K list sizes (pass A) or nullptr
  float log_thr;                 // log(threshold)
  float delta;                   // float64 window below the row's largest logit
  int m;                         // max_extra
};

// Insert (val, k) into a list sorted by value descending, index ascending.
// FULL = false: k is larger than every index already in the list (one wave's
// own stream), so an equal value ranks after the existing entries.
template <bool FULL>
__device__ __forceinline__ void top_insert(float (&tv)[kTopN], int (&tk)[kTopN], float val, int k) {
  auto better = [&](float v2, int k2) { return FULL ? (val > v2 || (val == v2 && k < k2)) : (val > v2); };
  if (!better(tv[kTopN - 1], tk[kTopN - 1])) return;
#pragma unroll
  for (int i = kTopN - 1; i > 0; --i) {
    if (better(tv[i - 1], tk[i - 1])) {
      tv[i] = tv[i - 1];
      tk[i] = tk[i - 1];
    } else if (better(tv[i], tk[i])) {
      tv[i] = val;
      tk[i] = k;
    }
  }
  if (better(tv[0], tk[0])) {
    tv[0] = val;
    tk[0] = k;
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// SPLIT: split-bfloat16 first-pass logits (refined mode, WD = 1); the tile's
// split operands are built once and serve every component group.
template <int WC, int WD, int DPW, int BN, int MODE, bool SPLIT = false>
__global__ void __launch_bounds__(kWave* WC* WD) k_assign(EArgs a, AArgs s) {
  using SH = Shape<WC, WD, DPW, BN>;
  constexpr bool REFINE = MODE == MODE_REFINE, F64 = MODE == MODE_FP64;
  static_assert(!SPLIT || (REFINE && WD == 1), "split-bf16 logits: refined mode, WD = 1");
  using SPR = SplitRow<DPW, false>;
  constexpr int NPB = SH::NPB;
  constexpr int TLW = 16 * (BN + 1);        // one wave's transposed 16-component block
  constexpr int LSTW = 2 * kTopN * BN;      // one wave's lists (values, indices)
  constexpr int TBW = TLW > LSTW ? TLW : LSTW;
  __shared__ __attribute__((aligned(16))) float xt[SH::TILE];
  __shared__ __attribute__((aligned(16))) float red[F64 ? 1 : SH::RED];
  __shared__ double red64[F64 ? SH::RED : 1];
  __shared__ float tbuf[WC][TBW];
  __shared__ float lpart[WC][BN];
  __shared__ float2 nrm[BN];
  __shared__ __attribute__((aligned(16))) float thrw[WC][BN];
  __shared__ float rlist[SH::COOP ? WC : WC * WD][kRefineCap];  // refinement lists (per group or wave)
  __shared__ unsigned short elist[SH::COOP ? WC : WC * WD][kRefineCap];
  __shared__ __attribute__((aligned(16))) __bf16 xsb[SPLIT ? BN * SPR::XSR : 8];  // split operands

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wc = w % WC, wd = w / WC;
  const int g = lane >> 4, r16 = lane & 15;
  const int ncg = a.Kpad / 32;
  const double C = *a.cshift;
  const int nt = (int)((a.nrows + BN - 1) / BN);
  const int stride = 1 + s.m;
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
    if constexpr (SPLIT) split_rows<SH, DPW, false>(xt, xsb, w);  // published by the barrier below
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
    float tv[kTopN];
    int tk[kTopN];
#pragma unroll
    for (int i = 0; i < kTopN; ++i) {
      tv[i] = kNegInf;
      tk[i] = INT_MAX;
    }
    float* tl = tbuf[wc];
    for (int cg = wc; cg < ncg; cg += WC) {
      const int compbase = cg * 32;
      f4 acc[NPB][2];
      if constexpr (F64) {
        logits_f64<SH, WC, WD, DPW>(xt, wop_block(a.wop64, compbase >> 4, WD, wd, DPW),
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
        if constexpr (SPLIT) {
          logit_tile_split<SH, DPW, false>(xsb, a.wsp + (size_t)(compbase >> 4) * SPR::WBLK,
                                           a.wsp + (size_t)((compbase >> 4) + 1) * SPR::WBLK, acc, lane);
        } else {
          logit_tile<SH, DPW>(xt, wop_block(a.wop, compbase >> 4, WD, wd, DPW),
                              wop_block(a.wop, (compbase >> 4) + 1, WD, wd, DPW), acc, lane, wd);
          reduce_partial_logits<SH, WC, WD>(red, acc, lane, wc, wd);
        }
      }
      if constexpr (REFINE) {
        // running maximum of guaranteed lower bounds L - E of the row's
        // logits; anything that can be selected lies within delta of the
        // row's largest logit, hence above this bound minus delta
        float co[6];
        lane_coefs(a, compbase, r16, co);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float2 nn = nrm[pb * 16 + 4 * g + v];
            const float lb = fmaxf(acc[pb][0][v] - err_bound(a.kappa, co[0], co[1], co[2], nn),
                                   acc[pb][1][v] - err_bound(a.kappa, co[3], co[4], co[5], nn));
            Rlb[pb][v] = fmaxf(Rlb[pb][v], row16_max(lb));
            if (r16 == 0 && wd == 0) thrw[wc][pb * 16 + 4 * g + v] = Rlb[pb][v] - s.delta;
          }
        if constexpr (WD > 1) __syncthreads();
        else wave_sync();
        refine_tile<SH, WD, DPW>(acc, thrw[wc], nrm, co, xt, rows, a, C, compbase, rlist[SH::COOP ? wc : w], elist[SH::COOP ? wc : w], lane,
                                 wd, nsel);
      }
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float mn = fmaxf(M[pb][v], fmaxf(acc[pb][0][v], acc[pb][1][v]));
          const float ms = (mn == kNegInf) ? 0.f : mn;
          S[pb][v] = S[pb][v] * __expf(M[pb][v] - ms) + __expf(acc[pb][0][v] - ms) +
                     __expf(acc[pb][1][v] - ms);
          M[pb][v] = mn;
        }
      // per-row top lists: transpose each 16-component block through LDS so
      // lane p sees row p's values, components in ascending order
      if (wd == 0) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
          for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
            for (int v = 0; v < 4; ++v) tl[r16 * (BN + 1) + pb * 16 + 4 * g + v] = acc[pb][cb][v];
          wave_sync();
          if (lane < BN) {
#pragma unroll 4
            for (int j = 0; j < 16; ++j) top_insert<false>(tv, tk, tl[j * (BN + 1) + lane], compbase + cb * 16 + j);
          }
          wave_sync();
        }
      }
    }
    // merge the WC waves' lists and log-sum-exp partials of each row
    if (wd == 0) {
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float mr = row16_max(M[pb][v]);
          const float ms = (mr == kNegInf) ? 0.f : mr;
          const float sm = row16_sum(S[pb][v] * __expf(M[pb][v] - ms));
          if (r16 == 0) lpart[wc][pb * 16 + 4 * g + v] = (sm > 0.f) ? ms + __logf(sm) : kNegInf;
        }
      if (wc > 0 && lane < BN) {
#pragma unroll
        for (int i = 0; i < kTopN; ++i) {
          tl[i * BN + lane] = tv[i];
          tl[(kTopN + i) * BN + lane] = __int_as_float(tk[i]);
        }
      }
    }
    __syncthreads();
    if (tid < BN) {  // wave 0 (wc = 0, wd = 0): lane = row
#pragma unroll 1
      for (int q = 1; q < WC; ++q) {
        const float* o = tbuf[q];
#pragma unroll 1
        for (int i = 0; i < kTopN; ++i) {
          const float v = o[i * BN + tid];
          if (v == kNegInf) break;
          top_insert<true>(tv, tk, v, __float_as_int(o[(kTopN + i) * BN + tid]));
        }
      }
      if (tid < rows) {
        float Mx = kNegInf, Sx = 0.f;
#pragma unroll
        for (int k = 0; k < WC; ++k) lse_merge(Mx, Sx, lpart[k][tid], 1.f);
        const float lz = lse_of(Mx, Sx);
        int32_t* out = s.sel + (trow + tid) * stride;
        const bool ok = (tv[0] != kNegInf) && (tv[0] == tv[0]) && (lz == lz) && (lz != kNegInf);
        if (!ok) {
          __hip_atomic_store(&a.flags[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int j = 0; j < stride; ++j) out[j] = -1;
        } else {
          out[0] = tk[0];
          if (s.counts) atomicAdd(&s.counts[tk[0]], 1ull);
          int n = 1;
#pragma unroll
          for (int i = 1; i < kTopN; ++i) {
            if (i <= s.m && tv[i] != kNegInf && tv[i] - lz >= s.log_thr) {
              out[n++] = tk[i];
              if (s.counts) atomicAdd(&s.counts[tk[i]], 1ull);
            }
          }
          for (; n < stride; ++n) out[n] = -1;
        }
      }
    }
    __syncthreads();
  }
  if constexpr (REFINE) count_refined(a, nsel);
}

// ---------------------------------------------------------------------------
// Inverted-list construction.

// offsets[0..K] = exclusive scan of counts; cursor = offsets[0..K-1];
// nnz = offsets[K].  One workgroup of 1024 threads, each owning a contiguous
// run of lists.
__global__ void __launch_bounds__(1024) k_list_offsets(const unsigned long long* __restrict__ counts, int K,
                                                       int64_t* __restrict__ offsets, int64_t* __restrict__ cursor,
                                                       int64_t* __restrict__ nnz) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  const int per = (K + 1023) / 1024;
  const int k0 = tid * per, k1 = min(K, k0 + per);
  int64_t sum = 0;
  for (int k = k0; k < k1; ++k) sum += (int64_t)counts[k];
  part[tid] = sum;
  __syncthreads();
  // inclusive Hillis-Steele scan of the 1024 run totals
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t v = (tid >= o) ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = (tid > 0) ? part[tid - 1] : 0;
  for (int k = k0; k < k1; ++k) {
    offsets[k] = run;
    cursor[k] = run;
    run += (int64_t)counts[k];
  }
  if (tid == 1023) {
    offsets[K] = part[1023];
    *nnz = part[1023];
  }
}

__global__ void k_fill_u32(unsigned* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
__global__ void k_fill_u64a(unsigned long long* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// cnt[b][k] = number of selections of list k among rows of block b.
__global__ void k_block_count(const int32_t* __restrict__ sel, int64_t rows, int stride, int BR, int NB,
                              unsigned* __restrict__ cnt, int Kpad) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= NB) return;
  unsigned* c = cnt + (size_t)b * Kpad;
  const int64_t r1 = min(rows, (int64_t)(b + 1) * BR);
  for (int64_t r = (int64_t)b * BR; r < r1; ++r)
    for (int j = 0; j < stride; ++j) {
      const int k = sel[r * stride + j];
      if (k >= 0) c[k] += 1u;
    }
}

// Per list: exclusive scan of the block counts (in place); tot = chunk total.
__global__ void k_block_scan(unsigned* __restrict__ cnt, int NB, int K, int Kpad, unsigned* __restrict__ tot) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  unsigned run = 0;
  for (int b = 0; b < NB; ++b) {
    const unsigned t = cnt[(size_t)b * Kpad + k];
    cnt[(size_t)b * Kpad + k] = run;
    run += t;
  }
  tot[k] = run;
}

// One thread per row block places the block's rows, in row order, after the
// rows of earlier blocks and earlier chunks: ids ascending within each list.
// A position past the list's end (the second selection pass disagreeing
// with the first) is not written and raises flags[2].
__global__ void k_block_scatter(const int32_t* __restrict__ sel, int64_t rows, int stride, int BR, int NB,
                                unsigned* __restrict__ cnt, int Kpad, const int64_t* __restrict__ cursor,
                                const int64_t* __restrict__ offsets, int64_t row0, int32_t* __restrict__ ids,
                                int* __restrict__ flags) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= NB) return;
  unsigned* c = cnt + (size_t)b * Kpad;
  const int64_t r1 = min(rows, (int64_t)(b + 1) * BR);
  for (int64_t r = (int64_t)b * BR; r < r1; ++r)
    for (int j = 0; j < stride; ++j) {
      const int k = sel[r * stride + j];
      if (k >= 0) {
        const unsigned o = c[k];
        c[k] = o + 1u;
        const int64_t pos = cursor[k] + o;
        if (pos < offsets[k + 1])
          ids[pos] = (int32_t)(row0 + r);
        else
          __hip_atomic_store(&flags[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
}

__global__ void k_cursor_advance(int64_t* __restrict__ cursor, const unsigned* __restrict__ tot, int K) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < K) cursor[k] += (int64_t)tot[k];
}

// ---------------------------------------------------------------------------
// Host side.

static int grid_n(size_t n) {
  size_t g = (n + 255) / 256;
  if (g > 65535 * 4) g = 65535 * 4;
  return (int)(g < 1 ? 1 : g);
}

template <int WC, int WD, int DPW>
struct AKern {
  static constexpr int BN = bn_for(WD, DPW);
  template <int M>
  static void* assign() { return (void*)&k_assign<WC, WD, DPW, BN, M>; }
  static void* assign_split() {
    if constexpr (WD == 1) return (void*)&k_assign<WC, WD, DPW, BN, MODE_REFINE, true>;
    else return nullptr;
  }
};

// t[0..2]: float32, refined, float64 logits; t[3]: refined with split-bf16
// first-pass logits (nullptr where not built)
static bool alookup(int WC, int WD, int DPW, void* (&t)[4]) {
#define GMM_A(wc, wd, dpw)                                           \
  if (WC == wc && WD == wd && DPW == dpw) {                          \
    t[0] = AKern<wc, wd, dpw>::assign<0>();                          \
    t[1] = AKern<wc, wd, dpw>::assign<1>();                          \
    t[2] = AKern<wc, wd, dpw>::assign<2>();                          \
    t[3] = AKern<wc, wd, dpw>::assign_split();                       \
    return true;                                                     \
  }
  GMM_A(1, 1, 16) GMM_A(1, 1, 32) GMM_A(1, 1, 64) GMM_A(1, 1, 128)
  GMM_A(2, 1, 16) GMM_A(2, 1, 32) GMM_A(2, 1, 64) GMM_A(2, 1, 128)
  GMM_A(4, 1, 16) GMM_A(4, 1, 32) GMM_A(4, 1, 64) GMM_A(4, 1, 128)
  GMM_A(8, 1, 16) GMM_A(8, 1, 32) GMM_A(8, 1, 64) GMM_A(8, 1, 128)
  GMM_A(1, 8, 32) GMM_A(1, 8, 64) GMM_A(1, 8, 96) GMM_A(1, 8, 128)
#undef GMM_A
  return false;
}

// The assignment kernel's own wave count: 8 component-group waves per
// workgroup when there are enough groups (one workgroup per CU fits its LDS),
// else the E-step shape.
static int assign_wc(const Plan& p) {
  if (p.WD != 1) return p.WC;
  const int groups = p.Kpad / 32;
  return groups >= 8 ? 8 : p.WC;
}

hipError_t assign_occupancy(const Plan& p, int* occ) {
  void* t[4];
  const int wc = assign_wc(p);
  *occ = 0;
  if (!alookup(wc, p.WD, p.DPW, t)) return hipSuccess;  // no assignment kernel for this shape
  int o0 = 0, o1 = 0, o3 = 1 << 30;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o0, (const void*)t[0], 64 * wc * p.WD, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o1, (const void*)t[1], 64 * wc * p.WD, 0);
  if (e == hipSuccess && t[3])
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o3, (const void*)t[3], 64 * wc * p.WD, 0);
  if (e != hipSuccess) return e;
  *occ = o0 < o1 ? o0 : o1;
  if (o3 < *occ) *occ = o3;
  return hipSuccess;
}

hipError_t launch_assign_select(const Plan& p, const Workspace& w, const float* X, int64_t row0, int64_t rows,
                                int64_t ldx, float threshold, int max_extra, bool count, hipStream_t s) {
  void* t[4];
  const int wc = assign_wc(p);
  if (!alookup(wc, p.WD, p.DPW, t)) return hipErrorInvalidValue;
  EArgs a{};
  a.X = X;
  a.ldx = ldx;
  a.row0 = row0;
  a.nrows = rows;
  a.wop = w.wop;
  a.cvec = w.cvec;
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
  a.dma = (p.D == p.Dp) ? 1 : 0;
  a.wop64 = w.wop64;
  a.cvec64 = w.cvec64;
  AArgs sa{};
  sa.sel = w.asel;
  sa.counts = count ? w.acounts : nullptr;
  const double lt = log((double)threshold);
  sa.log_thr = (float)lt;
  sa.delta = (float)(1.0 - lt > 16.0 ? 1.0 - lt : 16.0);
  sa.m = max_extra;
  void* args[] = {&a, &sa};
  const int64_t tiles = (rows + p.BN - 1) / p.BN;
  const int64_t gmax = (int64_t)p.numCU * (p.occAssign > 0 ? p.occAssign : 1);
  const int grid = (int)(tiles < gmax ? tiles : gmax);
  void* kern = t[w.f64 ? 2 : (w.refine ? 1 : 0)];
  if (!w.f64 && w.refine && w.split && t[3]) {
    // split-bf16 first-pass logits, the refinement bound widened to match
    kern = t[3];
    a.wsp = w.wsplit;
    a.kappa = (float)((6.0 * p.Dp + 8.0) * 5.9604644775390625e-08 * (1.0 + 1.0 / 64.0) + 3.1 * 1.52587890625e-05);
  }
  return hipLaunchKernel(kern, dim3(grid), dim3(64 * wc * p.WD), args, 0, s);
}

hipError_t launch_assign_begin(const Plan& p, const Workspace& w, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u64a, dim3((p.Kpad + 255) / 256), dim3(256), 0, s, w.acounts, (size_t)p.Kpad);
  return hipGetLastError();
}

hipError_t launch_assign_offsets(const Plan& p, const Workspace& w, int64_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(k_list_offsets, dim3(1), dim3(1024), 0, s, w.acounts, p.K, offsets, w.acursor, w.annz);
  return hipGetLastError();
}

hipError_t launch_assign_scatter(const Plan& p, const Workspace& w, int64_t row0, int64_t rows, int max_extra,
                                 const int64_t* offsets, int32_t* ids, hipStream_t s) {
  const int NB = p.assignBlocks;
  const int BR = (int)((p.assignChunk + NB - 1) / NB);
  const int stride = 1 + max_extra;
  const size_t n = (size_t)NB * p.Kpad;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_n(n)), dim3(256), 0, s, w.acnt, n);
  hipLaunchKernelGGL(k_block_count, dim3((NB + 63) / 64), dim3(64), 0, s, w.asel, rows, stride, BR, NB, w.acnt,
                     p.Kpad);
  hipLaunchKernelGGL(k_block_scan, dim3((p.K + 255) / 256), dim3(256), 0, s, w.acnt, NB, p.K, p.Kpad, w.atot);
  hipLaunchKernelGGL(k_block_scatter, dim3((NB + 63) / 64), dim3(64), 0, s, w.asel, rows, stride, BR, NB, w.acnt,
                     p.Kpad, w.acursor, offsets, row0, ids, w.flags);
  hipLaunchKernelGGL(k_cursor_advance, dim3((p.K + 255) / 256), dim3(256), 0, s, w.acursor, w.atot, p.K);
  return hipGetLastError();
}

}  // namespace gmm
