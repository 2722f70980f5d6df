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
//  * k_assign_ct (split-bf16 first-pass logits, D <= 128) is component-major:
//    W is the MFMA A operand, so each lane holds one row's logits against
//    four components of each 16-component block, and a row's maximum,
//    log-sum-exp and thresholds are per-lane registers with two permlane
//    steps per group.  Top lists (2, 4 or 9 entries, by max_extra) are kept
//    per row in the registers of one owner lane, value descending, index
//    ascending; only logits that can be selected are inserted.  Because r is
//    increasing in l, the extras are the list's entries 2..m+1 that clear
//    log(threshold) against the row's log Z.  k_assign (float32 or float64
//    logits, and the shapes with several dim segments per component group)
//    has the E-step's row-major layout and merges its lists through LDS.
//  * Every logit that can be the argmax or clear the threshold lies within
//    delta = max(16, 1 - log threshold) nats of the row's largest logit, and
//    each of those is recomputed in float64, so ranking and threshold tests
//    use float64-accurate values.
//  * Lists are built deterministically without sorting: the counting sweep
//    counts list sizes (integer atomics), a scan gives the offsets; per chunk
//    of rows the selections (kept from the counting sweep, or selected again
//    when they could not be kept) are counted per (row block, list), those
//    counts scanned per list, and one thread per row block places its rows in
//    row order.
#include "gmm_device.h"

#include <limits.h>

namespace gmm {

constexpr int kTopN = 9;  // 1 + the largest max_extra

struct AArgs {
  int32_t* sel;                  // chunk rows x (1 + m) component ids, -1 = none
  unsigned long long* counts;    // K list sizes (pass A) or nullptr
  float log_thr;                 // log(threshold)
  float delta;                   // float64 window below the row's largest logit
  float cand_off;                // candidate bound offset: min(log(threshold), 0) with extras, 0 without
  int m;                         // max_extra
  const float4* gco;             // Kpad / 32 per-group error-bound coefficients (k_assign_ct)
};

constexpr float kLag = 20.f;     // lag of the log-sum-exp reference (e^20 * K stays finite)

// Insert (val, k) into a list sorted by value descending, index ascending:
// the carried entry walks down the list and trades places with every entry
// it ranks before, so the list stays sorted and the last entry falls off.
// Branch-free: the same instructions for every lane and any input.
__device__ __forceinline__ void top_insert(float (&tv)[kTopN], int (&tk)[kTopN], float val, int k) {
#pragma unroll
  for (int i = 0; i < kTopN; ++i) {
    const bool b = (val > tv[i]) || (val == tv[i] && k < tk[i]);
    const float ov = tv[i];
    const int ok = tk[i];
    tv[i] = b ? val : ov;
    tk[i] = b ? k : ok;
    val = b ? ov : val;
    k = b ? ok : k;
  }
}

// Orders a wave's LDS writes before its later reads by other lanes of the
// same wave (the fence waits for the wave's outstanding LDS operations).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// Row-major accumulators (lane (g, r16), register v: row 4 g + v of a
// 16-row block, component r16 of a 16-component block) with float32 or
// float64 MFMA logits; the split-bf16 variant is k_assign_ct below.
template <int WC, int WD, int DPW, int BN, int MODE>
__global__ void __launch_bounds__(kWave* WC* WD) k_assign(EArgs a, AArgs s) {
  using SH = Shape<WC, WD, DPW, BN>;
  constexpr bool REFINE = MODE == MODE_REFINE, F64 = MODE == MODE_FP64;
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
      // online log-sum-exp with a lagging reference: the running reference
      // M moves only when a logit exceeds it by more than kLag nats, so the
      // rescaling exponential is rare; S then holds terms up to e^kLag
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float mn = fmaxf(acc[pb][0][v], acc[pb][1][v]);
          if (mn > M[pb][v] + kLag) {
            S[pb][v] = (M[pb][v] == kNegInf) ? 0.f : S[pb][v] * __expf(M[pb][v] - mn);
            M[pb][v] = mn;
          }
          const float ms = (M[pb][v] == kNegInf) ? 0.f : M[pb][v];
          S[pb][v] += __expf(acc[pb][0][v] - ms) + __expf(acc[pb][1][v] - ms);
        }
      // per-row top lists.  Only a logit at or above the row's candidate bound
      // can be selected: the argmax is at least the largest lower bound Rlb of
      // the row's logits seen so far (less one float32 rounding of a refined
      // value), and an extra needs l - log Z >= log(threshold) with
      // log Z >= that maximum.  The wave's candidates are compacted into a
      // list (lane-major); lane p then inserts the entries of row p.
      if (wd == 0) {
        unsigned cbits = 0;
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if constexpr (!REFINE) Rlb[pb][v] = fmaxf(Rlb[pb][v], row16_max(fmaxf(acc[pb][0][v], acc[pb][1][v])));
            const float rb = Rlb[pb][v];
            const float bound = rb + s.cand_off - (fabsf(rb) * 2.4e-7f + 1e-6f);
            const bool rok = pb * 16 + 4 * g + v < rows;
            cbits |= (rok && acc[pb][0][v] >= bound ? 1u : 0u) << (pb * 8 + v);
            cbits |= (rok && acc[pb][1][v] >= bound ? 1u : 0u) << (pb * 8 + 4 + v);
          }
        const int c = __popc(cbits);
        int pre = 0, total = 0;
#pragma unroll
        for (int b = 0; b < 6; ++b) {
          const unsigned long long m = __ballot((c >> b) & 1);
          pre += (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u)) << b;
          total += __popcll(m) << b;
        }
        if (total > 0) {
          // tl[0, CAPC): candidate values; tl[CAPC, 2 CAPC): their codes
          // (register << 6 | lane) as float bit patterns
          constexpr int CAPC = TBW / 2;
          for (int b0 = 0; b0 < total; b0 += CAPC) {
            const int n = min(CAPC, total - b0);
            {
              int idx = pre - b0;
#pragma unroll
              for (int r = 0; r < NPB * 8; ++r)
                if ((cbits >> r) & 1u) {
                  if (idx >= 0 && idx < CAPC) {
                    tl[idx] = acc[r >> 3][(r >> 2) & 1][r & 3];
                    tl[CAPC + idx] = __int_as_float((r << 6) | lane);
                  }
                  ++idx;
                }
            }
            wave_sync();
            if (lane < BN) {
#pragma unroll 1
              for (int e = 0; e < n; ++e) {
                const int code = __float_as_int(tl[CAPC + e]);
                const float cvv = tl[e];
                const int r = code >> 6, ln = code & 63;
                if ((r >> 3) * 16 + 4 * (ln >> 4) + (r & 3) == lane)
                  top_insert(tv, tk, cvv, compbase + ((r >> 2) & 1) * 16 + (ln & 15));
              }
            }
            wave_sync();
          }
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
          top_insert(tv, tk, v, __float_as_int(o[(kTopN + i) * BN + tid]));
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
// Component-major soft assignment: split-bf16 first-pass logits, float64
// refinement, one dim segment per wave.  The logit MFMA takes W as its A
// operand, so lane (g, r16) holds, for 16-row block pb, the logits of row
// pb * 16 + r16 against components 4 g .. 4 g + 3 of both 16-component
// blocks of the group: a row's 32 logits sit in the four lanes r16 + 16 g',
// eight per lane.  A row's per-group maximum is then an in-lane maximum and
// two cross-lane steps (lanes 32 and 16 apart), and its log-sum-exp,
// running bound and thresholds are per-lane registers.  The fp32 error
// bound uses the group's coefficient maxima (gco), at least every
// component's own bound, so every logit the per-component test would refine
// is refined.

// max / sum of v over lanes l and l ^ 32 (permlane32 swap: the two halves of
// the wave trade places), and over lanes l and l ^ 16 (permlane16 swap).
__device__ __forceinline__ float xmax32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Logits of one component group, component-major: W is the MFMA A operand
// and x the B operand (both have the same per-lane register form), so lane
// (g, r16), register v of block cb accumulates component cb * 16 + 4 g + v
// for row pb * 16 + r16.  Split-bf16, three passes per block as in
// logit_tile_split.  The W operands of each step are fetched one step ahead
// (two register sets, steps taken in pairs), and the last step fetches the
// first step of the next group (wn0, wn1; the current group's again when
// there is none), so the L2 latency of W overlaps MFMA work or the previous
// group's epilogue.  wf holds the step-0 operands on entry and the next
// group's on exit; cf, likewise, the starting values c of the next group's
// accumulators (cvn: its first component's c).
template <class SH, int DPW>
__device__ __forceinline__ void logit_group_ct(const __bf16* __restrict__ xsb, const __bf16* __restrict__ ws0,
                                               const __bf16* __restrict__ ws1, const __bf16* __restrict__ wn0,
                                               const __bf16* __restrict__ wn1, const float* __restrict__ cvn,
                                               bf16x8 (&wf)[4], f4 (&cf)[2], f4 (&acc)[SH::NPB][2], int lane) {
  using SR = SplitRow<DPW, false>;
  constexpr int S = SR::S;
  const int g = lane >> 4, r16 = lane & 15;
  const __bf16* arow = xsb + r16 * SR::XSR + g * 8;
  // W operands of step st of the blocks b0, b1 into wd (issued, not waited for)
  auto fetch = [&](bf16x8 (&wd)[4], const __bf16* b0, const __bf16* b1, int st) {
    wd[0] = *reinterpret_cast<const bf16x8*>(b0 + ((st * 2 + 0) * kWave + lane) * 8);
    wd[1] = *reinterpret_cast<const bf16x8*>(b0 + ((st * 2 + 1) * kWave + lane) * 8);
    wd[2] = *reinterpret_cast<const bf16x8*>(b1 + ((st * 2 + 0) * kWave + lane) * 8);
    wd[3] = *reinterpret_cast<const bf16x8*>(b1 + ((st * 2 + 1) * kWave + lane) * 8);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMA work
  };
  auto step = [&](const bf16x8 (&wc)[4], int st) {
    auto ld = [&](int pb, int off) {
      return *reinterpret_cast<const bf16x8*>(arow + pb * 16 * SR::XSR + off + st * 32);
    };
    bf16x8 ahn = ld(0, 0), aln = ld(0, SR::LO);
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb) {
      const bf16x8 ah = ahn, al = aln;
      if (pb + 1 < SH::NPB) {
        ahn = ld(pb + 1, 0);
        aln = ld(pb + 1, SR::LO);
      }
      // small terms first
      acc[pb][0] = mfma_bf16(wc[0], al, acc[pb][0]);
      acc[pb][1] = mfma_bf16(wc[2], al, acc[pb][1]);
      acc[pb][0] = mfma_bf16(wc[1], ah, acc[pb][0]);
      acc[pb][1] = mfma_bf16(wc[3], ah, acc[pb][1]);
      acc[pb][0] = mfma_bf16(wc[0], ah, acc[pb][0]);
      acc[pb][1] = mfma_bf16(wc[2], ah, acc[pb][1]);
    }
  };
  if constexpr (S % 2 == 0) {
    bf16x8 wb[4];
#pragma unroll 1
    for (int st = 0; st < S; st += 2) {
      fetch(wb, ws0, ws1, st + 1);
      step(wf, st);
      const bool last = st + 2 == S;  // uniform: pointer selects, no branch
      fetch(wf, last ? wn0 : ws0, last ? wn1 : ws1, last ? 0 : st + 2);
      step(wb, st + 1);
    }
  } else {
    static_assert(S == 1, "odd step count: one step");
    bf16x8 wb[4];
    fetch(wb, wn0, wn1, 0);
    step(wf, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) wf[i] = wb[i];
  }
  cf[0] = *reinterpret_cast<const f4*>(cvn + 4 * g);
  cf[1] = *reinterpret_cast<const f4*>(cvn + 16 + 4 * g);
}

__device__ __forceinline__ float max8(const f4& p, const f4& q) {
  return fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])), fmaxf(fmaxf(q[0], q[1]), fmaxf(q[2], q[3])));
}

// Order-preserving map of float32 onto int32 (LDS integer max of floats):
// non-negative floats keep their bits, negative ones have the magnitude
// bits flipped, so a < b as floats iff fkey(a) < fkey(b) as ints.
__device__ __forceinline__ int fkey(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float funkey(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }

// Float64 logits of the list entries [0, count) of one wave: entry codes
// (register << 6 | lane) in elist, component-major registers (register
// pb * 8 + cb * 4 + v of lane (g, r16): row pb * 16 + r16, component
// compbase + cb * 16 + 4 g + v); 16 lanes per logit, four logits per pass,
// results in rlist.  The same float64 arithmetic and order per logit as the
// row-major refine_tile.
template <class SH, int DPW>
__device__ __forceinline__ void refine_entries_ct(const unsigned short* __restrict__ elist, float* __restrict__ rlist,
                                                  int count, const float* __restrict__ xt, const EArgs& a, double C,
                                                  int compbase, int lane) {
  constexpr int DPT = DPW / 16;            // dims per lane (16 lanes per logit)
  constexpr int DCH = DPT;  // every load of a pass in flight together (one L2 round trip per pass)
  const int g = lane >> 4, r16 = lane & 15;
  for (int base = 0; base < count; base += 4) {
    const int e = base + g;
    const bool live = e < count;
    const int code = live ? (int)elist[e] : 0;
    const int r = code >> 6, ln = code & 63;
    const int pt = (r >> 3) * 16 + (ln & 15);
    const int comp = compbase + ((r >> 2) & 1) * 16 + 4 * (ln >> 4) + (r & 3);
    const double2* wr = a.w64 + (size_t)comp * a.Dp;
    const double cf = (live && r16 == 0) ? a.cfull[comp] : 0.0;
    double t = 0.0;
    if (live) {
#pragma unroll
      for (int j0 = 0; j0 < DPT; j0 += DCH) {
        double2 ab[DCH];
        float xv[DCH];
#pragma unroll
        for (int j = 0; j < DCH; ++j) {
          const int d = r16 + 16 * (j0 + j);  // < Dp: padded dims have a = b = 0
          ab[j] = wr[d];
          xv[j] = xt[pt * SH::RS + d];
        }
#pragma unroll
        for (int j = 0; j < DCH; ++j) {
          const double x = (double)xv[j];
          t = fma(ab[j].x, x * x, fma(ab[j].y, x, t));
        }
      }
    }
    t += __shfl_xor(t, 8);
    t += __shfl_xor(t, 4);
    t += __shfl_xor(t, 2);
    t += __shfl_xor(t, 1);
    if (live && r16 == 0) rlist[e] = (float)((cf - C) + t);
  }
}

// Mask of the lanes whose register e = pb * 8 + cb * 4 + v is >= lim[pb].
template <int NPB>
__device__ __forceinline__ unsigned long long sel_mask(const f4 (&acc)[NPB][2], const float (&lim)[NPB], int e) {
  return __ballot(acc[e >> 3][(e >> 2) & 1][e & 3] >= lim[e >> 3]);
}

// Lanes below this one in mask m.
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// List of the registers >= lim, register by register (register order, then
// lane order), one ballot per register: entry codes (register << 6 | lane)
// go to codes16[i], or, with vals given, the value to vals[i] and the code
// (as float bits) to codesf[i], for the first cap entries.  Returns the
// count over the wave (also past cap).
template <int NPB>
__device__ __forceinline__ int list_ge(const f4 (&acc)[NPB][2], const float (&lim)[NPB], int lane, int cap,
                                       unsigned short* __restrict__ codes16, float* __restrict__ vals,
                                       float* __restrict__ codesf) {
  int n = 0;
#pragma unroll
  for (int e = 0; e < NPB * 8; ++e) {
    const unsigned long long m = sel_mask(acc, lim, e);
    if (m) {
      if ((m >> lane) & 1ull) {
        const int i = n + lanes_below(m);
        if (i < cap) {
          if (codes16) codes16[i] = (unsigned short)((e << 6) | lane);
          if (vals) {
            vals[i] = acc[e >> 3][(e >> 2) & 1][e & 3];
            codesf[i] = __int_as_float((e << 6) | lane);
          }
        }
      }
      n += __popcll(m);
    }
  }
  return n;
}

// Marks the accumulators as changed (no instruction): later selection masks
// are recomputed from them instead of being kept in scalar registers.
template <int NPB>
__device__ __forceinline__ void opaque(f4 (&acc)[NPB][2]) {
#pragma unroll
  for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) asm volatile("" : "+v"(acc[pb][cb][v]));
}

// Float64 recomputation of the logits L >= tq[pb] of one wave's group
// (tq > -inf, so -inf logits, padding included, never qualify).  Up to
// kRefineCap of them: one list, built and taken back register by register;
// more: lane-major batches from per-lane bit masks.  Returns their number.
template <class SH, int DPW>
__device__ __forceinline__ int refine_ct(f4 (&acc)[SH::NPB][2], const float (&tq)[SH::NPB],
                                         const float* __restrict__ xt, const EArgs& a, double C, int compbase,
                                         float* __restrict__ rlist, unsigned short* __restrict__ elist, int lane) {
  constexpr int NREG = SH::NPB * 8;
  const int total = list_ge(acc, tq, lane, kRefineCap, elist, nullptr, nullptr);
  if (total == 0) return 0;
  if (total <= kRefineCap) {
    wave_sync();
    refine_entries_ct<SH, DPW>(elist, rlist, total, xt, a, C, compbase, lane);
    wave_sync();
    opaque(acc);
    int n = 0;
#pragma unroll
    for (int e = 0; e < NREG; ++e) {
      const unsigned long long m = sel_mask(acc, tq, e);
      if (m) {
        if ((m >> lane) & 1ull) acc[e >> 3][(e >> 2) & 1][e & 3] = rlist[n + lanes_below(m)];
        n += __popcll(m);
      }
    }
    wave_sync();
    return total;
  }
  unsigned sel = 0;
#pragma unroll
  for (int e = 0; e < NREG; ++e)
    sel |= (acc[e >> 3][(e >> 2) & 1][e & 3] >= tq[e >> 3] ? 1u : 0u) << e;
  const int c = __popc(sel);
  int pre = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) pre += lanes_below(__ballot((c >> b) & 1)) << b;
  wave_sync();  // the register-order list above is overwritten
  for (int b0 = 0; b0 < total; b0 += kRefineCap) {
    const int count = min(kRefineCap, total - b0);
    {
      unsigned bits = sel;
      int idx = pre - b0;
      while (bits) {
        const int r = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (idx >= 0 && idx < kRefineCap) elist[idx] = (unsigned short)((r << 6) | lane);
        ++idx;
      }
    }
    wave_sync();
    refine_entries_ct<SH, DPW>(elist, rlist, count, xt, a, C, compbase, lane);
    wave_sync();
    {
      int idx = pre - b0;
#pragma unroll
      for (int r = 0; r < NREG; ++r)
        if ((sel >> r) & 1u) {
          if (idx >= 0 && idx < kRefineCap) acc[r >> 3][(r >> 2) & 1][r & 3] = rlist[idx];
          ++idx;
        }
    }
    wave_sync();
  }
  return total;
}

// Insert (val, k) into a list of N entries sorted by value descending,
// index ascending (as top_insert).
template <int N>
__device__ __forceinline__ void top_insert_n(float (&tv)[N], int (&tk)[N], float val, int k) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool b = (val > tv[i]) || (val == tv[i] && k < tk[i]);
    const float ov = tv[i];
    const int ok = tk[i];
    tv[i] = b ? val : ov;
    tk[i] = b ? k : ok;
    val = b ? ov : val;
    k = b ? ok : k;
  }
}

// TOPN: list entries per row (1 + the largest max_extra it serves).
template <int WC, int DPW, int BN, int TOPN>
__global__ void __launch_bounds__(kWave* WC) k_assign_ct(EArgs a, AArgs s) {
  using SH = Shape<WC, 1, DPW, BN>;
  using SPR = SplitRow<DPW, false>;
  constexpr int NPB = SH::NPB;
  constexpr bool NIS = DPW == 128;       // row norms formed while splitting the rows
  constexpr int LSTW = 2 * TOPN * BN > 512 ? 2 * TOPN * BN : 512;  // per wave: lists, or candidates
  constexpr int CAPC = LSTW / 2;         // candidates per compaction batch
  __shared__ __attribute__((aligned(16))) float xt[SH::TILE];
  __shared__ __attribute__((aligned(16))) __bf16 xsb[BN * SPR::XSR];
  __shared__ float tbuf[WC][LSTW];
  __shared__ float lpart[WC][BN];
  __shared__ float2 nrm[BN];
  __shared__ int cbnd[BN];  // shared candidate bound per row (fkey), the largest any wave has shown
  __shared__ float rlist[WC][kRefineCap];
  __shared__ unsigned short elist[WC][kRefineCap];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int ncg = a.Kpad / 32;
  const double C = *a.cshift;
  const int nt = (int)((a.nrows + BN - 1) / BN);
  const int stride = 1 + s.m;
  unsigned nsel = 0;  // refined logits of this wave (counted once at the end)
  float* tl = tbuf[w];

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
    if (tid < BN) cbnd[tid] = fkey(kNegInf);  // published by the second barrier
    __syncthreads();
    split_rows<SH, DPW, false>(xt, xsb, w, NIS ? nrm : nullptr);
    if constexpr (!NIS) row_norms2<SH, DPW>(xt, nrm, a.Dp);
    __syncthreads();
    float2 nn[NPB];
    bool rok[NPB];
    float M[NPB], S[NPB], Rlb[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      nn[pb] = nrm[pb * 16 + r16];
      rok[pb] = pb * 16 + r16 < rows;
      M[pb] = kNegInf;
      S[pb] = 0.f;
      Rlb[pb] = kNegInf;
    }
    float tv[TOPN];
    int tk[TOPN];
#pragma unroll
    for (int i = 0; i < TOPN; ++i) {
      tv[i] = kNegInf;
      tk[i] = INT_MAX;
    }
    auto wblk = [&](int cb16) { return a.wsp + (size_t)cb16 * SPR::WBLK; };
    // the first step's W operands and the c values of this wave's next group
    bf16x8 wf[4];
    f4 cf[2];
    if (w < ncg) {
      const __bf16* b0 = wblk(2 * w);
      const __bf16* b1 = wblk(2 * w + 1);
      wf[0] = *reinterpret_cast<const bf16x8*>(b0 + lane * 8);
      wf[1] = *reinterpret_cast<const bf16x8*>(b0 + (kWave + lane) * 8);
      wf[2] = *reinterpret_cast<const bf16x8*>(b1 + lane * 8);
      wf[3] = *reinterpret_cast<const bf16x8*>(b1 + (kWave + lane) * 8);
      cf[0] = *reinterpret_cast<const f4*>(a.cvec + w * 32 + 4 * g);
      cf[1] = *reinterpret_cast<const f4*>(a.cvec + w * 32 + 16 + 4 * g);
    }
    for (int cg = w; cg < ncg; cg += WC) {
      const int compbase = cg * 32;
      const int cgn = (cg + WC < ncg) ? cg + WC : cg;
      const float4 gc = s.gco[cg];  // used after the contraction
      f4 acc[NPB][2];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        acc[pb][0] = cf[0];
        acc[pb][1] = cf[1];
      }
      logit_group_ct<SH, DPW>(xsb, wblk(2 * cg), wblk(2 * cg + 1), wblk(2 * cgn), wblk(2 * cgn + 1),
                              a.cvec + cgn * 32, wf, cf, acc, lane);
      // 1. running lower bound Rlb of the row's largest logit (the largest
      //    L - E seen so far) and the refinement test: L + E_k >= Rlb - delta
      //    implies L >= tq, since E_k <= Eg (the margin covers the roundings
      //    of both forms); tq > -inf keeps -inf logits (padding) out
      float tq[NPB];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        const float Eg = a.kappa * (gc.x * nn[pb].x + gc.y * nn[pb].y + gc.z);
        const float lb = xmax16(xmax32(max8(acc[pb][0], acc[pb][1]) - Eg));
        Rlb[pb] = fmaxf(Rlb[pb], lb);
        const float thr = Rlb[pb] - s.delta;
        tq[pb] = rok[pb] ? fmaxf((thr - Eg) - (fabsf(thr) + Eg) * 0x1p-21f, -__FLT_MAX__) : kPosInf;
      }
      nsel += (unsigned)refine_ct<SH, DPW>(acc, tq, xt, a, C, compbase, rlist[w], elist[w], lane);
      // 2. online log-sum-exp with a lagging reference: M moves only when a
      //    logit exceeds it by more than kLag nats
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        const float mn = max8(acc[pb][0], acc[pb][1]);
        if (mn > M[pb] + kLag) {
          S[pb] = (M[pb] == kNegInf) ? 0.f : S[pb] * __expf(M[pb] - mn);
          M[pb] = mn;
        }
        const float ms = (M[pb] == kNegInf) ? 0.f : M[pb];
        float sm = 0.f;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int v = 0; v < 4; ++v) sm += __expf(acc[pb][cb][v] - ms);
        S[pb] += sm;
      }
      // 3. top-list candidates.  A logit can be selected only if it is at
      //    least (a) the row's argmax lower bound Rlb (less one float32
      //    rounding of a refined value) plus min(log threshold, 0), since an
      //    extra needs l - log Z >= log threshold and log Z >= Rlb, and
      //    (b) the TOPN-th value of any wave's list of the row.  Every wave
      //    shows its bounds in cbnd (LDS integer max), so each filters with
      //    the largest bound shown so far; which bound a wave sees changes
      //    only which non-selectable logits it inserts, not the lists'
      //    selectable entries.  Candidates are listed register by register
      //    and lane p inserts the entries of row p.
      float bnd[NPB];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        const float rb = Rlb[pb];
        const float own = rb + s.cand_off - (fabsf(rb) * 2.4e-7f + 1e-6f);
        const int seen = atomicMax(&cbnd[pb * 16 + r16], fkey(own));
        bnd[pb] = rok[pb] ? fmaxf(own, funkey(seen)) : kPosInf;
      }
      const int ncand = list_ge(acc, bnd, lane, CAPC, nullptr, tl, tl + CAPC);
      if (ncand) {
        for (int b0 = 0; b0 < ncand; b0 += CAPC) {
          const int n = min(CAPC, ncand - b0);
          if (ncand > CAPC) {
            // more than one batch: lane-major order from per-lane bit masks
            unsigned cbits = 0;
#pragma unroll
            for (int e = 0; e < NPB * 8; ++e)
              cbits |= (acc[e >> 3][(e >> 2) & 1][e & 3] >= bnd[e >> 3] ? 1u : 0u) << e;
            const int c = __popc(cbits);
            int pre = 0;
#pragma unroll
            for (int b = 0; b < 6; ++b) pre += lanes_below(__ballot((c >> b) & 1)) << b;
            int idx = pre - b0;
#pragma unroll
            for (int r = 0; r < NPB * 8; ++r)
              if ((cbits >> r) & 1u) {
                if (idx >= 0 && idx < CAPC) {
                  tl[idx] = acc[r >> 3][(r >> 2) & 1][r & 3];
                  tl[CAPC + idx] = __int_as_float((r << 6) | lane);
                }
                ++idx;
              }
          }
          wave_sync();
          if (lane < BN) {
#pragma unroll 1
            for (int e = 0; e < n; ++e) {
              const int code = __float_as_int(tl[CAPC + e]);
              const float cvv = tl[e];
              const int r = code >> 6, ln = code & 63;
              if ((r >> 3) * 16 + (ln & 15) == lane)
                top_insert_n<TOPN>(tv, tk, cvv, compbase + ((r >> 2) & 1) * 16 + 4 * (ln >> 4) + (r & 3));
            }
            atomicMax(&cbnd[lane], fkey(tv[TOPN - 1]));
          }
          wave_sync();
        }
      }
    }
    // merge the four lanes of each row, then the WC waves
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      const float mr = xmax16(xmax32(M[pb]));
      const float ms = (mr == kNegInf) ? 0.f : mr;
      const float sm = xsum16(xsum32(S[pb] * __expf(M[pb] - ms)));
      if (g == 0) lpart[w][pb * 16 + r16] = (sm > 0.f) ? ms + __logf(sm) : kNegInf;
    }
    if (w > 0 && lane < BN) {
#pragma unroll
      for (int i = 0; i < TOPN; ++i) {
        tl[i * BN + lane] = tv[i];
        tl[(TOPN + i) * BN + lane] = __int_as_float(tk[i]);
      }
    }
    __syncthreads();
    if (tid < BN) {  // wave 0: lane = row
#pragma unroll 1
      for (int q = 1; q < WC; ++q) {
        const float* o = tbuf[q];
#pragma unroll 1
        for (int i = 0; i < TOPN; ++i) {
          const float v = o[i * BN + tid];
          if (v == kNegInf) break;
          top_insert_n<TOPN>(tv, tk, v, __float_as_int(o[(TOPN + i) * BN + tid]));
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
          for (int i = 1; i < TOPN; ++i) {
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
  count_refined(a, nsel);
}

// Per-group error-bound coefficients of k_assign_ct: for each 32-component
// group, the maxima over its components of max|a|, max|b| and |c - C|
// (padding contributes 0).  One wave per group.
__global__ void k_group_coefs(const float2* __restrict__ abmax, const float* __restrict__ cvec,
                              float4* __restrict__ gco, int ngroups) {
  const int grp = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & 63;
  if (grp >= ngroups) return;
  float ma = 0.f, mb = 0.f, mc = 0.f;
  if (lane < 32) {
    const int k = grp * 32 + lane;
    const float2 ab = abmax[k];
    const float c = cvec[k];
    ma = ab.x;
    mb = ab.y;
    mc = (c == kNegInf) ? 0.f : fabsf(c);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ma = fmaxf(ma, __shfl_xor(ma, o));
    mb = fmaxf(mb, __shfl_xor(mb, o));
    mc = fmaxf(mc, __shfl_xor(mc, o));
  }
  if (lane == 0) gco[grp] = make_float4(ma, mb, mc, 0.f);
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
  template <int TOPN>
  static void* assign_split() {
    if constexpr (WD == 1) return (void*)&k_assign_ct<WC, DPW, BN, TOPN>;
    else return nullptr;
  }
};

// t[0..2]: float32, refined, float64 logits; t[3..5]: refined with split-bf16
// first-pass logits (nullptr where not built)
static bool alookup(int WC, int WD, int DPW, void* (&t)[6]) {
#define GMM_A(wc, wd, dpw)                                           \
  if (WC == wc && WD == wd && DPW == dpw) {                          \
    t[0] = AKern<wc, wd, dpw>::assign<0>();                          \
    t[1] = AKern<wc, wd, dpw>::assign<1>();                          \
    t[2] = AKern<wc, wd, dpw>::assign<2>();                          \
    t[3] = AKern<wc, wd, dpw>::assign_split<2>();                    \
    t[4] = AKern<wc, wd, dpw>::assign_split<4>();                    \
    t[5] = AKern<wc, wd, dpw>::assign_split<kTopN>();                \
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
  void* t[6];
  const int wc = assign_wc(p);
  *occ = 0;
  if (!alookup(wc, p.WD, p.DPW, t)) return hipSuccess;  // no assignment kernel for this shape
  int o = 1 << 30;
  for (int i = 0; i < 6; ++i) {
    if (i == 2 || !t[i]) continue;  // the float64 variant has its own LDS; it takes the same grid
    int oi = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&oi, (const void*)t[i], 64 * wc * p.WD, 0);
    if (e != hipSuccess) return e;
    if (oi < o) o = oi;
  }
  *occ = o;
  return hipSuccess;
}

hipError_t launch_assign_select(const Plan& p, const Workspace& w, const float* X, int64_t row0, int64_t rows,
                                int64_t ldx, float threshold, int max_extra, bool count, int32_t* sel,
                                hipStream_t s) {
  void* t[6];
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
  sa.sel = sel;
  sa.counts = count ? w.acounts : nullptr;
  const double lt = log((double)threshold);
  sa.log_thr = (float)lt;
  sa.delta = (float)(1.0 - lt > 16.0 ? 1.0 - lt : 16.0);
  sa.cand_off = max_extra > 0 ? (float)(lt < 0.0 ? lt : 0.0) : 0.f;
  sa.m = max_extra;
  sa.gco = w.agco;
  void* args[] = {&a, &sa};
  const int64_t tiles = (rows + p.BN - 1) / p.BN;
  const int64_t gmax = (int64_t)p.numCU * (p.occAssign > 0 ? p.occAssign : 1);
  const int grid = (int)(tiles < gmax ? tiles : gmax);
  void* kern = t[w.f64 ? 2 : (w.refine ? 1 : 0)];
  void* ct = t[max_extra <= 1 ? 3 : (max_extra <= 3 ? 4 : 5)];  // list length 2, 4 or 9
  if (!w.f64 && w.refine && w.split && ct) {
    // split-bf16 first-pass logits, the refinement bound widened to match
    kern = ct;
    a.wsp = w.wsplit;
    a.kappa = (float)((6.0 * p.Dp + 8.0) * 5.9604644775390625e-08 * (1.0 + 1.0 / 64.0) + 3.1 * 1.52587890625e-05);
  }
  return hipLaunchKernel(kern, dim3(grid), dim3(64 * wc * p.WD), args, 0, s);
}

hipError_t launch_assign_begin(const Plan& p, const Workspace& w, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u64a, dim3((p.Kpad + 255) / 256), dim3(256), 0, s, w.acounts, (size_t)p.Kpad);
  const int ng = p.Kpad / 32;
  hipLaunchKernelGGL(k_group_coefs, dim3((ng + 3) / 4), dim3(256), 0, s, w.abmax, w.cvec, w.agco, ng);
  return hipGetLastError();
}

hipError_t launch_assign_offsets(const Plan& p, const Workspace& w, int64_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(k_list_offsets, dim3(1), dim3(1024), 0, s, w.acounts, p.K, offsets, w.acursor, w.annz);
  return hipGetLastError();
}

hipError_t launch_assign_scatter(const Plan& p, const Workspace& w, const int32_t* sel, int64_t row0, int64_t rows,
                                 int max_extra, const int64_t* offsets, int32_t* ids, hipStream_t s) {
  const int NB = p.assignBlocks;
  const int BR = (int)((p.assignChunk + NB - 1) / NB);
  const int stride = 1 + max_extra;
  const size_t n = (size_t)NB * p.Kpad;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_n(n)), dim3(256), 0, s, w.acnt, n);
  hipLaunchKernelGGL(k_block_count, dim3((NB + 63) / 64), dim3(64), 0, s, sel, rows, stride, BR, NB, w.acnt,
                     p.Kpad);
  hipLaunchKernelGGL(k_block_scan, dim3((p.K + 255) / 256), dim3(256), 0, s, w.acnt, NB, p.K, p.Kpad, w.atot);
  hipLaunchKernelGGL(k_block_scatter, dim3((NB + 63) / 64), dim3(64), 0, s, sel, rows, stride, BR, NB, w.acnt,
                     p.Kpad, w.acursor, offsets, row0, ids, w.flags);
  hipLaunchKernelGGL(k_cursor_advance, dim3((p.K + 255) / 256), dim3(256), 0, s, w.acursor, w.atot, p.K);
  return hipGetLastError();
}

}  // namespace gmm
