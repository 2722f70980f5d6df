// Device building blocks shared by the E-step and soft-assignment kernels
// (gfx950): MFMA and DPP helpers, the kernel argument block, the tile shape,
// X-tile staging into LDS, the logit contraction, and the float64 refinement
// of the logits that can matter.  Method: "Flash-GMM: A Memory-Efficient
// Kernel for Scalable Soft Clustering", Section 3.1 and Algorithm 1 (tiles of
// rows against blocks of components, log-densities computed on chip).
#pragma once
#include "gmm_internal.h"

#include <math.h>

namespace gmm {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef double d4 __attribute__((ext_vector_type(4)));

static constexpr float kNegInf = -__builtin_huge_valf();
static constexpr float kPosInf = __builtin_huge_valf();
static constexpr double kLog2Pi = 1.8378770664093454835606594728112;

// Logit precision of a kernel variant: float32 MFMA; float32 MFMA with the
// logits near each row's maximum recomputed in float64; float64 MFMA.
enum { MODE_FP32 = 0, MODE_REFINE = 1, MODE_FP64 = 2 };

__device__ __forceinline__ d4 mfma64(double a, double b, d4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Butterfly over the 16 lanes of a DPP row: mirror, half-mirror, xor 2, xor 1.
// IK: on order-preserving integer keys (non-negative floats keep their bits,
// negative ones have the magnitude bits flipped), so each step is one
// v_max_i32 / v_min_i32 with the DPP read folded in, where a float maximum of
// a DPP operand needs a separate move and a NaN-quieting pass; NaN takes the
// identity key, so NaN lanes are ignored as by fmaxf / fminf (a row of NaN
// gives NaN).  Measured: 0.5 % faster in the diagonal E-step, 2 % slower in
// the isotropic one (instruction scheduling), so each kernel picks.
template <int CTRL, int ID>
__device__ __forceinline__ int dppk(int k) {
  return __builtin_amdgcn_update_dpp(ID, k, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int okey(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float okey_inv(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }
// NANID = false (integer keys only): NaN is not mapped to the identity but
// keeps its key, above +inf's, so a NaN lane makes the row's maximum NaN
// (two instructions fewer per row; for rows whose NaN reaches the
// statistics anyway).
template <bool IK = false, bool NANID = true>
__device__ __forceinline__ float row16_max(float v) {
  if constexpr (IK) {
    constexpr int ID = (int)0x80000000;
    int k = (!NANID || v == v) ? okey(v) : ID;
    k = max(k, dppk<0x140, ID>(k));
    k = max(k, dppk<0x141, ID>(k));
    k = max(k, dppk<0x4E, ID>(k));
    k = max(k, dppk<0xB1, ID>(k));
    return okey_inv(k);
  } else {
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0xB1>(v));
    return v;
  }
}
template <bool IK = false>
__device__ __forceinline__ float row16_min(float v) {
  if constexpr (IK) {
    constexpr int ID = 0x7FFFFFFF;
    int k = (v == v) ? okey(v) : ID;
    k = min(k, dppk<0x140, ID>(k));
    k = min(k, dppk<0x141, ID>(k));
    k = min(k, dppk<0x4E, ID>(k));
    k = min(k, dppk<0xB1, ID>(k));
    return okey_inv(k);
  } else {
    v = fminf(v, dpp<0x140>(v));
    v = fminf(v, dpp<0x141>(v));
    v = fminf(v, dpp<0x4E>(v));
    v = fminf(v, dpp<0xB1>(v));
    return v;
  }
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0x140>(v);
  v += dpp<0x141>(v);
  v += dpp<0x4E>(v);
  v += dpp<0xB1>(v);
  return v;
}

// max(a, b) in one v_med3_f32 (the median of a, b and +inf), where fmaxf
// first quiets both operands.  With a NaN operand the result is the other
// operand or NaN; either way a NaN logit still reaches the row's sum of
// exponentials and the statistics, where the numeric check reports it.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, kPosInf); }

// Natural log of a row's sum of exponentials taken relative to its largest
// term, so s >= 1 (that term is exp(0)), or s = 0 for a row of -inf (giving
// -inf): the hardware base-2 logarithm times ln 2, without the denormal and
// range handling of the library logarithm, which such s never needs.
__device__ __forceinline__ float ln_rowsum(float s) { return __builtin_amdgcn_logf(s) * 0.693147180559945309f; }

// log(exp(a) + exp(b)) merge of two (max, sum) pairs; -inf safe.
__device__ __forceinline__ void lse_merge(float& M, float& S, float m2, float s2) {
  float mn = fmaxf(M, m2);
  float ms = (mn == kNegInf) ? 0.f : mn;
  S = S * __expf(M - ms) + s2 * __expf(m2 - ms);
  M = mn;
}
// S >= 1 (its largest term is exp(0)) or S = 0 with M = -inf
__device__ __forceinline__ float lse_of(float M, float S) { return (M == kNegInf ? 0.f : M) + ln_rowsum(S); }

struct EArgs {
  const float* X;
  int64_t ldx;
  int64_t row0;   // first row of this launch (two-sweep chunk)
  int64_t nrows;  // rows of this launch
  const float* wop;
  const float* cvec;
  float* logz;    // two-sweep: log Z per row of the chunk
  double* slots;
  double* llslots;
  unsigned long long* xbuf;
  int* flags;
  int K, D, Kpad, P, R, Dp;
  int slot_acc;   // 1: add into slots / llslots
  // float64 refinement of the logits that matter
  int refine;
  float kappa;           // fp32 logit error bound factor ((2 Dp + 8) 2^-24)
  const double2* w64;    // Kpad x Dp  (a, b) in float64
  const double* cfull;   // Kpad  float64 component constants
  const double* cshift;  // global logit offset C
  const float2* abmax;   // Kpad  (max_d |a_kd|, max_d |b_kd|)
  unsigned long long* nrefined;  // count of refined logits (statistics only)
  int dma;               // 1: X tiles by LDS DMA (D == Dp)
  const double* wop64;   // Kpad x 2 Dp  [a | b] in float64, MFMA-operand order (as wop)
  const double* cvec64;  // Kpad  c_k - C in float64 (-inf: padding)
  // isotropic kernel: W = mu / s^2 in its MFMA-operand order, 1 / (2 s^2)
  const float* wiso;     // Kpad x Dp
  const float* ivec;     // Kpad  (0: padding)
  // split-bf16 logits: W = W_hi + W_lo in bfloat16, in the operand order of
  // v_mfma_f32_16x16x32_bf16 (see logit_tile_split)
  const __bf16* wsp;     // Kpad x 2 Dp x 2
};

// ---------------------------------------------------------------------------
// Shared device pieces, parameterised by the workgroup shape.
template <int WC, int WD, int DPW, int BN>
struct Shape {
  static constexpr int NT = kWave * WC * WD;
  static constexpr int NPB = BN / 16;         // 16-row MFMA blocks per tile
  static constexpr int NFB = DPW / 8;         // 16-wide feature blocks per wave (2*DPW/16)
  static constexpr int SS = DPW;              // LDS floats per wave segment of a row (its dims)
  static constexpr int RS = WD * SS + 4;      // LDS floats per row: x (Dp) + 4 pad (rows 4 banks apart)
  static constexpr int TILE = BN * RS;        // LDS floats per tile buffer
  static constexpr int CPR = WD * SS / 4;     // 16-byte chunks of x per row
  // Two workgroups per CU for 4-wave shapes (their barrier, exchange and
  // refinement phases then overlap the other workgroup's MFMA work), one
  // otherwise.
  static constexpr int WGS_PER_CU = (WC * WD == 4) ? 2 : 1;
  // partial-logit exchange across the dim-segment waves, one 16-row block per
  // pass (the blocks of a tile go through it in turn): WD partials of 8 values
  // per lane, then the reduced values of every block (as float32)
  static constexpr int RED = (WD > 1) ? (WD + NPB) * WC * 8 * kWave : 1;
  static constexpr int NBUF = (TILE * 8 + RED * 4 <= (WGS_PER_CU == 1 ? 140 : 68) * 1024) ? 2 : 1;
  static constexpr int HALF = DPW / 2;
  // refinement: the WD waves of a component group share the float64 passes
  // when the group is the whole workgroup, else each wave refines its copy
  static constexpr bool COOP = (WD > 1) && (WC == 1);
};

// Stage rows [r0, r0+rows) of X into an LDS tile buffer: row p holds x
// (Dp floats, dims past D zero) at p * RS; rows past `rows` are zero.  x^2 is
// formed where it is used.  Register path, for any D; split into a
// global-load half and an LDS-store half.
template <class SH, int DPW>
struct Stage {
  static constexpr int Q4 = SH::CPR;
  static constexpr int ITEMS = (SH::TILE / SH::RS) * Q4;  // BN * Dp/4 float4s
  static constexpr int PER = (ITEMS + SH::NT - 1) / SH::NT;
  f4 v[PER];

  __device__ __forceinline__ void load(const float* __restrict__ X, int64_t ldx, int64_t r0, int rows, int D) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int it = threadIdx.x + k * SH::NT;
      const int pt = it / Q4;
      const int d = (it - pt * Q4) << 2;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (it < ITEMS && pt < rows && d < D) {
        // streamed once: a non-temporal load leaves the caches to the parameters
        x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(X + (r0 + pt) * ldx + d));
        if (d + 3 >= D) {
          if (d + 1 >= D) x[1] = 0.f;
          if (d + 2 >= D) x[2] = 0.f;
          x[3] = 0.f;
        }
      }
      v[k] = x;
    }
  }
  __device__ __forceinline__ void store(float* __restrict__ xt) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int it = threadIdx.x + k * SH::NT;
      if (it < ITEMS) {
        const int pt = it / Q4;
        const int c = it - pt * Q4;
        *reinterpret_cast<f4*>(xt + pt * SH::RS + c * 4) = v[k];
      }
    }
  }
};

// The same tile by LDS DMA (global_load_lds_dwordx4): no registers held, no
// VALU work; usable when every row has D == Dp valid floats (no dims to zero).
// One instruction moves up to 64 consecutive 16-byte chunks of one row (lane
// i -> LDS address M0 + 16 i, M0 = the row segment's start); rows past `rows`
// repeat the last valid row (finite, never used).  Completion is tracked by
// vmcnt: dma_wait() before the barrier that precedes reading the tile.
// The SH::NT / 64 waves that share the load pass their index w.
template <class SH>
__device__ __forceinline__ void stage_dma(float* __restrict__ xt, const float* __restrict__ X, int64_t ldx,
                                          int64_t r0, int rows, int w = (int)(threadIdx.x >> 6)) {
  constexpr int BN = SH::TILE / SH::RS;
  constexpr int IPR = (SH::CPR + 63) / 64;  // instructions per row
  constexpr int NW = SH::NT / kWave;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform: taken into a scalar register, the row
  // addresses are scalar arithmetic and only the lane offset is per lane
  w = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int i = w; i < BN * IPR; i += NW) {
    const int pt = i / IPR, part = i - pt * IPR;
    const int c = part * 64 + lane;
    const int row = pt < rows ? pt : rows - 1;
    if (c < SH::CPR) {
      const float* src = X + (r0 + row) * ldx + c * 4;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(xt + pt * SH::RS + part * 256), 16,
                                       0, 0);
    }
  }
}

// Segment-major staging: wave wd loads dims [wd * DPW, (wd + 1) * DPW) of rows
// [r0, r0 + BN) into its own block of LDS, row p of the block at p * SRS
// (SRS = DPW + 4: the pad keeps 16 rows of an MFMA operand load on distinct
// banks).  By LDS DMA, 16 bytes per lane, each instruction filling 1 KiB of
// the block (a pad slot loads the row's first chunk again), rows past `rows`
// repeating the last row; or through registers (any D: dims past D and rows
// past `rows` zero).  Only the wave itself reads the block, so its own wait
// makes it usable.
template <int DPW, int BN>
__device__ __forceinline__ void stage_seg(float* __restrict__ blk, const float* __restrict__ X, int64_t ldx,
                                          int64_t r0, int rows, int D, int wd, bool dma) {
  constexpr int SRS = DPW + 4;
  constexpr int CH = SRS / 4;         // 16-byte slots per block row (the last is pad)
  constexpr int UNITS = BN * CH;      // slots per block
  const int lane = threadIdx.x & 63;
  const int d0 = wd * DPW;
  if (dma) {
#pragma unroll
    for (int i = 0; i < (UNITS + 63) / 64; ++i) {
      const int u = i * 64 + lane;
      if (u < UNITS) {
        const int pt = u / CH, c = u - pt * CH;
        const int row = pt < rows ? pt : rows - 1;
        const float* src = X + (r0 + row) * ldx + d0 + (c < CH - 1 ? c * 4 : 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(blk + i * 256), 16, 0, 0);
      }
    }
  } else {
#pragma unroll 4
    for (int u = lane; u < UNITS; u += 64) {
      const int pt = u / CH, c = u - pt * CH;
      const int d = d0 + c * 4;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (c < CH - 1 && pt < rows && d < D) {
        const float* src = X + (r0 + pt) * ldx + d;
        if (d + 4 <= D) {
          x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src));
        } else {
          for (int q = 0; q < D - d; ++q) x[q] = src[q];
        }
      }
      *reinterpret_cast<f4*>(blk + u * 4) = x;
    }
  }
}

// Wait for this wave's outstanding global memory operations (LDS DMA
// included): s_waitcnt vmcnt(0).
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Isotropic logits x . (mu_k / s_k^2) of one wave (WD = 1): A = x of 16
// points, lane (g, r16) giving row r16's dims g*Q + 4 s4 .. +3 (Q = DPW / 4),
// B = the matching W values of 16 components, DPW/16 groups of four k-steps;
// W fetched one group ahead.  acc must hold the starting value.
template <class SH, int DPW>
__device__ __forceinline__ void logit_tile_iso(const float* __restrict__ xt, const float* __restrict__ w0,
                                               const float* __restrict__ w1, f4 (&acc)[SH::NPB][2], int lane) {
  const int g = lane >> 4, r16 = lane & 15;
  constexpr int Q = DPW / 4, S4 = DPW / 16;
  const float* arow = xt + r16 * SH::RS + g * Q;
  f4 b0 = *reinterpret_cast<const f4*>(w0 + lane * 4);
  f4 b1 = *reinterpret_cast<const f4*>(w1 + lane * 4);
#pragma unroll 2
  for (int s4 = 0; s4 < S4; ++s4) {
    const int nx = (s4 + 1 < S4) ? s4 + 1 : s4;
    const f4 b0n = *reinterpret_cast<const f4*>(w0 + (nx * kWave + lane) * 4);
    const f4 b1n = *reinterpret_cast<const f4*>(w1 + (nx * kWave + lane) * 4);
    auto ld = [&](int pb) { return *reinterpret_cast<const f4*>(arow + pb * 16 * SH::RS + s4 * 4); };
    f4 an = ld(0);
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb) {
      const f4 a = an;
      if (pb + 1 < SH::NPB) an = ld(pb + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[pb][0] = mfma(a[i], b0[i], acc[pb][0]);
        acc[pb][1] = mfma(a[i], b1[i], acc[pb][1]);
      }
    }
    b0 = b0n;
    b1 = b1n;
  }
}

// Row norms for the isotropic kernel: nrm as row_norms2 (rounded up, for the
// error bound) and xn2[pt] = ||x||^2 in float32 (fixed order) for the logits
// and Q.
template <class SH, int DPW>
__device__ __forceinline__ void row_norms_iso(const float* __restrict__ xt, float2* __restrict__ nrm,
                                              float* __restrict__ xn2) {
  constexpr int BN = SH::TILE / SH::RS;
  constexpr int TPR = SH::NT / BN;
  const int pt = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  float n2 = 0.f, n1 = 0.f;
  if (pt < BN) {
    const float* xrow = xt + pt * SH::RS;
#pragma unroll
    for (int q = sub; q < SH::CPR; q += TPR) {
      const f4 xv = *reinterpret_cast<const f4*>(xrow + q * 4);
      n2 += (xv[0] * xv[0] + xv[1] * xv[1]) + (xv[2] * xv[2] + xv[3] * xv[3]);
      n1 += (fabsf(xv[0]) + fabsf(xv[1])) + (fabsf(xv[2]) + fabsf(xv[3]));
    }
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) {
    n2 += __shfl_xor(n2, o);
    n1 += __shfl_xor(n1, o);
  }
  if (pt < BN && sub == 0) {
    nrm[pt] = make_float2(n2 * (1.f + 1e-6f), n1 * (1.f + 1e-6f));
    xn2[pt] = n2;
  }
}

// Partial logits of one wave: its 2 component blocks x NPB point blocks over
// its dim segment.  acc must hold the starting value (c or 0).  Per group of
// four k-steps the A operands (one ds_read_b128 per point block) are consumed
// point block by point block, so only two are live; the W operands (B, from
// L2) are fetched one group ahead.
template <class SH, int DPW>
__device__ __forceinline__ void logit_tile(const float* __restrict__ xt, const float* __restrict__ w0,
                                           const float* __restrict__ w1, f4 (&acc)[SH::NPB][2],
                                           int lane, int wd) {
  const int g = lane >> 4, r16 = lane & 15;
  // MFMA k index g: g = 0, 1 take dims [0, HALF) of the segment (x^2, x),
  // g = 2, 3 dims [HALF, DPW)
  const bool sq = (g & 1) == 0;
  const float* arow = xt + r16 * SH::RS + wd * DPW + (g >> 1) * SH::HALF;
  constexpr int S4 = DPW / 8;
  f4 b0 = *reinterpret_cast<const f4*>(w0 + lane * 4);
  f4 b1 = *reinterpret_cast<const f4*>(w1 + lane * 4);
#pragma unroll 2
  for (int s4 = 0; s4 < S4; ++s4) {
    const int nx = (s4 + 1 < S4) ? s4 + 1 : s4;
    const f4 b0n = *reinterpret_cast<const f4*>(w0 + (nx * kWave + lane) * 4);
    const f4 b1n = *reinterpret_cast<const f4*>(w1 + (nx * kWave + lane) * 4);
    auto ld = [&](int pb) { return *reinterpret_cast<const f4*>(arow + pb * 16 * SH::RS + s4 * 4); };
    f4 an = ld(0);
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb) {
      f4 a = an;
      if (pb + 1 < SH::NPB) an = ld(pb + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sq ? a[i] * a[i] : a[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[pb][0] = mfma(a[i], b0[i], acc[pb][0]);
        acc[pb][1] = mfma(a[i], b1[i], acc[pb][1]);
      }
    }
    b0 = b0n;
    b1 = b1n;
  }
}

// ---------------------------------------------------------------------------
// Split-bfloat16 logits.  A float x is carried as x_hi + x_lo with
// x_hi = bf16(x) and x_lo = bf16(x - x_hi) (x - x_hi is exact in float32), so
// |x - x_hi - x_lo| <= 2^-16 |x|; W likewise.  The logit contraction
// sum_f x_f w_f is then three bfloat16 MFMA passes, x_hi w_hi + x_hi w_lo +
// x_lo w_hi (products exact in float32, sums in float32), leaving out
// x_lo w_lo: at most about 3 * 2^-16 |x_f w_f| per feature on top of the
// float32 summation error of the 6 Dp partial products.  Each bfloat16 MFMA
// covers 32 features at 16x the float32 MFMA rate, so the three passes cost
// under a fifth of the float32 contraction.  The error bound of the float64
// refinement is widened to match, so the refined results are unchanged.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4 mfma_bf16(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS layout of one split row (WD = 1): hi operands then lo operands, each
// S MFMA steps x 4 lane groups x 8 features, plus 8 pad values (consecutive
// rows 4 banks apart).  Diagonal model (S = DPW / 16): step s, lane group g
// holds features x^2 (g even) or x (g odd) of dims (g / 2) * DPW / 2 + 8 s
// .. + 7.  Isotropic model (x only, S = DPW / 32): lane group g holds dims
// g * DPW / 4 + 8 s .. + 7.  Both keep the float32 kernels' assignment of
// dims to lane groups, so W needs only regrouping.
template <int DPW, bool ISO = false>
struct SplitRow {
  static constexpr int S = ISO ? DPW / 32 : DPW / 16;
  static constexpr int LO = ISO ? DPW : 2 * DPW;  // bf16 offset of the lo operands
  static constexpr int XSR = 2 * LO + 8;          // bf16 per row
  static constexpr int WBLK = S * 2 * 512;        // bf16 of split W per 16-component block
};

// Convert the rows this wave staged (rows w, w + NW, ... of the tile: the
// LDS-DMA row assignment with one instruction per row) from float32 in xt
// to split bfloat16 operands in xsb.  Called after this wave's dma_wait, so
// the rows it reads are its own DMA's; the next barrier publishes xsb.
// With nrm given (DPW = 128: one row per 16-lane DPP row and pass), the
// rows' ||x||^2 and ||x||_1 are formed on the way (slightly rounded up, as
// row_norms2) and written to nrm, published by the same barrier.
template <class SH, int DPW, bool ISO>
__device__ __forceinline__ void split_rows(const float* __restrict__ xt, __bf16* __restrict__ xsb, int w,
                                           float2* __restrict__ nrm = nullptr) {
  using SR = SplitRow<DPW, ISO>;
  constexpr int BN = SH::TILE / SH::RS;
  constexpr int NW = SH::NT / kWave;
  constexpr int CH = DPW / 8;                 // 8-dim chunks per row
  constexpr int RPW = (BN + NW - 1) / NW;     // rows per wave
  constexpr int HS = DPW / 16;                // chunks per half (= S)
  const int lane = threadIdx.x & 63;
  static_assert(CH == 16 || CH == 8 || CH == 4 || CH == 2, "8-dim chunks per row");
#pragma unroll 1  // one item at a time (registers, as in split_stats)
  for (int it = lane; it < RPW * CH; it += kWave) {
    const int rl = it / CH, c = it - rl * CH;
    const int pt = w + rl * NW;
    if (nrm) {
      // CH == 16: the 16 chunks of row rl sit in one DPP row of the wave
      // (uniform trip count: RPW * CH is a multiple of 64 for DPW = 128)
      float n2 = 0.f, n1 = 0.f;
      if (pt < BN) {
        const float* src = xt + pt * SH::RS + c * 8;
        const f4 u0 = *reinterpret_cast<const f4*>(src);
        const f4 u1 = *reinterpret_cast<const f4*>(src + 4);
        n2 = ((u0[0] * u0[0] + u0[1] * u0[1]) + (u0[2] * u0[2] + u0[3] * u0[3])) +
             ((u1[0] * u1[0] + u1[1] * u1[1]) + (u1[2] * u1[2] + u1[3] * u1[3]));
        n1 = ((fabsf(u0[0]) + fabsf(u0[1])) + (fabsf(u0[2]) + fabsf(u0[3]))) +
             ((fabsf(u1[0]) + fabsf(u1[1])) + (fabsf(u1[2]) + fabsf(u1[3])));
      }
      n2 = row16_sum(n2);
      n1 = row16_sum(n1);
      if (pt < BN && c == 0) nrm[pt] = make_float2(n2 * (1.f + 1e-6f), n1 * (1.f + 1e-6f));
    }
    if (pt < BN) {
      const float* src = xt + pt * SH::RS + c * 8;
      const f4 u0 = *reinterpret_cast<const f4*>(src);
      const f4 u1 = *reinterpret_cast<const f4*>(src + 4);
      __bf16* row = xsb + pt * SR::XSR;
      bf16x8 xh, xl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (i < 4) ? u0[i] : u1[i - 4];
        const __bf16 hx = (__bf16)x;
        xh[i] = hx;
        xl[i] = (__bf16)(x - (float)hx);
      }
      if constexpr (ISO) {
        const int st = c % SR::S, gg = c / SR::S;  // step, lane group
        *reinterpret_cast<bf16x8*>(row + (st * 4 + gg) * 8) = xh;
        *reinterpret_cast<bf16x8*>(row + SR::LO + (st * 4 + gg) * 8) = xl;
      } else {
        bf16x8 qh, ql;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = (i < 4) ? u0[i] : u1[i - 4];
          const float q = x * x;
          const __bf16 hq = (__bf16)q;
          qh[i] = hq;
          ql[i] = (__bf16)(q - (float)hq);
        }
        const int st = c % HS, gq = c / HS;  // step, half
        *reinterpret_cast<bf16x8*>(row + (st * 4 + 2 * gq) * 8) = qh;
        *reinterpret_cast<bf16x8*>(row + (st * 4 + 2 * gq + 1) * 8) = xh;
        *reinterpret_cast<bf16x8*>(row + SR::LO + (st * 4 + 2 * gq) * 8) = ql;
        *reinterpret_cast<bf16x8*>(row + SR::LO + (st * 4 + 2 * gq + 1) * 8) = xl;
      }
    }
  }
}

// Logits of one wave (WD = 1) from the split operands: per step the W hi/lo
// of both component blocks (from L2), per point block the x hi/lo of 16 rows
// (one ds_read_b128 each), three MFMAs per block.  No operand is fetched a
// step ahead and the step loop is not unrolled: the registers that would
// take cost more in spills of the whole kernel than the exposed load latency
// (measured 748 against 813 ms per EM iteration at N=1e8, K=1024).
// ws0/ws1: the two component blocks' split W, [step][hi, lo][lane][8].
// acc must hold the starting value.
template <class SH, int DPW, bool ISO>
__device__ __forceinline__ void logit_tile_split(const __bf16* __restrict__ xsb, const __bf16* __restrict__ ws0,
                                                 const __bf16* __restrict__ ws1, f4 (&acc)[SH::NPB][2], int lane) {
  using SR = SplitRow<DPW, ISO>;
  const int g = lane >> 4, r16 = lane & 15;
  const __bf16* arow = xsb + r16 * SR::XSR + g * 8;
  auto wl = [&](const __bf16* wb, int st, int hl) {
    return *reinterpret_cast<const bf16x8*>(wb + ((st * 2 + hl) * kWave + lane) * 8);
  };
#pragma unroll 1
  for (int st = 0; st < SR::S; ++st) {
    const bf16x8 h0 = wl(ws0, st, 0), l0 = wl(ws0, st, 1), h1 = wl(ws1, st, 0), l1 = wl(ws1, st, 1);
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
      acc[pb][0] = mfma_bf16(al, h0, acc[pb][0]);
      acc[pb][1] = mfma_bf16(al, h1, acc[pb][1]);
      acc[pb][0] = mfma_bf16(ah, l0, acc[pb][0]);
      acc[pb][1] = mfma_bf16(ah, l1, acc[pb][1]);
      acc[pb][0] = mfma_bf16(ah, h0, acc[pb][0]);
      acc[pb][1] = mfma_bf16(ah, h1, acc[pb][1]);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-bfloat16 statistics.  The statistics contraction has no float64
// safety net, so it takes the three-part split v = v_hi + v_mid + v_lo
// (bf16 each; v - v_hi and the next remainder are exact in float32, and the
// last remainder has at most 8 significant bits, so the three parts hold a
// float32 v exactly) for both operands, and the six products whose parts'
// orders add up to at most two: hi.hi, hi.mid, mid.hi, hi.lo, lo.hi,
// mid.mid.  The products left out are below 2^-23 of |r x|, at the float32
// rounding level of the fp32 MFMA it replaces, at six 16-cycle bf16 MFMAs
// per 32 rows against eight 32-cycle fp32 ones.
__device__ __forceinline__ void split3(float v, __bf16& h, __bf16& m, __bf16& l) {
  h = (__bf16)v;
  const float r1 = v - (float)h;
  m = (__bf16)r1;
  l = (__bf16)(r1 - (float)m);
}

// LDS layout of the statistics operands of one tile (WD = 1):
// [part][q][fb][lane][8] bf16, q the pair of 16-row blocks (rows 32 q ..),
// fb the 16-feature block; lane (g, f16) holds feature fb * 16 + f16 of the
// 8 rows 32 q + 4 g + {0..3} and 32 q + 16 + 4 g + {0..3}, the rows whose
// responsibilities lane group g holds in the logit accumulators of blocks
// 2q and 2q + 1.  Features follow the statistics slots.  Diagonal model:
// quarter f / HALF of the segment holds x^2 (even) or x (odd) of dims
// (quarter / 2) * HALF + f % HALF.  Isotropic model: feature f is x of dim f.
template <class SH, int DPW, bool ISO = false>
struct StatSplit {
  static constexpr int BN = SH::TILE / SH::RS;
  static constexpr int NQ = BN / 32;
  static constexpr int NFB = ISO ? DPW / 16 : DPW / 8;
  static constexpr int PS = NQ * NFB * 512;  // bf16 per part
  static constexpr int SIZE = 3 * PS;
};

// Raw tile -> statistics operands (all threads of the workgroup; reads rows
// any wave staged, so after a barrier that follows the staging).
template <class SH, int DPW, bool ISO>
__device__ __forceinline__ void split_stats(const float* __restrict__ xt, __bf16* __restrict__ xsb) {
  using ST = StatSplit<SH, DPW, ISO>;
  constexpr int HALF = DPW / 2;
  // one item at a time: the build runs while every accumulator is live, and
  // items in flight together would spill them
#pragma unroll 1
  for (int it = threadIdx.x; it < ST::NQ * ST::NFB * kWave; it += SH::NT) {
    const int ln = it & 63, rest = it >> 6;
    const int fb = rest % ST::NFB, q = rest / ST::NFB;
    const int gg = ln >> 4, f = fb * 16 + (ln & 15);
    const int quarter = f / HALF;
    const bool sq = !ISO && (quarter & 1) == 0;
    const int dim = ISO ? f : (quarter >> 1) * HALF + f % HALF;
    bf16x8 h, m, l;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int row = 32 * q + ((jj < 4) ? 0 : 16) + 4 * gg + (jj & 3);
      const float x = xt[row * SH::RS + dim];
      __bf16 a, b, c;
      split3(sq ? x * x : x, a, b, c);
      h[jj] = a;
      m[jj] = b;
      l[jj] = c;
    }
    __bf16* dst = xsb + (size_t)(q * ST::NFB + fb) * 512 + ln * 8;
    *reinterpret_cast<bf16x8*>(dst) = h;
    *reinterpret_cast<bf16x8*>(dst + ST::PS) = m;
    *reinterpret_cast<bf16x8*>(dst + 2 * ST::PS) = l;
  }
}

// Statistics of one wave from the split operands: r of the lane's rows
// (the logit accumulators, already responsibilities) split in registers per
// pair of row blocks, B operands from LDS per feature block (not fetched
// ahead, for the same register reason as the logits), six MFMAs per
// (component block, feature block), small products first.  ONEHOT (r is 0
// or 1, exact in bf16): r_mid = r_lo = 0, so three MFMAs, r against the three
// parts of x.
template <class SH, int DPW, bool ISO, bool ONEHOT>
__device__ __forceinline__ void stats_tile_split(const f4 (&r)[SH::NPB][2], const __bf16* __restrict__ xsb,
                                                 f4 (&sacc)[2][StatSplit<SH, DPW, ISO>::NFB], int lane) {
  using ST = StatSplit<SH, DPW, ISO>;
#pragma unroll
  for (int q = 0; q < ST::NQ; ++q) {
    bf16x8 ah[2], am[2], al[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        __bf16 a, b, c;
        split3((jj < 4) ? r[2 * q][cb][jj] : r[2 * q + 1][cb][jj - 4], a, b, c);
        ah[cb][jj] = a;
        am[cb][jj] = b;
        al[cb][jj] = c;
      }
    const __bf16* bq = xsb + (size_t)q * ST::NFB * 512 + lane * 8;
    auto ldb = [&](int fb, int part) { return *reinterpret_cast<const bf16x8*>(bq + fb * 512 + part * ST::PS); };
#pragma unroll
    for (int fb = 0; fb < ST::NFB; ++fb) {
      const bf16x8 bh = ldb(fb, 0), bm = ldb(fb, 1), bl = ldb(fb, 2);
      if constexpr (ONEHOT) {
        sacc[0][fb] = mfma_bf16(ah[0], bl, sacc[0][fb]);
        sacc[1][fb] = mfma_bf16(ah[1], bl, sacc[1][fb]);
        sacc[0][fb] = mfma_bf16(ah[0], bm, sacc[0][fb]);
        sacc[1][fb] = mfma_bf16(ah[1], bm, sacc[1][fb]);
        sacc[0][fb] = mfma_bf16(ah[0], bh, sacc[0][fb]);
        sacc[1][fb] = mfma_bf16(ah[1], bh, sacc[1][fb]);
        continue;
      }
      sacc[0][fb] = mfma_bf16(al[0], bh, sacc[0][fb]);
      sacc[1][fb] = mfma_bf16(al[1], bh, sacc[1][fb]);
      sacc[0][fb] = mfma_bf16(ah[0], bl, sacc[0][fb]);
      sacc[1][fb] = mfma_bf16(ah[1], bl, sacc[1][fb]);
      sacc[0][fb] = mfma_bf16(am[0], bm, sacc[0][fb]);
      sacc[1][fb] = mfma_bf16(am[1], bm, sacc[1][fb]);
      sacc[0][fb] = mfma_bf16(am[0], bh, sacc[0][fb]);
      sacc[1][fb] = mfma_bf16(am[1], bh, sacc[1][fb]);
      sacc[0][fb] = mfma_bf16(ah[0], bm, sacc[0][fb]);
      sacc[1][fb] = mfma_bf16(ah[1], bm, sacc[1][fb]);
      sacc[0][fb] = mfma_bf16(ah[0], bh, sacc[0][fb]);
      sacc[1][fb] = mfma_bf16(ah[1], bh, sacc[1][fb]);
    }
  }
}

// With WD > 1 the WD waves of a component group hold partial logits over
// their dim segments; sum them in a fixed order through LDS so every wave of
// the group ends with bit-identical full logits.
template <class SH, int WC, int WD>
__device__ __forceinline__ void reduce_partial_logits(float* __restrict__ red, f4 (&acc)[SH::NPB][2],
                                                      int lane, int wc, int wd) {
  if constexpr (WD > 1) {
    // wave wd sums values e = wd, wd + WD, ... of the 8 per lane over the WD
    // partials (in wave order) and posts the float32 sum; every wave then
    // reads the 8 sums it needs
    constexpr int PER = 8;  // values per lane and 16-row block
    float* mine = red + ((wd * WC + wc) * PER) * kWave + lane;
    float* sums = red + WD * WC * PER * kWave;
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) mine[(cb * 4 + v) * kWave] = acc[pb][cb][v];
      __syncthreads();
      for (int e = wd; e < PER; e += WD) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < WD; ++k) s += red[((k * WC + wc) * PER + e) * kWave + lane];
        sums[((pb * WC + wc) * PER + e) * kWave + lane] = s;
      }
      __syncthreads();
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[pb][cb][v] = sums[((pb * WC + wc) * PER + cb * 4 + v) * kWave + lane];
    }
  }
}

template <class T>
__device__ __forceinline__ const T* wop_block(const T* wop, int cb16, int WD, int wd, int DPW) {
  return wop + (size_t)(cb16 * WD + wd) * (DPW / 8) * 256;
}

// Float64 logits of one wave's 2 component blocks x NPB point blocks on
// v_mfma_f64_16x16x4_f64: A = x converted exactly, squared exactly for the x^2
// features; B = [a | b] in float64.  The f64 instruction's accumulator puts
// row g + 4v of the 16x16 result in lane g*16 + column, register v (the f32
// one puts row 4g + v there), so A's row r takes point 4 (r % 4) + r / 4 and
// the registers come out in the f32 point order.  With WD > 1 the dim-segment partials are
// summed in a fixed order through LDS (red64: WD*WC*8*64 doubles, one 16-row block at a time).  The
// result, (c_k - C) + sum, is rounded once to float32 into acc.  xw is the
// wave's dim segment of tile row 0, rows RSX floats apart.
template <class SH, int WC, int WD, int DPW, int RSX = SH::RS>
__device__ __forceinline__ void logits_f64(const float* __restrict__ xw, const double* __restrict__ w0,
                                           const double* __restrict__ w1, double c0, double c1,
                                           f4 (&acc)[SH::NPB][2], double* __restrict__ red64, int lane, int wc,
                                           int wd) {
  const int g = lane >> 4, r16 = lane & 15;
  const bool sq = (g & 1) == 0;
  const int prow = 4 * (r16 & 3) + (r16 >> 2);
  const float* arow = xw + prow * RSX + (g >> 1) * SH::HALF;
  constexpr int S4 = DPW / 8;
  d4 p[SH::NPB][2];
#pragma unroll
  for (int pb = 0; pb < SH::NPB; ++pb) {
    p[pb][0] = d4{c0, c0, c0, c0};
    p[pb][1] = d4{c1, c1, c1, c1};
  }
#pragma unroll 2
  for (int s4 = 0; s4 < S4; ++s4) {
    const d4 b0 = *reinterpret_cast<const d4*>(w0 + (s4 * kWave + lane) * 4);
    const d4 b1 = *reinterpret_cast<const d4*>(w1 + (s4 * kWave + lane) * 4);
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb) {
      const f4 a = *reinterpret_cast<const f4*>(arow + pb * 16 * RSX + s4 * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double x = (double)a[i];
        const double ai = sq ? x * x : x;
        p[pb][0] = mfma64(ai, b0[i], p[pb][0]);
        p[pb][1] = mfma64(ai, b1[i], p[pb][1]);
      }
    }
  }
  if constexpr (WD > 1) {
    // as reduce_partial_logits: wave wd sums values e = wd, wd + WD, ... over
    // the WD partials in float64 (in wave order), rounds the sum once to
    // float32 and posts it; every wave then reads the 8 sums it needs
    constexpr int PER = 8;  // values per lane and 16-row block
    double* mine = red64 + ((wd * WC + wc) * PER) * kWave + lane;
    float* sums = reinterpret_cast<float*>(red64 + WD * WC * PER * kWave);
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) mine[(cb * 4 + v) * kWave] = p[pb][cb][v];
      __syncthreads();
      for (int e = wd; e < PER; e += WD) {
        double t = 0.0;
#pragma unroll
        for (int k = 0; k < WD; ++k) t += red64[((k * WC + wc) * PER + e) * kWave + lane];
        sums[((pb * WC + wc) * PER + e) * kWave + lane] = (float)t;
      }
      __syncthreads();
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[pb][cb][v] = sums[((pb * WC + wc) * PER + cb * 4 + v) * kWave + lane];
    }
  } else {
#pragma unroll
    for (int pb = 0; pb < SH::NPB; ++pb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[pb][cb][v] = (float)p[pb][cb][v];
  }
}

// ---------------------------------------------------------------------------
// Float64 refinement of the logits that can matter.
//
// The fp32 expanded quadratic c + sum_d (a x^2 + b x) cancels terms whose
// magnitudes add up to S = sum_d (|a| x^2 + |b x|) + |c - C|, so its error is
// bounded by E = (2 Dp + 8) 2^-24 S (Dp k-step roundings of partial sums that
// never exceed S, plus the roundings of x^2, a, b and c).  For data spread
// over many cluster widths that is 1e-3..1e-2 nats, too much for overlapping
// components.  Every logit with L + E >= (a lower bound of the row's largest
// logit) - kDelta is recomputed from float64 a, b, c and exact float64 x^2;
// all others have responsibility < e^-kDelta relative to the row maximum, so
// their fp32 error is immaterial.  For clustered data a row has a handful of
// such logits, so the float64 work is a few percent of the MFMA work.
constexpr float kDelta = 16.f;
constexpr int kRefineCap = 256;  // list entries per component group and batch

// Bound on the fp32 error of one logit: kappa (max|a_k| ||x||^2 + max|b_k| ||x||_1 + |c_k - C|).
__device__ __forceinline__ float err_bound(float kappa, float al, float be, float cv, float2 nn) {
  return kappa * (al * nn.x + be * nn.y + cv);
}

// Per-lane error-bound coefficients of this wave's two component blocks:
// co = (max|a|, max|b|, |c - C|) for the lane's component in block 0, then 1.
__device__ __forceinline__ void lane_coefs(const EArgs& a, int compbase, int r16, float (&co)[6]) {
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int k = compbase + cb * 16 + r16;
    const float2 ab = a.abmax[k];
    const float c = a.cvec[k];
    co[3 * cb + 0] = ab.x;
    co[3 * cb + 1] = ab.y;
    co[3 * cb + 2] = (c == kNegInf) ? 0.f : fabsf(c);
  }
}

// ||x||^2 and ||x||_1 of each staged row into nrm[pt] (slightly rounded up).
// TPR threads per row read its chunks (any order) and combine with shuffles.
template <class SH, int DPW>
__device__ __forceinline__ void row_norms2(const float* __restrict__ xt, float2* __restrict__ nrm, int Dp) {
  constexpr int BN = SH::TILE / SH::RS;
  constexpr int TPR = SH::NT / BN;  // threads per row (power of two)
  const int pt = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  float n2 = 0.f, n1 = 0.f;
  if (pt < BN) {
    const float* xrow = xt + pt * SH::RS;
#pragma unroll
    for (int q = sub; q < SH::CPR; q += TPR) {
      const f4 xv = *reinterpret_cast<const f4*>(xrow + q * 4);
      n2 += (xv[0] * xv[0] + xv[1] * xv[1]) + (xv[2] * xv[2] + xv[3] * xv[3]);
      n1 += (fabsf(xv[0]) + fabsf(xv[1])) + (fabsf(xv[2]) + fabsf(xv[3]));
    }
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) {
    n2 += __shfl_xor(n2, o);
    n1 += __shfl_xor(n1, o);
  }
  if (pt < BN && sub == 0) nrm[pt] = make_float2(n2 * (1.f + 1e-6f), n1 * (1.f + 1e-6f));
}

// thr[pt]: the row's selection threshold (error-bound slack and kDelta
// included): a logit L is recomputed in float64 when L >= thr[pt].
template <class SH, int WD, int DPW>
__device__ __forceinline__ void refine_tile(f4 (&acc)[SH::NPB][2], const float* __restrict__ thr,
                                            const float2* __restrict__ nrm, const float (&co)[6],
                                            const float* __restrict__ xt, int rows, const EArgs& a, double C,
                                            int compbase, float* __restrict__ rlist,
                                            unsigned short* __restrict__ elist, int lane, int wd,
                                            unsigned& nsel) {
  constexpr int NREG = SH::NPB * 8;
  constexpr int DPT = DPW * WD / 16;           // dims per lane (16 lanes per logit)
  constexpr int DCH = DPT < 4 ? DPT : 4;       // dims with loads in flight together
  const int g = lane >> 4, r16 = lane & 15;
  // 1. one selection bit per register
  unsigned sel = 0;
  const bool cok0 = compbase + r16 < a.K, cok1 = compbase + 16 + r16 < a.K;
#pragma unroll
  for (int pb = 0; pb < SH::NPB; ++pb) {
    const f4 t4 = *reinterpret_cast<const f4*>(thr + pb * 16 + 4 * g);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int pt = pb * 16 + 4 * g + v;
      const bool rok = pt < rows;
      const float2 nn = nrm[pt];
      const float L0 = acc[pb][0][v], L1 = acc[pb][1][v];
      const float E0 = err_bound(a.kappa, co[0], co[1], co[2], nn);
      const float E1 = err_bound(a.kappa, co[3], co[4], co[5], nn);
      const bool b0 = rok && cok0 && (L0 != kNegInf) && (L0 + E0 >= t4[v]);
      const bool b1 = rok && cok1 && (L1 != kNegInf) && (L1 + E1 >= t4[v]);
      sel |= (b0 ? 1u : 0u) << (pb * 8 + v);
      sel |= (b1 ? 1u : 0u) << (pb * 8 + 4 + v);
    }
    __builtin_amdgcn_sched_barrier(0);  // bounds the LDS loads in flight (registers)
  }
  // 2. lane-major list: lane l's selected registers, in register order, take
  //    positions [pre, pre + popc(sel)) where pre is the exclusive prefix of
  //    the per-lane counts, built bit-slice by bit-slice from six ballots.
  const int c = __popc(sel);
  int pre = 0, total = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const unsigned long long m = __ballot((c >> b) & 1);
    // set bits of m in lanes below this one
    pre += (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u)) << b;
    total += __popcll(m) << b;
  }
  if (total == 0) return;  // uniform over the component group
  if (wd == 0) nsel += (unsigned)total;
  for (int b0 = 0; b0 < total; b0 += kRefineCap) {
    const int count = min(kRefineCap, total - b0);
    if (!SH::COOP || wd == 0) {
      // walk the set bits (a lane rarely has more than a few)
      unsigned bits = sel;
      int idx = pre - b0;
      while (bits) {
        const int r = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (idx >= 0 && idx < kRefineCap) elist[idx] = (unsigned short)((r << 6) | lane);
        ++idx;
      }
    }
    if constexpr (SH::COOP) __syncthreads();
    else { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); __builtin_amdgcn_wave_barrier(); }
    // 3. float64 logits: 16 lanes per entry, 4 entries per pass; in COOP
    //    mode the WD dim-segment waves of the group share the passes.
    for (int base = SH::COOP ? wd * 4 : 0; base < count; base += SH::COOP ? 4 * WD : 4) {
      const int e = base + g;
      const bool live = e < count;
      const int code = live ? (int)elist[e] : 0;
      const int r = code >> 6, ln = code & 63;
      const int pt = (r >> 3) * 16 + 4 * (ln >> 4) + (r & 3);
      const int comp = compbase + ((r >> 2) & 1) * 16 + (ln & 15);
      const double2* wr = a.w64 + (size_t)comp * a.Dp;
      const double cf = (live && r16 == 0) ? a.cfull[comp] : 0.0;  // issued with the (a, b) loads
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
    if constexpr (SH::COOP) __syncthreads();
    else { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); __builtin_amdgcn_wave_barrier(); }
    // 4. owners take their refined logits back, in the same order
    {
      int idx = pre - b0;
#pragma unroll
      for (int r = 0; r < NREG; ++r)
        if ((sel >> r) & 1u) {
          if (idx >= 0 && idx < kRefineCap) acc[r >> 3][(r >> 2) & 1][r & 3] = rlist[idx];
          ++idx;
        }
    }
    if constexpr (SH::COOP) __syncthreads();
    else { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); __builtin_amdgcn_wave_barrier(); }
  }
}

// The same refinement with the selected logits of all NW waves of a
// workgroup (WD = 1) pooled into one list: every wave then takes four
// entries per pass, so one pass serves up to 4 * NW logits of the
// workgroup and no wave waits on another's longer list.  Entry codes carry
// the owning wave (w << 11 | register << 6 | lane); comp0 is the first
// component of the workgroup (wave w owns comp0 + 32 w ...).  wtot: NW + 1
// ints of LDS.  Same float64 arithmetic and order per logit as refine_tile,
// so the refined values are bit-identical.
template <class SH, int DPW>
__device__ __forceinline__ void refine_pooled(f4 (&acc)[SH::NPB][2], const float* __restrict__ thr,
                                              const float2* __restrict__ nrm, const float (&co)[6],
                                              const float* __restrict__ xt, int rows, const EArgs& a, double C,
                                              int comp0, int compbase, float* __restrict__ rlist,
                                              unsigned short* __restrict__ elist, int* __restrict__ wtot, int cap,
                                              int lane, int w, unsigned& nsel) {
  constexpr int NREG = SH::NPB * 8;
  constexpr int NW = SH::NT / kWave;
  constexpr int DPT = DPW / 16;
  constexpr int DCH = DPT < 4 ? DPT : 4;
  static_assert(NW <= 32 && NREG <= 32, "entry code: 5 bits of wave, 5 of register, 6 of lane");
  const int g = lane >> 4, r16 = lane & 15;
  unsigned sel = 0;
  const bool cok0 = compbase + r16 < a.K, cok1 = compbase + 16 + r16 < a.K;
#pragma unroll
  for (int pb = 0; pb < SH::NPB; ++pb) {
    const f4 t4 = *reinterpret_cast<const f4*>(thr + pb * 16 + 4 * g);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int pt = pb * 16 + 4 * g + v;
      const bool rok = pt < rows;
      const float2 nn = nrm[pt];
      const float L0 = acc[pb][0][v], L1 = acc[pb][1][v];
      const float E0 = err_bound(a.kappa, co[0], co[1], co[2], nn);
      const float E1 = err_bound(a.kappa, co[3], co[4], co[5], nn);
      const bool b0 = rok && cok0 && (L0 != kNegInf) && (L0 + E0 >= t4[v]);
      const bool b1 = rok && cok1 && (L1 != kNegInf) && (L1 + E1 >= t4[v]);
      sel |= (b0 ? 1u : 0u) << (pb * 8 + v);
      sel |= (b1 ? 1u : 0u) << (pb * 8 + 4 + v);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const int c = __popc(sel);
  int pre = 0, total = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const unsigned long long m = __ballot((c >> b) & 1);
    pre += (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u)) << b;
    total += __popcll(m) << b;
  }
  if (lane == 0) wtot[w] = total;
  __syncthreads();
  int base = 0, T = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    const int tq = wtot[q];
    base += (q < w) ? tq : 0;
    T += tq;
  }
  if (T == 0) return;  // uniform over the workgroup
  nsel += (unsigned)total;
  for (int b0 = 0; b0 < T; b0 += cap) {
    const int count = min(cap, T - b0);
    {
      unsigned bits = sel;
      int idx = base + pre - b0;
      while (bits) {
        const int r = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (idx >= 0 && idx < cap) elist[idx] = (unsigned short)((w << 11) | (r << 6) | lane);
        ++idx;
      }
    }
    __syncthreads();
    for (int e0 = w * 4; e0 < count; e0 += NW * 4) {
      const int e = e0 + g;
      const bool live = e < count;
      const int code = live ? (int)elist[e] : 0;
      const int wo = code >> 11, r = (code >> 6) & 31, ln = code & 63;
      const int pt = (r >> 3) * 16 + 4 * (ln >> 4) + (r & 3);
      const int comp = comp0 + wo * 32 + ((r >> 2) & 1) * 16 + (ln & 15);
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
            const int d = r16 + 16 * (j0 + j);
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
    __syncthreads();
    {
      int idx = base + pre - b0;
#pragma unroll
      for (int r = 0; r < NREG; ++r)
        if ((sel >> r) & 1u) {
          if (idx >= 0 && idx < cap) acc[r >> 3][(r >> 2) & 1][r & 3] = rlist[idx];
          ++idx;
        }
    }
    __syncthreads();
  }
}

// Add a wave's refined-logit count to the global counter once per launch
// (one atomic per wave instead of one per tile keeps the counter off the
// critical path).
__device__ __forceinline__ void count_refined(const EArgs& a, unsigned nsel) {
  if ((threadIdx.x & 63) == 0 && nsel) atomicAdd(a.nrefined, (unsigned long long)nsel);
}

// Row group / member of a workgroup.  Members of one row group sit on one XCD
// when the grid allows (consecutive workgroup ids go round-robin over the 8
// XCDs), so the P re-reads of an X tile and the exchange stay in one L2.
__device__ __forceinline__ void rg_member(int G, int P, int& rg, int& p) {
  const int b = blockIdx.x;
  const int per = G / kNumXCD;
  if (G % kNumXCD == 0 && per % P == 0) {
    const int xcd = b % kNumXCD, s = b / kNumXCD;
    rg = xcd * (per / P) + s / P;
    p = s % P;
  } else {
    rg = b / P;
    p = b % P;
  }
}

}  // namespace gmm
