// bwd_common.h -- pieces shared by the two per-chunk backward kernels: the
// per-chunk gate load / scan and the masked Gram matrices of a chunk.
#pragma once

#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

// Slab (accumulator layout) of columns [col0, col0 + 16) of a [T, H, D] bf16
// tensor: raw bits loaded from rows clamped into the document, then masked and
// converted by slab_mask when consumed.
template <int D>
__device__ __forceinline__ void gslab_raw(u16 (&dst)[2][4], const u16 *src, int H, int h, int64_t t0g, int c0,
                                          int n, int col0) {
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dst[tr][r] = src[((t0g + min(c0 + slab_row(tr, r), n - 1)) * H + h) * D + col0 + acc_col()];
}
// The same for a noisy-stream tensor: its prompt rows (never used, they read
// as 0 through slab_mask) are loaded from the clean twin's same row instead,
// which the same lanes load too, so they cost no HBM traffic.
template <int D>
__device__ __forceinline__ void gslab_raw_noisy(u16 (&dst)[2][4], const u16 *src, const u16 *clean, int H, int h,
                                                int64_t t0g, int c0, int n, int P, int col0) {
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = c0 + slab_row(tr, r);
      dst[tr][r] = (row < P ? clean : src)[((t0g + min(row, n - 1)) * H + h) * D + col0 + acc_col()];
    }
}
// rows past the document end, and prompt rows of the noisy stream, read as 0
__device__ __forceinline__ Slab slab_mask(const u16 (&raw)[2][4], int c0, int n, int P, bool noisy) {
  Slab s;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tpos = c0 + slab_row(tr, r);
      const bool ok = tpos < n && (!noisy || tpos >= P);
      s.t[tr][r] = ok ? bf2f(raw[tr][r]) : 0.f;
    }
  return s;
}

enum { CC_AT = 0, CC_T, CC_MO, CC_MQ, CC_MK, CC_ANT, CC_TN, CC_MN };

// The hand-over from the backward pre-pass to the reverse scan, per (chunk
// slot, head), in fp32 words (bf16 io, d = 128).  With the end-state adjoint
// dS' of the chunk the scan's step is
//   dS_c = g_C dS' + R + K^T (W (K dS')),
// R the 128 x 128 state-independent right-hand side and W the 32 x 32 chain
// matrix W_ij = -exp(lg_i) T_ji b_j exp(lg_C - lg_j).  Every operand is stored
// in the register order of the wave that consumes it (16-byte units, lane
// fastest), so the scan reads each with plain coalesced loads:
//   R  [slab 8][tile 8][lane 64][4]  accumulator tile of d_v slab w, d_k tile kt
//        (the forward, whose R is K^T Z, stores the C x d_v matrix Z here
//        instead: [slab 8][tile 2][lane 64][4])
//   W  [tile 2][hi/lo 2][lane 64][8 bf16]  A fragment rows 16 tr + (l & 15),
//        columns in the slab k-permutation (slab.h)
//   KA [ks 4][tile 2][lane 64][8 bf16]  A fragments of K (rows: chunk tokens,
//        columns: d_k 32 ks + the slab k-permutation)
//   KT [tile 8][lane 64][8 bf16]  A fragments of K^T (rows: d_k 16 kt + (l & 15),
//        columns: chunk tokens in the slab k-permutation)
//   G  g_C = exp(lg_C) in word 0
constexpr int kPackR = 0, kPackW = kPackR + 16384, kPackKA = kPackW + 1024, kPackKT = kPackKA + 2048,
              kPackG = kPackKT + 2048, kPackWords = kPackG + 64;

// The gate value thread tid < 128 of a chunk reads: group g = tid / 32 of
// (a, b, a~, b~), position i = tid % 32 (padded tokens and noisy prompt tokens:
// a = 1, b = 0).
__device__ __forceinline__ float gate_load(const FwdArgs &f, int64_t t0g, int c0, int n, int P, int h, int tid) {
  const int g = tid / 32, i = tid % 32;
  const int tpos = c0 + i;
  bool ok = tpos < n;
  if (g >= 2) ok = ok && tpos >= P;
  // the four pointers are read into registers first: selecting among the
  // argument block's fields per lane would load the pointer itself per lane
  const float *const p0 = f.alpha, *const p1 = f.beta, *const p2 = f.alpha_n, *const p3 = f.beta_n;
  const float *src = g == 0 ? p0 : g == 1 ? p1 : g == 2 ? p2 : p3;
  // unconditional load from a row clamped into the document, masked afterwards
  const int64_t row = (t0g + min(tpos, n - 1)) * f.H + h;
  float v = src[row];
  if (f.l2f && (g & 1)) {  // the q/k L2 flag: folded write strengths (gdn_l2.hip)
    const float4 r = f.l2f[row];
    const float rk = g == 1 ? r.y : r.w;
    v *= rk * rk;
  }
  return ok ? v : ((g & 1) == 0 ? 1.f : 0.f);
}

// The same load, split: the raw value now (no use of it, so nothing waits),
// the mask and padding applied by gate_fix when the value is consumed.
// With the q/k L2 flag (f.l2f) the write strengths are the folded ones,
// b r_k^2 and b~ r_k~^2 (gdn_l2.hip).
__device__ __forceinline__ float gate_load_raw(const FwdArgs &f, int64_t t0g, int c0, int n, int h, int tid) {
  const int g = tid / 32, i = tid % 32;
  const float *const p0 = f.alpha, *const p1 = f.beta, *const p2 = f.alpha_n, *const p3 = f.beta_n;
  const float *src = g == 0 ? p0 : g == 1 ? p1 : g == 2 ? p2 : p3;
  const int64_t row = (t0g + min(c0 + i, n - 1)) * f.H + h;
  float v = src[row];
  if (f.l2f && (g & 1)) {
    const float4 r = f.l2f[row];
    const float rk = g == 1 ? r.y : r.w;
    v *= rk * rk;
  }
  return v;
}
__device__ __forceinline__ float gate_fix(float raw, int c0, int n, int P, int tid) {
  const int g = tid / 32, tpos = c0 + tid % 32;
  const bool ok = tpos < n && (g < 2 || tpos >= P);
  return ok ? raw : ((g & 1) == 0 ? 1.f : 0.f);
}

// The scan of gate_load's value (threads tid < 128): cumulative log a over the
// chunk, cumulative log a~ inside each noisy block of B.
__device__ __forceinline__ void gate_scan(float val, int B, int tid, float *lg, float *beta, float *lgn,
                                          float *betan) {
  const int g = tid / 32, i = tid % 32;
  if (g == 0 || g == 2) {
    float la = __logf(val);
    if (g == 0) {
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float y = __shfl_up(la, off, 32);
        if (i >= off) la += y;
      }
      lg[i] = la;
    } else {
      for (int off = 1; off < B; off <<= 1) {
        const float y = __shfl_up(la, off, B);
        if ((i & (B - 1)) >= off) la += y;
      }
      lgn[i] = la;
    }
  } else {
    (g == 1 ? beta : betan)[i] = val;
  }
}

// Per-chunk gates: lg = cumulative log a, lgn = cumulative log a~ inside each
// noisy block (padded tokens: a = 1, b = 0; noisy prompt tokens likewise).
__device__ __forceinline__ void load_gates(const FwdArgs &f, int64_t t0g, int c0, int n, int P, int h, int B,
                                           float *lg, float *beta, float *lgn, float *betan) {
  const int tid = threadIdx.x;
  if (tid < 128) {
    const int g = tid / 32, i = tid % 32;
    const int tpos = c0 + i;
    bool ok = tpos < n;
    if (g >= 2) ok = ok && tpos >= P;
    const float *src = g == 0 ? f.alpha : g == 1 ? f.beta : g == 2 ? f.alpha_n : f.beta_n;
    float val = (g & 1) == 0 ? 1.f : 0.f;
    if (ok) val = src[(t0g + tpos) * f.H + h];
    if (g == 0 || g == 2) {
      float la = __logf(val);
      if (g == 0) {
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          const float y = __shfl_up(la, off, 32);
          if (i >= off) la += y;
        }
        lg[i] = la;
      } else {
        for (int off = 1; off < B; off <<= 1) {
          const float y = __shfl_up(la, off, B);
          if ((i & (B - 1)) >= off) la += y;
        }
        lgn[i] = la;
      }
    } else {
      (g == 1 ? beta : betan)[i] = val;
    }
  }
}

// Gram tiles of one chunk (norm factors 1).  With fold_w the write strengths
// (b, b~) are multiplied in (pass 1); otherwise they are left out (pass 2,
// which needs the unweighted products for the gate gradients).  A and A~ are
// stored transposed (row j = column j of A) for the solve.
//   wave 0: A^T        wave 1: Mo        wave 2: Mq, M~        wave 3: Mk, A~^T
template <bool BF, int D, int LDX, int LDM, typename IO>
__device__ __forceinline__ void chunk_grams(IO (*x)[32][LDX], float (*cc)[32][LDM], const float *lg,
                                            const float *beta, const float *lgn, const float *betan, int c0,
                                            int n, int P, int B, bool has_noisy, bool fold_w) {
  constexpr int XL = BF ? RowU16 : RowF32;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {  // non-transposed tiles: acc[r] = G[16ti + g4 + r][16tj + cl]
      const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, D, XL, XL>(acc, &x[1][0][0], LDX, 16 * ti, &x[1][0][0], LDX, 16 * tj);
      const int j = 16 * tj + cl;
      const float wj = fold_w ? beta[j] : 1.f;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + g4 + r;
        o4[r] = j < i ? acc[r] * __expf(lg[i] - lg[j]) * wj : 0.f;
      }
      *reinterpret_cast<float4 *>(&cc[CC_AT][j][16 * ti + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
  } else if (wave == 1) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {  // transposed tiles: lane holds Mo[i][j0..j0+3]
      const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, D, XL, XL>(acc, &x[1][0][0], LDX, 16 * tj, &x[0][0][0], LDX, 16 * ti);
      const int i = 16 * ti + cl, j0 = 16 * tj + g4;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + r;
        o4[r] = j <= i ? acc[r] * __expf(lg[i] - lg[j]) * (fold_w ? beta[j] : 1.f) : 0.f;
      }
      *reinterpret_cast<float4 *>(&cc[CC_MO][i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
  } else if (has_noisy) {
    const bool qside = wave == 2;
    const int xm = qside ? 2 : 3;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, D, XL, XL>(acc, &x[1][0][0], LDX, 16 * tj, &x[xm][0][0], LDX, 16 * ti);
      const int i = 16 * ti + cl, j0 = 16 * tj + g4;
      const int pi = (i & -B);
      const bool resp = c0 + i < n && c0 + i >= P;
      const float lgp = pi > 0 ? lg[pi - 1] : 0.f;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + r;
        o4[r] = (resp && j < pi) ? acc[r] * __expf(lgp - lg[j]) * (fold_w ? beta[j] : 1.f) : 0.f;
      }
      *reinterpret_cast<float4 *>(&cc[qside ? CC_MQ : CC_MK][i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
    if (qside) {
      const int nt = B > 16 ? 4 : 2;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t >= nt) break;
        const int ti = (t == 0 || t == 2) ? 0 : 1, tj = (t == 0 || t == 3) ? 0 : 1;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, D, XL, XL>(acc, &x[3][0][0], LDX, 16 * tj, &x[2][0][0], LDX, 16 * ti);
        const int i = 16 * ti + cl, j0 = 16 * tj + g4;
        const int pi = (i & -B);
        const bool resp = c0 + i < n && c0 + i >= P;
        const float lge = lgn[pi + B - 1];
        float o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + r;
          o4[r] = (resp && j >= pi && j < pi + B) ? acc[r] * __expf(lge - lgn[j]) * (fold_w ? betan[j] : 1.f) : 0.f;
        }
        *reinterpret_cast<float4 *>(&cc[CC_MN][i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
    } else {
      const int nt = B > 16 ? 3 : 2;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        if (t >= nt) break;
        const int ti = t == 0 ? 0 : 1, tj = t == 1 ? 1 : 0;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, D, XL, XL>(acc, &x[3][0][0], LDX, 16 * ti, &x[3][0][0], LDX, 16 * tj);
        const int j = 16 * tj + cl;
        const int pj = (j & -B);
        const float wj = fold_w ? betan[j] : 1.f;
        float o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ti + g4 + r;
          const bool resp = c0 + i < n && c0 + i >= P;
          o4[r] = (resp && j < i && (i & -B) == pj) ? acc[r] * __expf(lgn[i] - lgn[j]) * wj : 0.f;
        }
        *reinterpret_cast<float4 *>(&cc[CC_ANT][j][16 * ti + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
    }
  }
}

// Chunk slot -> (document, chunk index); returns false for a slot past the end
// of its document.  Slots of document i start at floor(cu_i / 32) + i.
__device__ __forceinline__ bool slot_to_chunk(const FwdArgs &f, int slot, int &doc, int &c) {
  if (f.win_len > 0) {  // chunk windows: slot = doc * win_len + (c - win_lo)
    doc = slot / f.win_len;
    c = f.win_lo + slot % f.win_len;
    return doc < f.num_docs && c * 32 < f.cu[doc + 1] - f.cu[doc];
  }
  int lo = 0, hi = f.num_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)f.cu[mid] / 32 + mid <= slot) lo = mid; else hi = mid - 1;
  }
  doc = lo;
  c = slot - (int)(f.cu[doc] / 32) - doc;
  const int n = f.cu[doc + 1] - f.cu[doc];
  return c >= 0 && c * 32 < n;
}

// A^T of the chunk (one wave): A_ij = (k_i . k_j) exp(lg_i - lg_j) for j < i,
// without the write strengths, stored transposed (row j = column j of A).
template <int D, int LDX, int LDM>
__device__ __forceinline__ void gram_at(const u16 (*k)[LDX], float (*at)[LDM], const float *lg) {
  const int lane = lane_id(), g4 = 4 * (lane >> 4), cl = lane & 15;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    gemm_tile<true, D, RowU16, RowU16>(acc, &k[0][0], LDX, 16 * ti, &k[0][0], LDX, 16 * tj);
    const int j = 16 * tj + cl;
    float o4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + g4 + r;
      o4[r] = j < i ? acc[r] * __expf(lg[i] - lg[j]) : 0.f;
    }
    *reinterpret_cast<float4 *>(&at[j][16 * ti + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
  }
}

// A~^T (one wave): A~_ij = (k~_i . k~_j) exp(lgn_i - lgn_j) for j < i inside
// one noisy block of a response row, stored transposed.
template <int D, int LDX, int LDM>
__device__ __forceinline__ void gram_ant(const u16 (*kn)[LDX], float (*at)[LDM], const float *lgn, int c0, int n,
                                         int P, int B) {
  const int lane = lane_id(), g4 = 4 * (lane >> 4), cl = lane & 15;
  const int nt = B > 16 ? 3 : 2;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (t >= nt) break;
    const int ti = t == 0 ? 0 : 1, tj = t == 1 ? 1 : 0;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    gemm_tile<true, D, RowU16, RowU16>(acc, &kn[0][0], LDX, 16 * ti, &kn[0][0], LDX, 16 * tj);
    const int j = 16 * tj + cl;
    const int pj = (j & -B);
    float o4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + g4 + r;
      const bool resp = c0 + i < n && c0 + i >= P;
      o4[r] = (resp && j < i && (i & -B) == pj) ? acc[r] * __expf(lgn[i] - lgn[j]) : 0.f;
    }
    *reinterpret_cast<float4 *>(&at[j][16 * ti + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
  }
}

// The weighted masked Grams of a chunk (write strengths folded in), split over
// two waves: wave 0 Mwo and Mwq, wave 1 Mwk and Mw~.  x holds the rows of q, k,
// q~, k~; tiles that stay zero (above the diagonal, across noisy blocks) are
// not written, so the outputs must start zeroed.
//   Mwo[i][j] = (q_i . k_j) G_i / G_j b_j              j <= i
//   Mwq[i][j] = (q~_i . k_j) G_{p_i - 1} / G_j b_j     j < p_i, response row i
//   Mwk[i][j] = (k~_i . k_j) G_{p_i - 1} / G_j b_j     j < p_i, response row i
//   Mw~[i][j] = (q~_i . k~_j) G~_e(i) / G~_j b~_j       j in the block of i, response row i
template <int D, int LDX, int LDM>
__device__ __forceinline__ void grams_weighted(int wave, const u16 (*x)[32][LDX], float (*mo)[LDM],
                                               float (*mq)[LDM], float (*mk)[LDM], float (*mn)[LDM],
                                               const float *lg, const float *beta, const float *lgn,
                                               const float *betan, int c0, int n, int P, int B, bool has_noisy) {
  const int lane = lane_id(), g4 = 4 * (lane >> 4), cl = lane & 15;
  const int ti_t[3] = {0, 1, 1}, tj_t[3] = {0, 0, 1};
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int ti = ti_t[t], tj = tj_t[t];
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<true, D, RowU16, RowU16>(acc, &x[1][0][0], LDX, 16 * tj, &x[0][0][0], LDX, 16 * ti);
      const int i = 16 * ti + cl, j0 = 16 * tj + g4;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + r;
        o4[r] = j <= i ? acc[r] * __expf(lg[i] - lg[j]) * beta[j] : 0.f;
      }
      *reinterpret_cast<float4 *>(&mo[i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
  }
  if (!has_noisy) return;
  const int xm = wave == 0 ? 2 : 3;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int ti = ti_t[t], tj = tj_t[t];
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    gemm_tile<true, D, RowU16, RowU16>(acc, &x[1][0][0], LDX, 16 * tj, &x[xm][0][0], LDX, 16 * ti);
    const int i = 16 * ti + cl, j0 = 16 * tj + g4;
    const int pi = (i & -B);
    const bool resp = c0 + i < n && c0 + i >= P;
    const float lgp = pi > 0 ? lg[pi - 1] : 0.f;
    float o4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + r;
      o4[r] = (resp && j < pi) ? acc[r] * __expf(lgp - lg[j]) * beta[j] : 0.f;
    }
    *reinterpret_cast<float4 *>(&(wave == 0 ? mq : mk)[i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
  }
  if (wave == 1) {
    const int nt = B > 16 ? 4 : 2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= nt) break;
      const int ti = (t == 0 || t == 2) ? 0 : 1, tj = (t == 0 || t == 3) ? 0 : 1;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<true, D, RowU16, RowU16>(acc, &x[3][0][0], LDX, 16 * tj, &x[2][0][0], LDX, 16 * ti);
      const int i = 16 * ti + cl, j0 = 16 * tj + g4;
      const int pi = (i & -B);
      const bool resp = c0 + i < n && c0 + i >= P;
      const float lge = lgn[pi + B - 1];
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + r;
        o4[r] = (resp && j >= pi && j < pi + B) ? acc[r] * __expf(lge - lgn[j]) * betan[j] : 0.f;
      }
      *reinterpret_cast<float4 *>(&mn[i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
  }
}

}  // namespace flare
