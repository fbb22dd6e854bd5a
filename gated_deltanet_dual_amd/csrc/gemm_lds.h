// gemm_lds.h -- one 16x16 output tile of a product of two LDS-resident
// operands, acc[i][j] += sum_k A(ra + i, k) * Bt(rb + j, k), for the operand
// layouts the dual-stream kernels use:
//   RowU16 : element (r, k) = p[r * ld + k], bf16 exact
//   ColU16 : element (r, k) = p[k * ld + r], bf16 exact (transposed read)
//   RowF32 : element (r, k) = p[r * ld + k], fp32
//   ColF32 : element (r, k) = p[k * ld + r], fp32 (transposed read)
// On the bf16 path fp32 operands are split hi + lo (two bf16 values, ~2^-16
// relative) when SPLIT is set, else rounded once; the product then issues
// hi*hi (+ hi*lo) (+ lo*hi) on v_mfma_f32_16x16x32_bf16.  On the fp32 path every
// operand is read as fp32 and v_mfma_f32_16x16x4f32 is used.  K is the
// contraction depth: a multiple of 32, or 16 (then lanes 32..63, which carry
// k = 16..31, supply zeros).
#pragma once

#include "device_common.h"

namespace flare {

enum Layout { RowU16 = 0, ColU16 = 1, RowF32 = 2, ColF32 = 3 };

template <int L> __device__ __forceinline__ constexpr bool is_f32() { return L == RowF32 || L == ColF32; }

// fp32 column-gather fragment split into hi + lo.
__device__ __forceinline__ void frag_f32_split_T(const float *base, int ld, int row0, int k0, bf16x8 &hi,
                                                 bf16x8 &lo) {
  const int l = lane_id();
  const float *p = base + (k0 + 8 * (l >> 4)) * ld + row0 + (l & 15);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = p[e * ld];
  uint32_t h[4], o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    o[e] = pack_bf16x2(x[2 * e] - __uint_as_float(h[e] << 16), x[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

template <int L>
__device__ __forceinline__ void frag_any(const void *p, int ld, int r0, int k0, bf16x8 &hi, bf16x8 &lo,
                                         bool want_lo) {
  if constexpr (L == RowU16) {
    hi = frag_bf16(reinterpret_cast<const u16 *>(p), ld, r0, k0);
  } else if constexpr (L == ColU16) {
    hi = frag_bf16_T(reinterpret_cast<const u16 *>(p), ld, r0, k0);
  } else if constexpr (L == RowF32) {
    if (want_lo) frag_f32_split(reinterpret_cast<const float *>(p), ld, r0, k0, hi, lo);
    else hi = frag_f32_hi(reinterpret_cast<const float *>(p), ld, r0, k0);
  } else {
    frag_f32_split_T(reinterpret_cast<const float *>(p), ld, r0, k0, hi, lo);
  }
}

template <int L>
__device__ __forceinline__ float frag1_any(const void *p, int ld, int r0, int k0) {
  const int l = lane_id();
  const int r = r0 + (l & 15), k = k0 + (l >> 4);
  if constexpr (L == RowU16) return bf2f(reinterpret_cast<const u16 *>(p)[r * ld + k]);
  else if constexpr (L == ColU16) return bf2f(reinterpret_cast<const u16 *>(p)[k * ld + r]);
  else if constexpr (L == RowF32) return reinterpret_cast<const float *>(p)[r * ld + k];
  else return reinterpret_cast<const float *>(p)[k * ld + r];
}

// BF: bf16 MFMA path (else fp32 MFMA); SPLIT: hi/lo for fp32 operands.
template <bool BF, int K, int LA, int LB, bool SPLIT = true>
__device__ __forceinline__ void gemm_tile(floatx4 &acc, const void *A, int lda, int ra, const void *Bt, int ldb,
                                          int rb) {
  if constexpr (BF) {
    constexpr bool sa = SPLIT && is_f32<LA>(), sb = SPLIT && is_f32<LB>();
    if constexpr (K % 32 == 0) {
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += 32) {
        bf16x8 ah, al, bh, bl;
        frag_any<LA>(A, lda, ra, k0, ah, al, sa);
        frag_any<LB>(Bt, ldb, rb, k0, bh, bl, sb);
        mma_bf16(acc, ah, bh);
        if constexpr (sb) mma_bf16(acc, ah, bl);
        if constexpr (sa) mma_bf16(acc, al, bh);
      }
    } else {
      static_assert(K == 16, "contraction depth must be 16 or a multiple of 32");
      bf16x8 ah, al, bh, bl;
      frag_any<LA>(A, lda, ra, 0, ah, al, sa);
      frag_any<LB>(Bt, ldb, rb, 0, bh, bl, sb);
      if (lane_id() >= 32) {
        const bf16x8 z = as_bf16x8(u16x8{});
        ah = al = bh = bl = z;
      }
      mma_bf16(acc, ah, bh);
      if constexpr (sb) mma_bf16(acc, ah, bl);
      if constexpr (sa) mma_bf16(acc, al, bh);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) mma_f32(acc, frag1_any<LA>(A, lda, ra, k0), frag1_any<LB>(Bt, ldb, rb, k0));
  }
}

// Sum of x over the 16 lanes that share an accumulator row group (the 16
// columns of a 16x16 tile); every lane of the group gets the total.
__device__ __forceinline__ float sum16(float x) { return dpp_sum16(x); }

}  // namespace flare
