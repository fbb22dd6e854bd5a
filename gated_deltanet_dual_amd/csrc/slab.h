// slab.h -- register-resident column slabs for the chunked delta-rule kernels.
//
// Most of the chunk algebra is separable over the columns of d_v: U, the noisy
// reads, their adjoints, ... are C x d_v matrices whose columns never mix, and
// they are produced by C x C (or C x d_k) matrices acting from the left.  A
// wave therefore owns a 16-column slab and keeps every such C x 16 matrix in
// MFMA accumulator layout for its whole dependency chain, with no LDS round
// trip and no barrier between steps.
//
// Slab layout (C = 32 rows, 16 columns): t[tr][r] holds X[16*tr + 4*(l>>4) + r][l & 15].
//
// A slab is fed back into v_mfma_f32_16x16x32_bf16 as the B operand of a
// product contracting over the chunk index: lane l supplies k-slots
// e = 0..7 as the rows pk(g, e) = 4g + e (e < 4) and 16 + 4g + e - 4 (e >= 4),
// g = l >> 4 -- exactly the rows the lane already holds.  The A operand is
// loaded with the same column permutation, so the product is unchanged.
#pragma once

#include "device_common.h"

namespace flare {

struct Slab {
  floatx4 t[2];
};

__device__ __forceinline__ Slab slab_zero() {
  Slab s;
  s.t[0] = floatx4{0.f, 0.f, 0.f, 0.f};
  s.t[1] = floatx4{0.f, 0.f, 0.f, 0.f};
  return s;
}

// chunk row held by accumulator register r of tile tr in this lane
__device__ __forceinline__ int slab_row_l(int l, int tr, int r) { return 16 * tr + 4 * (l >> 4) + r; }
__device__ __forceinline__ int slab_row(int tr, int r) { return slab_row_l(lane_id(), tr, r); }

// bf16 B fragment (k-permuted) of a slab: hi only.
__device__ __forceinline__ bf16x8 slab_b_hi(const Slab &s) {
  const uint4 h = make_uint4(pack_bf16x2(s.t[0][0], s.t[0][1]), pack_bf16x2(s.t[0][2], s.t[0][3]),
                             pack_bf16x2(s.t[1][0], s.t[1][1]), pack_bf16x2(s.t[1][2], s.t[1][3]));
  return __builtin_bit_cast(bf16x8, h);
}

// hi + lo split of 8 fp32 values into two bf16x8 (x ~= hi + lo to ~2^-16).
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
  uint32_t h[4], o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    o[e] = pack_bf16x2(x[2 * e] - __uint_as_float(h[e] << 16), x[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ void slab_b_split(const Slab &s, bf16x8 &hi, bf16x8 &lo) {
  const float x[8] = {s.t[0][0], s.t[0][1], s.t[0][2], s.t[0][3], s.t[1][0], s.t[1][1], s.t[1][2], s.t[1][3]};
  split8(x, hi, lo);
}

// A fragment of rows m0 .. m0+15 of a C x C fp32 LDS matrix M (row-major,
// pitch ld), columns in the slab's k-permutation, split hi + lo.
__device__ __forceinline__ void cc_a_split(const float *M, int ld, int m0, bf16x8 &hi, bf16x8 &lo) {
  const int l = lane_id(), g = l >> 4;
  const float *p = M + (m0 + (l & 15)) * ld;
  const float4 a0 = *reinterpret_cast<const float4 *>(p + 4 * g);
  const float4 a1 = *reinterpret_cast<const float4 *>(p + 16 + 4 * g);
  const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  split8(x, hi, lo);
}

// The same for the transpose: A[m][k] = M[k][m].
__device__ __forceinline__ void cc_aT_split(const float *M, int ld, int m0, bf16x8 &hi, bf16x8 &lo) {
  const int l = lane_id(), g = l >> 4, col = m0 + (l & 15);
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = M[(4 * g + e) * ld + col];
    x[4 + e] = M[(16 + 4 * g + e) * ld + col];
  }
  split8(x, hi, lo);
}

// out += op(M) * in, op(M) = M or M^T (C x C fp32 in LDS), in a slab.
// TERMS = 3: both operands split (hi*hi + hi*lo + lo*hi, ~2^-16 relative);
// TERMS = 2: `in` is exact in bf16 (hi*hi + lo*hi).
template <int TERMS, bool TRANS>
__device__ __forceinline__ void cc_mul(Slab &out, const float *M, int ld, const Slab &in) {
  bf16x8 bh, bl;
  if constexpr (TERMS == 3) slab_b_split(in, bh, bl);
  else bh = slab_b_hi(in);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
    bf16x8 ah, al;
    if constexpr (TRANS) cc_aT_split(M, ld, 16 * tr, ah, al);
    else cc_a_split(M, ld, 16 * tr, ah, al);
    mma_bf16(out.t[tr], ah, bh);
    if constexpr (TERMS == 3) mma_bf16(out.t[tr], ah, bl);
    mma_bf16(out.t[tr], al, bh);
  }
}

// A fragment of rows m0 .. m0+15 of a C x C bf16 plane in LDS (row-major,
// pitch ld elements, a multiple of 4), columns in the slab's k-permutation:
// two 8-byte reads, no conversion.
__device__ __forceinline__ bf16x8 plane_a_l(int l, const u16 *P, int ld, int m0) {
  const int g = l >> 4;
  const u16 *p = P + (m0 + (l & 15)) * ld + 4 * g;
  const uint2 lo4 = *reinterpret_cast<const uint2 *>(p);
  const uint2 hi4 = *reinterpret_cast<const uint2 *>(p + 16);
  return __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
}
__device__ __forceinline__ bf16x8 plane_a(const u16 *P, int ld, int m0) { return plane_a_l(lane_id(), P, ld, m0); }

// out += A * in, A (C x C) given as its bf16 hi and lo planes, already in the
// orientation of the product (a transposed operand is stored transposed).
// TERMS as for cc_mul.
template <int TERMS>
__device__ __forceinline__ void cc_mul_planes_l(int l, Slab &out, const u16 *Ah, const u16 *Al, int ld,
                                                const Slab &in) {
  bf16x8 bh, bl;
  if constexpr (TERMS == 3) slab_b_split(in, bh, bl);
  else bh = slab_b_hi(in);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
    const bf16x8 ah = plane_a_l(l, Ah, ld, 16 * tr), al = plane_a_l(l, Al, ld, 16 * tr);
    mma_bf16(out.t[tr], ah, bh);
    if constexpr (TERMS == 3) mma_bf16(out.t[tr], ah, bl);
    mma_bf16(out.t[tr], al, bh);
  }
}
template <int TERMS>
__device__ __forceinline__ void cc_mul_planes(Slab &out, const u16 *Ah, const u16 *Al, int ld, const Slab &in) {
  cc_mul_planes_l<TERMS>(lane_id(), out, Ah, Al, ld, in);
}

// Sum of x over the 16 lanes that share an accumulator row group.
__device__ __forceinline__ float row_sum16(float x) { return dpp_sum16(x); }

}  // namespace flare
