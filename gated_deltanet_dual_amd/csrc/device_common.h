// device_common.h -- small device helpers shared by the gfx950 kernels:
// bf16 <-> fp32 conversion, the 16x16 MFMA tile primitives and the LDS
// fragment loaders that feed them.
//
// MFMA tile conventions (CDNA 16x16 output tiles, wave64):
//   output/accumulator: lane l holds D[4*(l>>4) + r][l & 15], r = 0..3
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[l & 15][8*(l>>4) + e] and
//     B[8*(l>>4) + e][l & 15], e = 0..7 (A and B use the same k assignment, so a
//     permutation of k inside the hardware cannot change the product)
//   v_mfma_f32_16x16x4f32:    lane l supplies A[l & 15][l >> 4], B[l >> 4][l & 15]
// Every product in the kernels is written as D[i][j] = sum_k A[i][k] * Bt[j][k],
// with A and Bt both row-major in LDS, so both operands are fetched with the
// same row-fragment loader.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flare {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

struct __align__(16) u16x8 { u16 v[8]; };

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Round to nearest, ties to even, on the gfx950 conversion unit
// (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }
// Two values rounded by one instruction: lo in bits 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2v v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

template <typename IO> struct io_traits;
template <> struct io_traits<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct io_traits<u16> {
  static __device__ __forceinline__ float to_f(u16 x) { return bf2f(x); }
  static __device__ __forceinline__ u16 from_f(float x) { return f2bf(x); }
};

__device__ __forceinline__ bf16x8 as_bf16x8(const u16x8 &x) {
  return __builtin_bit_cast(bf16x8, x);
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ void mma_bf16(floatx4 &acc, const bf16x8 &a, const bf16x8 &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_f32(floatx4 &acc, float a, float b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// 16-byte non-temporal loads (for data a kernel reads once): the builtin
// takes native vectors only
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt_u4(const void *p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 ld_nt_f4(const void *p) {
  const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
// 16-byte non-temporal stores (for data a kernel writes once and no later
// access of the same kernel reads)
__device__ __forceinline__ void st_nt_u4(void *p, const uint4 &v) {
  __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v *>(p));
}
__device__ __forceinline__ void st_nt_f4(void *p, const float4 &v) {
  __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, reinterpret_cast<floatx4 *>(p));
}

// ---------------------------------------------------------------- fragments
// Row fragment of a row-major bf16 matrix: rows row0 + (l & 15), columns
// k0 + 8*(l>>4) .. +7 (one 16-byte LDS read).
// The _l variants take the lane index as an argument: a kernel that loops
// over work items passes a per-item opaque copy, so the per-lane offsets are
// formed inside the loop instead of being hoisted out of it.
__device__ __forceinline__ bf16x8 frag_bf16_l(int l, const u16 *base, int ld, int row0, int k0) {
  const u16x8 *p = reinterpret_cast<const u16x8 *>(base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
  return as_bf16x8(*p);
}
__device__ __forceinline__ bf16x8 frag_bf16(const u16 *base, int ld, int row0, int k0) {
  return frag_bf16_l(lane_id(), base, ld, row0, k0);
}

// Row fragment of a row-major fp32 matrix rounded to bf16 (hi part).
__device__ __forceinline__ bf16x8 frag_f32_hi(const float *base, int ld, int row0, int k0) {
  const int l = lane_id();
  const float4 *p = reinterpret_cast<const float4 *>(base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
  const float4 x0 = p[0], x1 = p[1];
  const uint4 h = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                             pack_bf16x2(x1.z, x1.w));
  return __builtin_bit_cast(bf16x8, h);
}

// Row fragment of a row-major fp32 matrix split as hi + lo, both bf16, with
// hi = bf16(x) and lo = bf16(x - hi): x is represented to ~2^-16 relative.
__device__ __forceinline__ void frag_f32_split(const float *base, int ld, int row0, int k0,
                                               bf16x8 &hi, bf16x8 &lo) {
  const int l = lane_id();
  const float4 *p = reinterpret_cast<const float4 *>(base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
  const float4 x0 = p[0], x1 = p[1];
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint32_t h[4], o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    const float r0 = x[2 * e] - __uint_as_float(h[e] << 16);
    const float r1 = x[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u);
    o[e] = pack_bf16x2(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// Column-gather fragment: element (r, k) = base[(k0 + 8*(l>>4) + e) * ld + row0 + (l&15)],
// i.e. the row fragment of the TRANSPOSE of a row-major bf16 matrix.
__device__ __forceinline__ bf16x8 frag_bf16_T_l(int l, const u16 *base, int ld, int row0, int k0) {
  const u16 *p = base + (k0 + 8 * (l >> 4)) * ld + row0 + (l & 15);
  u16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h.v[e] = p[e * ld];
  return as_bf16x8(h);
}
__device__ __forceinline__ bf16x8 frag_bf16_T(const u16 *base, int ld, int row0, int k0) {
  return frag_bf16_T_l(lane_id(), base, ld, row0, k0);
}

// fp32 MFMA operands (16x16x4): one element per lane.
__device__ __forceinline__ float frag1_f32(const float *base, int ld, int row0, int k0) {
  const int l = lane_id();
  return base[(row0 + (l & 15)) * ld + k0 + (l >> 4)];
}
__device__ __forceinline__ float frag1_f32_T(const float *base, int ld, int row0, int k0) {
  const int l = lane_id();
  return base[(k0 + (l >> 4)) * ld + row0 + (l & 15)];
}

// Workgroup barrier for LDS traffic only: waits until this wave's LDS operations
// have completed, then meets the other waves.  Unlike __syncthreads() it does
// not wait for outstanding global loads, so a prefetch of the next tile stays in
// flight across it.  Global memory written before it is NOT made visible.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// x from another lane of the same 16-lane row through the DPP network (no LDS
// traffic): CTRL is a gfx9 DPP control code.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum of x over the 16 lanes of this lane's DPP row (lanes 16q .. 16q + 15);
// every lane of the row gets the total.  xor 1 and xor 2 inside each quad
// (quad_perm), then the mirrored quad and the mirrored half-row.
__device__ __forceinline__ float dpp_sum16(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror: quad 0 <-> quad 1, quad 2 <-> quad 3
  x += dpp_f32<0x140>(x);  // row_mirror: lanes 0-7 <-> 15-8
  return x;
}

// x + x of lane l ^ 16, and x + x of lane l ^ 32: sums across the 16-lane rows
// with the gfx950 permlane swaps (VALU, no LDS traffic).  A swap of a value
// with itself leaves each lane holding its own value in one output and its
// partner's in the other.
__device__ __forceinline__ float xsum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Output element coordinates of accumulator register r for this lane.
__device__ __forceinline__ int acc_row(int r) { return 4 * (lane_id() >> 4) + r; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

}  // namespace flare
