// conv_common.h -- pieces shared by the ShortConv forward and reverse
// kernels: a lane's slice of a [T, C] row and static iteration over the slots
// of a register ring.
#pragma once

#include <utility>

#include "device_common.h"

namespace flare {
namespace conv {

// A lane's slice of one row: N channels of type IO, loaded as one word.
template <typename IO, int N> struct Slice;
template <> struct Slice<u16, 4> {
  using Raw = uint2;
  static __device__ __forceinline__ Raw load(const u16 *p) { return *reinterpret_cast<const uint2 *>(p); }
  static __device__ __forceinline__ void cvt(Raw r, float *f) {
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xffff0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(u16 *p, const float *f) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  }
};
template <> struct Slice<u16, 2> {
  using Raw = uint32_t;
  static __device__ __forceinline__ Raw load(const u16 *p) { return *reinterpret_cast<const uint32_t *>(p); }
  static __device__ __forceinline__ void cvt(Raw r, float *f) {
    f[0] = __uint_as_float(r << 16);
    f[1] = __uint_as_float(r & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(u16 *p, const float *f) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(f[0], f[1]);
  }
};
template <> struct Slice<float, 2> {
  using Raw = float2;
  static __device__ __forceinline__ Raw load(const float *p) { return *reinterpret_cast<const float2 *>(p); }
  static __device__ __forceinline__ void cvt(Raw r, float *f) { f[0] = r.x; f[1] = r.y; }
  static __device__ __forceinline__ void store(float *p, const float *f) {
    *reinterpret_cast<float2 *>(p) = make_float2(f[0], f[1]);
  }
};
template <> struct Slice<float, 1> {
  using Raw = float;
  static __device__ __forceinline__ Raw load(const float *p) { return *p; }
  static __device__ __forceinline__ void cvt(Raw r, float *f) { f[0] = r; }
  static __device__ __forceinline__ void store(float *p, const float *f) { *p = f[0]; }
};

// Sum of x over aligned groups of G consecutive lanes (G a power of two, at
// most 64, wave-uniform); every lane of a group gets its group's total.  xor 1
// and xor 2 inside quads, then mirrored quads (8), mirrored half-rows (16), and
// the permlane swaps across rows (32, 64).  The steps past G are switched off
// by 0/1 factors (GroupSum::f, formed once) rather than by branches, so a loop
// that calls it holds six scalars instead of a mask per call.
// Each step adds the partner lane's value in an order both lanes share, so all
// lanes of a group hold the same bits.
struct GroupSum {
  float f[6], g4, g5;  // f: step on (1) or off (0); g4, g5 = 1 - f[4], 1 - f[5]
  __device__ __forceinline__ explicit GroupSum(int G) {
#pragma unroll
    for (int i = 0; i < 6; ++i) f[i] = G >= (2 << i) ? 1.f : 0.f;
    g4 = 1.f - f[4];
    g5 = 1.f - f[5];
  }
  __device__ __forceinline__ float operator()(float x) const {
    x = fmaf(f[0], dpp_f32<0xB1>(x), x);   // quad_perm [1,0,3,2]
    x = fmaf(f[1], dpp_f32<0x4E>(x), x);   // quad_perm [2,3,0,1]
    x = fmaf(f[2], dpp_f32<0x141>(x), x);  // row_half_mirror
    x = fmaf(f[3], dpp_f32<0x140>(x), x);  // row_mirror
    x = fmaf(f[4], xsum16(x), g4 * x);     // rows 2k + 2k+1 (even row's value first in both)
    x = fmaf(f[5], xsum32(x), g5 * x);     // halves of the wave
    return x;
  }
};

// f(integral_constant<int, J>) for J = 0, 1, ... in order (static slot indices)
template <typename F, int... J>
__device__ __forceinline__ void for_each_slot(std::integer_sequence<int, J...>, F &&f) {
  (f(std::integral_constant<int, J>{}), ...);
}


}  // namespace conv
}  // namespace flare
