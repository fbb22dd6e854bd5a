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

// f(integral_constant<int, J>) for J = 0, 1, ... in order (static slot indices)
template <typename F, int... J>
__device__ __forceinline__ void for_each_slot(std::integer_sequence<int, J...>, F &&f) {
  (f(std::integral_constant<int, J>{}), ...);
}


}  // namespace conv
}  // namespace flare
