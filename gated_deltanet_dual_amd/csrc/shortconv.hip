// shortconv.hip -- dual-source depthwise causal ShortConv over packed documents.
//
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
// designs item 3: the width-W causal convolution in front of the GDN layer must
// not let the noisy stream see noisy tokens of an earlier block.  A noisy tap
// that lies before the start of the output token's block reads the clean input
// (clean history), a tap inside the block reads the noisy input; taps before
// the document start read zero (cu_seqlens guard).  Clean taps always read the
// clean input.  Noisy prompt rows are written as zeros.
//
// Layout: x, xn, y, yn are [T, C] with channels contiguous.  Each thread owns
// 16 bytes of channels (8 bf16 or 4 fp32) and walks a run of R consecutive
// tokens, keeping the last WMAX rows of both streams in registers, so every
// input row is fetched from HBM about once (plus a W-1 row halo per run).  The
// kernel is a pure streaming kernel: bound by HBM bandwidth.
#include "device_common.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

constexpr int kConvRun = 32;   // tokens per thread
constexpr int kConvWMax = 8;   // largest supported width
constexpr int kConvThreads = 256;

template <typename IO> struct ConvVec;
template <> struct ConvVec<u16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const u16 *p, float *f) {
    const uint4 r = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(u16 *p, const float *f) {
    uint4 r;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    r.x = w[0]; r.y = w[1]; r.z = w[2]; r.w = w[3];
    *reinterpret_cast<uint4 *>(p) = r;
  }
};
template <> struct ConvVec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float *p, float *f) {
    const float4 r = *reinterpret_cast<const float4 *>(p);
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
  static __device__ __forceinline__ void store(float *p, const float *f) {
    *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};

template <typename IO>
__global__ __launch_bounds__(kConvThreads) void shortconv_dual_kernel(ShortConvArgs a) {
  using V = ConvVec<IO>;
  constexpr int N = V::N;
  const int64_t c0 = ((int64_t)blockIdx.x * kConvThreads + threadIdx.x) * N;
  if (c0 >= a.C) return;
  const int64_t t_begin = (int64_t)blockIdx.y * kConvRun;
  const int64_t t_end = min(t_begin + kConvRun, a.T);
  const int W = a.W;
  const IO *x = reinterpret_cast<const IO *>(a.x);
  const IO *xn = reinterpret_cast<const IO *>(a.xn);
  IO *y = reinterpret_cast<IO *>(a.y);
  IO *yn = reinterpret_cast<IO *>(a.yn);

  // weights by lag: wl[L][c] multiplies x[t - L]; lags >= W are zero
  float wl[kConvWMax][N];
#pragma unroll
  for (int L = 0; L < kConvWMax; ++L)
#pragma unroll
    for (int c = 0; c < N; ++c) wl[L][c] = L < W ? a.w[(c0 + c) * W + (W - 1 - L)] : 0.f;
  float bias[N];
#pragma unroll
  for (int c = 0; c < N; ++c) bias[c] = a.bias ? a.bias[c0 + c] : 0.f;

  // start W-1 tokens early to fill the history window
  const int64_t ts = max((int64_t)0, t_begin - (W - 1));
  // document containing ts (binary search over cu_seqlens)
  int lo = 0, hi = a.num_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu[mid] <= ts) lo = mid; else hi = mid - 1;
  }
  int doc = lo;
  int64_t ds = a.cu[doc], de = a.cu[doc + 1];
  int64_t P = a.plen[doc];

  float hx[kConvWMax][N], hn[kConvWMax][N];
#pragma unroll
  for (int L = 0; L < kConvWMax; ++L)
#pragma unroll
    for (int c = 0; c < N; ++c) hx[L][c] = hn[L][c] = 0.f;

  for (int64_t t = ts; t < t_end; ++t) {
    while (t >= de) {  // next document: reset the history (taps before its start read 0)
      ++doc;
      ds = a.cu[doc];
      de = a.cu[doc + 1];
      P = a.plen[doc];
#pragma unroll
      for (int L = 0; L < kConvWMax; ++L)
#pragma unroll
        for (int c = 0; c < N; ++c) hx[L][c] = hn[L][c] = 0.f;
    }
    if (t == ds) {
#pragma unroll
      for (int L = 0; L < kConvWMax; ++L)
#pragma unroll
        for (int c = 0; c < N; ++c) hx[L][c] = hn[L][c] = 0.f;
    }
    const int64_t tp = t - ds;  // position inside the document
    const bool resp = tp >= P;
#pragma unroll
    for (int L = kConvWMax - 1; L > 0; --L)
#pragma unroll
      for (int c = 0; c < N; ++c) {
        hx[L][c] = hx[L - 1][c];
        hn[L][c] = hn[L - 1][c];
      }
    V::load(x + t * a.C + c0, hx[0]);
    if (resp) V::load(xn + t * a.C + c0, hn[0]);
    else {
#pragma unroll
      for (int c = 0; c < N; ++c) hn[0][c] = 0.f;
    }
    if (t < t_begin) continue;
    float yc[N], ynv[N];
#pragma unroll
    for (int c = 0; c < N; ++c) yc[c] = bias[c];
#pragma unroll
    for (int L = 0; L < kConvWMax; ++L)
#pragma unroll
      for (int c = 0; c < N; ++c) yc[c] += wl[L][c] * hx[L][c];
    if (resp) {
      // taps at lag L <= tp - blk lie inside the block and read the noisy input
      const int64_t blk = P + ((tp - P) / a.B) * a.B;
      const int64_t inside = tp - blk;
#pragma unroll
      for (int c = 0; c < N; ++c) ynv[c] = bias[c];
#pragma unroll
      for (int L = 0; L < kConvWMax; ++L) {
        const bool noisy = L <= inside;
#pragma unroll
        for (int c = 0; c < N; ++c) ynv[c] += wl[L][c] * (noisy ? hn[L][c] : hx[L][c]);
      }
    }
    if (a.activation == 1) {
#pragma unroll
      for (int c = 0; c < N; ++c) {
        yc[c] = yc[c] / (1.f + __expf(-yc[c]));
        ynv[c] = ynv[c] / (1.f + __expf(-ynv[c]));
      }
    }
    if (!resp) {
#pragma unroll
      for (int c = 0; c < N; ++c) ynv[c] = 0.f;
    }
    V::store(y + t * a.C + c0, yc);
    V::store(yn + t * a.C + c0, ynv);
  }
}

hipError_t launch_shortconv(const ShortConvArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int N = a.bf16 ? 8 : 4;
  const int64_t vecs = a.C / N;
  const dim3 grid((unsigned)((vecs + kConvThreads - 1) / kConvThreads),
                  (unsigned)((a.T + kConvRun - 1) / kConvRun));
  TimedLaunch tl(K_SHORTCONV, st);
  if (a.bf16)
    hipLaunchKernelGGL(shortconv_dual_kernel<u16>, grid, dim3(kConvThreads), 0, st, a);
  else
    hipLaunchKernelGGL(shortconv_dual_kernel<float>, grid, dim3(kConvThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
