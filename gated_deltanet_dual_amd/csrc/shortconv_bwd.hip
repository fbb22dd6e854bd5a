// shortconv_bwd.hip -- reverse mode of the dual-source depthwise causal
// ShortConv (shortconv.hip) over packed documents.
//
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
// designs item 3: a noisy output's tap that lies before the start of the
// output's block read the clean input, a tap inside the block read the noisy
// input, taps before the document start read zero.  With the lag weights
// wl[L] = w[W-1-L] (wl[L] multiplies the input L tokens back), the
// pre-activation sums z, z~ and
//   g(t) = dy(t) act'(z(t)),  g~(t) = dy~(t) act'(z~(t)) on response rows (else 0),
// the gradients are, over the outputs t = m + L of m's document,
//   dx(m)  = sum_L wl[L] (g(t) + [L > in(t)] g~(t))
//   dx~(m) = sum_L wl[L] [L <= in(t)] g~(t)
//   dwl[L] = sum_t g(t) x(t-L) + g~(t) (L <= in(t) ? x~(t-L) : x(t-L))
//   dbias  = sum_t g(t) + g~(t)
// with in(t) = t - (start of t's block) (-1 on prompt rows).
//
// Layout: [T, C] with channels contiguous.  A thread owns N channels (16 or 8
// bytes) and a run of R tokens, walking positions in order with three sliding
// register windows of WM rows: the inputs (to rebuild z and for dwl), the
// output gradients g, g~ with each row's in(t) (dx(m) needs the W rows
// m .. m + W - 1, so it is emitted W - 1 steps after m), and the per-lag
// weight-gradient partials of the run.  Those partials go to a workspace
// [run][C][W + 1] (taps, then bias) and a second kernel sums them over the
// runs in a fixed order, so the result is deterministic.  Streaming: bound by
// HBM bandwidth.
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

namespace {

constexpr int kBRun = kConvBwdRun;  // tokens per thread (the workspace is sized by it)
constexpr int kBThreads = 256;

template <typename IO, int N> struct BVec;
template <> struct BVec<u16, 8> {
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
    *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                               pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
};
template <> struct BVec<u16, 4> {
  static __device__ __forceinline__ void load(const u16 *p, float *f) {
    const uint2 r = *reinterpret_cast<const uint2 *>(p);
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xffff0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(u16 *p, const float *f) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  }
};
template <> struct BVec<float, 4> {
  static __device__ __forceinline__ void load(const float *p, float *f) {
    const float4 r = *reinterpret_cast<const float4 *>(p);
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
  static __device__ __forceinline__ void store(float *p, const float *f) {
    *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};

__device__ __forceinline__ float silu_grad(float z) {
  const float sg = 1.f / (1.f + __expf(-z));
  return sg * (1.f + z * (1.f - sg));
}

// the document containing position t (uniform: every thread of a workgroup
// walks the same positions), advanced monotonically
struct DocCursor {
  int doc;
  int64_t ds, de, P;
  __device__ __forceinline__ void seek(const ShortConvBwdArgs &a, int64_t t) {
    int lo = 0, hi = a.num_docs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    doc = lo;
    ds = a.cu[doc];
    de = a.cu[doc + 1];
    P = a.plen[doc];
  }
  // true when t starts a new document (also past empty ones)
  __device__ __forceinline__ bool advance(const ShortConvBwdArgs &a, int64_t t) {
    bool moved = false;
    while (t >= de && doc + 1 < a.num_docs) {
      ++doc;
      ds = a.cu[doc];
      de = a.cu[doc + 1];
      P = a.plen[doc];
      moved = true;
    }
    return moved || t == ds;
  }
};

}  // namespace

template <typename IO, int W, int N>
__global__ __launch_bounds__(kBThreads) void shortconv_dual_bwd_kernel(ShortConvBwdArgs a) {
  constexpr int WM = W;
  using V = BVec<IO, N>;
  const int64_t c0 = ((int64_t)blockIdx.y * kBThreads + threadIdx.x) * N;
  if (c0 >= a.C) return;
  const int run = blockIdx.x;
  const int64_t t_begin = (int64_t)run * kBRun;
  const int64_t t_end = min(t_begin + kBRun, a.T);
  const IO *x = reinterpret_cast<const IO *>(a.x), *xn = reinterpret_cast<const IO *>(a.xn);
  const IO *dy = reinterpret_cast<const IO *>(a.dy), *dyn = reinterpret_cast<const IO *>(a.dyn);
  IO *dx = reinterpret_cast<IO *>(a.dx), *dxn = reinterpret_cast<IO *>(a.dxn);

  float wl[WM][N];
#pragma unroll
  for (int L = 0; L < WM; ++L)
#pragma unroll
    for (int c = 0; c < N; ++c) wl[L][c] = a.w[(c0 + c) * W + (W - 1 - L)];
  float bias[N];
#pragma unroll
  for (int c = 0; c < N; ++c) bias[c] = a.bias ? a.bias[c0 + c] : 0.f;

  // windows: inputs at t - L, output gradients at t - L (row L = 0 newest)
  float hx[WM][N], hn[WM][N], gc[WM][N], gn[WM][N];
  int ins[WM];
#pragma unroll
  for (int L = 0; L < WM; ++L) {
    ins[L] = -1;
#pragma unroll
    for (int c = 0; c < N; ++c) hx[L][c] = hn[L][c] = gc[L][c] = gn[L][c] = 0.f;
  }
  float dwl[WM][N], db[N];
#pragma unroll
  for (int c = 0; c < N; ++c) {
    db[c] = 0.f;
#pragma unroll
    for (int L = 0; L < WM; ++L) dwl[L][c] = 0.f;
  }

  const int64_t t_lo = max((int64_t)0, t_begin - (W - 1));
  const int64_t t_hi = t_end + (W - 1);
  DocCursor dt, dm;
  dt.seek(a, t_lo);
  dm.seek(a, t_begin);

  for (int64_t t = t_lo; t < t_hi; ++t) {
    const bool valid = t < a.T;
    // ---- inputs at t (a new document starts with an empty history)
    if (valid && dt.advance(a, t)) {
#pragma unroll
      for (int L = 0; L < WM; ++L)
#pragma unroll
        for (int c = 0; c < N; ++c) hx[L][c] = hn[L][c] = 0.f;
    }
    const int64_t tp = t - dt.ds;
    const bool resp = valid && tp >= dt.P;
#pragma unroll
    for (int L = WM - 1; L > 0; --L) {
      ins[L] = ins[L - 1];
#pragma unroll
      for (int c = 0; c < N; ++c) {
        hx[L][c] = hx[L - 1][c];
        hn[L][c] = hn[L - 1][c];
        gc[L][c] = gc[L - 1][c];
        gn[L][c] = gn[L - 1][c];
      }
    }
#pragma unroll
    for (int c = 0; c < N; ++c) hx[0][c] = hn[0][c] = gc[0][c] = gn[0][c] = 0.f;
    ins[0] = -1;
    if (valid) V::load(x + t * a.C + c0, hx[0]);
    if (resp) V::load(xn + t * a.C + c0, hn[0]);
    // ---- output gradients at t (needed from t_begin on)
    if (valid && t >= t_begin) {
      const int64_t inside = resp ? tp - (dt.P + ((tp - dt.P) / a.B) * a.B) : -1;
      ins[0] = (int)inside;
      float g[N], gv[N];
      V::load(dy + t * a.C + c0, g);
      if (a.activation == 1) {
        float z[N];
#pragma unroll
        for (int c = 0; c < N; ++c) z[c] = bias[c];
#pragma unroll
        for (int L = 0; L < WM; ++L)
#pragma unroll
          for (int c = 0; c < N; ++c) z[c] += wl[L][c] * hx[L][c];
#pragma unroll
        for (int c = 0; c < N; ++c) g[c] *= silu_grad(z[c]);
      }
#pragma unroll
      for (int c = 0; c < N; ++c) gv[c] = 0.f;
      if (resp) {
        V::load(dyn + t * a.C + c0, gv);
        if (a.activation == 1) {
          float z[N];
#pragma unroll
          for (int c = 0; c < N; ++c) z[c] = bias[c];
#pragma unroll
          for (int L = 0; L < WM; ++L) {
            const bool noisy = L <= inside;
#pragma unroll
            for (int c = 0; c < N; ++c) z[c] += wl[L][c] * (noisy ? hn[L][c] : hx[L][c]);
          }
#pragma unroll
          for (int c = 0; c < N; ++c) gv[c] *= silu_grad(z[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < N; ++c) {
        gc[0][c] = g[c];
        gn[0][c] = gv[c];
      }
      // ---- weight and bias partials over this run's outputs
      if (t < t_end) {
#pragma unroll
        for (int L = 0; L < WM; ++L) {
          const bool noisy = L <= inside;
#pragma unroll
          for (int c = 0; c < N; ++c) dwl[L][c] += g[c] * hx[L][c] + gv[c] * (noisy ? hn[L][c] : hx[L][c]);
        }
#pragma unroll
        for (int c = 0; c < N; ++c) db[c] += g[c] + gv[c];
      }
    }
    // ---- dx(m), dx~(m) for m = t - (W - 1): rows m + L sit in window row W - 1 - L
    const int64_t m = t - (W - 1);
    if (m >= t_begin && m < t_end) {
      dm.advance(a, m);
      float ox[N], on[N];
#pragma unroll
      for (int c = 0; c < N; ++c) ox[c] = on[c] = 0.f;
#pragma unroll
      for (int L = 0; L < W; ++L) {
        const int r = W - 1 - L;  // window row of output m + L
        // outputs of m's document only
        const bool in_doc = m + L < dm.de;
        const bool noisy = L <= ins[r];
#pragma unroll
        for (int c = 0; c < N; ++c) {
          const float gcr = in_doc ? gc[r][c] : 0.f, gnr = in_doc ? gn[r][c] : 0.f;
          ox[c] += wl[L][c] * (gcr + (noisy ? 0.f : gnr));
          on[c] += noisy ? wl[L][c] * gnr : 0.f;
        }
      }
      V::store(dx + m * a.C + c0, ox);
      V::store(dxn + m * a.C + c0, on);
    }
  }
  // ---- partials: [run][C][W + 1], taps by index j = W - 1 - L, then the bias
  float *part = a.part + ((size_t)run * a.C + c0) * (W + 1);
#pragma unroll
  for (int c = 0; c < N; ++c) {
#pragma unroll
    for (int L = 0; L < W; ++L) part[(size_t)c * (W + 1) + (W - 1 - L)] = dwl[L][c];
    part[(size_t)c * (W + 1) + W] = db[c];
  }
}

// dweight[c][j] and dbias[c]: the run partials summed in run order
__global__ __launch_bounds__(256) void shortconv_bwd_reduce_kernel(ShortConvBwdArgs a, int runs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int W1 = a.W + 1;
  if (i >= (int64_t)a.C * W1) return;
  float s = 0.f;
  for (int r = 0; r < runs; ++r) s += a.part[(size_t)r * a.C * W1 + i];
  const int64_t c = i / W1, j = i % W1;
  if (j < a.W) a.dw[c * a.W + j] = s;
  else if (a.dbias) a.dbias[c] = s;
}

template <typename IO, int W>
static hipError_t launch_bwd_w(const ShortConvBwdArgs &a, int runs, hipStream_t st) {
  // up to 4 taps 16-byte rows of channels per thread; wider windows take half
  // as many channels, so the four windows still fit in registers
  constexpr int N = (sizeof(IO) == 2 && W <= 4) ? 8 : 4;
  // runs on x (no 65535 limit there), channel groups on y
  const dim3 grid((unsigned)runs, (unsigned)((a.C / N + kBThreads - 1) / kBThreads));
  if (grid.y > 65535u) return hipErrorInvalidValue;
  hipLaunchKernelGGL((shortconv_dual_bwd_kernel<IO, W, N>), grid, dim3(kBThreads), 0, st, a);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_bwd_io(const ShortConvBwdArgs &a, int runs, hipStream_t st) {
  switch (a.W) {
    case 1: return launch_bwd_w<IO, 1>(a, runs, st);
    case 2: return launch_bwd_w<IO, 2>(a, runs, st);
    case 3: return launch_bwd_w<IO, 3>(a, runs, st);
    case 4: return launch_bwd_w<IO, 4>(a, runs, st);
    case 5: return launch_bwd_w<IO, 5>(a, runs, st);
    case 6: return launch_bwd_w<IO, 6>(a, runs, st);
    case 7: return launch_bwd_w<IO, 7>(a, runs, st);
    case 8: return launch_bwd_w<IO, 8>(a, runs, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shortconv_bwd(const ShortConvBwdArgs &a, hipStream_t st) {
  const int runs = (int)((a.T + kBRun - 1) / kBRun);
  if (a.C <= 0) return hipSuccess;
  TimedLaunch tl(K_SHORTCONV_BWD, st);
  if (runs > 0) {
    hipError_t e = a.bf16 ? launch_bwd_io<u16>(a, runs, st) : launch_bwd_io<float>(a, runs, st);
    if (e != hipSuccess) return e;
  }
  // with no tokens (runs = 0) this writes the zero sums
  const int64_t outs = (int64_t)a.C * (a.W + 1);
  hipLaunchKernelGGL(shortconv_bwd_reduce_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st, a, runs);
  return hipGetLastError();
}

}  // namespace flare
