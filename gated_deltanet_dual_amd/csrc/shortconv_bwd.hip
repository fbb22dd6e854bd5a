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
// Layout: [T, C] with channels contiguous.  A lane owns an 8-byte slice of
// channels (4 bytes for W > 4) and walks a run of 64 tokens; the four waves of
// a workgroup take four consecutive runs over the same channels.  Scatter form:
// at step t the lane turns g(t), g~(t) into their contributions to the pending
// dx, dx~ rows t - L, L < W; row t - W + 1 is then complete and stored.  Since
// t is uniform over the wave, which lags are noisy (L <= in(t)) and which still
// lie in the document (L <= t - doc start) are uniform branches, not selects.
//
// Registers are indexed by step modulo U (U = max(W, 4); the loop is unrolled
// by U, so no window ever shifts), and the four input rows of step t + U - 1
// are loaded at step t.  Every load and store of the loop is unconditional
// (rows clamped into the batch, rows that are not needed redirected to the
// clean input row of the same step, which the same step loads anyway), so the
// compiler's wait counts never have to assume a skipped access and U - 1 steps
// of loads stay in flight.  The per-lag weight-gradient partials of the four
// runs are summed in LDS in a fixed order and written to a workspace
// [256-token block][C][W + 1] (taps, then bias); a second kernel sums them
// over the blocks in a fixed order, so the result is run-to-run identical.  Streaming:
// bound by HBM bandwidth.
#include "conv_common.h"
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

using conv::Slice;
using conv::for_each_slot;
using conv::GroupSum;

namespace {

constexpr int kBWaves = 4;                       // runs per workgroup
constexpr int kBRun = kConvBwdRun / kBWaves;     // tokens per wave (64)
static_assert(kBRun * kBWaves == kConvBwdRun, "workspace rows must be whole workgroups");

__device__ __forceinline__ float silu_grad(float z) {
  const float sg = 1.f / (1.f + __expf(-z));
  return sg * (1.f + z * (1.f - sg));
}

template <typename IO, int W> struct BwdCfg {
  static constexpr int N = (W <= 4 ? 8 : 4) / (int)sizeof(IO);  // channels per lane
  static constexpr int U = W < 4 ? 4 : W;                        // ring slots
  static constexpr int RED = 64 * N * (W + 1);                   // partials per wave
};

}  // namespace

// NRM: the forward L2-normalised the section's outputs per group of a.hd
// channels, so the incoming gradients are w.r.t. the normalised rows
template <typename IO, int W, bool ACT, bool NRM>
__global__ __launch_bounds__(256) void shortconv_dual_bwd_kernel(ShortConvBwdArgs a, const int32_t *__restrict__ cu,
                                                                 const int32_t *__restrict__ plen, int sec0,
                                                                 int64_t part_stride) {
  using Cfg = BwdCfg<IO, W>;
  constexpr int N = Cfg::N, U = Cfg::U;
  using S = Slice<IO, N>;
  using Raw = typename S::Raw;
  __shared__ float red[kBWaves][Cfg::RED];

  // the wave index through readfirstlane: everything derived from it (the
  // run, the documents, the per-step lag counts) is then known to be uniform
  // and lives in scalar registers.  Positions are 32-bit (the entry point
  // checks T < 2^31).
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sec = sec0 + (int)blockIdx.z;
  const IO *const x = reinterpret_cast<const IO *>(a.x[sec]), *const xn = reinterpret_cast<const IO *>(a.xn[sec]);
  const IO *const dy = reinterpret_cast<const IO *>(a.dy[sec]);
  const IO *const dyn = reinterpret_cast<const IO *>(a.dyn[sec]);
  IO *const dx = reinterpret_cast<IO *>(a.dx[sec]), *const dxn = reinterpret_cast<IO *>(a.dxn[sec]);
  const float *const wsec = a.w[sec];
  float *const part = a.part + sec * part_stride;
  const int64_t C = a.C;
  const int T = (int)a.T;
  const int64_t cb = (int64_t)blockIdx.y * 64 * N;
  // lanes past the last channel repeat the matching lanes of the last group
  // (head) of channels: same inputs, same results, duplicate stores of
  // identical values, group sums that never mix live and repeated lanes
  const int64_t grp = NRM ? a.hd : N;
  const int64_t c0 = cb + (int64_t)lane * N;
  const int64_t cl = c0 < C ? c0 : C - grp + c0 % grp;
  const GroupSum group_sum((int)(grp / N));  // sums over the lanes of a group
  const uint32_t lo = (uint32_t)(cl * (int64_t)sizeof(IO));  // byte offset in a row
  const int tb = (int)blockIdx.x * kConvBwdRun + wave * kBRun;
  const int te = min(tb + kBRun, T);
  auto at = [&](const IO *row) { return S::load(reinterpret_cast<const IO *>(reinterpret_cast<const char *>(row) + lo)); };

  float dwl[W][N], db[N];
#pragma unroll
  for (int c = 0; c < N; ++c) {
    db[c] = 0.f;
#pragma unroll
    for (int L = 0; L < W; ++L) dwl[L][c] = 0.f;
  }

  if (te > tb) {
    float wl[W][N], bias[N];
#pragma unroll
    for (int L = 0; L < W; ++L)
#pragma unroll
      for (int c = 0; c < N; ++c) wl[L][c] = wsec[(cl + c) * W + (W - 1 - L)];
#pragma unroll
    for (int c = 0; c < N; ++c) bias[c] = ACT && a.bias ? a.bias[cl + c] : 0.f;

    // steps t in [t0, te + W - 1), a whole number of U-step groups: output
    // m = t - W + 1 is complete at step t; the first steps only fill the
    // windows (their stores go to row tb, which its own step rewrites later)
    const int nsteps = (te - tb + 2 * (W - 1) + U - 1) / U * U;
    const int t0 = te + W - 1 - nsteps;
    // documents of the computed step (dc) and of the loaded one (dl)
    int dc = 0;
    {
      const int t1 = max(t0, 0);
      int hi = a.num_docs - 1;
      while (dc < hi) {
        const int mid = (dc + hi + 1) >> 1;
        if (cu[mid] <= t1) dc = mid; else hi = mid - 1;
      }
    }
    int cds = cu[dc], cde = cu[dc + 1], cP = plen[dc];
    int dl = dc, lds_ = cds, lde = cde, lP = cP;
    // position in the block at the step before the first valid one; stepped
    // after (blocks start at the prompt end, prompts are whole blocks)
    int inb = 0;
    {
      const int tp1 = max(t0, 0) - cds;
      if (tp1 > cP) inb = (tp1 - 1 - cP) % a.B;
    }

    Raw rx[U], rn[U], rg[U], rgn[U];
    // windows start at zero: the first steps read slots no step has filled
    // yet, with zero weight (0 * garbage could be NaN)
    float hx[U][N], hn[U][N], ax[U][N], an[U][N];
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int c = 0; c < N; ++c) hx[j][c] = hn[j][c] = ax[j][c] = an[j][c] = 0.f;
    auto issue = [&](int slot, int t) {
      const int tc = min(max(t, 0), T - 1);
      while (tc >= lde && dl + 1 < a.num_docs) {
        ++dl;
        lds_ = cu[dl];
        lde = cu[dl + 1];
        lP = plen[dl];
      }
      const bool resp = t >= 0 && t < T && tc - lds_ >= lP;
      const bool grad = t >= tb && t < T;
      const int64_t o = (int64_t)tc * C;
      rx[slot] = at(x + o);
      rn[slot] = at((resp ? xn : x) + o);
      rg[slot] = at((grad ? dy : x) + o);
      rgn[slot] = at((grad && resp ? dyn : x) + o);
    };
#pragma unroll
    for (int j = 0; j < U - 1; ++j) issue(j, t0 + j);

    for (int s0 = 0; s0 < nsteps; s0 += U) {
      for_each_slot(std::make_integer_sequence<int, U>{}, [&](auto jc) {
        constexpr int J = decltype(jc)::value;
        const int t = t0 + s0 + J;
        float g[N], gn[N];
        S::cvt(rx[J], hx[J]);
        S::cvt(rn[J], hn[J]);
        S::cvt(rg[J], g);
        S::cvt(rgn[J], gn);
        issue((J + U - 1) % U, t + U - 1);
        const bool valid = t >= 0 && t < T;
        if (valid) {
          while (t >= cde && dc + 1 < a.num_docs) {
            ++dc;
            cds = cu[dc];
            cde = cu[dc + 1];
            cP = plen[dc];
          }
        }
        const int tp = t - cds;
        const bool resp = valid && tp >= cP;
        if (resp) inb = tp == cP || inb + 1 == a.B ? 0 : inb + 1;
        // lags L < nb read inside the document, L < na inside the block
        // (noisy); no gradient before the run or past the batch
        const bool grad = valid && t >= tb;
        const int nb = grad ? min(tp + 1, W) : 0;
        const int na = grad && resp ? min(inb + 1, W) : 0;
        const bool own = grad && t < te;
        if (ACT || NRM) {
          // the forward's pre-activation sums of row t
          float z[N], zn[N];
#pragma unroll
          for (int c = 0; c < N; ++c) z[c] = zn[c] = bias[c];
#pragma unroll
          for (int L = 0; L < W; ++L) {
            const int r = (J - L + U * W) % U;
#pragma unroll
            for (int c = 0; c < N; ++c) {
              const float hxu = L < nb ? hx[r][c] : 0.f;
              z[c] = fmaf(wl[L][c], hxu, z[c]);
              zn[c] = fmaf(wl[L][c], L < na ? hn[r][c] : hxu, zn[c]);
            }
          }
          if (NRM) {
            // through y / sqrt(|y|^2 + 1e-6) per head: dy = r dyhat - y r^3 (y . dyhat)
            float yv[N], yvn[N], ss = 0.f, ssn = 0.f, dt = 0.f, dtn = 0.f;
#pragma unroll
            for (int c = 0; c < N; ++c) {
              yv[c] = ACT ? z[c] / (1.f + __expf(-z[c])) : z[c];
              yvn[c] = ACT ? zn[c] / (1.f + __expf(-zn[c])) : zn[c];
              ss = fmaf(yv[c], yv[c], ss);
              ssn = fmaf(yvn[c], yvn[c], ssn);
              dt = fmaf(yv[c], g[c], dt);
              dtn = fmaf(yvn[c], gn[c], dtn);
            }
            const float r = rsqrtf(group_sum(ss) + 1e-6f), rn = rsqrtf(group_sum(ssn) + 1e-6f);
            const float k3 = r * r * r * group_sum(dt), k3n = rn * rn * rn * group_sum(dtn);
#pragma unroll
            for (int c = 0; c < N; ++c) {
              g[c] = r * g[c] - yv[c] * k3;
              gn[c] = rn * gn[c] - yvn[c] * k3n;
            }
          }
          if (ACT) {
#pragma unroll
            for (int c = 0; c < N; ++c) {
              g[c] *= silu_grad(z[c]);
              gn[c] *= silu_grad(zn[c]);
            }
          }
        }
        float gs[N];
#pragma unroll
        for (int c = 0; c < N; ++c) gs[c] = na > 0 ? g[c] + gn[c] : g[c];
#pragma unroll
        for (int L = 0; L < W; ++L) {
          const int r = (J - L + U * W) % U;
          const bool live = L < nb, noisy = L < na;
#pragma unroll
          for (int c = 0; c < N; ++c) {
            // the part of the output gradient that reads x (q) and x~ (p)
            const float q = noisy ? g[c] : live ? gs[c] : 0.f;
            const float p = noisy ? gn[c] : 0.f;
            dwl[L][c] = fmaf(own ? q : 0.f, hx[r][c], dwl[L][c]);
            dwl[L][c] = fmaf(own ? p : 0.f, hn[r][c], dwl[L][c]);
            if (L == 0) {
              ax[J][c] = wl[0][c] * q;
              an[J][c] = wl[0][c] * p;
            } else {
              ax[r][c] = fmaf(wl[L][c], q, ax[r][c]);
              an[r][c] = fmaf(wl[L][c], p, an[r][c]);
            }
          }
        }
#pragma unroll
        for (int c = 0; c < N; ++c) db[c] += own ? gs[c] : 0.f;
        // row t - W + 1 has all its contributions
        constexpr int r = (J - (W - 1) + U * W) % U;
        const int64_t m = (int64_t)max(t - (W - 1), tb) * C;
        S::store(reinterpret_cast<IO *>(reinterpret_cast<char *>(dx + m) + lo), ax[r]);
        S::store(reinterpret_cast<IO *>(reinterpret_cast<char *>(dxn + m) + lo), an[r]);
      });
    }
  }

  // ---- weight and bias partials of the four runs, summed in wave order
  float *mine = red[wave] + lane * N * (W + 1);
#pragma unroll
  for (int c = 0; c < N; ++c) {
#pragma unroll
    for (int L = 0; L < W; ++L) mine[c * (W + 1) + (W - 1 - L)] = dwl[L][c];
    mine[c * (W + 1) + W] = db[c];
  }
  __syncthreads();
  const int nel = (int)min((int64_t)64 * N, C - cb) * (W + 1);
  float *dst = part + ((size_t)blockIdx.x * C + cb) * (W + 1);
  for (int e = threadIdx.x; e < nel; e += 256) dst[e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// dweight[c][j] and dbias[c]: the block partials summed in a fixed order.
// A workgroup owns 64 consecutive outputs; wave w sums the blocks r = w mod 4
// (eight loads in flight per lane), then the four sums are added in wave order.
__global__ __launch_bounds__(256) void shortconv_bwd_reduce_kernel(ShortConvBwdArgs a, int blocks,
                                                                   int64_t part_stride) {
  __shared__ float sums[4][64];
  const int sec = (int)blockIdx.y;
  const float *const part = a.part + sec * part_stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W1 = a.W + 1;
  const int64_t n = (int64_t)a.C * W1;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  const int64_t ic = min(i, n - 1);
  const size_t stride = (size_t)n;
  float s = 0.f;
  int r = wave;
  for (; r + 28 < blocks; r += 32) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = part[(size_t)(r + 4 * k) * stride + ic];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; r < blocks; r += 4) s += part[(size_t)r * stride + ic];
  sums[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && i < n) {
    const float t = ((sums[0][lane] + sums[1][lane]) + sums[2][lane]) + sums[3][lane];
    const int64_t c = i / W1, j = i % W1;
    if (j < a.W) a.dw[sec][c * a.W + j] = t;
    else if (a.dbias) a.dbias[c] = t;  // one section only
  }
}

template <typename IO, int W, bool NRM>
static hipError_t launch_bwd_wn(const ShortConvBwdArgs &a, int blocks, int64_t part_stride, int sec0, int nsec,
                                hipStream_t st) {
  constexpr int N = BwdCfg<IO, W>::N;
  // token blocks on x (no 65535 limit there), channel groups on y, sections on z
  const dim3 grid((unsigned)blocks, (unsigned)((a.C + 64 * N - 1) / (64 * N)), (unsigned)nsec);
  if (grid.y > 65535u) return hipErrorInvalidValue;
  if (a.activation == 1)
    hipLaunchKernelGGL((shortconv_dual_bwd_kernel<IO, W, true, NRM>), grid, dim3(256), 0, st, a, a.cu, a.plen, sec0,
                       part_stride);
  else
    hipLaunchKernelGGL((shortconv_dual_bwd_kernel<IO, W, false, NRM>), grid, dim3(256), 0, st, a, a.cu, a.plen,
                       sec0, part_stride);
  return hipGetLastError();
}

template <typename IO, int W>
static hipError_t launch_bwd_w(const ShortConvBwdArgs &a, int blocks, hipStream_t st) {
  const int64_t part_stride = (int64_t)blocks * a.C * (W + 1);
  if (a.nnorm > 0) {
    const hipError_t e = launch_bwd_wn<IO, W, true>(a, blocks, part_stride, 0, a.nnorm, st);
    if (e != hipSuccess) return e;
  }
  if (a.nsec > a.nnorm) return launch_bwd_wn<IO, W, false>(a, blocks, part_stride, a.nnorm, a.nsec - a.nnorm, st);
  return hipSuccess;
}

template <typename IO>
static hipError_t launch_bwd_io(const ShortConvBwdArgs &a, int blocks, hipStream_t st) {
  switch (a.W) {
    case 1: return launch_bwd_w<IO, 1>(a, blocks, st);
    case 2: return launch_bwd_w<IO, 2>(a, blocks, st);
    case 3: return launch_bwd_w<IO, 3>(a, blocks, st);
    case 4: return launch_bwd_w<IO, 4>(a, blocks, st);
    case 5: return launch_bwd_w<IO, 5>(a, blocks, st);
    case 6: return launch_bwd_w<IO, 6>(a, blocks, st);
    case 7: return launch_bwd_w<IO, 7>(a, blocks, st);
    case 8: return launch_bwd_w<IO, 8>(a, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shortconv_bwd(const ShortConvBwdArgs &a, hipStream_t st) {
  const int blocks = (int)((a.T + kConvBwdRun - 1) / kConvBwdRun);
  if (a.C <= 0) return hipSuccess;
  TimedLaunch tl(K_SHORTCONV_BWD, st);
  if (blocks > 0) {
    hipError_t e = a.bf16 ? launch_bwd_io<u16>(a, blocks, st) : launch_bwd_io<float>(a, blocks, st);
    if (e != hipSuccess) return e;
  }
  // with no tokens (blocks = 0) this writes the zero sums
  const int64_t outs = (int64_t)a.C * (a.W + 1);
  hipLaunchKernelGGL(shortconv_bwd_reduce_kernel, dim3((unsigned)((outs + 63) / 64), (unsigned)a.nsec), dim3(256), 0,
                     st, a, blocks, (int64_t)blocks * outs);
  return hipGetLastError();
}

}  // namespace flare
