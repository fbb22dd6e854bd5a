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
// Layout: x, xn, y, yn are [T, C] with channels contiguous.  A lane owns an
// 8-byte slice of channels (4 bytes for W > 4) and walks a run of 64 tokens,
// keeping the last W rows of both inputs in registers, so every input row is
// read from HBM about once (plus a W - 1 row halo per run); the four waves of
// a workgroup take four consecutive runs.  Since the step's position is
// uniform over the wave, which taps lie inside the document and which inside
// the block are wave-uniform masks.  The input rows of step t + U - 1 are
// loaded at step t into a register ring of U = max(W, 4) slots (the loop is
// unrolled by U, so slots are static), and every load and store is
// unconditional -- rows clamped into the batch, the noisy row of a prompt
// position redirected to the clean row the step loads anyway -- so U - 1
// steps of loads stay in flight.  A pure streaming kernel: bound by HBM
// bandwidth.
#include "conv_common.h"
#include "device_common.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

using conv::Slice;
using conv::for_each_slot;
using conv::GroupSum;

namespace {

constexpr int kConvWaves = 4;   // runs per workgroup
constexpr int kConvRun = 64;    // tokens per wave

template <typename IO, int W> struct FwdCfg {
  static constexpr int N = (W <= 4 ? 8 : 4) / (int)sizeof(IO);  // channels per lane
  static constexpr int U = W < 4 ? 4 : W;                        // ring slots
};

}  // namespace

// NRM: the section's outputs are L2-normalised per group of a.hd channels
// (sections sec0 + blockIdx.z, all with or all without the normalisation)
template <typename IO, int W, bool ACT, bool NRM>
__global__ __launch_bounds__(256) void shortconv_dual_kernel(ShortConvArgs a, const int32_t *__restrict__ cu,
                                                             const int32_t *__restrict__ plen, int sec0) {
  using Cfg = FwdCfg<IO, W>;
  constexpr int N = Cfg::N, U = Cfg::U;
  using S = Slice<IO, N>;
  using Raw = typename S::Raw;

  // the wave index through readfirstlane: the run, its documents and the
  // per-step tap masks are then uniform (scalar registers)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sec = sec0 + (int)blockIdx.z;
  const IO *const x = reinterpret_cast<const IO *>(a.x[sec]), *const xn = reinterpret_cast<const IO *>(a.xn[sec]);
  IO *const y = reinterpret_cast<IO *>(a.y[sec]), *const yn = reinterpret_cast<IO *>(a.yn[sec]);
  const float *const wsec = a.w[sec];
  const int64_t C = a.C;
  const int T = (int)a.T;
  const int64_t cb = (int64_t)blockIdx.y * 64 * N;
  // lanes past the last channel repeat the matching lanes of the last group
  // (head) of channels: same inputs, same results, duplicate stores of
  // identical values, and group sums that never mix live and repeated lanes
  const int64_t grp = NRM ? a.hd : N;
  const int64_t c0 = cb + (int64_t)lane * N;
  const int64_t cl = c0 < C ? c0 : C - grp + c0 % grp;
  const GroupSum group_sum((int)(grp / N));  // sums over the lanes of a group
  const uint32_t lo = (uint32_t)(cl * (int64_t)sizeof(IO));
  const int tb = (int)blockIdx.x * (kConvWaves * kConvRun) + wave * kConvRun;
  const int te = min(tb + kConvRun, T);
  if (te <= tb) return;
  auto at = [&](const IO *row) { return S::load(reinterpret_cast<const IO *>(reinterpret_cast<const char *>(row) + lo)); };

  // weights by lag: wl[L] multiplies the input L tokens back
  float wl[W][N], bias[N];
#pragma unroll
  for (int L = 0; L < W; ++L)
#pragma unroll
    for (int c = 0; c < N; ++c) wl[L][c] = wsec[(cl + c) * W + (W - 1 - L)];
#pragma unroll
  for (int c = 0; c < N; ++c) bias[c] = a.bias ? a.bias[cl + c] : 0.f;

  // steps t in [t0, te), a whole number of U-step groups; the first W - 1 (or
  // more) only fill the window, and their stores go to row tb, which its own
  // step rewrites later
  const int nsteps = (te - tb + W - 1 + U - 1) / U * U;
  const int t0 = te - nsteps;
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
  // position in the block at the step before the first valid one, stepped
  // after (blocks start at the prompt end; prompts are whole blocks)
  int inb = 0;
  {
    const int tp1 = max(t0, 0) - cds;
    if (tp1 > cP) inb = (tp1 - 1 - cP) % a.B;
  }

  Raw rx[U], rn[U];
  float hx[U][N], hn[U][N];
#pragma unroll
  for (int j = 0; j < U; ++j)
#pragma unroll
    for (int c = 0; c < N; ++c) hx[j][c] = hn[j][c] = 0.f;
  auto issue = [&](int slot, int t) {
    const int tc = min(max(t, 0), T - 1);
    while (tc >= lde && dl + 1 < a.num_docs) {
      ++dl;
      lds_ = cu[dl];
      lde = cu[dl + 1];
      lP = plen[dl];
    }
    const bool resp = t >= 0 && t < T && tc - lds_ >= lP;
    const int64_t o = (int64_t)tc * C;
    rx[slot] = at(x + o);
    rn[slot] = at((resp ? xn : x) + o);
  };
#pragma unroll
  for (int j = 0; j < U - 1; ++j) issue(j, t0 + j);

  for (int s0 = 0; s0 < nsteps; s0 += U) {
    for_each_slot(std::make_integer_sequence<int, U>{}, [&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int t = t0 + s0 + J;
      S::cvt(rx[J], hx[J]);
      S::cvt(rn[J], hn[J]);
      issue((J + U - 1) % U, t + U - 1);
      const bool valid = t >= 0;  // t < te <= T always
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
      // taps L < nb read inside the document (earlier ones read zero), taps
      // L < na inside the block (the noisy input)
      const int nb = valid ? min(tp + 1, W) : 0;
      const int na = resp ? min(inb + 1, W) : 0;
      float yc[N], ynv[N];
#pragma unroll
      for (int c = 0; c < N; ++c) yc[c] = ynv[c] = bias[c];
#pragma unroll
      for (int L = 0; L < W; ++L) {
        const int r = (J - L + U * W) % U;
#pragma unroll
        for (int c = 0; c < N; ++c) {
          const float hxu = L < nb ? hx[r][c] : 0.f;
          yc[c] = fmaf(wl[L][c], hxu, yc[c]);
          ynv[c] = fmaf(wl[L][c], L < na ? hn[r][c] : hxu, ynv[c]);
        }
      }
      if (ACT) {
#pragma unroll
        for (int c = 0; c < N; ++c) {
          yc[c] = yc[c] / (1.f + __expf(-yc[c]));
          ynv[c] = ynv[c] / (1.f + __expf(-ynv[c]));
        }
      }
#pragma unroll
      for (int c = 0; c < N; ++c) ynv[c] = resp ? ynv[c] : 0.f;  // noisy prompt rows are zero
      if (NRM) {
        // divide each head's row by sqrt(sum y^2 + 1e-6) (zero rows stay zero)
        float ss = 0.f, ssn = 0.f;
#pragma unroll
        for (int c = 0; c < N; ++c) {
          ss = fmaf(yc[c], yc[c], ss);
          ssn = fmaf(ynv[c], ynv[c], ssn);
        }
        const float r = rsqrtf(group_sum(ss) + 1e-6f), rn = rsqrtf(group_sum(ssn) + 1e-6f);
#pragma unroll
        for (int c = 0; c < N; ++c) {
          yc[c] *= r;
          ynv[c] *= rn;
        }
      }
      const int64_t m = (int64_t)max(t, tb) * C;
      S::store(reinterpret_cast<IO *>(reinterpret_cast<char *>(y + m) + lo), yc);
      S::store(reinterpret_cast<IO *>(reinterpret_cast<char *>(yn + m) + lo), ynv);
    });
  }
}

template <typename IO, int W, bool NRM>
static hipError_t launch_fwd_wn(const ShortConvArgs &a, int sec0, int nsec, hipStream_t st) {
  constexpr int N = FwdCfg<IO, W>::N;
  // token blocks on x (no 65535 limit there), channel groups on y, sections on z
  const dim3 grid((unsigned)((a.T + kConvWaves * kConvRun - 1) / (kConvWaves * kConvRun)),
                  (unsigned)((a.C + 64 * N - 1) / (64 * N)), (unsigned)nsec);
  if (grid.y > 65535u) return hipErrorInvalidValue;
  if (a.activation == 1)
    hipLaunchKernelGGL((shortconv_dual_kernel<IO, W, true, NRM>), grid, dim3(256), 0, st, a, a.cu, a.plen, sec0);
  else
    hipLaunchKernelGGL((shortconv_dual_kernel<IO, W, false, NRM>), grid, dim3(256), 0, st, a, a.cu, a.plen, sec0);
  return hipGetLastError();
}

template <typename IO, int W>
static hipError_t launch_fwd_w(const ShortConvArgs &a, hipStream_t st) {
  // the normalised sections first, then the others
  if (a.nnorm > 0) {
    const hipError_t e = launch_fwd_wn<IO, W, true>(a, 0, a.nnorm, st);
    if (e != hipSuccess) return e;
  }
  if (a.nsec > a.nnorm) return launch_fwd_wn<IO, W, false>(a, a.nnorm, a.nsec - a.nnorm, st);
  return hipSuccess;
}

template <typename IO>
static hipError_t launch_fwd_io(const ShortConvArgs &a, hipStream_t st) {
  switch (a.W) {
    case 1: return launch_fwd_w<IO, 1>(a, st);
    case 2: return launch_fwd_w<IO, 2>(a, st);
    case 3: return launch_fwd_w<IO, 3>(a, st);
    case 4: return launch_fwd_w<IO, 4>(a, st);
    case 5: return launch_fwd_w<IO, 5>(a, st);
    case 6: return launch_fwd_w<IO, 6>(a, st);
    case 7: return launch_fwd_w<IO, 7>(a, st);
    case 8: return launch_fwd_w<IO, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shortconv(const ShortConvArgs &a, hipStream_t st) {
  if (a.T == 0 || a.C <= 0) return hipSuccess;
  TimedLaunch tl(K_SHORTCONV, st);
  return a.bf16 ? launch_fwd_io<u16>(a, st) : launch_fwd_io<float>(a, st);
}

}  // namespace flare
