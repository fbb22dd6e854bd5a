// gdn_bwd_scan.hip -- reverse scan of the state adjoint for bf16 io at
// d_k = d_v = 128 (the other shapes use the generic scan in gdn_bwd.hip).
//
// The pre-pass (gdn_bwd_pre.hip) has reduced the chunk step to
//   dS_c = g_C dS' + R + K^T (W (K dS'))
// (R: 128 x 128 right-hand side, W: 32 x 32 chain matrix, K: the chunk's keys),
// so what stays sequential is three small products per chunk.  Every column
// of dS evolves on its own, so a wave owns a 16-column slab of d_v: its
// 128 x 16 slab of dS lives in MFMA accumulators for the whole document (8
// tiles over d_k) and every operand arrives already in register order, read
// with 16-byte coalesced loads one chunk ahead (two register sets, used in
// turn).  No LDS but a per-wave staging area for the 16-byte stores of dS',
// no barrier.  Eight single-wave workgroups per (document, head), on one XCD
// so the operands they share stay in that XCD's L2.
#include "bwd_common.h"
#include "device_common.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int sC = 32, sD = 128, sNS = sD / 16;  // slabs (single-wave workgroups) per (doc, head)

// one chunk's operands in the order the step consumes them
struct ScanOps {
  float4 r[8];   // R, accumulator tile kt of this slab
  uint4 w[4];    // W fragments [tr][hi / lo]
  uint4 ka[8];   // K fragments [ks][tr]
  uint4 kt[8];   // K^T fragments [kt]
  float gc;      // g_C
};

}  // namespace

__global__ __launch_bounds__(64) void gdn_bwd_scan_d128_kernel(BwdArgs a) {
  constexpr int C = sC, D = sD;
  __shared__ alignas(16) float stage[D][16 + 4];  // dS' slab staging for 16-byte stores
  const FwdArgs &f = a.f;
  const int lane = threadIdx.x;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  // ---- workgroup -> (document, head, slab); the slabs of a pair share an XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * sNS), rem = L % (8 * sNS);
  const int slab = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= f.num_docs * f.H) return;
  const int doc = pair / f.H, h = pair % f.H;
  const int H = f.H;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int nchunks = (n + C - 1) / C;
  const int dv0 = 16 * slab;
  const int64_t ck_base = (int64_t)(t0g / C) + doc;
  float *const ws = reinterpret_cast<float *>(a.workspace);

  // ---- dS slab: tile kt holds rows 16 kt + 4 g + r (d_k), column dv0 + cl
  floatx4 dS[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    dS[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (a.dh_final) {
      const float *src = a.dh_final + ((size_t)doc * H + h) * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) dS[kt][r] = src[(size_t)(16 * kt + g4 + r) * D + dv0 + cl];
    }
  }
  // the dS slab -> global, row-major [d_k][d_v], through this wave's LDS:
  // 8 16-byte stores per lane instead of 32 scalar ones
  auto store_dS = [&](float *dst) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) stage[16 * kt + g4 + r][cl] = dS[kt][r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = j * 64 + lane, row = u >> 2, c4 = u & 3;
      *reinterpret_cast<float4 *>(dst + (size_t)row * D + dv0 + 4 * c4) =
          *reinterpret_cast<const float4 *>(&stage[row][4 * c4]);
    }
  };
  // Loads are unconditional (the chunk index is clamped to 0 at the end), so
  // no load sits under a branch: the compiler would otherwise wait for every
  // load issued before it.
  auto load_ops = [&](ScanOps &p, int c) {
    const float *pk = a.pack + ((size_t)(ck_base + max(c, 0)) * H + h) * kPackWords;
    const float4 *pr = reinterpret_cast<const float4 *>(pk + kPackR) + (size_t)slab * 8 * 64;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) p.r[kt] = pr[kt * 64 + lane];
    const uint4 *pw = reinterpret_cast<const uint4 *>(pk + kPackW);
#pragma unroll
    for (int j = 0; j < 4; ++j) p.w[j] = pw[j * 64 + lane];
    const uint4 *pa = reinterpret_cast<const uint4 *>(pk + kPackKA);
#pragma unroll
    for (int j = 0; j < 8; ++j) p.ka[j] = pa[j * 64 + lane];
    const uint4 *pt = reinterpret_cast<const uint4 *>(pk + kPackKT);
#pragma unroll
    for (int j = 0; j < 8; ++j) p.kt[j] = pt[j * 64 + lane];
    p.gc = pk[kPackG];
  };
  auto bf = [](const uint4 &v) { return __builtin_bit_cast(bf16x8, v); };
  // one chunk: store dS' (the chunk's end-state adjoint, for the per-chunk
  // pass), fetch the next chunk's operands, then the step
  auto step = [&](const ScanOps &p, ScanOps &nxt, int c) {
    store_dS(ws + ((ck_base + c) * H + h) * (size_t)D * D);
    load_ops(nxt, c - 1);
    // X = K dS' (dS' from the accumulators: k-slots of step ks are d_k rows
    // 32 ks + 4 g + e (e < 4) and 32 ks + 16 + 4 g + e - 4, split hi + lo)
    Slab X = slab_zero();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float xv[8] = {dS[2 * ks][0], dS[2 * ks][1], dS[2 * ks][2], dS[2 * ks][3],
                           dS[2 * ks + 1][0], dS[2 * ks + 1][1], dS[2 * ks + 1][2], dS[2 * ks + 1][3]};
      bf16x8 bh, bl;
      split8(xv, bh, bl);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        mma_bf16(X.t[tr], bf(p.ka[2 * ks + tr]), bh);
        mma_bf16(X.t[tr], bf(p.ka[2 * ks + tr]), bl);
      }
    }
    // Y = W X
    bf16x8 xh, xl;
    slab_b_split(X, xh, xl);
    Slab Y = slab_zero();
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      mma_bf16(Y.t[tr], bf(p.w[2 * tr]), xh);
      mma_bf16(Y.t[tr], bf(p.w[2 * tr]), xl);
      mma_bf16(Y.t[tr], bf(p.w[2 * tr + 1]), xh);
    }
    // dS_c = g_C dS' + R + K^T Y
    bf16x8 yh, yl;
    slab_b_split(Y, yh, yl);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      dS[kt] = p.gc * dS[kt] + floatx4{p.r[kt].x, p.r[kt].y, p.r[kt].z, p.r[kt].w};
      mma_bf16(dS[kt], bf(p.kt[kt]), yh);
      mma_bf16(dS[kt], bf(p.kt[kt]), yl);
    }
  };

  ScanOps pa, pb;
  load_ops(pa, nchunks - 1);
  for (int c = nchunks - 1; c >= 0; c -= 2) {
    step(pa, pb, c);
    if (c == 0) break;
    step(pb, pa, c - 1);
  }
  if (a.dh0) {
    float *dst = a.dh0 + ((size_t)doc * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * kt + g4 + r) * D + dv0 + cl] = dS[kt][r];
  }
}

hipError_t launch_bwd_scan_d128(const BwdArgs &a, hipStream_t st) {
  const int pairs = a.f.num_docs * a.f.H;
  const int groups = (pairs + 7) / 8;
  hipLaunchKernelGGL(gdn_bwd_scan_d128_kernel, dim3((unsigned)(groups * 8 * sNS)), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
