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
// with 16-byte coalesced loads two chunks ahead (three register sets, used in
// turn).  No LDS but a per-wave staging area for the 16-byte stores of dS',
// no barrier.  Eight single-wave workgroups per (document, head), on one XCD
// so the operands they share stay in that XCD's L2.
#include "bwd_common.h"
#include "device_common.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int sC = 32, sD = 128, sNW = 2, sNQ = sD / (16 * sNW);  // waves per workgroup, workgroups per (doc, head)
constexpr int sRING = 4;                                            // register ring depth (chunks)
// the operands every slab needs (W, then K and K^T fragments: contiguous in the
// hand-over), in 1 KB units of 64 lanes x 16 bytes, split between the waves
constexpr int sSH = (kPackKT + 2048 - kPackW) / 256, sSHW = sSH / sNW;
static_assert(kPackKA == kPackW + 1024 && kPackKT == kPackKA + 2048, "shared operands must be contiguous");
static_assert(sSH == 20 && sSH % sNW == 0, "shared units");

// one chunk's loads for one wave: its R slab and its half of the shared units
struct ScanRing {
  uint4 r[8];
  uint4 sh[sSHW];
  float gc;  // g_C
};

struct ScanSmem {
  alignas(16) uint4 sh[2][sSH][64];          // shared units, double-buffered by chunk parity
  alignas(16) float stage[sNW][sD][16 + 4];  // per-wave dS' staging for 16-byte stores
};

}  // namespace

__global__ __launch_bounds__(64 * sNW) void gdn_bwd_scan_d128_kernel(BwdArgs a) {
  constexpr int C = sC, D = sD;
  __shared__ ScanSmem sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  // ---- workgroup -> (document, head, quarter); the quarters of a pair share an XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * sNQ), rem = L % (8 * sNQ);
  const int quarter = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= f.num_docs * f.H) return;
  const int doc = pair / f.H, h = pair % f.H;
  const int H = f.H;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int nchunks = (n + C - 1) / C;
  const int slab = sNW * quarter + wave;
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
      for (int r = 0; r < 4; ++r) sm.stage[wave][16 * kt + g4 + r][cl] = dS[kt][r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = j * 64 + lane, row = u >> 2, c4 = u & 3;
      *reinterpret_cast<float4 *>(dst + (size_t)row * D + dv0 + 4 * c4) =
          *reinterpret_cast<const float4 *>(&sm.stage[wave][row][4 * c4]);
    }
  };
  auto pack_of = [&](int c) { return a.pack + ((size_t)(ck_base + c) * H + h) * kPackWords; };
  // Loads are unconditional (the chunk index is clamped to 0 at the end), so
  // no load sits under a branch: the compiler would otherwise wait for every
  // load issued before it.
  auto load_ring = [&](ScanRing &p, int c) {
    const float *pk = pack_of(max(c, 0));
    const uint4 *pr = reinterpret_cast<const uint4 *>(pk + kPackR) + (size_t)slab * 8 * 64;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) p.r[kt] = pr[kt * 64 + lane];
    const uint4 *ps = reinterpret_cast<const uint4 *>(pk + kPackW) + (size_t)wave * sSHW * 64;
#pragma unroll
    for (int j = 0; j < sSHW; ++j) p.sh[j] = ps[j * 64 + lane];
    p.gc = pk[kPackG];
  };
  auto bf = [](const uint4 &v) { return __builtin_bit_cast(bf16x8, v); };
  // one chunk: store dS' (the chunk's end-state adjoint, for the per-chunk
  // pass), publish this wave's half of the shared operands, then the step;
  // the ring slot is refilled with the chunk sRING steps on once R is used
  auto step = [&](ScanRing &p, int c) {
    store_dS(ws + ((ck_base + c) * H + h) * (size_t)D * D);
    uint4 (*sh)[64] = sm.sh[c & 1];
#pragma unroll
    for (int j = 0; j < sSHW; ++j) sh[wave * sSHW + j][lane] = p.sh[j];
    lds_barrier();
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
        const bf16x8 ak = bf(sh[4 + 2 * ks + tr][lane]);
        mma_bf16(X.t[tr], ak, bh);
        mma_bf16(X.t[tr], ak, bl);
      }
    }
    // Y = W X
    bf16x8 xh, xl;
    slab_b_split(X, xh, xl);
    Slab Y = slab_zero();
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const bf16x8 wh = bf(sh[2 * tr][lane]), wl = bf(sh[2 * tr + 1][lane]);
      mma_bf16(Y.t[tr], wh, xh);
      mma_bf16(Y.t[tr], wh, xl);
      mma_bf16(Y.t[tr], wl, xh);
    }
    // dS_c = g_C dS' + R + K^T Y
    bf16x8 yh, yl;
    slab_b_split(Y, yh, yl);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const float4 rv = __builtin_bit_cast(float4, p.r[kt]);
      dS[kt] = p.gc * dS[kt] + floatx4{rv.x, rv.y, rv.z, rv.w};
      mma_bf16(dS[kt], bf(sh[12 + kt][lane]), yh);
      mma_bf16(dS[kt], bf(sh[12 + kt][lane]), yl);
    }
    load_ring(p, c - sRING);
  };

  // sRING operand sets in rotation: sRING - 1 chunks in flight while one computes
  ScanRing p0, p1, p2, p3;
  static_assert(sRING == 4, "the rotation below names four sets");
  load_ring(p0, nchunks - 1);
  load_ring(p1, nchunks - 2);
  load_ring(p2, nchunks - 3);
  load_ring(p3, nchunks - 4);
  for (int c = nchunks - 1; c >= 0; c -= 4) {
    step(p0, c);
    if (c == 0) break;
    step(p1, c - 1);
    if (c == 1) break;
    step(p2, c - 2);
    if (c == 2) break;
    step(p3, c - 3);
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
  hipLaunchKernelGGL(gdn_bwd_scan_d128_kernel, dim3((unsigned)(groups * 8 * sNQ)), dim3(64 * sNW), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
