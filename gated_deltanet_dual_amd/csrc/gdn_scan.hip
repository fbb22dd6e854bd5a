// gdn_scan.hip -- the sequential part of the chunked recurrence, forward
// (the clean state) and reverse (the state adjoint), for bf16 io at
// d_k = d_v = 128.
//
// A pre-pass (gdn_fwd_pre.hip, gdn_bwd_pre.hip) reduces every chunk's step to
//   X <- g_C X + R + K^T (W (K X))
// (forward: R = K^T Z with Z only C x d_v, so the scan adds Z to W (K X) and
// reads a quarter of the bytes)
// (R: 128 x 128 right-hand side, W: 32 x 32 chain matrix, K: the chunk's keys,
// g_C: the chunk's decay), forward for the state S over the chunks of a
// document, in reverse for the adjoint dS; so what stays sequential is three
// small products per chunk.  The carried value before each chunk's step is
// stored at that chunk's slot: the chunk-start states S_c (the checkpoints)
// forward, the chunk end-state adjoints dS' in reverse.
//
// Every column of X evolves on its own, so a wave owns a 16-column slab of
// d_v: its 128 x 16 slab of X lives in MFMA accumulators for the whole
// document (8 tiles over d_k).  Every operand arrives in register order (the
// pre-pass stores it so): a wave's R slab and its share of the operands all
// slabs need (W and two fragment sets of K) are loaded four chunks ahead into
// a register ring with 16-byte coalesced loads; the shared operands are
// published to the other waves through a double-buffered LDS area, one
// barrier per chunk.  Two slabs form a workgroup, four workgroups per
// (document, head), on one XCD so the operands they share stay in its L2.
// A third wave per workgroup only stores: the compute waves stage each
// chunk's carried slabs in LDS and it writes them out, so the stores never sit
// in the compute waves' (in-order) memory counters ahead of their loads.
#include "bwd_common.h"
#include "device_common.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int sC = 32, sD = 128, sNW = 2, sNQ = sD / (16 * sNW);  // waves per workgroup, workgroups per (doc, head)
constexpr int sRING = 4;                                            // register ring depth (chunks)
// the operands every slab needs (W, then K and K^T fragments: contiguous in the
// hand-over), in 1 KB units of 64 lanes x 16 bytes, dealt round-robin to the waves
constexpr int sSH = (kPackKT + 2048 - kPackW) / 256, sSHW = (sSH + sNW - 1) / sNW;
static_assert(kPackKA == kPackW + 1024 && kPackKT == kPackKA + 2048, "shared operands must be contiguous");
static_assert(sSH == 20, "shared units");

// one chunk's loads for one wave: its right-hand side (the R slab, or the Z
// slab when the right-hand side is K^T Z) and its half of the shared units
template <bool ZRHS>
struct ScanRing {
  uint4 r[ZRHS ? 2 : 8];
  uint4 sh[sSHW];
  float gc;  // g_C
};

struct ScanSmem {
  alignas(16) uint4 sh[2][sSH][64];             // shared units, double-buffered by chunk parity
  alignas(16) float stage[2][sNW][sD][16 + 4];  // the carried slabs for the store wave, by chunk parity
};

}  // namespace

// ZRHS: the right-hand side is K^T Z with Z a C x d_v matrix (stored as
// slabs, [slab 8][tile 2][lane 64][4], in the R area of the hand-over), added
// to W (K X) before the K^T product; else a full 128 x 128 R.
template <bool REVERSE, bool ZRHS>
__global__ __launch_bounds__(64 * (sNW + 1)) void gdn_scan_d128_kernel(ScanArgs a) {
  using ScanRing = ScanRing<ZRHS>;
  constexpr int C = sC, D = sD;
  __shared__ ScanSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  // ---- workgroup -> (document, head, quarter); the quarters of a pair share an XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * sNQ), rem = L % (8 * sNQ);
  const int quarter = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= a.num_docs * a.H) return;
  const int doc = pair / a.H, h = pair % a.H;
  const int H = a.H;
  const int64_t t0g = a.cu[doc];
  const int n = a.cu[doc + 1] - a.cu[doc];
  const int nchunks = (n + C - 1) / C;
  const int64_t ck_base = (int64_t)(t0g / C) + doc;
  // step i handles chunk at(i)
  auto at = [&](int i) { return REVERSE ? nchunks - 1 - i : i; };

  // ---- the store wave: after each chunk's barrier, the carried slabs the
  // compute waves staged for that chunk -> global, row-major [d_k][d_v], as
  // 16-byte stores.  Its stores never hold up the compute waves' loads (each
  // wave's memory counter is in order).  Same barrier count as the compute
  // waves: one per chunk.
  if (wave == sNW) {
    for (int i = 0; i < nchunks; ++i) {
      const int c = at(i);
      lds_barrier();
      float *dst = a.states + ((ck_base + c) * H + h) * (size_t)D * D;
#pragma unroll
      for (int w = 0; w < sNW; ++w)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int u = j * 64 + lane, row = u >> 2, c4 = u & 3;
          *reinterpret_cast<float4 *>(dst + (size_t)row * D + 16 * (sNW * quarter + w) + 4 * c4) =
              *reinterpret_cast<const float4 *>(&sm.stage[c & 1][w][row][4 * c4]);
        }
    }
    return;
  }
  const int slab = sNW * quarter + wave;
  const int dv0 = 16 * slab;

  // ---- X slab: tile kt holds rows 16 kt + 4 g + r (d_k), column dv0 + cl
  floatx4 X[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    X[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (a.init) {
      const float *src = a.init + ((size_t)(a.slot ? a.slot[doc] : doc) * H + h) * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) X[kt][r] = src[(size_t)(16 * kt + g4 + r) * D + dv0 + cl];
    }
  }
  // the X slab -> the store wave's staging area for chunk parity `par`
  auto stage_X = [&](int par) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.stage[par][wave][16 * kt + g4 + r][cl] = X[kt][r];
  };
  // Loads are unconditional (the chunk index is clamped into the document:
  // an empty document still owns one slot), so no load sits under a branch:
  // the compiler would otherwise wait for every load issued before it.
  auto load_ring = [&](ScanRing &p, int c) {
    c = max(0, min(c, nchunks - 1));
    const float *pk = a.pack + ((size_t)(ck_base + c) * H + h) * kPackWords;
    constexpr int NR = ZRHS ? 2 : 8;
    const uint4 *pr = reinterpret_cast<const uint4 *>(pk + kPackR) + (size_t)slab * NR * 64;
#pragma unroll
    for (int j = 0; j < NR; ++j) p.r[j] = pr[j * 64 + lane];
    // shared unit j * sNW + wave (clamped: the last round is partial, and
    // its surplus loads are repeats that are never published)
    const uint4 *ps = reinterpret_cast<const uint4 *>(pk + kPackW);
#pragma unroll
    for (int j = 0; j < sSHW; ++j) p.sh[j] = ps[min(j * sNW + wave, sSH - 1) * 64 + lane];
    p.gc = pk[kPackG];
  };
  auto bf = [](const uint4 &v) { return __builtin_bit_cast(bf16x8, v); };
  // one chunk: stage the carried X for the store wave (it goes to the chunk's
  // slot), publish this wave's half of the shared operands, then the step;
  // the ring slot is refilled with chunk `refill` once R is used
  auto step = [&](ScanRing &p, int c, int refill) {
    stage_X(c & 1);
    uint4 (*sh)[64] = sm.sh[c & 1];
#pragma unroll
    for (int j = 0; j < sSHW; ++j)
      if (j * sNW + wave < sSH) sh[j * sNW + wave][lane] = p.sh[j];
    lds_barrier();
    // KX = K X (X from the accumulators: k-slots of step ks are d_k rows
    // 32 ks + 4 g + e (e < 4) and 32 ks + 16 + 4 g + e - 4, split hi + lo)
    Slab KX = slab_zero();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float xv[8] = {X[2 * ks][0], X[2 * ks][1], X[2 * ks][2], X[2 * ks][3],
                           X[2 * ks + 1][0], X[2 * ks + 1][1], X[2 * ks + 1][2], X[2 * ks + 1][3]};
      bf16x8 bh, bl;
      split8(xv, bh, bl);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const bf16x8 ak = bf(sh[4 + 2 * ks + tr][lane]);
        mma_bf16(KX.t[tr], ak, bh);
        mma_bf16(KX.t[tr], ak, bl);
      }
    }
    // Y = W KX
    bf16x8 xh, xl;
    slab_b_split(KX, xh, xl);
    Slab Y = slab_zero();
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const bf16x8 wh = bf(sh[2 * tr][lane]), wl = bf(sh[2 * tr + 1][lane]);
      mma_bf16(Y.t[tr], wh, xh);
      mma_bf16(Y.t[tr], wh, xl);
      mma_bf16(Y.t[tr], wl, xh);
    }
    // X <- g_C X + R + K^T Y, or g_C X + K^T (Y + Z)
    if constexpr (ZRHS) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const float4 zv = __builtin_bit_cast(float4, p.r[tr]);
        Y.t[tr] += floatx4{zv.x, zv.y, zv.z, zv.w};
      }
    }
    bf16x8 yh, yl;
    slab_b_split(Y, yh, yl);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      if constexpr (ZRHS) {
        X[kt] = p.gc * X[kt];
      } else {
        const float4 rv = __builtin_bit_cast(float4, p.r[kt]);
        X[kt] = p.gc * X[kt] + floatx4{rv.x, rv.y, rv.z, rv.w};
      }
      mma_bf16(X[kt], bf(sh[12 + kt][lane]), yh);
      mma_bf16(X[kt], bf(sh[12 + kt][lane]), yl);
    }
    load_ring(p, refill);
  };

  // sRING operand sets in rotation, sRING - 1 chunks in flight while one computes
  ScanRing p0, p1, p2, p3;
  static_assert(sRING == 4, "the rotation below names four sets");
  load_ring(p0, at(0));
  load_ring(p1, at(1));
  load_ring(p2, at(2));
  load_ring(p3, at(3));
  for (int i = 0; i < nchunks; i += 4) {
    step(p0, at(i), at(i + 4));
    if (i + 1 >= nchunks) break;
    step(p1, at(i + 1), at(i + 5));
    if (i + 2 >= nchunks) break;
    step(p2, at(i + 2), at(i + 6));
    if (i + 3 >= nchunks) break;
    step(p3, at(i + 3), at(i + 7));
  }
  if (a.final_out) {
    float *dst = a.final_out + ((size_t)(a.slot ? a.slot[doc] : doc) * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * kt + g4 + r) * D + dv0 + cl] = X[kt][r];
  }
}

hipError_t launch_scan_d128(const ScanArgs &a, bool reverse, hipStream_t st) {
  const int pairs = a.num_docs * a.H;
  const int groups = (pairs + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * sNQ)), block(64 * (sNW + 1));
  // the reverse recurrence carries a full R, the forward one K^T Z
  if (reverse) hipLaunchKernelGGL((gdn_scan_d128_kernel<true, false>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((gdn_scan_d128_kernel<false, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
