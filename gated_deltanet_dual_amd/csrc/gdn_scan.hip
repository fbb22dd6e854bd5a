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
// In reverse the store wave also writes each chunk's K dS' (the step's first
// product) over the chunk's R slabs in the hand-over, for the per-chunk
// gradient kernel (ScanArgs::kx).
//
// A long document is one long chain.  Its chunks can be cut into runs
// scanned in parallel (the affine segment scan): the step is affine in X, so
// a run maps its start value X_0 to M X_0 + N, with M the run's transfer map
// (the run scanned from the identity without the right-hand side) and N its
// offset (the run scanned from zero).  The runs' start values then follow
// from one short sequential pass over the runs (gdn_scan_compose_kernel), and
// a last parallel scan of every run from its start value writes the states.
//
// Chunk windows bound the memory of the per-chunk buffers: a launch then
// covers one window of chunks of every document, its chain carried from the
// previous window's launch through init / final_out.  Inside a window, runs
// that start at strided checkpoints rebuild every chunk-start state in
// parallel (the backward's rebuild when only every s-th state was kept).
#include "bwd_common.h"
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int sC = 32, sD = 128, sNW = 2, sNQ = sD / (16 * sNW);  // waves per workgroup, workgroups per (doc, head)
// register ring depth (chunks): 4 keeps one workgroup per CU (the deep
// ring's registers take a SIMD's whole file per wave); 2 lets the scan's
// registers fit two workgroups per CU (2 waves per SIMD), so that a second
// chain hides each one's latency (launch_scan_d128 picks per launch)
constexpr int sRING_DEEP = 4, sRING_SHALLOW = 2;
typedef unsigned v4u __attribute__((ext_vector_type(4)));           // a native vector for the nontemporal builtin
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
  // the carried slabs for the store wave, by chunk parity; the reverse scan
  // stages its K X slab in the row padding (row 64 tr + lane, columns 16-19)
  alignas(16) float stage[2][sNW][sD][16 + 4];
};

}  // namespace

// ZRHS: the right-hand side is K^T Z with Z a C x d_v matrix (stored as
// slabs, [slab 8][tile 2][lane 64][4], in the R area of the hand-over), added
// to W (K X) before the K^T product; else a full 128 x 128 R.
template <bool REVERSE, bool ZRHS, int RING>
__global__ __launch_bounds__(64 * (sNW + 1), RING == sRING_SHALLOW ? 2 : 1) void gdn_scan_d128_kernel(ScanArgs a) {
  using ScanRing = ScanRing<ZRHS>;
  constexpr int C = sC, D = sD;
  __shared__ ScanSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  // ---- workgroup -> (unit, head, quarter); the quarters of a pair share an XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * sNQ), rem = L % (8 * sNQ);
  const int quarter = rem / 8;
  const int64_t pair = (int64_t)grp * 8 + (rem % 8);
  const bool win = a.win_len > 0;
  const int64_t npairs = (a.seg_span > 0 || win ? a.units : a.num_docs) * a.H;
  if (pair >= npairs) return;
  const int64_t unit = pair / a.H;
  const int h = (int)(pair % a.H);
  const int H = a.H;
  int doc = (int)unit, seg = 0;
  if (win) {  // unit -> (document, run inside the window)
    if (a.seg_span > 0) {
      const int per = a.win_len / a.seg_span;
      doc = (int)(unit / per);
      seg = (int)(unit % per);
    }
  } else if (a.seg_span > 0) {  // unit -> (document, run): the checkpoint-slot numbering of stride seg_span
    const int64_t span = (int64_t)C * a.seg_span;
    int lo = 0, hi = a.num_docs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)a.cu[mid] / span + mid <= unit) lo = mid; else hi = mid - 1;
    }
    doc = lo;
    seg = (int)(unit - (int64_t)a.cu[doc] / span - doc);
  }
  const int64_t t0g = a.cu[doc];
  const int n = a.cu[doc + 1] - a.cu[doc];
  const int nchunks_doc = (n + C - 1) / C;
  // this chain's chunks [c_lo, c_hi); an empty document (or, in a window, a
  // document with no chunk there) is one empty chain: its init passes through
  const int c_base = (win ? a.win_lo : 0) + (a.seg_span > 0 ? seg * a.seg_span : 0);
  const int c_len = a.seg_span > 0 ? a.seg_span : win ? a.win_len : nchunks_doc;
  const int c_lo = c_base;
  const int c_hi = min(c_base + c_len, nchunks_doc);
  if (a.seg_span > 0 && c_lo > 0 && c_lo >= nchunks_doc) return;  // a unit no run maps to
  const int nchunks = max(c_hi - c_lo, 0);
  // where the chain starts (init, or seg_init of its unit) and whether it
  // ends in final_out: whole chains and window chains take both; runs of a
  // document take init only for its first run in scan order and write
  // final_out only from its last; runs inside a window start from seg_init
  bool use_init, write_final;
  if (win) {
    use_init = write_final = a.seg_span == 0;
  } else {
    use_init = !a.seg_init_all && (REVERSE ? c_hi == nchunks_doc : c_lo == 0);
    write_final = REVERSE ? c_lo == 0 : c_hi == nchunks_doc;
  }
  // seg_init / seg_final index: the unit, or in a window the run's checkpoint slot
  const int64_t ck_unit = win && a.seg_span > 0 ? t0g / ((int64_t)C * a.seg_span) + doc + c_lo / a.seg_span : unit;
  const int64_t ck_init = a.seg_init_stride > 0
                              ? t0g / ((int64_t)C * a.seg_init_stride) + doc + c_lo / a.seg_init_stride
                              : ck_unit;
  const int64_t ck_base = (int64_t)(t0g / C) + doc;
  // the slot of chunk c in pack and states
  auto wslot = [&](int c) -> int64_t { return win ? (int64_t)doc * a.win_len + (c - a.win_lo) : ck_base + c; };
  const int sstride = a.states_stride > 1 ? a.states_stride : 1;
  // step i handles chunk at(i)
  auto at = [&](int i) { return REVERSE ? c_hi - 1 - i : c_lo + i; };

  // The step order (measured per direction): the forward scan stages the
  // carried X for the store wave and publishes the chunk's shared operands
  // before each step's barrier; the reverse scan (LAG) does both after it,
  // during the step's products, with the store wave one chunk behind.
  constexpr bool LAG = REVERSE;

  // ---- the store wave: after barrier i (LAG: i + 1) the carried slabs the
  // compute waves staged for step i (chunk at(i), staging parity i & 1) ->
  // global, row-major [d_k][d_v], as 16-byte stores.  Its stores never hold
  // up the compute waves' loads (each wave's memory counter is in order).
  // Same barrier count as the compute waves: one per step (LAG: and one
  // after the last).
  if (wave == sNW) {
    if constexpr (LAG) lds_barrier();
    for (int i = 0; i < nchunks; ++i) {
      const int c = at(i);
      lds_barrier();
      float *dst = nullptr, *dck = nullptr;
      if (a.states && c % sstride == 0) {
        const int64_t sslot = sstride == 1 ? wslot(c) : t0g / ((int64_t)C * sstride) + doc + c / sstride;
        dst = a.states + (sslot * H + h) * (size_t)D * D;
      }
      if (a.ckpt && c % a.ckpt_stride == 0)
        dck = a.ckpt + ((t0g / ((int64_t)C * a.ckpt_stride) + doc + c / a.ckpt_stride) * H + h) * (size_t)D * D;
      float *const dkx = REVERSE && a.kx ? a.kx + ((size_t)wslot(c) * H + h) * kPackWords + kPackR : nullptr;
      if (dkx) {  // slab s of K X at the start of the chunk's R slab s
#pragma unroll
        for (int w = 0; w < sNW; ++w)
#pragma unroll
          for (int tr = 0; tr < 2; ++tr)
            *reinterpret_cast<floatx4 *>(dkx + (size_t)(sNW * quarter + w) * (8 * 256) + tr * 256 + 4 * lane) =
                *reinterpret_cast<const floatx4 *>(&sm.stage[i & 1][w][64 * tr + lane][16]);
      }
      if (!dst && !dck) continue;
#pragma unroll
      for (int w = 0; w < sNW; ++w)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int u = j * 64 + lane, row = u >> 2, c4 = u & 3;
          const size_t off = (size_t)row * D + 16 * (sNW * quarter + w) + 4 * c4;
          const float4 v4 = *reinterpret_cast<const float4 *>(&sm.stage[i & 1][w][row][4 * c4]);
          if (dst) *reinterpret_cast<float4 *>(dst + off) = v4;
          if (dck) *reinterpret_cast<float4 *>(dck + off) = v4;
        }
    }
    return;
  }
  const int slab = sNW * quarter + wave;
  const int dv0 = 16 * slab;

  // ---- X slab: tile kt holds rows 16 kt + 4 g + r (d_k), column dv0 + cl
  floatx4 X[8];
  const float *src = nullptr;
  if (!a.identity_init) {
    if (use_init) src = a.init ? a.init + ((size_t)(a.slot ? a.slot[doc] : doc) * H + h) * D * D : nullptr;
    else src = a.seg_init ? a.seg_init + ((size_t)ck_init * H + h) * D * D : nullptr;
  }
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    X[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (src) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X[kt][r] = src[(size_t)(16 * kt + g4 + r) * D + dv0 + cl];
    } else if (a.identity_init) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X[kt][r] = 16 * kt + g4 + r == dv0 + cl ? 1.f : 0.f;
    }
  }
  const bool homog = a.homog != 0;
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
    c = max(c_lo, min(c, c_hi - 1));
    const float *pk = a.pack + ((size_t)wslot(c) * H + h) * kPackWords;
    constexpr int NR = ZRHS ? 2 : 8;
    const uint4 *pr = reinterpret_cast<const uint4 *>(pk + kPackR) + (size_t)slab * NR * 64;
#pragma unroll
    for (int j = 0; j < NR; ++j) {  // read once: non-temporal
      const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(pr) + j * 64 + lane);
      p.r[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    // shared unit j * sNW + wave (clamped: the last round is partial, and
    // its surplus loads are repeats that are never published); the K units
    // (all but W's first four) from kpack's hand-over when it is given
    const uint4 *ps = reinterpret_cast<const uint4 *>(pk + kPackW);
    const uint4 *psk = ps;  // (the forward scan is compiled without kpack)
    if constexpr (REVERSE)
      if (a.kpack) psk = reinterpret_cast<const uint4 *>(a.kpack + ((size_t)wslot(c) * H + h) * kPackWords + kPackW);
    // (round j holds units j sNW .. j sNW + sNW - 1: W's in the first rounds)
    static_assert(((kPackKA - kPackW) / 256) % sNW == 0, "W's units must fill whole rounds");
#pragma unroll
    for (int j = 0; j < sSHW; ++j)
      p.sh[j] = (j * sNW < (kPackKA - kPackW) / 256 ? ps : psk)[min(j * sNW + wave, sSH - 1) * 64 + lane];
    p.gc = pk[kPackG];
  };
  auto bf = [](const uint4 &v) { return __builtin_bit_cast(bf16x8, v); };
  // this wave's half of a chunk's shared operands -> the LDS area of parity par
  auto publish = [&](const ScanRing &p, int par) {
    uint4 (*sh)[64] = sm.sh[par];
#pragma unroll
    for (int j = 0; j < sSHW; ++j)
      if (j * sNW + wave < sSH) sh[j * sNW + wave][lane] = p.sh[j];
  };
  // step i (chunk c = at(i)): after barrier i its shared operands are in
  // sh[i & 1].  LAG: the carried X is staged for the store wave and the next
  // chunk's operands (ring slot pn) published while the products run, every
  // operand fragment read first so those writes never queue ahead of a read
  // the products wait for.  The ring slot is refilled with chunk `refill`
  // once R is used.
  auto step = [&](ScanRing &p, const ScanRing &pn, int i, int refill) {
    if constexpr (!LAG) {
      stage_X(i & 1);
      publish(p, i & 1);
    }
    lds_barrier();
    const uint4 (*sh)[64] = sm.sh[i & 1];
    bf16x8 fka[8], fw[4], fkt[8];
    if constexpr (LAG) {
#pragma unroll
      for (int j = 0; j < 8; ++j) fka[j] = bf(sh[4 + j][lane]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fw[j] = bf(sh[j][lane]);
#pragma unroll
      for (int j = 0; j < 8; ++j) fkt[j] = bf(sh[12 + j][lane]);
    }
    auto KA = [&](int j) { if constexpr (LAG) return fka[j]; else return bf(sh[4 + j][lane]); };
    auto WF = [&](int j) { if constexpr (LAG) return fw[j]; else return bf(sh[j][lane]); };
    auto KT = [&](int j) { if constexpr (LAG) return fkt[j]; else return bf(sh[12 + j][lane]); };
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
        const bf16x8 ak = KA(2 * ks + tr);
        mma_bf16(KX.t[tr], ak, bh);
        mma_bf16(KX.t[tr], ak, bl);
      }
    }
    if constexpr (LAG) {
      stage_X(i & 1);
      if (REVERSE && a.kx) {
        *reinterpret_cast<floatx4 *>(&sm.stage[i & 1][wave][lane][16]) = KX.t[0];
        *reinterpret_cast<floatx4 *>(&sm.stage[i & 1][wave][64 + lane][16]) = KX.t[1];
      }
      if (i + 1 < nchunks) publish(pn, (i + 1) & 1);
    }
    // Y = W KX
    bf16x8 xh, xl;
    slab_b_split(KX, xh, xl);
    Slab Y = slab_zero();
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const bf16x8 wh = WF(2 * tr), wl = WF(2 * tr + 1);
      mma_bf16(Y.t[tr], wh, xh);
      mma_bf16(Y.t[tr], wh, xl);
      mma_bf16(Y.t[tr], wl, xh);
    }
    // X <- g_C X + R + K^T Y, or g_C X + K^T (Y + Z)
    if constexpr (ZRHS) {
      if (!homog) {
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          const float4 zv = __builtin_bit_cast(float4, p.r[tr]);
          Y.t[tr] += floatx4{zv.x, zv.y, zv.z, zv.w};
        }
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
        X[kt] = p.gc * X[kt] + (homog ? floatx4{0.f, 0.f, 0.f, 0.f} : floatx4{rv.x, rv.y, rv.z, rv.w});
      }
      mma_bf16(X[kt], KT(kt), yh);
      mma_bf16(X[kt], KT(kt), yl);
    }
    load_ring(p, refill);
  };

  // RING operand sets in rotation, RING - 1 chunks in flight while one
  // computes; LAG: the first chunk's shared operands are published up front
  static_assert(RING == sRING_DEEP || RING == sRING_SHALLOW, "the rotations below name four or two sets");
  if constexpr (RING == sRING_DEEP) {
    ScanRing p0, p1, p2, p3;
    load_ring(p0, at(0));
    load_ring(p1, at(1));
    load_ring(p2, at(2));
    load_ring(p3, at(3));
    if constexpr (LAG) publish(p0, 0);
    for (int i = 0; i < nchunks; i += 4) {
      step(p0, p1, i, at(i + 4));
      if (i + 1 >= nchunks) break;
      step(p1, p2, i + 1, at(i + 5));
      if (i + 2 >= nchunks) break;
      step(p2, p3, i + 2, at(i + 6));
      if (i + 3 >= nchunks) break;
      step(p3, p0, i + 3, at(i + 7));
    }
  } else {
    ScanRing p0, p1;
    load_ring(p0, at(0));
    load_ring(p1, at(1));
    if constexpr (LAG) publish(p0, 0);
    for (int i = 0; i < nchunks; i += 2) {
      step(p0, p1, i, at(i + 2));
      if (i + 1 >= nchunks) break;
      step(p1, p0, i + 1, at(i + 3));
    }
  }
  if constexpr (LAG) lds_barrier();  // the last step's staging, for the store wave
  if (a.final_out && write_final) {
    float *dst = a.final_out + ((size_t)(a.slot ? a.slot[doc] : doc) * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * kt + g4 + r) * D + dv0 + cl] = X[kt][r];
  }
  if (a.seg_final) {
    float *dst = a.seg_final + ((size_t)ck_unit * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * kt + g4 + r) * D + dv0 + cl] = X[kt][r];
  }
}

// The runs' start values, one workgroup of 8 waves per (document, head), wave
// w the 16-column slab w of X, in scan order over the document's runs:
//   seg_out[unit_g] = X_g,  X_{g+1} = M_g X_g + N_g
// (M_g X_g on the matrix cores, M split hi + lo as A fragments, X as split B
// fragments from its accumulators, the slab k-permutation of slab.h over
// d_k).  The maps pass through LDS, double-buffered by step parity: the
// workgroup loads the next map (8 float4s per thread, once for all waves)
// and the next offset slab while the current step runs from the other
// buffer, so the sequential steps do not wait on HBM.  MT: the maps are
// given transposed (M_g^T stored), and the A fragments are read down the
// staged columns.
constexpr int sLDM = sD + 4;  // map rows in LDS, padded
template <bool REVERSE, bool MT>
__global__ __launch_bounds__(512) void gdn_scan_compose_kernel(ScanArgs a, const float *M, const float *Nb,
                                                               float *seg_out) {
  constexpr int C = sC, D = sD, NT = 512;
  __shared__ float mb[2][D][sLDM];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  const int doc = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int H = a.H;
  const int n = a.cu[doc + 1] - a.cu[doc];
  const int nchunks = (n + C - 1) / C;
  const int nruns = nchunks == 0 ? 0 : (nchunks + a.seg_span - 1) / a.seg_span;
  const int64_t ubase = (int64_t)a.cu[doc] / ((int64_t)C * a.seg_span) + doc;
  const int dv0 = 16 * wave;
  // run unit of step j (scan order)
  auto unit_of = [&](int j) { return ubase + (REVERSE ? nruns - 1 - j : j); };
  // thread tid's share of a map: float4 f = e NT + tid, row f / 32, columns 4 (f % 32) ..
  constexpr int NE = D * D / 4 / NT;
  float4 m0r, m1r, m2r, m3r, m4r, m5r, m6r, m7r;  // named: an array here would live in scratch
  static_assert(NE == 8, "eight float4s per thread");
#define FLARE_MAP_LOAD(Mg)                                                                       \
  do {                                                                                         \
    const float *mg_ = (Mg);                                                                   \
    m0r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(0 * NT + tid));                  \
    m1r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(1 * NT + tid));                  \
    m2r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(2 * NT + tid));                  \
    m3r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(3 * NT + tid));                  \
    m4r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(4 * NT + tid));                  \
    m5r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(5 * NT + tid));                  \
    m6r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(6 * NT + tid));                  \
    m7r = *reinterpret_cast<const float4 *>(mg_ + 4 * (size_t)(7 * NT + tid));                  \
  } while (0)
  auto put_one = [&](int buf, int e, const float4 &v) {
    const int f = e * NT + tid;
    *reinterpret_cast<float4 *>(&mb[buf][f >> 5][4 * (f & 31)]) = v;
  };
  auto put_map = [&](int buf) {
    put_one(buf, 0, m0r); put_one(buf, 1, m1r); put_one(buf, 2, m2r); put_one(buf, 3, m3r);
    put_one(buf, 4, m4r); put_one(buf, 5, m5r); put_one(buf, 6, m6r); put_one(buf, 7, m7r);
  };
  floatx4 Yn[8];  // the next step's offset slab
  auto load_off = [&](int j) {
    const float *Ng = Nb + ((size_t)unit_of(j) * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Yn[kt][r] = Ng[(size_t)(16 * kt + g4 + r) * D + dv0 + cl];
  };
  auto map_ptr = [&](int j) { return M + ((size_t)unit_of(j) * H + h) * D * D; };
  floatx4 X[8];
  const float *src = a.init ? a.init + ((size_t)(a.slot ? a.slot[doc] : doc) * H + h) * D * D : nullptr;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) X[kt][r] = src ? src[(size_t)(16 * kt + g4 + r) * D + dv0 + cl] : 0.f;
  if (nruns > 1) {
    FLARE_MAP_LOAD(map_ptr(0));
    load_off(0);
    put_map(0);
  }
  lds_barrier();
  for (int j = 0; j < nruns; ++j) {
    float *so = seg_out + ((size_t)unit_of(j) * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) so[(size_t)(16 * kt + g4 + r) * D + dv0 + cl] = X[kt][r];
    if (j == nruns - 1) break;  // the last run's end value is the scan's own
    floatx4 Y[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) Y[kt] = Yn[kt];
    const bool more = j + 1 < nruns - 1;  // the next step multiplies too
    if (more) {
      FLARE_MAP_LOAD(map_ptr(j + 1));
      load_off(j + 1);
    }
    const float (*Mg)[sLDM] = mb[j & 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // X rows 32 ks + 4 g + e (e < 4) and 32 ks + 16 + 4 g + e - 4 as the B operand
      const float xv[8] = {X[2 * ks][0], X[2 * ks][1], X[2 * ks][2], X[2 * ks][3],
                           X[2 * ks + 1][0], X[2 * ks + 1][1], X[2 * ks + 1][2], X[2 * ks + 1][3]};
      bf16x8 bh, bl;
      split8(xv, bh, bl);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        // A: rows 16 kt + (l & 15) of M, columns in the same permutation
        float mv[8];
        if constexpr (MT) {  // M[i][k] = staged[k][i]: one column down the staged rows
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mv[e] = Mg[32 * ks + g4 + e][16 * kt + cl];
            mv[4 + e] = Mg[32 * ks + 16 + g4 + e][16 * kt + cl];
          }
        } else {
          const float *mr = &Mg[16 * kt + cl][32 * ks];
          const float4 m0 = *reinterpret_cast<const float4 *>(mr + g4);
          const float4 m1 = *reinterpret_cast<const float4 *>(mr + 16 + g4);
          mv[0] = m0.x; mv[1] = m0.y; mv[2] = m0.z; mv[3] = m0.w;
          mv[4] = m1.x; mv[5] = m1.y; mv[6] = m1.z; mv[7] = m1.w;
        }
        bf16x8 ah, al;
        split8(mv, ah, al);
        mma_bf16(Y[kt], ah, bh);
        mma_bf16(Y[kt], ah, bl);
        mma_bf16(Y[kt], al, bh);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) X[kt] = Y[kt];
    // the next map into the other buffer (its last reader was step j - 1,
    // before the previous barrier)
    if (more) put_map((j + 1) & 1);
    lds_barrier();
  }
#undef FLARE_MAP_LOAD
}

hipError_t launch_scan_compose_d128(const ScanArgs &a, const float *M, const float *Nb, float *seg_out, bool reverse,
                                    hipStream_t st, bool m_transposed) {
  const dim3 grid((unsigned)(a.num_docs * a.H)), block(512);
  if (reverse && m_transposed)
    hipLaunchKernelGGL((gdn_scan_compose_kernel<true, true>), grid, block, 0, st, a, M, Nb, seg_out);
  else if (reverse)
    hipLaunchKernelGGL((gdn_scan_compose_kernel<true, false>), grid, block, 0, st, a, M, Nb, seg_out);
  else if (m_transposed)
    hipLaunchKernelGGL((gdn_scan_compose_kernel<false, true>), grid, block, 0, st, a, M, Nb, seg_out);
  else
    hipLaunchKernelGGL((gdn_scan_compose_kernel<false, false>), grid, block, 0, st, a, M, Nb, seg_out);
  return hipGetLastError();
}

hipError_t scan_d128_runs(const ScanArgs &a, bool reverse, int span, int64_t units, float *ws, hipStream_t st,
                          const float *maps_t) {
  if (span <= 0) return launch_scan_d128(a, reverse, st);
  const size_t per = (size_t)units * a.H * sD * sD;
  float *const M = ws, *const Nb = ws + per, *const S = ws + 2 * per;
  ScanArgs r = a;
  r.seg_span = span;
  r.units = units;
  r.states = nullptr;
  r.ckpt = nullptr;
  r.kx = nullptr;
  r.final_out = nullptr;
  r.seg_init = nullptr;
  // the runs' transfer maps (from the identity, no right-hand side), unless given
  hipError_t e = hipSuccess;
  if (!maps_t) {
    ScanArgs m = r;
    m.init = nullptr;
    m.identity_init = 1;
    m.homog = 1;
    m.seg_final = M;
    e = launch_scan_d128(m, reverse, st);
    if (e != hipSuccess) return e;
  }
  // their offsets (from zero)
  ScanArgs z = r;
  z.init = nullptr;
  z.seg_final = Nb;
  e = launch_scan_d128(z, reverse, st);
  if (e != hipSuccess) return e;
  // the runs' start values in scan order, then every run from its start value
  ScanArgs c = a;
  c.seg_span = span;
  e = launch_scan_compose_d128(c, maps_t ? maps_t : M, Nb, S, reverse, st, maps_t != nullptr);
  if (e != hipSuccess) return e;
  c.units = units;
  c.seg_init = S;
  c.seg_final = nullptr;
  return launch_scan_d128(c, reverse, st);
}

hipError_t launch_scan_d128(const ScanArgs &a, bool reverse, hipStream_t st) {
  const int64_t pairs = (a.seg_span > 0 || a.win_len > 0 ? a.units : a.num_docs) * a.H;
  const int64_t groups = (pairs + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * sNQ)), block(64 * (sNW + 1));
  // the reverse recurrence carries a full R, the forward one K^T Z.  The
  // shallow ring (two workgroups per CU) when the launch has more workgroups
  // than CUs and either stores nothing per chunk (a long document's transfer
  // map and offset runs: latency-bound, a second chain per CU hides it) or
  // has many short chains (their start-up latency dominates); a launch that
  // streams every chunk's state out keeps the deep ring, one per CU (measured
  // at 8 x 4096 and 32 x 1024 tokens, 16 heads: the shallow ring was 4-27 %
  // slower there, 20-26 % faster for the runs and at 128 x 256)
  const bool stores = a.states || a.ckpt || a.kx;
  const bool shallow = grid.x > (unsigned)kScanWorkgroupTarget &&
                       (!stores || grid.x >= 16u * (unsigned)kScanWorkgroupTarget);
  if (reverse) {
    if (shallow) hipLaunchKernelGGL((gdn_scan_d128_kernel<true, false, sRING_SHALLOW>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gdn_scan_d128_kernel<true, false, sRING_DEEP>), grid, block, 0, st, a);
  } else {
    if (shallow) hipLaunchKernelGGL((gdn_scan_d128_kernel<false, true, sRING_SHALLOW>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gdn_scan_d128_kernel<false, true, sRING_DEEP>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace flare
