// gdn_bwd_scan.hip -- reverse scan of the state adjoint for bf16 io at
// d_k = d_v = 128 (the other shapes use the generic scan in gdn_bwd.hip).
//
// Per chunk (reverse order), with the end-state adjoint dS' of the chunk
// (algebra at the top of gdn_bwd.hip):
//   dU   = diag(D) K dS' + s Mwo^T do + Mwq^T dr_q + Mwk^T dr_k     (Mw: b folded in)
//   dS_c = G_C dS' + Q^T (s G do) + q~^T (G_p dr_q) + k~^T (G_p dr_k) - K^T (G T^T dU)
// with dr_q = s G~_e do~, dr_k = -G~ T~^T (s Mw~^T do~).  Every term is
// separable over the columns of d_v.
//
// Layout: four workgroups of 2 waves per (document, head), on one XCD; wave w
// of quarter q owns d_v columns [32 q + 16 w, +16).  Its 128 x 16 slab of dS
// lives in MFMA accumulators for the whole document (8 tiles over d_k), and
// every C x 16 quantity of a chunk is a register slab (slab.h).  K dS' takes
// dS straight from the accumulators as its B operand; dS += X^T Y takes X^T
// from a transposed copy of the chunk's q/k rows kept in LDS.  T and T~ come
// precomputed, with the weighted Gram matrices, by the chunk-matrix kernel
// (gdn_tri.hip), so neither a solve nor a Gram sits on the sequential chain;
// the next chunk's rows, those six matrices, gates and do/do~ columns are
// fetched into registers while the current chunk computes.
#include "bwd_common.h"
#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int sC = 32, sD = 128, sNW = 2, sNT = 64 * sNW, sQ = 4;  // quarters per (doc, head)
constexpr int sLDX = sD + 8, sLDT = sC + 4, sLDM = sC + 4;
enum { SC_T = 0, SC_TN, SC_MO, SC_MQ, SC_MK, SC_MN };  // the chunk-matrix pass's order

struct ScanSmem2 {
  alignas(16) u16 xr[4][sC][sLDX];  // q, k, q~, k~ rows
  alignas(16) u16 xt[4][sD][sLDT];  // the same, transposed ([d_k][chunk row])
  alignas(16) float cc[6][sC][sLDM];  // T, T~, Mwo, Mwq, Mwk, Mw~ (b folded)
  alignas(16) u16 dob[2][sC][32 + 8];  // do, do~ columns of this quarter
  alignas(16) float dst[sNW][sD][16 + 4];  // per-wave staging of the dS slab for 16-byte stores
  alignas(16) float lg[sC], beta[sC], lgn[sC], betan[sC];
};

// The next chunk's inputs, held in registers while the current one computes.
// Raw bits only: masking and conversion happen when they are consumed, so no
// instruction touches a loaded register before the next chunk (and nothing
// waits for the loads early).
struct ScanPrefetch {
  uint4 x[4][4];  // [array][row rr]: rows 4 (t % 8) + rr, 16-byte unit t / 8
  float4 tri[12];
  float gate;
  uint4 dob[2];  // do / do~ rows: unit (j * 128 + t) -> array, row, 16-byte unit of the quarter
};

}  // namespace

__global__ __launch_bounds__(sNT) void gdn_bwd_scan_d128_kernel(BwdArgs a) {
  constexpr int C = sC, D = sD, NT = sNT, LDX = sLDX, LDT = sLDT, LDM = sLDM;
  __shared__ ScanSmem2 sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  // ---- workgroup -> (document, head, quarter); the quarters of a pair share an XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * sQ), rem = L % (8 * sQ);
  const int quarter = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= f.num_docs * f.H) return;
  const int doc = pair / f.H, h = pair % f.H;
  const int H = f.H;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int P = f.plen[doc];
  const int B = f.B;
  const int nchunks = (n + C - 1) / C;
  const int dv0 = 32 * quarter + 16 * wave;
  const float s = f.scale;
  const int64_t ck_base = (int64_t)(t0g / C) + doc;
  float *ws = reinterpret_cast<float *>(a.workspace);
  const u16 *const px[4] = {reinterpret_cast<const u16 *>(f.q), reinterpret_cast<const u16 *>(f.k),
                            reinterpret_cast<const u16 *>(f.qn), reinterpret_cast<const u16 *>(f.kn)};
  const u16 *const pdo = reinterpret_cast<const u16 *>(a.d_o), *const pdon = reinterpret_cast<const u16 *>(a.d_on);

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
  // the dS slab -> global through this wave's own LDS staging rows, so it
  // leaves as 8 16-byte stores per lane instead of 32 scalar ones (few enough
  // vector-memory operations in flight for the prefetch to be tracked exactly)
  auto store_dS = [&](float *dst) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.dst[wave][16 * kt + g4 + r][cl] = dS[kt][r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = j * 64 + lane, row = u >> 2, c4 = u & 3;
      *reinterpret_cast<float4 *>(dst + (size_t)row * D + dv0 + 4 * c4) =
          *reinterpret_cast<const float4 *>(&sm.dst[wave][row][4 * c4]);
    }
  };

  // ---- prefetch of chunk c into registers
  // 4 rows x one 16-byte unit per array; neighbouring lanes take neighbouring
  // rows, so the transposed 8-byte LDS writes spread over the banks
  const int prow = 4 * (tid & 7), pu = tid >> 3;
  // Loads are unconditional, from a row clamped into the document (always in
  // bounds), and masked afterwards: a load under a branch would make the
  // compiler wait for it, and for every load issued before it.
  // do / do~ slab of this wave from the quarter's LDS rows
  auto slab_lds = [&](int m) {
    Slab sl;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) sl.t[tr][r] = bf2f(sm.dob[m][slab_row(tr, r)][16 * wave + cl]);
    return sl;
  };
  auto prefetch = [&](ScanPrefetch &pf, int c) {
    const int c0 = c * C;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        pf.x[m][rr] = *reinterpret_cast<const uint4 *>(px[m] + ((t0g + min(c0 + prow + rr, n - 1)) * H + h) * D + 8 * pu);
    const float *tri = a.tri + ((size_t)(ck_base + c) * H + h) * 6 * C * C;
#pragma unroll
    for (int j = 0; j < 12; ++j) pf.tri[j] = *reinterpret_cast<const float4 *>(tri + 4 * (j * NT + tid));
    pf.gate = gate_load_raw(f, t0g, c0, n, h, tid);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = (tid >> 2), un = tid & 3;
      pf.dob[j] = *reinterpret_cast<const uint4 *>((j == 0 ? pdo : pdon) +
                                                   ((t0g + min(c0 + row, n - 1)) * H + h) * D + 32 * quarter + 8 * un);
    }
  };
  auto fill_lds = [&](const ScanPrefetch &pf, int c0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint4 xv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tpos = c0 + prow + rr;
        const bool ok = tpos < n && (m < 2 || tpos >= P);
        xv[rr] = ok ? pf.x[m][rr] : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4 *>(&sm.xr[m][prow + rr][8 * pu]) = xv[rr];
      }
      // transposed: element e of the unit is column 8 pu + e; four rows -> one 8-byte write
      const uint32_t w[4][4] = {{xv[0].x, xv[0].y, xv[0].z, xv[0].w},
                                {xv[1].x, xv[1].y, xv[1].z, xv[1].w},
                                {xv[2].x, xv[2].y, xv[2].z, xv[2].w},
                                {xv[3].x, xv[3].y, xv[3].z, xv[3].w}};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xffffu, v1 = (w[1][e >> 1] >> sh) & 0xffffu;
        const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xffffu, v3 = (w[3][e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2 *>(&sm.xt[m][8 * pu + e][prow]) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
      }
    }
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int u = j * NT + tid, which = u / (C * C / 4), rr = u % (C * C / 4);
      *reinterpret_cast<float4 *>(&sm.cc[which][rr / (C / 4)][4 * (rr % (C / 4))]) = pf.tri[j];
    }
    gate_scan(gate_fix(pf.gate, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = tid >> 2, un = tid & 3, tpos = c0 + row;
      const bool ok = tpos < n && (j == 0 || tpos >= P);
      *reinterpret_cast<uint4 *>(&sm.dob[j][row][8 * un]) = ok ? pf.dob[j] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  ScanPrefetch pf;
  if (nchunks > 0) prefetch(pf, nchunks - 1);

  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * C;
    const bool has_noisy = (c0 + C > P) && (P < n);
    lds_barrier();  // every wave is done with the previous chunk's LDS
    fill_lds(pf, c0);
    // the adjoint of this chunk's end state, for the per-chunk pass (issued
    // before the next prefetch, so waiting for that prefetch never waits on it)
    store_dS(ws + ((ck_base + c) * H + h) * (size_t)D * D);
    if (c > 0) prefetch(pf, c - 1);
    lds_barrier();
    const Slab DO = slab_lds(0), DON = slab_lds(1);

    const float lgC = sm.lg[C - 1];
    // ---- the column-separable chain of this slab
    Slab Y1, Y2 = slab_zero(), Y3 = slab_zero(), DRQ = slab_zero(), DRK = slab_zero();
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) Y1.t[tr][r] = s * __expf(sm.lg[slab_row(tr, r)]) * DO.t[tr][r];
    if (has_noisy) {
      Slab dun = slab_zero();
      cc_mul<2, true>(dun, &sm.cc[SC_MN][0][0], LDM, DON);  // Mw~^T do~
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = slab_row(tr, r), pi = i - (i % B);
          dun.t[tr][r] *= s;
          DRQ.t[tr][r] = s * __expf(sm.lgn[pi + B - 1]) * DON.t[tr][r];
          Y2.t[tr][r] = (pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f) * DRQ.t[tr][r];
        }
      Slab drn = slab_zero();
      cc_mul<3, true>(drn, &sm.cc[SC_TN][0][0], LDM, dun);  // T~^T du~
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = slab_row(tr, r), pi = i - (i % B);
          DRK.t[tr][r] = -__expf(sm.lgn[i]) * drn.t[tr][r];
          Y3.t[tr][r] = (pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f) * DRK.t[tr][r];
        }
    }
    // K dS' (dS' from the accumulators: k-slots of step ks are d_k rows
    // 32 ks + 4g + e (e < 4) and 32 ks + 16 + 4g + e - 4, split hi + lo)
    Slab dU = slab_zero();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float xv[8] = {dS[2 * ks][0], dS[2 * ks][1], dS[2 * ks][2], dS[2 * ks][3],
                           dS[2 * ks + 1][0], dS[2 * ks + 1][1], dS[2 * ks + 1][2], dS[2 * ks + 1][3]};
      bf16x8 bh, bl;
      split8(xv, bh, bl);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const u16 *row = &sm.xr[1][16 * tr + cl][32 * ks];
        const uint2 lo4 = *reinterpret_cast<const uint2 *>(row + g4);
        const uint2 hi4 = *reinterpret_cast<const uint2 *>(row + 16 + g4);
        const bf16x8 ak = __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
        mma_bf16(dU.t[tr], ak, bh);
        mma_bf16(dU.t[tr], ak, bl);
      }
    }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        dU.t[tr][r] *= sm.beta[i] * __expf(lgC - sm.lg[i]);  // diag(D) K dS'
      }
    {
      Slab t2 = slab_zero();
      cc_mul<2, true>(t2, &sm.cc[SC_MO][0][0], LDM, DO);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) dU.t[tr] += s * t2.t[tr];
    }
    if (has_noisy) {
      cc_mul<3, true>(dU, &sm.cc[SC_MQ][0][0], LDM, DRQ);
      cc_mul<3, true>(dU, &sm.cc[SC_MK][0][0], LDM, DRK);
    }
    Slab Y4 = slab_zero();
    cc_mul<3, true>(Y4, &sm.cc[SC_T][0][0], LDM, dU);  // drhs = T^T dU
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) Y4.t[tr][r] *= -__expf(sm.lg[slab_row(tr, r)]);

    // ---- dS_c = G_C dS' + Q^T Y1 + K^T Y4 (+ q~^T Y2 + k~^T Y3)
    const float gC = __expf(lgC);
    bf16x8 yh[4], yl[4];
    slab_b_split(Y1, yh[0], yl[0]);
    slab_b_split(Y4, yh[1], yl[1]);
    if (has_noisy) {
      slab_b_split(Y2, yh[2], yl[2]);
      slab_b_split(Y3, yh[3], yl[3]);
    }
    // A = X^T from the transposed rows (k-slots in the slab permutation); the
    // noisy terms in a loop of their own, so each loop is one basic block
    auto xt_frag = [&](int xm, int kt) {
      const u16 *col = &sm.xt[xm][16 * kt + cl][0];
      const uint2 lo4 = *reinterpret_cast<const uint2 *>(col + g4);
      const uint2 hi4 = *reinterpret_cast<const uint2 *>(col + 16 + g4);
      return __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
    };
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      dS[kt] *= gC;
      const bf16x8 aq = xt_frag(0, kt), ak = xt_frag(1, kt);  // Y1 <- q, Y4 <- k
      mma_bf16(dS[kt], aq, yh[0]);
      mma_bf16(dS[kt], aq, yl[0]);
      mma_bf16(dS[kt], ak, yh[1]);
      mma_bf16(dS[kt], ak, yl[1]);
    }
    if (has_noisy) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const bf16x8 aqn = xt_frag(2, kt), akn = xt_frag(3, kt);  // Y2 <- q~, Y3 <- k~
        mma_bf16(dS[kt], aqn, yh[2]);
        mma_bf16(dS[kt], aqn, yl[2]);
        mma_bf16(dS[kt], akn, yh[3]);
        mma_bf16(dS[kt], akn, yl[3]);
      }
    }
  }
  if (a.dh0) store_dS(a.dh0 + ((size_t)doc * H + h) * D * D);
}

hipError_t launch_bwd_scan_d128(const BwdArgs &a, hipStream_t st) {
  const int pairs = a.f.num_docs * a.f.H;
  const int groups = (pairs + 7) / 8;
  hipLaunchKernelGGL(gdn_bwd_scan_d128_kernel, dim3((unsigned)(groups * 8 * sQ)), dim3(sNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
