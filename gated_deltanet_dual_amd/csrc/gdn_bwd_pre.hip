// gdn_bwd_pre.hip -- the part of the reverse scan's chunk step that does not
// depend on the state adjoint (bf16 io, d_k = d_v = 128), fully in parallel
// over (chunk, head), ahead of the scan.
//
// With the chunk's end-state adjoint dS' (algebra at the top of gdn_bwd.hip)
//   dU   = diag(D) K dS' + dU0,   dU0 = s Mwo^T do + Mwq^T dr_q + Mwk^T dr_k
//   dS_c = G_C dS' + Q^T (s G do) + q~^T (G_p dr_q) + k~^T (G_p dr_k) - K^T (G T^T dU)
// with dr_q = s G~_e do~ and dr_k = -G~ T~^T (s Mw~^T do~).  Only the first
// term of dU carries dS', so
//   dS_c = G_C dS' + R + K^T (W (K dS')),   W = -diag(G) T^T diag(D),
//   R    = Q^T (s G do) + q~^T (G_p dr_q) + k~^T (G_p dr_k) - K^T (G T^T dU0).
// This kernel forms R, W, G_C and the two fragment sets of K the scan uses,
// in the register order the scan consumes them (bwd_common.h), so the scan's
// sequential chain is three short products per chunk.
//
// One workgroup of 8 waves per (chunk slot, head); wave w owns d_v columns
// [16 w, 16 w + 16) of R (a register slab, slab.h) and one of the fragment
// sets.  LDS holds only what the waves share: q, k, q~, k~ transposed
// ([d_k][chunk row]) and the six chunk matrices -- 64 KB, two workgroups per CU.
// L2: the q/k L2 flag folded into per-row factors (gdn_l2.hip): the write
// strengths arrive folded from the gate load and the output gradients are
// r_q do, r_q~ do~.
#include "bwd_common.h"
#include "chunk_common.h"
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "slab.h"

static_assert(flare::kPackWords == flare::kScanPackFloats, "scan hand-over size");

namespace flare {

namespace {

constexpr int pC = 32, pD = 128, pNW = 8, pNT = 64 * pNW;
constexpr int pLDT = pC + 4, pLDM = pC + 4;
enum { PT_T = 0, PT_TN, PT_MO, PT_MQ, PT_MK, PT_MN };  // the chunk-matrix pass's order

struct PreSmem {
  alignas(16) u16 xt[4][pD][pLDT];    // q, k, q~, k~ transposed
  alignas(16) float cc[6][pC][pLDM];  // T, T~, Mwo, Mwq, Mwk, Mw~ (b folded)
  alignas(16) float lg[pC], beta[pC], lgn[pC], betan[pC];
  alignas(16) float rq[2][pC];  // L2: r_q, r_q~ of the chunk's rows
};

}  // namespace

template <bool L2>
__global__ __launch_bounds__(pNT) void gdn_bwd_pre_d128_kernel(BwdArgs a) {
  constexpr int C = pC, D = pD, NT = pNT, LDM = pLDM;
  __shared__ PreSmem sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  const int H = f.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  int doc, c;
  if (!slot_to_chunk(f, slot, doc, c)) return;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int P = f.plen[doc];
  const int B = f.B;  // a power of two up to 32 (checked by the host): i % B = i & (B - 1)
  const int c0 = c * C;
  const bool has_noisy = (c0 + C > P) && (P < n);
  const float s = f.scale;
  const int col0 = 16 * wave;
  const u16 *const px[4] = {reinterpret_cast<const u16 *>(f.q), reinterpret_cast<const u16 *>(f.k),
                            reinterpret_cast<const u16 *>(f.qn), reinterpret_cast<const u16 *>(f.kn)};
  const u16 *const pdo = reinterpret_cast<const u16 *>(a.d_o), *const pdon = reinterpret_cast<const u16 *>(a.d_on);
  float *const pack = a.pack + ((size_t)slot * H + h) * kPackWords;

  // ---- every global load first (unconditional, rows clamped into the document)
  // rows: array m = tid / 128; four consecutive rows 4 (t % 8) .. +3 of the
  // 16-byte unit t / 8 (t = tid % 128), so the transposed writes are 8 bytes
  const int m = tid >> 7, tq = tid & 127, prow = 4 * (tq & 7), pu = tq >> 3;
  uint4 xv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    // a noisy prompt row (masked below) is read from the clean twin, which
    // another wave of the workgroup loads (selects, not an indexed array: no scratch)
    const int ms = m >= 2 && c0 + prow + rr < P ? m - 2 : m;
    const u16 *src = ms == 0 ? px[0] : ms == 1 ? px[1] : ms == 2 ? px[2] : px[3];
    xv[rr] = *reinterpret_cast<const uint4 *>(src + ((t0g + min(c0 + prow + rr, n - 1)) * H + h) * D + 8 * pu);
  }
  const float *tri = a.tri + ((size_t)slot * H + h) * 6 * C * C;
  float4 tv[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) tv[j] = cm_load_f4<false>(tri, j * NT + tid, B, has_noisy);  // live half-rows only
  const float graw = tid < 4 * C ? gate_load_raw(f, t0g, c0, n, h, tid) : 0.f;
  float l2r = 1.f;  // L2, thread tid < 64: r_q (tid < 32) or r_q~ of row tid % 32
  if (L2 && tid < 2 * C) l2r = reinterpret_cast<const float *>(f.l2f + (t0g + min(c0 + (tid & (C - 1)), n - 1)) * H +
                                                               h)[2 * (tid / C)];
  u16 rdo[2][4], rdon[2][4];
  gslab_raw<D>(rdo, pdo, H, h, t0g, c0, n, col0);
  gslab_raw_noisy<D>(rdon, pdon, pdo, H, h, t0g, c0, n, P, col0);
  // this wave's K fragment (ks, tr) = (wave / 2, wave % 2): row 16 tr + (l & 15),
  // d_k 32 ks + 4 g .. +3 and 32 ks + 16 + 4 g .. +3
  uint2 ka0, ka1;
  const int ka_row = 16 * (wave & 1) + cl, ka_col = 32 * (wave >> 1) + g4;
  {
    const u16 *src = px[1] + ((t0g + min(c0 + ka_row, n - 1)) * H + h) * D;
    ka0 = *reinterpret_cast<const uint2 *>(src + ka_col);
    ka1 = *reinterpret_cast<const uint2 *>(src + ka_col + 16);
  }

  // ---- LDS: transposed rows (masked), chunk matrices, gates
  {
    uint4 w4[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int tpos = c0 + prow + rr;
      const bool ok = tpos < n && (m < 2 || tpos >= P);
      w4[rr] = ok ? xv[rr] : make_uint4(0u, 0u, 0u, 0u);
    }
    const uint32_t w[4][4] = {{w4[0].x, w4[0].y, w4[0].z, w4[0].w},
                              {w4[1].x, w4[1].y, w4[1].z, w4[1].w},
                              {w4[2].x, w4[2].y, w4[2].z, w4[2].w},
                              {w4[3].x, w4[3].y, w4[3].z, w4[3].w}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xffffu, v1 = (w[1][e >> 1] >> sh) & 0xffffu;
      const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xffffu, v3 = (w[3][e >> 1] >> sh) & 0xffffu;
      *reinterpret_cast<uint2 *>(&sm.xt[m][8 * pu + e][prow]) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int u = j * NT + tid, which = u / (C * C / 4);
    *reinterpret_cast<float4 *>(&sm.cc[which][cm_row(u)][cm_col(u)]) = tv[j];
  }
  if (tid < 4 * C) gate_scan(gate_fix(graw, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  if (L2 && tid < 2 * C) sm.rq[tid / C][tid & (C - 1)] = l2r;
  lds_barrier();

  const float lgC = sm.lg[C - 1];
  // the fragment sets (one per wave, stored as they are consumed), unless
  // the scan reads the forward's (the same values: k rows, zero past the
  // document end)
  if (!a.kpack) {
    // K: rows past the document end are zero
    const bool ok = c0 + ka_row < n;
    const uint4 v = ok ? make_uint4(ka0.x, ka0.y, ka1.x, ka1.y) : make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4 *>(pack + kPackKA)[wave * 64 + lane] = v;
  }
  if (!a.kpack) {
    // K^T tile kt = wave: d_k row 16 kt + (l & 15), tokens 4 g .. +3, 16 + 4 g .. +3
    const u16 *col = &sm.xt[1][16 * wave + cl][0];
    const uint2 lo4 = *reinterpret_cast<const uint2 *>(col + g4);
    const uint2 hi4 = *reinterpret_cast<const uint2 *>(col + 16 + g4);
    reinterpret_cast<uint4 *>(pack + kPackKT)[wave * 64 + lane] = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
  }
  if (wave < 2) {
    // W rows i = 16 tr + (l & 15), columns j in the slab permutation; zero on
    // rows and columns past the document end
    const int tr = wave, i = 16 * tr + cl;
    const bool iok = c0 + i < n;
    const float gi = -__expf(sm.lg[i]);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = e < 4 ? g4 + e : 16 + g4 + e - 4;
      const bool ok = iok && c0 + j < n;
      x[e] = ok ? gi * sm.cc[PT_T][j][i] * sm.beta[j] * __expf(lgC - sm.lg[j]) : 0.f;
    }
    bf16x8 wh, wl;
    split8(x, wh, wl);
    uint4 *dst = reinterpret_cast<uint4 *>(pack + kPackW);
    dst[(2 * tr) * 64 + lane] = __builtin_bit_cast(uint4, wh);
    dst[(2 * tr + 1) * 64 + lane] = __builtin_bit_cast(uint4, wl);
  }
  if (tid == 0) pack[kPackG] = __expf(lgC);

  // ---- the state-independent chain of this wave's slab
  auto Gm = [&](int i) { return __expf(sm.lg[i]); };
  auto Gp = [&](int i) { const int pi = (i & -B); return pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f; };
  Slab DO = slab_mask(rdo, c0, n, P, false), DON = slab_mask(rdon, c0, n, P, true);
  if constexpr (L2) {
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        DO.t[tr][r] *= sm.rq[0][i];
        DON.t[tr][r] *= sm.rq[1][i];
      }
  }
  // with L2 the scaled gradients are no longer exact in bf16: both operands split
  constexpr int DT = L2 ? 3 : 2;
  Slab Y1, Y2 = slab_zero(), Y3 = slab_zero(), DRQ = slab_zero(), DRK = slab_zero();
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) Y1.t[tr][r] = s * Gm(slab_row(tr, r)) * DO.t[tr][r];
  if (has_noisy) {
    Slab dun = slab_zero();
    cc_mul<DT, true>(dun, &sm.cc[PT_MN][0][0], LDM, DON);  // Mw~^T do~
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r), pi = (i & -B);
        dun.t[tr][r] *= s;
        DRQ.t[tr][r] = s * __expf(sm.lgn[pi + B - 1]) * DON.t[tr][r];
        Y2.t[tr][r] = Gp(i) * DRQ.t[tr][r];
      }
    Slab drn = slab_zero();
    cc_mul<3, true>(drn, &sm.cc[PT_TN][0][0], LDM, dun);  // T~^T du~
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        DRK.t[tr][r] = -__expf(sm.lgn[i]) * drn.t[tr][r];
        Y3.t[tr][r] = Gp(i) * DRK.t[tr][r];
      }
  }
  Slab dU0 = slab_zero();
  cc_mul<DT, true>(dU0, &sm.cc[PT_MO][0][0], LDM, DO);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) dU0.t[tr] *= s;
  if (has_noisy) {
    cc_mul<3, true>(dU0, &sm.cc[PT_MQ][0][0], LDM, DRQ);
    cc_mul<3, true>(dU0, &sm.cc[PT_MK][0][0], LDM, DRK);
  }
  Slab Y4 = slab_zero();
  cc_mul<3, true>(Y4, &sm.cc[PT_T][0][0], LDM, dU0);  // T^T dU0
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) Y4.t[tr][r] *= -Gm(slab_row(tr, r));

  // ---- R = Q^T Y1 + K^T Y4 (+ q~^T Y2 + k~^T Y3), d_k tile kt per accumulator
  bf16x8 yh[4], yl[4];
  slab_b_split(Y1, yh[0], yl[0]);
  slab_b_split(Y4, yh[1], yl[1]);
  slab_b_split(Y2, yh[2], yl[2]);
  slab_b_split(Y3, yh[3], yl[3]);
  auto xt_frag = [&](int xm, int kt) {
    const u16 *col = &sm.xt[xm][16 * kt + cl][0];
    const uint2 lo4 = *reinterpret_cast<const uint2 *>(col + g4);
    const uint2 hi4 = *reinterpret_cast<const uint2 *>(col + 16 + g4);
    return __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
  };
  float4 *rdst = reinterpret_cast<float4 *>(pack + kPackR) + (size_t)wave * 8 * 64;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 aq = xt_frag(0, kt), ak = xt_frag(1, kt);
    mma_bf16(acc, aq, yh[0]);
    mma_bf16(acc, aq, yl[0]);
    mma_bf16(acc, ak, yh[1]);
    mma_bf16(acc, ak, yl[1]);
    if (has_noisy) {
      const bf16x8 aqn = xt_frag(2, kt), akn = xt_frag(3, kt);
      mma_bf16(acc, aqn, yh[2]);
      mma_bf16(acc, aqn, yl[2]);
      mma_bf16(acc, akn, yh[3]);
      mma_bf16(acc, akn, yl[3]);
    }
    st_nt_f4(&rdst[kt * 64 + lane], make_float4(acc[0], acc[1], acc[2], acc[3]));
  }
}

hipError_t launch_bwd_pre_d128(const BwdArgs &a, hipStream_t st, int64_t slots) {
  if (a.f.l2f)
    hipLaunchKernelGGL(gdn_bwd_pre_d128_kernel<true>, dim3((unsigned)(slots * a.f.H)), dim3(pNT), 0, st, a);
  else
    hipLaunchKernelGGL(gdn_bwd_pre_d128_kernel<false>, dim3((unsigned)(slots * a.f.H)), dim3(pNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
