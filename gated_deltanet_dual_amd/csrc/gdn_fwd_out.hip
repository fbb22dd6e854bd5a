// gdn_fwd_out.hip -- the dual-stream forward's outputs for bf16 io at
// d_k = d_v = 128 without flags, fully in parallel over (chunk, head), from
// the chunk-start states the forward scan stored (gdn_scan.hip).
//
// Method ("FLARE: Diffusion for Hybrid Language Model", papernotes.org notes,
// Key designs item 2; Overall framework): the clean stream follows the gated
// delta rule; a noisy block starts from the clean state at its boundary,
// applies its own updates, and every position of the block reads the
// block-end state.  Per chunk of C = 32 tokens, with start state S_c and the
// chunk matrices T, T~, Mwo, Mwq, Mwk, Mw~ of the chunk-matrix pass
// (gdn_tri.hip):
//   U   = T (V - diag(G) K S_c)
//   o   = s (diag(G) Q S_c + Mwo U)
//   r_q = diag(G_p) q~ S_c + Mwq U,   r_k = diag(G_p) k~ S_c + Mwk U
//   u~  = T~ (v~ - diag(G~) r_k),     o~ = s (diag(G~_e) r_q + Mw~ u~)
// r_q and r_k are the reads of the noisy blocks' boundary states, which are
// never formed.  Prompt rows of o~ are written 0.
//
// One workgroup of 8 waves per (chunk slot, head); wave w owns d_v columns
// [16 w, 16 w + 16): every C x 16 quantity is a register slab (slab.h) and
// S_c's columns are the B operand of X S_c, split hi + lo.  The outputs leave
// through LDS staging (over the q/k rows) as 16-byte row stores.
#include "bwd_common.h"
#include "device_common.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int oC = 32, oD = 128, oNW = 8, oNT = 64 * oNW;
constexpr int oLDX = oD + 8, oLDM = oC + 4;
enum { OC_T = 0, OC_TN, OC_MO, OC_MQ, OC_MK, OC_MN };  // the chunk-matrix pass's order

struct OutSmem {
  alignas(16) u16 x[4][oC][oLDX];     // q, k, q~, k~ rows; then the o, o~ staging
  alignas(16) float cc[6][oC][oLDM];  // T, T~, Mwo, Mwq, Mwk, Mw~
  alignas(16) float lg[oC], beta[oC], lgn[oC], betan[oC];
};

}  // namespace

__global__ __launch_bounds__(oNT) void gdn_fwd_out_d128_kernel(FwdArgs f, const float *cmat, const float *states) {
  constexpr int C = oC, D = oD, NT = oNT, LDM = oLDM;
  __shared__ OutSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  const int H = f.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  int doc, c;
  if (!slot_to_chunk(f, slot, doc, c)) return;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int P = f.plen[doc];
  const int B = f.B;
  const int c0 = c * C;
  const bool has_noisy = (c0 + C > P) && (P < n);
  const float s = f.scale;
  const int col0 = 16 * wave;
  const u16 *const px[4] = {reinterpret_cast<const u16 *>(f.q), reinterpret_cast<const u16 *>(f.k),
                            reinterpret_cast<const u16 *>(f.qn), reinterpret_cast<const u16 *>(f.kn)};
  const u16 *const pv = reinterpret_cast<const u16 *>(f.v), *const pvn = reinterpret_cast<const u16 *>(f.vn);
  const float *const Sc = states + ((size_t)slot * H + h) * D * D;

  // ---- every global load first (unconditional, rows clamped into the document)
  constexpr int RU = D / 8, PU = C * RU, UX = 4 * PU / NT;
  uint4 xr[UX];
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    xr[e] = *reinterpret_cast<const uint4 *>(px[m] + ((t0g + min(c0 + row, n - 1)) * H + h) * D + cu16 * 8);
  }
  const float *cm = cmat + ((size_t)slot * H + h) * 6 * C * C;
  float4 cv[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) cv[j] = reinterpret_cast<const float4 *>(cm)[j * NT + tid];
  const float graw = tid < 4 * C ? gate_load_raw(f, t0g, c0, n, h, tid) : 0.f;
  u16 rv[2][4], rvn[2][4];
  gslab_raw<D>(rv, pv, H, h, t0g, c0, n, col0);
  gslab_raw<D>(rvn, pvn, H, h, t0g, c0, n, col0);
  // S_c column slab as B fragments: k-slots of step ks are d_k rows
  // 32 ks + 4 g + e (e < 4) and 32 ks + 16 + 4 g + e - 4
  float xs[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 32 * ks + (e < 4 ? g4 + e : 16 + g4 + e - 4);
      xs[ks][e] = Sc[(size_t)row * D + col0 + cl];
    }

  // ---- LDS: rows (masked), chunk matrices, gates
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    const int tpos = c0 + row;
    const bool ok = tpos < n && (m < 2 || tpos >= P);
    *reinterpret_cast<uint4 *>(&sm.x[m][row][cu16 * 8]) = ok ? xr[e] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int u = j * NT + tid, which = u / (C * C / 4), rr = u % (C * C / 4);
    *reinterpret_cast<float4 *>(&sm.cc[which][rr / (C / 4)][4 * (rr % (C / 4))]) = cv[j];
  }
  if (tid < 4 * C) gate_scan(gate_fix(graw, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  lds_barrier();

  // A fragment of rows 16 tr .. of a row tile over d_k step ks, columns in the
  // slab k-permutation (32 ks + 4 g .. +3 and 32 ks + 16 + 4 g .. +3)
  auto xrow_frag = [&](int m, int tr, int ks) {
    const u16 *row = &sm.x[m][16 * tr + cl][32 * ks];
    const uint2 lo4 = *reinterpret_cast<const uint2 *>(row + g4);
    const uint2 hi4 = *reinterpret_cast<const uint2 *>(row + 16 + g4);
    return __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
  };
  auto Gm = [&](int i) { return __expf(sm.lg[i]); };
  auto Gp = [&](int i) { const int pi = i - (i % B); return pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f; };

  bf16x8 sh[4], sl[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) split8(xs[ks], sh[ks], sl[ks]);
  Slab KS = slab_zero(), QS = slab_zero();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const bf16x8 ak = xrow_frag(1, tr, ks), aq = xrow_frag(0, tr, ks);
      mma_bf16(KS.t[tr], ak, sh[ks]);
      mma_bf16(KS.t[tr], ak, sl[ks]);
      mma_bf16(QS.t[tr], aq, sh[ks]);
      mma_bf16(QS.t[tr], aq, sl[ks]);
    }
  // U = T (v - G K S_c)
  const Slab V = slab_mask(rv, c0, n, P, false);
  Slab rhs;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) rhs.t[tr][r] = V.t[tr][r] - Gm(slab_row(tr, r)) * KS.t[tr][r];
  Slab U = slab_zero();
  cc_mul<3, false>(U, &sm.cc[OC_T][0][0], LDM, rhs);
  // o = s (G Q S_c + Mwo U)
  Slab O = slab_zero();
  cc_mul<3, false>(O, &sm.cc[OC_MO][0][0], LDM, U);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = slab_row(tr, r);
      O.t[tr][r] = s * (Gm(i) * QS.t[tr][r] + O.t[tr][r]);
    }
  // the noisy blocks: reads of their boundary states, then the block
  Slab ON = slab_zero();
  if (has_noisy) {
    Slab RQ = slab_zero(), RK = slab_zero();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const bf16x8 aqn = xrow_frag(2, tr, ks), akn = xrow_frag(3, tr, ks);
        mma_bf16(RQ.t[tr], aqn, sh[ks]);
        mma_bf16(RQ.t[tr], aqn, sl[ks]);
        mma_bf16(RK.t[tr], akn, sh[ks]);
        mma_bf16(RK.t[tr], akn, sl[ks]);
      }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gp = Gp(slab_row(tr, r));
        RQ.t[tr][r] *= gp;
        RK.t[tr][r] *= gp;
      }
    cc_mul<3, false>(RQ, &sm.cc[OC_MQ][0][0], LDM, U);
    cc_mul<3, false>(RK, &sm.cc[OC_MK][0][0], LDM, U);
    const Slab VN = slab_mask(rvn, c0, n, P, true);
    Slab rhsn;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rhsn.t[tr][r] = VN.t[tr][r] - __expf(sm.lgn[slab_row(tr, r)]) * RK.t[tr][r];
    Slab UN = slab_zero();
    cc_mul<3, false>(UN, &sm.cc[OC_TN][0][0], LDM, rhsn);
    cc_mul<3, false>(ON, &sm.cc[OC_MN][0][0], LDM, UN);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r), pi = i - (i % B);
        const bool resp = c0 + i < n && c0 + i >= P;
        ON.t[tr][r] = resp ? s * (__expf(sm.lgn[pi + B - 1]) * RQ.t[tr][r] + ON.t[tr][r]) : 0.f;
      }
  }

  // ---- o, o~ -> LDS staging over the q / k rows -> 16-byte row stores
  lds_barrier();  // every wave is done with the rows
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = slab_row(tr, r);
      sm.x[0][i][col0 + cl] = f2bf(O.t[tr][r]);
      sm.x[1][i][col0 + cl] = f2bf(ON.t[tr][r]);
    }
  lds_barrier();
  u16 *const po = reinterpret_cast<u16 *>(f.o), *const pon = reinterpret_cast<u16 *>(f.on);
#pragma unroll
  for (int e = 0; e < 2 * PU / NT; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    if (c0 + row < n) {
      u16 *dst = (m == 0 ? po : pon) + ((t0g + c0 + row) * H + h) * D + cu16 * 8;
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(&sm.x[m][row][cu16 * 8]);
    }
  }
}

hipError_t launch_fwd_out_d128(const FwdArgs &a, const float *cmat, const float *states, hipStream_t st,
                               int64_t slots) {
  hipLaunchKernelGGL(gdn_fwd_out_d128_kernel, dim3((unsigned)(slots * a.H)), dim3(oNT), 0, st, a, cmat, states);
  return hipGetLastError();
}

}  // namespace flare
