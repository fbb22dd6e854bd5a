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
// L2: the q/k L2 flag folded into per-row factors (gdn_l2.hip): the write
// strengths arrive folded from the gate load, v and v~ rows are divided by
// r_k and r_k~, and the rows of o and o~ multiplied by r_q and r_q~.
// CW > 0: the ShortConv in the loads (conv_load.h): the q, k, q~, k~ rows and
// the v, v~ rows are formed from the raw projections, two rows of one section
// and stream per thread; v and v~ are staged in LDS for the slabs.
#include <type_traits>

#include "bwd_common.h"
#include "chunk_common.h"
#include "conv_load.h"
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
  alignas(16) float fac[4][oC];  // L2: r_q, 1 / r_k, r_q~, 1 / r_k~ of the chunk's rows
};
struct OutSmemConv : OutSmem {
  alignas(16) u16 v[2][oC][oLDX];  // the v, v~ rows formed by the conv loads
};

}  // namespace

template <bool L2, int CW>
__global__ __launch_bounds__(oNT) void gdn_fwd_out_d128_kernel(FwdArgs f, const float *cmat, const float *states) {
  constexpr int C = oC, D = oD, NT = oNT, LDM = oLDM;
  using Smem = typename std::conditional<(CW > 0), OutSmemConv, OutSmem>::type;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  const int H = f.H;
  // the slot: in document order, or (equal documents) chunk-major from the
  // last chunks down, so the chunk-start states the scan wrote last are read
  // while they are still in the last-level cache
  const int q = blockIdx.x / H, h = blockIdx.x % H;
  const int slot = f.slot_order > 0 ? (q % f.num_docs) * f.slot_order + (f.slot_order - 1 - q / f.num_docs) : q;
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
  const u16 *const pv = reinterpret_cast<const u16 *>(f.v), *const pvn = reinterpret_cast<const u16 *>(f.vn);
  const float *const Sc = states + ((size_t)slot * H + h) * D * D;

  // ---- every global load first (unconditional, rows clamped into the document)
  constexpr int RU = D / 8, PU = C * RU, UX = CW > 0 ? 1 : 4 * PU / NT;
  constexpr int CWW = CW > 0 ? CW : 1;
  uint4 xr[UX];
  ConvRows<CWW, 2> cqk, cvr;  // CW: rows 2 (tid / 16 % 16) .. +1 of q / k (by tid / 256), and of v / v~
  const int csel = tid >> 8, crg = (tid >> 4) & 15, cu16 = tid & 15;
  if constexpr (CW > 0) {
    cqk.load(f, csel, t0g, c0, 2 * crg, n, h, cu16, has_noisy);
  } else {
#pragma unroll
    for (int e = 0; e < UX; ++e) {
      const int u = e * NT + tid;
      const int m = u / PU, r = u % PU, row = r / RU, cu = r % RU;
      // a noisy prompt row (masked below) is read from the clean twin this thread loads too
      const int ms = m >= 2 && c0 + row < P ? m - 2 : m;  // (selects, not an indexed array: no scratch)
      const u16 *src = ms == 0 ? px[0] : ms == 1 ? px[1] : ms == 2 ? px[2] : px[3];
      xr[e] = *reinterpret_cast<const uint4 *>(src + ((t0g + min(c0 + row, n - 1)) * H + h) * D + cu * 8);
    }
  }
  const float *cm = cmat + ((size_t)slot * H + h) * 6 * C * C;
  // three named registers, not an array: an array the compiler leaves
  // un-unrolled would live in scratch
  // (only the half-rows that can be non-zero are read; the others are zero)
  const float4 cv0 = cm_load_f4<false>(cm, tid, B, has_noisy);
  const float4 cv1 = cm_load_f4<false>(cm, NT + tid, B, has_noisy);
  const float4 cv2 = cm_load_f4<false>(cm, 2 * NT + tid, B, has_noisy);
  const float graw = tid < 4 * C ? gate_load_raw(f, t0g, c0, n, h, tid) : 0.f;
  float l2r = 1.f;  // thread tid < 128: factor tid / 32 of row tid % 32
  if (L2 && tid < 4 * C) {
    const float *fr = reinterpret_cast<const float *>(f.l2f + (t0g + min(c0 + (tid & (C - 1)), n - 1)) * H + h);
    l2r = fr[tid / C];
  }
  u16 rv[2][4], rvn[2][4];
  if constexpr (CW == 0) {
    gslab_raw<D>(rv, pv, H, h, t0g, c0, n, col0);
    gslab_raw_noisy<D>(rvn, pvn, pv, H, h, t0g, c0, n, P, col0);
  }
  // S_c column slab as B fragments: k-slots of step ks are d_k rows
  // 32 ks + 4 g + e (e < 4) and 32 ks + 16 + 4 g + e - 4
  float xs[4][8];
  auto load_sc = [&]() {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = 32 * ks + (e < 4 ? g4 + e : 16 + g4 + e - 4);
        xs[ks][e] = Sc[(size_t)row * D + col0 + cl];
      }
  };
  if constexpr (CW == 0) load_sc();

  // ---- LDS: rows (masked), chunk matrices, gates
  if constexpr (CW > 0) {
    uint4 y[2], yn[2];
    cqk.rows(c0, 2 * crg, P, B, f.cact != 0, y, yn);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 2 * crg + i, tpos = c0 + row;
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4 *>(&sm.x[csel][row][cu16 * 8]) = sel4(tpos < n, y[i], z);
      *reinterpret_cast<uint4 *>(&sm.x[2 + csel][row][cu16 * 8]) = sel4(tpos < n && tpos >= P, yn[i], z);
    }
    // the S_c columns and the v, v~ rows after the q, k rows (their loads
    // all at once would double the registers live)
    lds_barrier();
    load_sc();
    cvr.load(f, 2, t0g, c0, 2 * crg, n, h, cu16, csel == 1 && has_noisy);
    uint4 vy[2], vyn[2];
    cvr.rows(c0, 2 * crg, P, B, f.cact != 0, vy, vyn);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 2 * crg + i, tpos = c0 + row;
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4 *>(&sm.v[csel][row][cu16 * 8]) =
          sel4(csel == 0, sel4(tpos < n, vy[i], z), sel4(tpos < n && tpos >= P, vyn[i], z));
    }
  } else {
#pragma unroll
    for (int e = 0; e < UX; ++e) {
      const int u = e * NT + tid;
      const int m = u / PU, r = u % PU, row = r / RU, cu = r % RU;
      const int tpos = c0 + row;
      const bool ok = tpos < n && (m < 2 || tpos >= P);
      *reinterpret_cast<uint4 *>(&sm.x[m][row][cu * 8]) = ok ? xr[e] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  auto put_cm = [&](int j, const float4 &v) {
    const int u = j * NT + tid, which = u / (C * C / 4);
    *reinterpret_cast<float4 *>(&sm.cc[which][cm_row(u)][cm_col(u)]) = v;
  };
  put_cm(0, cv0);
  put_cm(1, cv1);
  put_cm(2, cv2);

  if (tid < 4 * C) gate_scan(gate_fix(graw, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  if (L2 && tid < 4 * C) sm.fac[tid / C][tid & (C - 1)] = (tid / C) & 1 ? (l2r > 0.f ? 1.f / l2r : 0.f) : l2r;
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
  auto Gp = [&](int i) { const int pi = (i & -B); return pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f; };

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
  // the v, v~ slabs: staged rows (the conv loads, already masked) or the raw loads
  auto vslab = [&](int m) {
    Slab sl;
    if constexpr (CW > 0) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) sl.t[tr][r] = bf2f(sm.v[m][slab_row(tr, r)][col0 + cl]);
    } else {
      sl = slab_mask(m == 0 ? rv : rvn, c0, n, P, m == 1);
    }
    return sl;
  };
  // U = T (v - G K S_c)
  const Slab V = vslab(0);
  Slab rhs;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = slab_row(tr, r);
      rhs.t[tr][r] = (L2 ? V.t[tr][r] * sm.fac[1][i] : V.t[tr][r]) - Gm(i) * KS.t[tr][r];
    }
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
      if constexpr (L2) O.t[tr][r] *= sm.fac[0][i];
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
    const Slab VN = vslab(1);
    Slab rhsn;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rhsn.t[tr][r] = (L2 ? VN.t[tr][r] * sm.fac[3][slab_row(tr, r)] : VN.t[tr][r]) -
                        __expf(sm.lgn[slab_row(tr, r)]) * RK.t[tr][r];
    Slab UN = slab_zero();
    cc_mul<3, false>(UN, &sm.cc[OC_TN][0][0], LDM, rhsn);
    cc_mul<3, false>(ON, &sm.cc[OC_MN][0][0], LDM, UN);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r), pi = (i & -B);
        const bool resp = c0 + i < n && c0 + i >= P;
        ON.t[tr][r] = resp ? s * (__expf(sm.lgn[pi + B - 1]) * RQ.t[tr][r] + ON.t[tr][r]) : 0.f;
        if constexpr (L2) ON.t[tr][r] = resp ? ON.t[tr][r] * sm.fac[2][i] : 0.f;
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
      st_nt_u4(dst, *reinterpret_cast<const uint4 *>(&sm.x[m][row][cu16 * 8]));
    }
  }
}

template <int CW>
static void launch_out_w(const FwdArgs &a, const float *cmat, const float *states, hipStream_t st, int64_t slots) {
  const dim3 grid((unsigned)(slots * a.H)), block(oNT);
  if (a.l2f) hipLaunchKernelGGL((gdn_fwd_out_d128_kernel<true, CW>), grid, block, 0, st, a, cmat, states);
  else hipLaunchKernelGGL((gdn_fwd_out_d128_kernel<false, CW>), grid, block, 0, st, a, cmat, states);
}

hipError_t launch_fwd_out_d128(const FwdArgs &a, const float *cmat, const float *states, hipStream_t st,
                               int64_t slots) {
  switch (a.cw) {
    case 0: launch_out_w<0>(a, cmat, states, st, slots); break;
    case 1: launch_out_w<1>(a, cmat, states, st, slots); break;
    case 2: launch_out_w<2>(a, cmat, states, st, slots); break;
    case 3: launch_out_w<3>(a, cmat, states, st, slots); break;
    case 4: launch_out_w<4>(a, cmat, states, st, slots); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace flare
