// gdn_fwd_prep.hip -- the forward's state-independent chunk work in one pass
// (bf16 io, d_k = d_v = 128): the chunk matrices of gdn_tri.hip and the scan
// hand-over of gdn_fwd_pre.hip, from one load of the chunk's rows.
//
// Method ("FLARE: Diffusion for Hybrid Language Model", papernotes.org notes,
// Key designs item 2; Overall framework): per chunk of C = 32 tokens,
//   T = (I + A)^-1, A_ij = b_j exp(lg_i - lg_j) k_i . k_j (j < i), T~ for the
//   noisy blocks, the weighted masked Grams Mwo, Mwq, Mwk, Mw~;
//   Z = diag(D) T V, W = -diag(D) T diag(G), D_i = b_i G_C / G_i,
// so that the scan's step is S_{c+1} = G_C S_c + K^T (Z + W (K S_c)).
// The chunk matrices go to the workspace for the output pass (and for the
// backward), the hand-over in the scan's register order (bwd_common.h).
//
// One workgroup of 4 waves per (chunk slot, head).  All loads first; then the
// four chunk-matrix jobs in parallel (wave 0 T, wave 1 T~, waves 2-3 the
// Grams) while every wave also writes its two fragment sets of K and K^T from
// the staged k rows; after one barrier, W (waves 0-1), the decay, and Z for
// two 16-column d_v slabs per wave.  Against the two separate passes this
// reads k, the gates and the chunk matrices once instead of twice.
// L2: the q/k L2 flag folded into per-row factors (gdn_l2.hip): the write
// strengths arrive folded from the gate load, the v rows are divided by r_k.
// CW > 0: the ShortConv in the loads (conv_load.h): the q, k, q~, k~ rows and
// the v rows are formed from the raw projections (each thread four rows of one
// section and both streams, the v rows two at a time), and with the L2 flag
// this pass also forms the factors from those rows (the same sums as the
// factor pass) and writes them for the output pass.
#include "bwd_common.h"
#include "chunk_common.h"
#include "conv_load.h"
#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {
constexpr int pC = 32, pD = 128, pNW = 4, pNT = 64 * pNW, pLDX = pD + 8, pLDM = pC + 4;
struct PrepSmem {
  alignas(16) u16 x[4][pC][pLDX];     // q, k, q~, k~ rows (masked)
  alignas(16) float at[2][pC][pLDM];  // A^T, A~^T (gated, without b)
  alignas(16) float tm[6][pC][pLDM];  // T, T~, Mwo, Mwq, Mwk, Mw~
  alignas(16) float tmp[2][16][17];
  alignas(16) float lg[pC], beta[pC], lgn[pC], betan[pC];
  alignas(16) float vsc[pC];  // L2: 1 / r_k of the chunk's rows
  alignas(16) float fac[4][pC];  // L2 with the conv loads: r_q, r_k, r_q~, r_k~ of the chunk's rows
};
}  // namespace

template <bool L2, int CW>
__global__ __launch_bounds__(pNT) void gdn_fwd_prep_d128_kernel(FwdArgs f, float *cmat, float *pack_all) {
  constexpr int C = pC, D = pD, NT = pNT, LDX = pLDX, LDM = pLDM;
  __shared__ PrepSmem sm;
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
  const u16 *const px[4] = {reinterpret_cast<const u16 *>(f.q), reinterpret_cast<const u16 *>(f.k),
                            reinterpret_cast<const u16 *>(f.qn), reinterpret_cast<const u16 *>(f.kn)};
  const u16 *const pv = reinterpret_cast<const u16 *>(f.v);
  float *const pack = pack_all + ((size_t)slot * H + h) * kPackWords;

  // ---- every global load first (unconditional, rows clamped into the
  // document): q, k, q~, k~ rows (8 16-byte units per thread), gates, the v
  // columns of this wave's two d_v slabs, the L2 factors
  constexpr int RU = D / 8, PU = C * RU, UX = CW > 0 ? 1 : 4 * PU / NT;
  constexpr int CWW = CW > 0 ? CW : 1;
  uint4 xr[UX];
  u16 rv[2][2][4];
  ConvRows<CWW, 4> cqk;  // CW: rows 4 (tid / 16 % 8) .. +3 of q (tid < 128) or k, both streams
  ConvRows<CWW, 2> cvr;  // CW: rows 2 (tid / 16) .. +1 of v
  const int csec = tid >> 7, crg = (tid >> 4) & 7, cvg = tid >> 4, cu16 = tid & 15;
  if constexpr (CW > 0) {
    cqk.load(f, csec, t0g, c0, 4 * crg, n, h, cu16, has_noisy);
    cvr.load(f, 2, t0g, c0, 2 * cvg, n, h, cu16, false);
  } else {
#pragma unroll
    for (int e = 0; e < UX; ++e) {
      const int u = e * NT + tid;
      const int m = u / PU, r = u % PU, row = r / RU, cu = r % RU;
      // a noisy prompt row (masked later) is read from the clean twin this thread loads too
      const int ms = m >= 2 && c0 + row < P ? m - 2 : m;  // (selects, not an indexed array: no scratch)
      const u16 *src = ms == 0 ? px[0] : ms == 1 ? px[1] : ms == 2 ? px[2] : px[3];
      xr[e] = ld_nt_u4(src + ((t0g + min(c0 + row, n - 1)) * H + h) * D + cu * 8);  // read once here
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) gslab_raw<D>(rv[sb], pv, H, h, t0g, c0, n, 32 * wave + 16 * sb);
  }
  // the gates (with the conv loads unfolded: this pass forms the factors)
  FwdArgs fg = f;
  if (CW > 0) fg.l2f = nullptr;
  const float graw = tid < 4 * C ? gate_load_raw(fg, t0g, c0, n, h, tid) : 0.f;
  float rkl = 1.f;
  if (L2 && CW == 0 && tid < C) rkl = f.l2f[(t0g + min(c0 + tid, n - 1)) * H + h].y;

  // ---- LDS: zeroed chunk matrices, the masked rows, gates
  for (int e = tid; e < 8 * C * LDM; e += NT) (&sm.at[0][0][0])[e] = 0.f;  // at and tm
  uint4 yv[2];  // CW: the v rows, kept until the rows' LDS is free
  if constexpr (CW > 0) {
    uint4 y[4], yn[4];
    cqk.rows(c0, 4 * crg, P, B, f.cact != 0, y, yn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * crg + i, tpos = c0 + row;
      const uint4 yc = sel4(tpos < n, y[i], make_uint4(0u, 0u, 0u, 0u));
      const uint4 ynv = sel4(tpos < n && tpos >= P, yn[i], make_uint4(0u, 0u, 0u, 0u));
      *reinterpret_cast<uint4 *>(&sm.x[csec][row][cu16 * 8]) = yc;
      *reinterpret_cast<uint4 *>(&sm.x[2 + csec][row][cu16 * 8]) = ynv;
      if (L2) {  // the row factors, from the same sums as the factor pass
        const float rc = l2_factor(l2_rowsum16(yc)), rn = l2_factor(l2_rowsum16(ynv));
        if (cu16 == 0) {
          sm.fac[csec][row] = rc;
          sm.fac[2 + csec][row] = rn;
        }
      }
    }
    uint4 vdum[2];
    cvr.rows(c0, 2 * cvg, P, B, f.cact != 0, yv, vdum);
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
  if constexpr (CW > 0 && L2) {
    lds_barrier();  // the factors: fold them into the write strengths, hand them to the output pass
    if (tid < C) {
      rkl = sm.fac[1][tid];
      if (c0 + tid < n)
        const_cast<float4 *>(f.l2f)[(t0g + c0 + tid) * H + h] =
            make_float4(sm.fac[0][tid], sm.fac[1][tid], sm.fac[2][tid], sm.fac[3][tid]);
    }
  }
  if (tid < 4 * C) {
    float gv = graw;
    if (CW > 0 && L2 && ((tid / C) & 1)) {  // folded write strengths b r_k^2 (gdn_l2.hip)
      const float rk = sm.fac[tid / C][tid & (C - 1)];
      gv *= rk * rk;
    }
    gate_scan(gate_fix(gv, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  }
  if (L2 && tid < C) sm.vsc[tid] = rkl > 0.f ? 1.f / rkl : 0.f;
  lds_barrier();

  // ---- the chunk matrices, each wave its own jobs (ordered per wave)
  if (wave == 0) {
    gram_at<D, LDX, LDM>(sm.x[1], sm.at[0], sm.lg);
    solve_unit_lower<LDM>(&sm.at[0][0][0], &sm.tm[0][0][0], &sm.tmp[0][0][0], true, sm.beta);
  } else if (wave == 1) {
    if (has_noisy) {
      gram_ant<D, LDX, LDM>(sm.x[3], sm.at[1], sm.lgn, c0, n, P, B);
      solve_unit_lower<LDM>(&sm.at[1][0][0], &sm.tm[1][0][0], &sm.tmp[1][0][0], B > 16, sm.betan);
    }
  } else {
    grams_weighted<D, LDX, LDM>(wave - 2, sm.x, sm.tm[2], sm.tm[3], sm.tm[4], sm.tm[5], sm.lg, sm.beta, sm.lgn,
                                sm.betan, c0, n, P, B, has_noisy);
  }
  // wave 0 wrote T (0), wave 1 T~ (1), wave 2 Mwo, Mwq (2, 3), wave 3 Mwk, Mw~ (4, 5)
  {
    float *dst = cmat + ((size_t)slot * H + h) * 6 * C * C;
    const int nm = wave < 2 ? 1 : 2;
    for (int mi = 0; mi < nm; ++mi) {
      const int mtx = wave < 2 ? wave : (wave == 2 ? 2 : 4) + mi;
#pragma unroll
      for (int e = 0; e < C * C / 4 / 64; ++e) {
        const int u = mtx * (C * C / 4) + e * 64 + lane;  // the record's tile-major order
        if (cm_f4_live(u, B, has_noisy))  // structurally zero parts are not stored
          *reinterpret_cast<float4 *>(dst + 4 * (size_t)u) =
              *reinterpret_cast<const float4 *>(&sm.tm[mtx][cm_row(u)][cm_col(u)]);
      }
    }
  }
  // ---- the fragment sets of K (sets wave and wave + 4): KA set s holds rows
  // 16 (s & 1) + (l & 15), d_k columns 32 (s >> 1) + the slab k-permutation;
  // KT set s holds the columns d_k 16 s + (l & 15), chunk rows in the slab
  // k-permutation.  Rows past the document end are zero in the staged rows.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = wave + 4 * j;
    const u16 *kr = &sm.x[1][16 * (s & 1) + cl][32 * (s >> 1)];
    const uint2 lo = *reinterpret_cast<const uint2 *>(kr + g4);
    const uint2 hi = *reinterpret_cast<const uint2 *>(kr + 16 + g4);
    reinterpret_cast<uint4 *>(pack + kPackKA)[s * 64 + lane] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    const int col = 16 * s + cl;
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = e < 2 ? g4 + 2 * e : 16 + g4 + 2 * (e - 2);
      w4[e] = (uint32_t)sm.x[1][row][col] | ((uint32_t)sm.x[1][row + 1][col] << 16);
    }
    reinterpret_cast<uint4 *>(pack + kPackKT)[s * 64 + lane] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  lds_barrier();  // T visible to every wave

  const float lgC = sm.lg[C - 1];
  auto Dd = [&](int i) { return sm.beta[i] * __expf(lgC - sm.lg[i]); };
  if (wave < 2) {
    // W_ij = -D_i T_ij G_j, rows i = 16 tr + (l & 15), columns j in the slab
    // permutation; zero on rows and columns past the document end
    const int tr = wave, i = 16 * tr + cl;
    const bool iok = c0 + i < n;
    const float di = -Dd(i);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = e < 4 ? g4 + e : 16 + g4 + e - 4;
      const bool ok = iok && c0 + j < n;
      x[e] = ok ? di * sm.tm[0][i][j] * __expf(sm.lg[j]) : 0.f;
    }
    bf16x8 wh, wl;
    split8(x, wh, wl);
    uint4 *dst = reinterpret_cast<uint4 *>(pack + kPackW);
    dst[(2 * tr) * 64 + lane] = __builtin_bit_cast(uint4, wh);
    dst[(2 * tr + 1) * 64 + lane] = __builtin_bit_cast(uint4, wl);
  }
  if (tid == 0) pack[kPackG] = __expf(lgC);
  if constexpr (CW > 0) {  // the v rows -> the q rows' LDS (every wave is done with them)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 2 * cvg + i;
      *reinterpret_cast<uint4 *>(&sm.x[0][row][cu16 * 8]) = sel4(c0 + row < n, yv[i], make_uint4(0u, 0u, 0u, 0u));
    }
    lds_barrier();
  }

  // ---- Z = diag(D) T V for this wave's two slabs, stored as [slab][tile][lane][4]
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int slab = 2 * wave + sb;
    Slab V;
    if constexpr (CW > 0) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) V.t[tr][r] = bf2f(sm.x[0][slab_row(tr, r)][16 * slab + cl]);
    } else {
      V = slab_mask(rv[sb], c0, n, P, false);
    }
    Slab Z = slab_zero();
    if constexpr (L2) {  // v' = v / r_k is no longer exact in bf16: both operands split
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) V.t[tr][r] *= sm.vsc[slab_row(tr, r)];
      cc_mul<3, false>(Z, &sm.tm[0][0][0], LDM, V);
    } else {
      cc_mul<2, false>(Z, &sm.tm[0][0][0], LDM, V);
    }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) Z.t[tr][r] *= Dd(slab_row(tr, r));
    float4 *zdst = reinterpret_cast<float4 *>(pack + kPackR) + (size_t)slab * 2 * 64;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) st_nt_f4(&zdst[tr * 64 + lane], make_float4(Z.t[tr][0], Z.t[tr][1], Z.t[tr][2], Z.t[tr][3]));
  }
}

template <int CW>
static void launch_prep_w(const FwdArgs &a, float *cmat, float *pack, hipStream_t st, int64_t slots) {
  const dim3 grid((unsigned)(slots * a.H)), block(pNT);
  if (a.l2f) hipLaunchKernelGGL((gdn_fwd_prep_d128_kernel<true, CW>), grid, block, 0, st, a, cmat, pack);
  else hipLaunchKernelGGL((gdn_fwd_prep_d128_kernel<false, CW>), grid, block, 0, st, a, cmat, pack);
}

hipError_t launch_fwd_prep_d128(const FwdArgs &a, float *cmat, float *pack, hipStream_t st, int64_t slots) {
  switch (a.cw) {
    case 0: launch_prep_w<0>(a, cmat, pack, st, slots); break;
    case 1: launch_prep_w<1>(a, cmat, pack, st, slots); break;
    case 2: launch_prep_w<2>(a, cmat, pack, st, slots); break;
    case 3: launch_prep_w<3>(a, cmat, pack, st, slots); break;
    case 4: launch_prep_w<4>(a, cmat, pack, st, slots); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace flare
