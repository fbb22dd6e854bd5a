// gdn_fwd_march.hip -- dual-stream forward for bf16 io at d_k = d_v = 128
// without the q/k normalisation flag (other configurations use the fused
// kernel in gdn_fwd.hip).
//
// Method ("FLARE: Diffusion for Hybrid Language Model", papernotes.org notes,
// Key designs item 2; Overall framework): the clean stream follows the gated
// delta rule; a noisy block starts from the clean state at its boundary,
// applies its own updates, and every position of the block reads the
// block-end state.  Per chunk of C = 32 tokens, with start state S_c and the
// chunk matrices T, T~, Mwo, Mwq, Mwk, Mw~ formed in parallel beforehand by
// the chunk-matrix kernel (gdn_tri.hip):
//   U   = T (V - diag(G) K S_c)
//   o   = s (diag(G) Q S_c + Mwo U)
//   r_q = diag(G_p) q~ S_c + Mwq U,   r_k = diag(G_p) k~ S_c + Mwk U
//   u~  = T~ (v~ - diag(G~) r_k),     o~ = s (diag(G~_e) r_q + Mw~ u~)
//   S  <- G_C S_c + K^T diag(b G_C / G) U
// The boundary states of the noisy blocks are never formed: r_q and r_k are
// their reads.
//
// Layout: four workgroups of 2 waves per (document, head), on one XCD; wave w
// of quarter q owns d_v columns [32 q + 16 w, +16).  Its 128 x 16 slab of S
// lives in MFMA accumulators for the whole document and is fed straight back
// (bf16) as the B operand of K S_c, Q S_c, q~ S_c, k~ S_c; every C x 16
// quantity is a register slab (slab.h); K^T comes from a transposed copy of
// the chunk's k rows in LDS.  The next chunk's rows, matrices, gates and v, v~
// columns are fetched as raw bits while the current chunk computes; outputs,
// checkpoints and the final state leave through LDS staging as 16-byte stores.
#include "bwd_common.h"
#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int mC = 32, mD = 128, mNW = 2, mNT = 64 * mNW, mQ = 4;
constexpr int mLDX = mD + 8, mLDT = mC + 4, mLDM = mC + 4, mLDQ = 32 + 8;
enum { MC_T = 0, MC_TN, MC_MO, MC_MQ, MC_MK, MC_MN };  // the chunk-matrix kernel's order

struct MarchSmem {
  alignas(16) u16 xr[4][mC][mLDX];   // q, k, q~, k~ rows
  alignas(16) u16 kt[mD][mLDT];      // k transposed ([d_k][chunk row])
  alignas(16) float cc[6][mC][mLDM];  // T, T~, Mwo, Mwq, Mwk, Mw~
  alignas(16) u16 vq[2][mC][mLDQ];   // v, v~ columns of this quarter
  alignas(16) u16 oq[2][mC][mLDQ];   // o, o~ staging
  alignas(16) float st[mNW][mD][16 + 4];  // per-wave staging of the state slab
  alignas(16) float lg[mC], beta[mC], lgn[mC], betan[mC];
};

struct MarchPrefetch {
  uint4 x[4][4];  // [array][row rr]: rows 4 (t % 8) + rr, 16-byte unit t / 8
  float4 cm[12];  // the six chunk matrices
  float gate;
  uint4 vq[2];    // v / v~: row t / 4, 16-byte unit t % 4 of the quarter
};

}  // namespace

__global__ __launch_bounds__(mNT) void gdn_fwd_march_d128_kernel(FwdArgs a, const float *cmat) {
  constexpr int C = mC, D = mD, NT = mNT;
  __shared__ MarchSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  // ---- workgroup -> (document, head, quarter); the quarters of a pair share an XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * mQ), rem = L % (8 * mQ);
  const int quarter = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= a.num_docs * a.H) return;
  const int doc = pair / a.H, h = pair % a.H;
  const int H = a.H;
  const int64_t t0g = a.cu[doc];
  const int n = a.cu[doc + 1] - a.cu[doc];
  const int P = a.plen[doc];
  const int B = a.B;
  const int nchunks = (n + C - 1) / C;
  const int dv0 = 32 * quarter + 16 * wave;
  const float s = a.scale;
  const int64_t ck_base = (int64_t)(t0g / C) + doc;
  const u16 *const px[4] = {reinterpret_cast<const u16 *>(a.q), reinterpret_cast<const u16 *>(a.k),
                            reinterpret_cast<const u16 *>(a.qn), reinterpret_cast<const u16 *>(a.kn)};
  const u16 *const pv = reinterpret_cast<const u16 *>(a.v), *const pvn = reinterpret_cast<const u16 *>(a.vn);
  u16 *const po = reinterpret_cast<u16 *>(a.o), *const pon = reinterpret_cast<u16 *>(a.on);

  // ---- state slab: tile kt holds rows 16 kt + 4 g + r (d_k), column dv0 + cl
  floatx4 S[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    S[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (a.h0) {
      const float *src = a.h0 + ((size_t)doc * H + h) * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kt][r] = src[(size_t)(16 * kt + g4 + r) * D + dv0 + cl];
    }
  }
  // the state slab -> global [D][D] through this wave's LDS staging rows
  auto store_state = [&](float *dst) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.st[wave][16 * kt + g4 + r][cl] = S[kt][r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = j * 64 + lane, row = u >> 2, c4 = u & 3;
      *reinterpret_cast<float4 *>(dst + (size_t)row * D + dv0 + 4 * c4) =
          *reinterpret_cast<const float4 *>(&sm.st[wave][row][4 * c4]);
    }
  };

  // ---- prefetch (raw bits; rows clamped into the document, masked at the fill)
  const int prow = 4 * (tid & 7), pu = tid >> 3;
  auto prefetch = [&](MarchPrefetch &pf, int c) {
    const int c0 = c * C;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        pf.x[m][rr] = *reinterpret_cast<const uint4 *>(px[m] + ((t0g + min(c0 + prow + rr, n - 1)) * H + h) * D + 8 * pu);
    const float *cm = cmat + ((size_t)(ck_base + c) * H + h) * 6 * C * C;
#pragma unroll
    for (int j = 0; j < 12; ++j) pf.cm[j] = *reinterpret_cast<const float4 *>(cm + 4 * (j * NT + tid));
    pf.gate = gate_load_raw(a, t0g, c0, n, h, tid);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pf.vq[j] = *reinterpret_cast<const uint4 *>((j == 0 ? pv : pvn) +
                                                  ((t0g + min(c0 + (tid >> 2), n - 1)) * H + h) * D + 32 * quarter +
                                                  8 * (tid & 3));
  };
  auto fill_lds = [&](const MarchPrefetch &pf, int c0) {
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
      if (m == 1) {  // k transposed: four rows of one column -> one 8-byte write
        const uint32_t w[4][4] = {{xv[0].x, xv[0].y, xv[0].z, xv[0].w},
                                  {xv[1].x, xv[1].y, xv[1].z, xv[1].w},
                                  {xv[2].x, xv[2].y, xv[2].z, xv[2].w},
                                  {xv[3].x, xv[3].y, xv[3].z, xv[3].w}};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xffffu, v1 = (w[1][e >> 1] >> sh) & 0xffffu;
          const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xffffu, v3 = (w[3][e >> 1] >> sh) & 0xffffu;
          *reinterpret_cast<uint2 *>(&sm.kt[8 * pu + e][prow]) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int u = j * NT + tid, which = u / (C * C / 4), rr = u % (C * C / 4);
      *reinterpret_cast<float4 *>(&sm.cc[which][rr / (C / 4)][4 * (rr % (C / 4))]) = pf.cm[j];
    }
    gate_scan(gate_fix(pf.gate, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = tid >> 2, un = tid & 3, tpos = c0 + row;
      const bool ok = tpos < n && (j == 0 || tpos >= P);
      *reinterpret_cast<uint4 *>(&sm.vq[j][row][8 * un]) = ok ? pf.vq[j] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto slab_lds = [&](const u16 (*src)[mLDQ]) {
    Slab sl;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) sl.t[tr][r] = bf2f(src[slab_row(tr, r)][16 * wave + cl]);
    return sl;
  };
  // A fragment of rows 16 tr .. of an LDS row tile over d_k step ks, columns in
  // the state slab's k-permutation (32 ks + 4g .. +3 and 32 ks + 16 + 4g .. +3)
  auto xrow_frag = [&](int m, int tr, int ks) {
    const u16 *row = &sm.xr[m][16 * tr + cl][32 * ks];
    const uint2 lo4 = *reinterpret_cast<const uint2 *>(row + g4);
    const uint2 hi4 = *reinterpret_cast<const uint2 *>(row + 16 + g4);
    return __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
  };

  MarchPrefetch pf;
  if (nchunks > 0) prefetch(pf, 0);

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * C;
    const bool has_noisy = (c0 + C > P) && (P < n);
    lds_barrier();  // every wave is done with the previous chunk's LDS
    fill_lds(pf, c0);
    if (a.ckpt) store_state(a.ckpt + ((size_t)(ck_base + c) * H + h) * D * D);
    if (c + 1 < nchunks) prefetch(pf, c + 1);
    lds_barrier();

    const float lgC = sm.lg[C - 1];
    const Slab V = slab_lds(sm.vq[0]);
    // S_c as B fragments (bf16), k-slots 32 ks + 4g + e / 32 ks + 16 + 4g + e - 4
    bf16x8 sb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 hbits = make_uint4(pack_bf16x2(S[2 * ks][0], S[2 * ks][1]), pack_bf16x2(S[2 * ks][2], S[2 * ks][3]),
                                     pack_bf16x2(S[2 * ks + 1][0], S[2 * ks + 1][1]),
                                     pack_bf16x2(S[2 * ks + 1][2], S[2 * ks + 1][3]));
      sb[ks] = __builtin_bit_cast(bf16x8, hbits);
    }
    Slab KS = slab_zero(), QS = slab_zero();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        mma_bf16(KS.t[tr], xrow_frag(1, tr, ks), sb[ks]);
        mma_bf16(QS.t[tr], xrow_frag(0, tr, ks), sb[ks]);
      }
    // U = T (v - G K S_c)
    Slab rhs;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) rhs.t[tr][r] = V.t[tr][r] - __expf(sm.lg[slab_row(tr, r)]) * KS.t[tr][r];
    Slab U = slab_zero();
    cc_mul<3, false>(U, &sm.cc[MC_T][0][0], mLDM, rhs);
    // o = s (G Q S_c + Mwo U)
    Slab O = slab_zero();
    cc_mul<3, false>(O, &sm.cc[MC_MO][0][0], mLDM, U);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        O.t[tr][r] = s * (__expf(sm.lg[i]) * QS.t[tr][r] + O.t[tr][r]);
      }
    // noisy reads of the block-boundary states and the noisy blocks
    Slab ON = slab_zero();
    if (has_noisy) {
      Slab RQ = slab_zero(), RK = slab_zero();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tr = 0; tr < 2; ++tr) {
          mma_bf16(RQ.t[tr], xrow_frag(2, tr, ks), sb[ks]);
          mma_bf16(RK.t[tr], xrow_frag(3, tr, ks), sb[ks]);
        }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = slab_row(tr, r), pi = i - (i % B);
          const float gp = pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f;
          RQ.t[tr][r] *= gp;
          RK.t[tr][r] *= gp;
        }
      cc_mul<3, false>(RQ, &sm.cc[MC_MQ][0][0], mLDM, U);
      cc_mul<3, false>(RK, &sm.cc[MC_MK][0][0], mLDM, U);
      const Slab VN = slab_lds(sm.vq[1]);
      Slab rhsn;
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          rhsn.t[tr][r] = VN.t[tr][r] - __expf(sm.lgn[slab_row(tr, r)]) * RK.t[tr][r];
      Slab UN = slab_zero();
      cc_mul<3, false>(UN, &sm.cc[MC_TN][0][0], mLDM, rhsn);
      cc_mul<3, false>(ON, &sm.cc[MC_MN][0][0], mLDM, UN);
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = slab_row(tr, r), pi = i - (i % B);
          const bool resp = c0 + i < n && c0 + i >= P;
          ON.t[tr][r] = resp ? s * (__expf(sm.lgn[pi + B - 1]) * RQ.t[tr][r] + ON.t[tr][r]) : 0.f;
        }
    }
    // S <- G_C S_c + K^T diag(b G_C / G) U
    Slab DU;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        DU.t[tr][r] = sm.beta[i] * __expf(lgC - sm.lg[i]) * U.t[tr][r];
      }
    {
      const float gC = __expf(lgC);
      bf16x8 dh, dl;
      slab_b_split(DU, dh, dl);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const u16 *col = &sm.kt[16 * kt + cl][0];
        const uint2 lo4 = *reinterpret_cast<const uint2 *>(col + g4);
        const uint2 hi4 = *reinterpret_cast<const uint2 *>(col + 16 + g4);
        const bf16x8 ak = __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
        S[kt] *= gC;
        mma_bf16(S[kt], ak, dh);
        mma_bf16(S[kt], ak, dl);
      }
    }
    // o, o~ of this slab -> LDS staging -> 16-byte stores of the quarter's rows
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        sm.oq[0][i][16 * wave + cl] = f2bf(O.t[tr][r]);
        sm.oq[1][i][16 * wave + cl] = f2bf(ON.t[tr][r]);
      }
    lds_barrier();
    {
      const int row = tid >> 2, un = tid & 3;
      if (c0 + row < n) {
        const int64_t off = ((t0g + c0 + row) * H + h) * D + 32 * quarter + 8 * un;
        *reinterpret_cast<uint4 *>(po + off) = *reinterpret_cast<const uint4 *>(&sm.oq[0][row][8 * un]);
        *reinterpret_cast<uint4 *>(pon + off) = *reinterpret_cast<const uint4 *>(&sm.oq[1][row][8 * un]);
      }
    }
  }
  if (a.h_final) store_state(a.h_final + ((size_t)doc * H + h) * D * D);
}

hipError_t launch_fwd_march_d128(const FwdArgs &a, const float *cmat, hipStream_t st) {
  const int pairs = a.num_docs * a.H;
  const int groups = (pairs + 7) / 8;
  hipLaunchKernelGGL(gdn_fwd_march_d128_kernel, dim3((unsigned)(groups * 8 * mQ)), dim3(mNT), 0, st, a, cmat);
  return hipGetLastError();
}

}  // namespace flare
