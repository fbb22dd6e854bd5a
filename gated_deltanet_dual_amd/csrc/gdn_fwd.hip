// gdn_fwd.hip -- fused dual-stream Gated DeltaNet forward for gfx950.
//
// Method ("FLARE: Diffusion for Hybrid Language Model", papernotes.org notes):
//   * Overall framework: the prompt is clean causal context; the response is cut
//     into consecutive blocks of B tokens.
//   * Key designs item 2: clean stream S_t = a_t (I - b_t k_t k_t^T) S_{t-1}
//     + b_t k_t v_t^T, o_t = s S_t^T q_t.  A noisy block starts from the clean
//     boundary state, applies its own noisy updates, and all its positions read
//     the block-end state.  Block-boundary states are rebuilt on chip instead of
//     being kept in HBM; only strided clean checkpoints may be written.
//   * Key designs item 3: documents are packed with per-document reset.
//
// Design (gfx950, wave64, MFMA):
//   One workgroup of 4 waves per (document, head, 32-column tile of d_v).  The
//   tiles of a (document, head) are placed on the same XCD so that the q/k rows
//   they all read are shared through that XCD's L2.  The workgroup marches the
//   document's chunks of C = 32 tokens in order; the clean state tile
//   (d_k x 32, fp32) lives in MFMA accumulator registers for the whole document.
//   The next chunk's inputs are prefetched into registers while the current one
//   is computed.  Per chunk, with G_i = exp(cumulative log a) inside the chunk:
//     A   = strictly-lower((K K^T) o G_i/G_j) diag(b),  T = (I + A)^-1
//     U   = T (V - diag(G) K S_c)                         (WY/UT form)
//     o   = s (diag(G) Q S_c + tril((Q K^T) o G_i/G_j) diag(b) U)
//     S  <- G_C S_c + K^T diag(b G_C/G) U
//   Noisy block reads never materialise the boundary state S_p: for a noisy
//   token l whose block starts after p chunk tokens,
//     S_p^T x = G_p S_c^T x + sum_{j<p} (G_p/G_j) b_j (k_j . x) u_j,  x in {q~_l, k~_l},
//   i.e. the clean output formula with the mask j < p.  The block itself is
//   another small UT solve with block-diagonal masks:
//     u~ = T~ (v~ - diag(G~) S_p^T k~),  o~_l = s (G~_e S_p^T q~_l + sum_{j in blk} (G~_e/G~_j) b~_j (q~_l.k~_j) u~_j).
//   Every contraction over d_k (Gram matrices, X S_c, K^T U) runs on
//   v_mfma_f32_16x16x32_bf16 with bf16 inputs that are exact (q, k) or the
//   bf16 rounding of the fp32 state; the C x C by C x 32 products whose both
//   operands are fp32 (T rhs, M U) use a two/three-term bf16 hi+lo split, which
//   keeps them at ~2^-16 relative error.  fp32 io uses v_mfma_f32_16x16x4f32
//   throughout.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace flare {

template <typename IO, int D> struct FwdCfg {
  static constexpr bool BF = std::is_same<IO, u16>::value;
  static constexpr int C = 32;                 // chunk
  static constexpr int NW = 4;                 // waves
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int DV = D >= 32 ? 32 : D;  // d_v columns per workgroup
  static constexpr int NTILE = D / DV;
  static constexpr int LDX = D + 8;            // q/k tile pitch (elements)
  static constexpr int LDM = C + 4;            // C x C and [DV][C] fp32 pitch
  static constexpr int LDV = DV + 4;           // value tile pitch (fp32)
  static constexpr int ES = sizeof(IO);
  static constexpr int PU = C * D * ES / 16;   // 16-byte units per q/k tile
  static constexpr int RU = D * ES / 16;       // units per q/k row
  static constexpr int UX = 4 * PU / NT;       // q/k units per thread
  static constexpr int PV = C * DV * ES / 16;  // units per value tile
  static constexpr int RV = DV * ES / 16;      // units per value row
  static constexpr int NST = (D / 16) * (DV / 16);        // 16x16 state tiles
  static constexpr int SPW = (NST + NW - 1) / NW;         // state tiles per wave
  static_assert(4 * PU % NT == 0, "q/k tile units must divide the threads");
  static_assert(2 * PV <= NT, "at most one value unit per thread");
};

template <typename IO, int D> struct FwdSmem {
  using Cfg = FwdCfg<IO, D>;
  static constexpr int C = Cfg::C, DV = Cfg::DV, LDX = Cfg::LDX, LDM = Cfg::LDM, LDV = Cfg::LDV;
  using ST = typename std::conditional<Cfg::BF, u16, float>::type;  // S^T storage
  alignas(16) IO x[4][C][LDX];           // 0 q, 1 k, 2 q~, 3 k~
  alignas(16) ST st[DV][LDX];            // S_c^T (bf16 hi, or fp32)
  alignas(16) float v[2][C][LDV];        // v, v~ tiles (fp32)
  alignas(16) float cc[8][C][LDM];       // 0 A, 1 T, 2 Mo, 3 Mq, 4 Mk, 5 A~, 6 T~, 7 M~
  alignas(16) float vt[7][DV][LDM];      // 0 rhs, 1 QS, 2 rq, 3 rk/rhs~, 4 U, 5 DU, 6 u~
  alignas(16) float tmp[2][16][17];      // off-diagonal block solve scratch
  alignas(16) IO out[2][C][DV];          // o, o~ staging
  alignas(16) float rawg[4][C];          // a, b, a~, b~ of the chunk
  alignas(16) float lg[C], beta[C], lgn[C], betan[C];
  alignas(16) float nrm[4][C];  // 1/|x| per row (1 without the L2 flag)
};

enum { CC_A = 0, CC_T, CC_MO, CC_MQ, CC_MK, CC_AN, CC_TN, CC_MN };
enum { VT_RHS = 0, VT_QS, VT_RQ, VT_RK, VT_U, VT_DU, VT_UN };

// ------------------------------------------------------------------ products
// All compute acc[i][j] += sum_k A[ra + i][k] * Bt[rb + j][k] for one 16x16 tile.
template <int K>
__device__ __forceinline__ void mm_u16(floatx4 &acc, const u16 *A, int lda, int ra, const u16 *Bt,
                                       int ldb, int rb) {
  if constexpr (K % 32 == 0) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) mma_bf16(acc, frag_bf16(A, lda, ra, k0), frag_bf16(Bt, ldb, rb, k0));
  } else {
    static_assert(K == 16, "a contraction shorter than one MFMA step must be 16 deep");
    // one 32-deep step whose upper half (lanes 32..63 carry k = 16..31) is zero
    const bool live = lane_id() < 32;
    const bf16x8 z = as_bf16x8(u16x8{});
    mma_bf16(acc, live ? frag_bf16(A, lda, ra, 0) : z, live ? frag_bf16(Bt, ldb, rb, 0) : z);
  }
}
template <int K>
__device__ __forceinline__ void mm_f32(floatx4 &acc, const float *A, int lda, int ra, const float *Bt,
                                       int ldb, int rb) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4) mma_f32(acc, frag1_f32(A, lda, ra, k0), frag1_f32(Bt, ldb, rb, k0));
}
// A fp32 -> bf16 hi, Bt fp32 -> hi + lo   (2 MFMA per k-step)
template <int K>
__device__ __forceinline__ void mm_split2(floatx4 &acc, const float *A, int lda, int ra,
                                          const float *Bt, int ldb, int rb) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const bf16x8 a = frag_f32_hi(A, lda, ra, k0);
    bf16x8 bh, bl;
    frag_f32_split(Bt, ldb, rb, k0, bh, bl);
    mma_bf16(acc, a, bh);
    mma_bf16(acc, a, bl);
  }
}
// A, Bt fp32 -> hi + lo each; hi*hi + hi*lo + lo*hi   (3 MFMA per k-step)
template <int K>
__device__ __forceinline__ void mm_split3(floatx4 &acc, const float *A, int lda, int ra,
                                          const float *Bt, int ldb, int rb) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    bf16x8 ah, al, bh, bl;
    frag_f32_split(A, lda, ra, k0, ah, al);
    frag_f32_split(Bt, ldb, rb, k0, bh, bl);
    mma_bf16(acc, ah, bh);
    mma_bf16(acc, ah, bl);
    mma_bf16(acc, al, bh);
  }
}

// dispatch on the io precision: "exact-ish" product of two fp32 LDS matrices
template <bool BF, int K, int TERMS>
__device__ __forceinline__ void mm_ff(floatx4 &acc, const float *A, int lda, int ra, const float *Bt,
                                      int ldb, int rb) {
  if constexpr (BF) {
    if constexpr (TERMS == 2) mm_split2<K>(acc, A, lda, ra, Bt, ldb, rb);
    else mm_split3<K>(acc, A, lda, ra, Bt, ldb, rb);
  } else {
    mm_f32<K>(acc, A, lda, ra, Bt, ldb, rb);
  }
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

template <typename IO, int D>
__global__ __launch_bounds__(256) void gdn_dual_fwd_kernel(FwdArgs a) {
  using Cfg = FwdCfg<IO, D>;
  using Sm = FwdSmem<IO, D>;
  constexpr bool BF = Cfg::BF;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, DV = Cfg::DV, NTILE = Cfg::NTILE;
  constexpr int LDX = Cfg::LDX, LDM = Cfg::LDM, LDV = Cfg::LDV;
  constexpr int SPW = Cfg::SPW, NST = Cfg::NST;
  using ST = typename Sm::ST;

  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- workgroup -> (document, head, d_v tile), tiles of one pair on one XCD
  const int L = blockIdx.x;
  const int grp = L / (8 * NTILE), rem = L % (8 * NTILE);
  const int tile = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= a.num_docs * a.H) return;
  const int doc = pair / a.H, h = pair % a.H;
  const int H = a.H;
  const int64_t t0g = a.cu[doc];
  const int n = a.cu[doc + 1] - a.cu[doc];
  const int P = a.plen[doc];
  const int B = a.B;
  const int nchunks = (n + C - 1) / C;
  const int dv0 = tile * DV;
  const float scale = a.scale;
  const bool l2 = (a.flags & 1) != 0;

  const IO *gx[4] = {reinterpret_cast<const IO *>(a.q), reinterpret_cast<const IO *>(a.k),
                     reinterpret_cast<const IO *>(a.qn), reinterpret_cast<const IO *>(a.kn)};
  const IO *gv[2] = {reinterpret_cast<const IO *>(a.v), reinterpret_cast<const IO *>(a.vn)};
  const float *gg[4] = {a.alpha, a.beta, a.alpha_n, a.beta_n};

  // ---- one-time LDS init: zero all C x C matrices (upper blocks stay zero)
  for (int e = tid; e < 8 * C * LDM; e += NT) (&sm.cc[0][0][0])[e] = 0.f;
  for (int e = tid; e < 4 * C; e += NT) (&sm.nrm[0][0])[e] = 1.f;

  // ---- state tiles owned by this wave: tile q -> rows 16*(q / (DV/16)), cols 16*(q % (DV/16))
  floatx4 S[SPW];
#pragma unroll
  for (int e = 0; e < SPW; ++e) {
    const int q = wave * SPW + e;
    S[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (q < NST && a.h0) {
      const int rt = q / (DV / 16), ct = q % (DV / 16);
      const float *src = a.h0 + ((size_t)doc * H + h) * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[e][r] = src[(size_t)(16 * rt + acc_row(r)) * D + dv0 + 16 * ct + acc_col()];
    }
  }
  auto write_state_t = [&]() {  // S -> st (S^T, bf16 hi or fp32)
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int q = wave * SPW + e;
      if (q < NST) {
        const int rt = q / (DV / 16), ct = q % (DV / 16);
        ST *dst = &sm.st[16 * ct + acc_col()][16 * rt + acc_row(0)];
        if constexpr (BF) {
          uint2 w;
          w.x = (uint32_t)f2bf(S[e][0]) | ((uint32_t)f2bf(S[e][1]) << 16);
          w.y = (uint32_t)f2bf(S[e][2]) | ((uint32_t)f2bf(S[e][3]) << 16);
          *reinterpret_cast<uint2 *>(dst) = w;
        } else {
          *reinterpret_cast<float4 *>(dst) = make_float4(S[e][0], S[e][1], S[e][2], S[e][3]);
        }
      }
    }
  };
  auto write_state_global = [&](float *dst_base) {  // fp32 [D][D] of this head
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int q = wave * SPW + e;
      if (q < NST) {
        const int rt = q / (DV / 16), ct = q % (DV / 16);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst_base[(size_t)(16 * rt + acc_row(r)) * D + dv0 + 16 * ct + acc_col()] = S[e][r];
      }
    }
  };
  write_state_t();

  // ---- prefetch registers
  uint4 pfx[Cfg::UX];
  uint4 pfv = make_uint4(0u, 0u, 0u, 0u);
  float pfg = 0.f;
  auto prefetch = [&](int c) {
    const int c0 = c * C;
#pragma unroll
    for (int e = 0; e < Cfg::UX; ++e) {
      const int u = e * NT + tid;
      const int m = u / Cfg::PU, r = u % Cfg::PU;
      const int row = r / Cfg::RU, cu16 = r % Cfg::RU;
      const int tpos = c0 + row;
      bool ok = tpos < n;
      if (m >= 2) ok = ok && tpos >= P;
      pfx[e] = make_uint4(0u, 0u, 0u, 0u);
      if (ok)
        pfx[e] = *reinterpret_cast<const uint4 *>(gx[m] + ((t0g + tpos) * H + h) * D + cu16 * (16 / Cfg::ES));
    }
    if (tid < 2 * Cfg::PV) {
      const int m = tid / Cfg::PV, r = tid % Cfg::PV;
      const int row = r / Cfg::RV, cu16 = r % Cfg::RV;
      const int tpos = c0 + row;
      bool ok = tpos < n;
      if (m == 1) ok = ok && tpos >= P;
      pfv = make_uint4(0u, 0u, 0u, 0u);
      if (ok)
        pfv = *reinterpret_cast<const uint4 *>(gv[m] + ((t0g + tpos) * H + h) * D + dv0 + cu16 * (16 / Cfg::ES));
    }
    if (tid < 4 * C) {
      const int g = tid / C, i = tid % C;
      const int tpos = c0 + i;
      bool ok = tpos < n;
      if (g >= 2) ok = ok && tpos >= P;
      const bool is_alpha = (g & 1) == 0;
      pfg = is_alpha ? 1.f : 0.f;
      if (ok) pfg = gg[g][(t0g + tpos) * H + h];
    }
  };
  auto store_prefetch = [&]() {
#pragma unroll
    for (int e = 0; e < Cfg::UX; ++e) {
      const int u = e * NT + tid;
      const int m = u / Cfg::PU, r = u % Cfg::PU;
      const int row = r / Cfg::RU, cu16 = r % Cfg::RU;
      *reinterpret_cast<uint4 *>(&sm.x[m][row][cu16 * (16 / Cfg::ES)]) = pfx[e];
    }
    if (tid < 2 * Cfg::PV) {
      const int m = tid / Cfg::PV, r = tid % Cfg::PV;
      const int row = r / Cfg::RV, cu16 = r % Cfg::RV;
      float *dst = &sm.v[m][row][cu16 * (16 / Cfg::ES)];
      if constexpr (BF) {
        const uint32_t w[4] = {pfv.x, pfv.y, pfv.z, pfv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[2 * i] = __uint_as_float(w[i] << 16);
          dst[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        dst[0] = __uint_as_float(pfv.x); dst[1] = __uint_as_float(pfv.y);
        dst[2] = __uint_as_float(pfv.z); dst[3] = __uint_as_float(pfv.w);
      }
    }
    if (tid < 4 * C) sm.rawg[tid / C][tid % C] = pfg;
  };

  if (nchunks > 0) prefetch(0);
  const int64_t ck_base = a.ckpt ? (int64_t)(t0g / ((int64_t)C * a.ckpt_stride)) + doc : 0;

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * C;
    const bool has_noisy = (c0 + C > P) && (P < n);

    // ---------------------------------------------------------- [A] inputs
    __syncthreads();
    store_prefetch();
    if (c + 1 < nchunks) prefetch(c + 1);
    if (a.ckpt && (c % a.ckpt_stride) == 0)
      write_state_global(a.ckpt + ((ck_base + c / a.ckpt_stride) * H + h) * (size_t)D * D);
    __syncthreads();

    // ---------------------------------------------------------- [B] gates, norms
    if (wave == 0) {
      const int i = lane & 31;
      const bool noisy = lane >= 32;
      float la = __logf(sm.rawg[noisy ? 2 : 0][i]);
      const float be = sm.rawg[noisy ? 3 : 1][i];
      if (!noisy) {
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          const float y = __shfl_up(la, off, 32);
          if (i >= off) la += y;
        }
        sm.lg[i] = la;
        sm.beta[i] = be;
      } else {
        // segmented scan inside blocks of B tokens (blocks are B-aligned in the chunk)
        for (int off = 1; off < B; off <<= 1) {
          const float y = __shfl_up(la, off, B);
          if ((i % B) >= off) la += y;
        }
        sm.lgn[i] = la;
        sm.betan[i] = be;
      }
    }
    if (l2 && tid < 4 * C) {
      const int m = tid / C, row = tid % C;
      float ss = 0.f;
      for (int e = 0; e < D; ++e) {
        const float xv = io_traits<IO>::to_f(sm.x[m][row][e]);
        ss += xv * xv;
      }
      sm.nrm[m][row] = rsqrtf(ss + 1e-6f);
    }
    __syncthreads();

    // ---------------------------------------------------------- [C1] Gram matrices
    {
      // job list: (kind, ti, tj); kinds 0 A, 1 Mo, 2 Mq, 3 Mk use tiles (0,0),(1,0),(1,1);
      // 4 A~ and 5 M~ use the diagonal tiles, plus (1,0) [and (0,1) for M~] when B > 16.
      const int nclean = 6;
      const int nnoisy = has_noisy ? (6 + (B > 16 ? 7 : 4)) : 0;
      for (int job = wave; job < nclean + nnoisy; job += NW) {
        int kind, tsub;
        if (job < 6) { kind = job / 3; tsub = job % 3; }
        else if (job < 12) { kind = 2 + (job - 6) / 3; tsub = (job - 6) % 3; }
        else { const int jj = job - 12; const int na = B > 16 ? 3 : 2;
               if (jj < na) { kind = 4; tsub = jj; } else { kind = 5; tsub = jj - na; } }
        int ti, tj;
        if (kind < 4) { ti = tsub == 0 ? 0 : 1; tj = tsub == 2 ? 1 : 0; }
        else if (kind == 4) { ti = tsub == 0 ? 0 : (tsub == 1 ? 1 : 1); tj = tsub == 2 ? 0 : ti; }
        else { const int na = B > 16 ? 4 : 2;
               if (na == 2) { ti = tsub; tj = tsub; }
               else { ti = tsub >> 1; tj = tsub & 1; } }
        // X (rows i) and Y (rows j) for G[i][j] = x_i . y_j
        const int xm = kind == 0 ? 1 : kind == 1 ? 0 : kind == 2 ? 2 : kind == 3 ? 3 : kind == 4 ? 3 : 2;
        const int ym = kind <= 3 ? 1 : 3;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) mm_u16<D>(acc, &sm.x[ym][0][0], LDX, 16 * tj, &sm.x[xm][0][0], LDX, 16 * ti);
        else mm_f32<D>(acc, &sm.x[ym][0][0], LDX, 16 * tj, &sm.x[xm][0][0], LDX, 16 * ti);
        // acc[r] = G^T[j][i] with j = 16 tj + acc_row(r), i = 16 ti + acc_col()
        const int i = 16 * ti + acc_col();
        const int pi = i - (i % B);  // chunk-local start of i's block
        const int tpos = c0 + i;
        const bool resp = tpos < n && tpos >= P;
        float outv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * tj + acc_row(r);
          const float g = acc[r] * sm.nrm[xm][i] * sm.nrm[ym][j];
          float val = 0.f;
          if (kind == 0) {
            if (j < i) val = g * fast_exp(sm.lg[i] - sm.lg[j]) * sm.beta[j];
          } else if (kind == 1) {
            if (j <= i) val = g * fast_exp(sm.lg[i] - sm.lg[j]) * sm.beta[j];
          } else if (kind <= 3) {
            if (resp && j < pi) val = g * fast_exp(sm.lg[pi - 1] - sm.lg[j]) * sm.beta[j];
          } else if (kind == 4) {
            if (resp && j < i && j >= pi) val = g * fast_exp(sm.lgn[i] - sm.lgn[j]) * sm.betan[j];
          } else {
            if (resp && j >= pi && j < pi + B) val = g * fast_exp(sm.lgn[pi + B - 1] - sm.lgn[j]) * sm.betan[j];
          }
          outv[r] = val;
        }
        const int cc = kind == 0 ? CC_A : kind == 1 ? CC_MO : kind == 2 ? CC_MQ : kind == 3 ? CC_MK
                     : kind == 4 ? CC_AN : CC_MN;
        *reinterpret_cast<float4 *>(&sm.cc[cc][i][16 * tj + acc_row(0)]) =
            make_float4(outv[0], outv[1], outv[2], outv[3]);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- [C2] X S_c (waves 1..) | diagonal solves (wave 0)
    if (wave == 0) {
      // lanes: (matrix m = lane >> 5: 0 clean, 1 noisy), (block bb = (lane >> 4) & 1), column cl
      const int m = lane >> 5, bb = (lane >> 4) & 1, cl = lane & 15;
      if (m == 0 || has_noisy) {
        const float(*Am)[LDM] = sm.cc[m ? CC_AN : CC_A];
        float(*Tm)[LDM] = sm.cc[m ? CC_TN : CC_T];
        const int r0 = 16 * bb;
        for (int ii = 0; ii < 16; ++ii) {
          float x = 0.f;
          if (ii == cl) {
            x = 1.f;
          } else if (ii > cl) {
            float acc0 = 0.f, acc1 = 0.f;
            int mm = cl;
            for (; mm + 1 < ii; mm += 2) {
              acc0 += Am[r0 + ii][r0 + mm] * Tm[r0 + mm][r0 + cl];
              acc1 += Am[r0 + ii][r0 + mm + 1] * Tm[r0 + mm + 1][r0 + cl];
            }
            if (mm < ii) acc0 += Am[r0 + ii][r0 + mm] * Tm[r0 + mm][r0 + cl];
            x = -(acc0 + acc1);
          }
          Tm[r0 + ii][r0 + cl] = x;
        }
      }
    } else {
      constexpr int CT = DV / 16;             // column tiles
      constexpr int JOBS_PER_X = 2 * CT;      // (C/16) row tiles x CT
      const int nx = has_noisy ? 4 : 2;
      for (int job = wave - 1; job < nx * JOBS_PER_X; job += NW - 1) {
        const int xsel = job / JOBS_PER_X;    // 0 K, 1 Q, 2 K~, 3 Q~
        const int jr = job % JOBS_PER_X;
        const int tr = jr / CT, tc = jr % CT;
        const int xm = xsel == 0 ? 1 : xsel == 1 ? 0 : xsel == 2 ? 3 : 2;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) mm_u16<D>(acc, &sm.x[xm][0][0], LDX, 16 * tr, &sm.st[0][0], LDX, 16 * tc);
        else mm_f32<D>(acc, &sm.x[xm][0][0], LDX, 16 * tr, &sm.st[0][0], LDX, 16 * tc);
        // acc[r] = (X S)[tok][dv], tok = 16 tr + acc_row(r), dv = 16 tc + acc_col()
        const int dv = 16 * tc + acc_col();
        const int tok0 = 16 * tr + acc_row(0);
        float out4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = tok0 + r;
          const float xs = acc[r] * sm.nrm[xm][tok];
          if (xsel == 0) {
            out4[r] = sm.v[0][tok][dv] - fast_exp(sm.lg[tok]) * xs;
          } else if (xsel == 1) {
            out4[r] = xs;
          } else {
            const int pt = tok - (tok % B);
            out4[r] = (pt > 0 ? fast_exp(sm.lg[pt - 1]) : 1.f) * xs;
          }
        }
        const int vt = xsel == 0 ? VT_RHS : xsel == 1 ? VT_QS : xsel == 2 ? VT_RK : VT_RQ;
        *reinterpret_cast<float4 *>(&sm.vt[vt][dv][tok0]) = make_float4(out4[0], out4[1], out4[2], out4[3]);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- [D] off-diagonal block T_10 = -T_11 A_10 T_00
    {
      const int nm = (has_noisy && B > 16) ? 2 : 1;
      for (int e = tid; e < nm * 256; e += NT) {
        const int m = e >> 8, ii = (e >> 4) & 15, cl = e & 15;
        const float(*Am)[LDM] = sm.cc[m ? CC_AN : CC_A];
        const float(*Tm)[LDM] = sm.cc[m ? CC_TN : CC_T];
        float acc = 0.f;
        for (int mm = cl; mm < 16; ++mm) acc += Am[16 + ii][mm] * Tm[mm][cl];
        sm.tmp[m][ii][cl] = acc;
      }
      __syncthreads();
      for (int e = tid; e < nm * 256; e += NT) {
        const int m = e >> 8, ii = (e >> 4) & 15, cl = e & 15;
        float(*Tm)[LDM] = sm.cc[m ? CC_TN : CC_T];
        float acc = 0.f;
        for (int mm = 0; mm <= ii; ++mm) acc += Tm[16 + ii][16 + mm] * sm.tmp[m][mm][cl];
        Tm[16 + ii][cl] = -acc;
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- [E] U = T rhs, DU
    {
      constexpr int CT = DV / 16;
      const float lgC = sm.lg[C - 1];
      for (int job = wave; job < 2 * CT; job += NW) {
        const int tr = job / CT, tc = job % CT;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        mm_ff<BF, C, 2>(acc, &sm.cc[CC_T][0][0], LDM, 16 * tr, &sm.vt[VT_RHS][0][0], LDM, 16 * tc);
        const int dv = 16 * tc + acc_col();
        const int i0 = 16 * tr + acc_row(0);
        float du[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          du[r] = acc[r] * sm.beta[i] * fast_exp(lgC - sm.lg[i]) * sm.nrm[1][i];
        }
        *reinterpret_cast<float4 *>(&sm.vt[VT_U][dv][i0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4 *>(&sm.vt[VT_DU][dv][i0]) = make_float4(du[0], du[1], du[2], du[3]);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- [F] outputs, noisy reads, state update
    {
      constexpr int CT = DV / 16;
      const int njobs = 2 * CT * (has_noisy ? 3 : 1);
      for (int job = wave; job < njobs; job += NW) {
        const int kind = job / (2 * CT);  // 0 o, 1 r_q, 2 r_k
        const int jr = job % (2 * CT);
        const int tr = jr / CT, tc = jr % CT;
        const int dv = 16 * tc + acc_col();
        const int i0 = 16 * tr + acc_row(0);
        const int src = kind == 0 ? VT_QS : kind == 1 ? VT_RQ : VT_RK;
        const float4 init = *reinterpret_cast<const float4 *>(&sm.vt[src][dv][i0]);
        floatx4 acc = {init.x, init.y, init.z, init.w};
        if (kind == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= fast_exp(sm.lg[i0 + r]);
        }
        const int cc = kind == 0 ? CC_MO : kind == 1 ? CC_MQ : CC_MK;
        mm_ff<BF, C, 3>(acc, &sm.cc[cc][0][0], LDM, 16 * tr, &sm.vt[VT_U][0][0], LDM, 16 * tc);
        if (kind == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.out[0][i0 + r][dv] = io_traits<IO>::from_f(scale * acc[r]);
        } else if (kind == 1) {
          *reinterpret_cast<float4 *>(&sm.vt[VT_RQ][dv][i0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = sm.v[1][i0 + r][dv] - fast_exp(sm.lgn[i0 + r]) * acc[r];
          *reinterpret_cast<float4 *>(&sm.vt[VT_RK][dv][i0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
      }
      // state update on the wave's own tiles: S <- G_C S + K^T (DU)
      const float gC = fast_exp(sm.lg[C - 1]);
#pragma unroll
      for (int e = 0; e < SPW; ++e) {
        const int q = wave * SPW + e;
        if (q < NST) {
          const int rt = q / (DV / 16), ct = q % (DV / 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[e][r] *= gC;
          if constexpr (BF) {
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += 32)
              mma_bf16(S[e], frag_bf16_T(&sm.x[1][0][0], LDX, 16 * rt, k0),
                       frag_f32_hi(&sm.vt[VT_DU][0][0], LDM, 16 * ct, k0));
          } else {
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += 4)
              mma_f32(S[e], frag1_f32_T(&sm.x[1][0][0], LDX, 16 * rt, k0),
                      frag1_f32(&sm.vt[VT_DU][0][0], LDM, 16 * ct, k0));
          }
        }
      }
      write_state_t();
    }
    __syncthreads();

    if (has_noisy) {
      // -------------------------------------------------------- [G] u~ = T~ rhs~
      constexpr int CT = DV / 16;
      for (int job = wave; job < 2 * CT; job += NW) {
        const int tr = job / CT, tc = job % CT;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        mm_ff<BF, C, 2>(acc, &sm.cc[CC_TN][0][0], LDM, 16 * tr, &sm.vt[VT_RK][0][0], LDM, 16 * tc);
        const int dv = 16 * tc + acc_col();
        const int i0 = 16 * tr + acc_row(0);
        *reinterpret_cast<float4 *>(&sm.vt[VT_UN][dv][i0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
      __syncthreads();
      // -------------------------------------------------------- [H] o~ = s (G~_e r_q + M~ u~)
      for (int job = wave; job < 2 * CT; job += NW) {
        const int tr = job / CT, tc = job % CT;
        const int dv = 16 * tc + acc_col();
        const int i0 = 16 * tr + acc_row(0);
        const float4 init = *reinterpret_cast<const float4 *>(&sm.vt[VT_RQ][dv][i0]);
        floatx4 acc = {init.x, init.y, init.z, init.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          const int pi = i - (i % B);
          acc[r] *= fast_exp(sm.lgn[pi + B - 1]);
        }
        mm_ff<BF, C, 3>(acc, &sm.cc[CC_MN][0][0], LDM, 16 * tr, &sm.vt[VT_UN][0][0], LDM, 16 * tc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tpos = c0 + i0 + r;
          const bool resp = tpos < n && tpos >= P;
          sm.out[1][i0 + r][dv] = io_traits<IO>::from_f(resp ? scale * acc[r] : 0.f);
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- [I] write o, o~
    {
      constexpr int UPR = DV * Cfg::ES / 16;  // 16-byte units per row
      IO *go[2] = {reinterpret_cast<IO *>(a.o), reinterpret_cast<IO *>(a.on)};
      for (int e = tid; e < 2 * C * UPR; e += NT) {
        const int m = e / (C * UPR), rr = e % (C * UPR);
        const int row = rr / UPR, cu16 = rr % UPR;
        const int tpos = c0 + row;
        if (tpos >= n) continue;
        uint4 val = *reinterpret_cast<const uint4 *>(&sm.out[m][row][cu16 * (16 / Cfg::ES)]);
        if (m == 1 && !has_noisy) val = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4 *>(go[m] + ((t0g + tpos) * H + h) * D + dv0 + cu16 * (16 / Cfg::ES)) = val;
      }
    }
  }

  if (a.h_final) write_state_global(a.h_final + ((size_t)doc * H + h) * D * D);
}

template <typename IO, int D>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t st) {
  using Cfg = FwdCfg<IO, D>;
  const int pairs = a.num_docs * a.H;
  const int groups = (pairs + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * Cfg::NTILE));
  hipLaunchKernelGGL((gdn_dual_fwd_kernel<IO, D>), grid, dim3(Cfg::NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gdn_fwd(const FwdArgs &a, hipStream_t st) {
  if (a.num_docs == 0) return hipSuccess;
  // fp32 io is instantiated at d = 16 only (the fp32 tiles at d = 128 exceed the LDS budget)
  if (a.bf16) return a.D == 128 ? launch_fwd_t<u16, 128>(a, st) : launch_fwd_t<u16, 16>(a, st);
  return a.D == 16 ? launch_fwd_t<float, 16>(a, st) : hipErrorInvalidValue;
}

}  // namespace flare
