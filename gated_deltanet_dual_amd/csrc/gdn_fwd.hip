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
//   is computed.  The waves are specialised so that each dependency chain of a
//   chunk stays inside one wave (LDS traffic of one wave is ordered, so it needs
//   no barrier) and the chunk needs four workgroup barriers:
//     wave 0: A Gram -> T solve ; K S_c -> rhs -> U, DU      (clean chain)
//     wave 1: Mo Gram ; Q S_c (registers) -> o
//     wave 2: Mq, M~ Grams ; q~ S_c (registers) -> r_q -> o~
//     wave 3: Mk, A~ Grams -> T~ solve ; k~ S_c -> r_k -> rhs~ -> u~
//   and every wave updates its quarter of the state with K^T DU.
//   Per chunk, with G_i = exp(cumulative log a) inside the chunk:
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

#include "chunk_common.h"
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

template <typename IO, int D> struct FwdCfg {
  static constexpr bool BF = std::is_same<IO, u16>::value;
  static constexpr int C = 32;                 // chunk
  static constexpr int NW = 4;                 // waves
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int DV = D >= 32 ? 32 : D;  // d_v columns per workgroup
  static constexpr int NTILE = D / DV;
  static constexpr int CT = DV / 16;           // 16-column tiles of d_v
  static constexpr int LDX = D + 8;            // q/k tile pitch (elements)
  static constexpr int LDM = C + 4;            // C x C and [DV][C] fp32 pitch
  static constexpr int LDV = DV + 4;           // value tile pitch (fp32)
  static constexpr int ES = sizeof(IO);
  static constexpr int PU = C * D * ES / 16;   // 16-byte units per q/k tile
  static constexpr int RU = D * ES / 16;       // units per q/k row
  static constexpr int UX = 4 * PU / NT;       // q/k units per thread
  static constexpr int PV = C * DV * ES / 16;  // units per value tile
  static constexpr int RV = DV * ES / 16;      // units per value row
  static constexpr int NST = (D / 16) * CT;    // 16x16 state tiles
  static constexpr int SPW = (NST + NW - 1) / NW;  // state tiles per wave
  static_assert(4 * PU % NT == 0, "q/k tile units must divide the threads");
  static_assert(2 * PV <= NT, "at most one value unit per thread");
};

template <typename IO, int D> struct FwdSmem {
  using Cfg = FwdCfg<IO, D>;
  static constexpr int C = Cfg::C, DV = Cfg::DV, LDX = Cfg::LDX, LDM = Cfg::LDM, LDV = Cfg::LDV;
  using ST = typename std::conditional<Cfg::BF, u16, float>::type;  // S^T storage
  alignas(16) IO x[4][C][LDX];      // 0 q, 1 k, 2 q~, 3 k~
  alignas(16) ST st[DV][LDX];       // S_c^T (bf16 hi, or fp32)
  alignas(16) float v[2][C][LDV];   // v, v~ tiles (fp32)
  alignas(16) float cc[8][C][LDM];  // A^T, T, Mo, Mq, Mk, A~^T, T~, M~
  alignas(16) float vt[5][DV][LDM]; // rhs^T, U^T, DU^T, rhs~^T, u~^T
  alignas(16) float tmp[2][16][17]; // off-diagonal block solve scratch
  alignas(16) IO out[2][C][DV];     // o, o~ staging
  alignas(16) float lg[C];          // cumulative log a inside the chunk
  alignas(16) float beta[C];
  alignas(16) float lgn[C];         // cumulative log a~ inside each noisy block
  alignas(16) float betan[C];
  alignas(16) float nrm[4][C];      // 1/|x| per row (1 without the L2 flag)
};

enum { CC_AT = 0, CC_T, CC_MO, CC_MQ, CC_MK, CC_ANT, CC_TN, CC_MN };
enum { VT_RHS = 0, VT_U, VT_DU, VT_RHSN, VT_UN };

// ------------------------------------------------------------------ products
// Register-cached row fragments of a 32-row (or DV-row) LDS tile over a K-deep
// contraction: f[h][ks] covers rows 16h..16h+15 and k-step ks.
template <bool BF, int K, int NH> struct Frags {
  static constexpr int KS = BF ? (K >= 32 ? K / 32 : 1) : K / 4;
  using F = typename std::conditional<BF, bf16x8, float>::type;
  F f[NH][KS];
};

template <bool BF, int K, int NH, typename T>
__device__ __forceinline__ void load_frags(Frags<BF, K, NH> &fr, const T *base, int ld) {
  using FR = Frags<BF, K, NH>;
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ks = 0; ks < FR::KS; ++ks) {
      if constexpr (BF) {
        if constexpr (K >= 32) {
          fr.f[h][ks] = frag_bf16(reinterpret_cast<const u16 *>(base), ld, 16 * h, 32 * ks);
        } else {
          // a 16-deep contraction: lanes 32..63 carry k = 16..31 and must be zero
          const bf16x8 z = as_bf16x8(u16x8{});
          fr.f[h][ks] = lane_id() < 32 ? frag_bf16(reinterpret_cast<const u16 *>(base), ld, 16 * h, 0) : z;
        }
      } else {
        fr.f[h][ks] = frag1_f32(reinterpret_cast<const float *>(base), ld, 16 * h, 4 * ks);
      }
    }
}

// acc[i][j] += sum_k a[ha][i][k] * b[hb][j][k]
template <bool BF, int K, int NA, int NB>
__device__ __forceinline__ void mma_frags(floatx4 &acc, const Frags<BF, K, NA> &a, int ha,
                                          const Frags<BF, K, NB> &b, int hb) {
#pragma unroll
  for (int ks = 0; ks < Frags<BF, K, NA>::KS; ++ks) {
    if constexpr (BF) mma_bf16(acc, a.f[ha][ks], b.f[hb][ks]);
    else mma_f32(acc, a.f[ha][ks], b.f[hb][ks]);
  }
}

// Products of two fp32 LDS matrices, acc[i][j] += sum_k A[ra+i][k] Bt[rb+j][k].
template <int K>
__device__ __forceinline__ void mm_f32(floatx4 &acc, const float *A, int lda, int ra, const float *Bt,
                                       int ldb, int rb) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4) mma_f32(acc, frag1_f32(A, lda, ra, k0), frag1_f32(Bt, ldb, rb, k0));
}
// A -> bf16 hi, Bt -> hi + lo   (2 MFMA per k-step)
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
// A, Bt -> hi + lo each; hi*hi + hi*lo + lo*hi   (3 MFMA per k-step)
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
  constexpr int C = Cfg::C, NT = Cfg::NT, DV = Cfg::DV, NTILE = Cfg::NTILE, CT = Cfg::CT;
  constexpr int LDX = Cfg::LDX, LDM = Cfg::LDM;
  constexpr int SPW = Cfg::SPW, NST = Cfg::NST;
  using ST = typename Sm::ST;
  using XF = Frags<BF, D, 2>;   // 32 rows of q/k/q~/k~ over d_k
  using SF = Frags<BF, D, CT>;  // DV rows of S^T over d_k

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
  const int B = a.B;  // a power of two up to 32 (checked by the host): i % B = i & (B - 1)
  const int nchunks = (n + C - 1) / C;
  const int dv0 = tile * DV;
  const float scale = a.scale;
  const bool l2 = (a.flags & 1) != 0;

  // Input pointers copied to (uniform) locals first: selecting among them per
  // lane is then a register select, not a per-lane load from the argument block.
  const IO *const pq = reinterpret_cast<const IO *>(a.q), *const pk = reinterpret_cast<const IO *>(a.k);
  const IO *const pqn = reinterpret_cast<const IO *>(a.qn), *const pkn = reinterpret_cast<const IO *>(a.kn);
  const IO *const pv = reinterpret_cast<const IO *>(a.v), *const pvn = reinterpret_cast<const IO *>(a.vn);
  const float *const pa = a.alpha, *const pb = a.beta, *const pan = a.alpha_n, *const pbn = a.beta_n;
  auto gx = [=](int m) { return m == 0 ? pq : m == 1 ? pk : m == 2 ? pqn : pkn; };
  auto gv = [=](int m) { return m == 0 ? pv : pvn; };
  auto gg = [=](int g) { return g == 0 ? pa : g == 1 ? pb : g == 2 ? pan : pbn; };

  // ---- one-time LDS init: zero all C x C matrices (blocks never written stay zero)
  for (int e = tid; e < 8 * C * LDM; e += NT) (&sm.cc[0][0][0])[e] = 0.f;
  for (int e = tid; e < 4 * C; e += NT) (&sm.nrm[0][0])[e] = 1.f;

  // ---- state tiles owned by this wave: tile q -> rows 16*(q / CT), cols 16*(q % CT)
  floatx4 S[SPW];
#pragma unroll
  for (int e = 0; e < SPW; ++e) {
    const int q = wave * SPW + e;
    S[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (q < NST && a.h0) {
      const int rt = q / CT, ct = q % CT;
      const float *src = a.h0 + ((size_t)(a.state_slot ? a.state_slot[doc] : doc) * H + h) * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[e][r] = src[(size_t)(16 * rt + acc_row(r)) * D + dv0 + 16 * ct + acc_col()];
    }
  }
  auto write_state_t = [&]() {  // S -> st (S^T, bf16 hi or fp32)
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int q = wave * SPW + e;
      if (q < NST) {
        const int rt = q / CT, ct = q % CT;
        ST *dst = &sm.st[16 * ct + acc_col()][16 * rt + acc_row(0)];
        if constexpr (BF) {
          uint2 w;
          w.x = pack_bf16x2(S[e][0], S[e][1]);
          w.y = pack_bf16x2(S[e][2], S[e][3]);
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
        const int rt = q / CT, ct = q % CT;
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
        pfx[e] = *reinterpret_cast<const uint4 *>(gx(m) + ((t0g + tpos) * H + h) * D + cu16 * (16 / Cfg::ES));
    }
    if (tid < 2 * Cfg::PV) {
      const int m = tid / Cfg::PV, r = tid % Cfg::PV;
      const int row = r / Cfg::RV, cu16 = r % Cfg::RV;
      const int tpos = c0 + row;
      bool ok = tpos < n;
      if (m == 1) ok = ok && tpos >= P;
      pfv = make_uint4(0u, 0u, 0u, 0u);
      if (ok)
        pfv = *reinterpret_cast<const uint4 *>(gv(m) + ((t0g + tpos) * H + h) * D + dv0 + cu16 * (16 / Cfg::ES));
    }
    if (tid < 4 * C) {
      const int g = tid / C, i = tid % C;
      const int tpos = c0 + i;
      bool ok = tpos < n;
      if (g >= 2) ok = ok && tpos >= P;
      pfg = (g & 1) == 0 ? 1.f : 0.f;
      if (ok) pfg = gg(g)[(t0g + tpos) * H + h];
    }
  };
  // prefetch registers -> LDS; the gates are scanned straight from registers:
  // wave 0 lanes 0..31 hold alpha, 32..63 beta; wave 1 the noisy pair.
  auto store_prefetch = [&]() {
#pragma unroll
    for (int e = 0; e < Cfg::UX; ++e) {
      const int u = e * NT + tid;
      const int m = u / Cfg::PU, r = u % Cfg::PU;
      const int row = r / Cfg::RU, cu16 = r % Cfg::RU;
      *reinterpret_cast<uint4 *>(&sm.x[m][row][cu16 * (16 / Cfg::ES)]) = pfx[e];
      if (l2) {
        // sum of squares of this 16-byte unit, reduced over the RU lanes of the row
        const uint32_t w[4] = {pfx[e].x, pfx[e].y, pfx[e].z, pfx[e].w};
        float ss = 0.f;
        if constexpr (BF) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
            ss += lo * lo + hi * hi;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) ss += __uint_as_float(w[i]) * __uint_as_float(w[i]);
        }
#pragma unroll
        for (int off = 1; off < Cfg::RU; off <<= 1) ss += __shfl_xor(ss, off, 64);
        if (cu16 == 0) sm.nrm[m][row] = rsqrtf(ss + 1e-6f);
      }
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
    if (tid < 4 * C) {
      const int g = tid / C, i = tid % C;
      if (g == 0 || g == 2) {
        float la = __logf(pfg);
        if (g == 0) {
#pragma unroll
          for (int off = 1; off < C; off <<= 1) {
            const float y = __shfl_up(la, off, C);
            if (i >= off) la += y;
          }
          sm.lg[i] = la;
        } else {
          // segmented scan inside blocks of B tokens (blocks are B-aligned in the chunk)
          for (int off = 1; off < B; off <<= 1) {
            const float y = __shfl_up(la, off, B);
            if ((i & (B - 1)) >= off) la += y;
          }
          sm.lgn[i] = la;
        }
      } else {
        (g == 1 ? sm.beta : sm.betan)[i] = pfg;
      }
    }
  };
  // staged o, o~ rows of chunk cprev -> global (16-byte stores)
  auto store_outputs = [&](int cprev, bool noisy_prev) {
    constexpr int UPR = DV * Cfg::ES / 16;  // 16-byte units per row
    IO *go[2] = {reinterpret_cast<IO *>(a.o), reinterpret_cast<IO *>(a.on)};
    for (int e = tid; e < 2 * C * UPR; e += NT) {
      const int m = e / (C * UPR), rr = e % (C * UPR);
      const int row = rr / UPR, cu16 = rr % UPR;
      const int tpos = cprev * C + row;
      if (tpos >= n) continue;
      uint4 val = *reinterpret_cast<const uint4 *>(&sm.out[m][row][cu16 * (16 / Cfg::ES)]);
      if (m == 1 && !noisy_prev) val = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4 *>(go[m] + ((t0g + tpos) * H + h) * D + dv0 + cu16 * (16 / Cfg::ES)) = val;
    }
  };

  if (nchunks > 0) prefetch(0);
  const int64_t ck_base = a.ckpt ? (int64_t)(t0g / ((int64_t)C * a.ckpt_stride)) + doc : 0;
  bool prev_noisy = false;

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * C;
    const bool has_noisy = (c0 + C > P) && (P < n);

    // ============================================================ [A] inputs
    lds_barrier();                                       // B0
    if (c > 0) store_outputs(c - 1, prev_noisy);
    store_prefetch();
    if (c + 1 < nchunks) prefetch(c + 1);
    if (a.ckpt && (c % a.ckpt_stride) == 0)
      write_state_global(a.ckpt + ((ck_base + c / a.ckpt_stride) * H + h) * (size_t)D * D);
    lds_barrier();                                       // B1

    // ============================================================ [P1] Grams, X S_c, solves
    // Floating-point io helpers for the row-side factors used in the epilogues.
    const int g4 = 4 * (lane >> 4);  // accumulator row offset of this lane
    const int cl = lane & 15;        // accumulator column of this lane
    floatx4 xs[2][CT];               // q S_c (wave 1), q~ S_c -> r_q (wave 2), k~ S_c -> r_k (wave 3)
    if (wave == 0) {
      XF kf;
      SF sf;
      load_frags(kf, &sm.x[1][0][0], LDX);
      load_frags(sf, &sm.st[0][0], LDX);
      // A^T: non-transposed Gram tiles G[i = 16ti + g4 + r][j = 16tj + cl] of K K^T
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        mma_frags(acc, kf, ti, kf, tj);
        const int j = 16 * tj + cl;
        const float lgj = sm.lg[j], bj = sm.beta[j] * sm.nrm[1][j];
        float o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ti + g4 + r;
          o4[r] = j < i ? acc[r] * sm.nrm[1][i] * fast_exp(sm.lg[i] - lgj) * bj : 0.f;
        }
        *reinterpret_cast<float4 *>(&sm.cc[CC_AT][j][16 * ti + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
      // rhs = V - diag(G) K S_c  ->  rhs^T
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mma_frags(acc, kf, tr, sf, tc);
          const int dv = 16 * tc + cl;
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tr + g4 + r;
            o4[r] = sm.v[0][tok][dv] - fast_exp(sm.lg[tok]) * sm.nrm[1][tok] * acc[r];
          }
          *reinterpret_cast<float4 *>(&sm.vt[VT_RHS][dv][16 * tr + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
      solve_unit_lower<LDM>(&sm.cc[CC_AT][0][0], &sm.cc[CC_T][0][0], &sm.tmp[0][0][0], true);
      // U = T rhs ; DU = diag(b G_C / G) U (the K row norm folded in)
      const float lgC = sm.lg[C - 1];
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mm_ff<BF, C, 2>(acc, &sm.cc[CC_T][0][0], LDM, 16 * tr, &sm.vt[VT_RHS][0][0], LDM, 16 * tc);
          const int dv = 16 * tc + cl, i0 = 16 * tr + g4;
          float du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            du[r] = acc[r] * sm.beta[i0 + r] * fast_exp(lgC - sm.lg[i0 + r]) * sm.nrm[1][i0 + r];
          *reinterpret_cast<float4 *>(&sm.vt[VT_U][dv][i0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
          *reinterpret_cast<float4 *>(&sm.vt[VT_DU][dv][i0]) = make_float4(du[0], du[1], du[2], du[3]);
        }
    } else if (wave == 1) {
      XF kf, qf;
      SF sf;
      load_frags(kf, &sm.x[1][0][0], LDX);
      load_frags(qf, &sm.x[0][0][0], LDX);
      load_frags(sf, &sm.st[0][0], LDX);
      // Mo[i][j] = (q_i.k_j) G_i/G_j b_j, j <= i  (transposed Gram tiles: lane holds Mo[i][j0..j0+3])
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        mma_frags(acc, kf, tj, qf, ti);
        const int i = 16 * ti + cl, j0 = 16 * tj + g4;
        const float lgi = sm.lg[i], ni = sm.nrm[0][i];
        float o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + r;
          o4[r] = j <= i ? acc[r] * ni * sm.nrm[1][j] * fast_exp(lgi - sm.lg[j]) * sm.beta[j] : 0.f;
        }
        *reinterpret_cast<float4 *>(&sm.cc[CC_MO][i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mma_frags(acc, qf, tr, sf, tc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tr + g4 + r;
            acc[r] *= sm.nrm[0][tok] * fast_exp(sm.lg[tok]);
          }
          xs[tr][tc] = acc;
        }
    } else if (has_noisy) {
      // waves 2 (q~ side) and 3 (k~ side)
      const bool qside = wave == 2;
      const int xm = qside ? 2 : 3;
      XF kf, xf, knf;
      SF sf;
      load_frags(kf, &sm.x[1][0][0], LDX);
      load_frags(xf, &sm.x[xm][0][0], LDX);
      load_frags(sf, &sm.st[0][0], LDX);
      if (qside) load_frags(knf, &sm.x[3][0][0], LDX);
      // Mq / Mk[i][j] = (x~_i.k_j) (G_p(i)/G_j) b_j for j < p(i), x~ in {q~, k~}
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int ti = t == 0 ? 0 : 1, tj = t == 2 ? 1 : 0;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        mma_frags(acc, kf, tj, xf, ti);
        const int i = 16 * ti + cl, j0 = 16 * tj + g4;
        const int pi = (i & -B);
        const bool resp = c0 + i < n && c0 + i >= P;
        const float lgp = pi > 0 ? sm.lg[pi - 1] : 0.f;
        const float ni = sm.nrm[xm][i];
        float o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + r;
          o4[r] = (resp && j < pi) ? acc[r] * ni * sm.nrm[1][j] * fast_exp(lgp - sm.lg[j]) * sm.beta[j] : 0.f;
        }
        *reinterpret_cast<float4 *>(&sm.cc[qside ? CC_MQ : CC_MK][i][j0]) =
            make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
      if (qside) {
        // M~[i][j] = (q~_i.k~_j) (G~_e/G~_j) b~_j for j in i's block (transposed Gram tiles)
        const int nt = B > 16 ? 4 : 2;
#pragma unroll
        for (int t = 0; t < 4; ++t) {  // tiles (0,0), (1,1), then (0,1), (1,0) when B > 16
          if (t >= nt) break;
          const int ti = (t == 0 || t == 2) ? 0 : 1, tj = (t == 0 || t == 3) ? 0 : 1;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mma_frags(acc, knf, tj, xf, ti);
          const int i = 16 * ti + cl, j0 = 16 * tj + g4;
          const int pi = (i & -B);
          const bool resp = c0 + i < n && c0 + i >= P;
          const float lge = sm.lgn[pi + B - 1], ni = sm.nrm[2][i];
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            o4[r] = (resp && j >= pi && j < pi + B)
                        ? acc[r] * ni * sm.nrm[3][j] * fast_exp(lge - sm.lgn[j]) * sm.betan[j] : 0.f;
          }
          *reinterpret_cast<float4 *>(&sm.cc[CC_MN][i][j0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
      } else {
        // A~^T: non-transposed Gram tiles of K~ K~^T inside blocks, then T~ = (I + A~)^-1
        const int nt = B > 16 ? 3 : 2;
#pragma unroll
        for (int t = 0; t < 3; ++t) {  // tiles (0,0), (1,1), then (1,0) when B > 16
          if (t >= nt) break;
          const int ti = t == 0 ? 0 : 1, tj = t == 1 ? 1 : 0;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mma_frags(acc, xf, ti, xf, tj);
          const int j = 16 * tj + cl;
          const int pj = (j & -B);
          const float lgj = sm.lgn[j], bj = sm.betan[j] * sm.nrm[3][j];
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + g4 + r;
            const bool resp = c0 + i < n && c0 + i >= P;
            o4[r] = (resp && j < i && (i & -B) == pj) ? acc[r] * sm.nrm[3][i] * fast_exp(sm.lgn[i] - lgj) * bj : 0.f;
          }
          *reinterpret_cast<float4 *>(&sm.cc[CC_ANT][j][16 * ti + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
        solve_unit_lower<LDM>(&sm.cc[CC_ANT][0][0], &sm.cc[CC_TN][0][0], &sm.tmp[1][0][0], B > 16);
      }
      // x~ S_c, scaled by G_p: the S_c part of S_p^T x~
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mma_frags(acc, xf, tr, sf, tc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tr + g4 + r;
            const int pt = (tok & -B);
            acc[r] *= sm.nrm[xm][tok] * (pt > 0 ? fast_exp(sm.lg[pt - 1]) : 1.f);
          }
          xs[tr][tc] = acc;
        }
    }
    lds_barrier();                                       // B2

    // ============================================================ [P2] state, o, r_q, r_k -> u~
    {
      const float gC = fast_exp(sm.lg[C - 1]);
#pragma unroll
      for (int e = 0; e < SPW; ++e) {
        const int q = wave * SPW + e;
        if (q < NST) {
          const int rt = q / CT, ct = q % CT;
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
    if (wave == 1) {
      // o = s (G q S_c + Mo U)
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = xs[tr][tc];
          mm_ff<BF, C, 3>(acc, &sm.cc[CC_MO][0][0], LDM, 16 * tr, &sm.vt[VT_U][0][0], LDM, 16 * tc);
          const int dv = 16 * tc + cl;
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.out[0][16 * tr + g4 + r][dv] = io_traits<IO>::from_f(scale * acc[r]);
        }
    } else if (has_noisy && wave == 2) {
      // r_q = S_p^T q~ = G_p q~ S_c + Mq U   (kept in registers for [P3])
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc)
          mm_ff<BF, C, 3>(xs[tr][tc], &sm.cc[CC_MQ][0][0], LDM, 16 * tr, &sm.vt[VT_U][0][0], LDM, 16 * tc);
    } else if (has_noisy && wave == 3) {
      // r_k = S_p^T k~ ; rhs~ = v~ - diag(G~) r_k ; u~ = T~ rhs~
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = xs[tr][tc];
          mm_ff<BF, C, 3>(acc, &sm.cc[CC_MK][0][0], LDM, 16 * tr, &sm.vt[VT_U][0][0], LDM, 16 * tc);
          const int dv = 16 * tc + cl;
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tr + g4 + r;
            o4[r] = sm.v[1][tok][dv] - fast_exp(sm.lgn[tok]) * acc[r];
          }
          *reinterpret_cast<float4 *>(&sm.vt[VT_RHSN][dv][16 * tr + g4]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          mm_ff<BF, C, 2>(acc, &sm.cc[CC_TN][0][0], LDM, 16 * tr, &sm.vt[VT_RHSN][0][0], LDM, 16 * tc);
          *reinterpret_cast<float4 *>(&sm.vt[VT_UN][16 * tc + cl][16 * tr + g4]) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
    lds_barrier();                                       // B3

    // ============================================================ [P3] o~ = s (G~_e r_q + M~ u~)
    if (has_noisy && wave == 2) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = xs[tr][tc];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * tr + g4 + r;
            acc[r] *= fast_exp(sm.lgn[(i & -B) + B - 1]);
          }
          mm_ff<BF, C, 3>(acc, &sm.cc[CC_MN][0][0], LDM, 16 * tr, &sm.vt[VT_UN][0][0], LDM, 16 * tc);
          const int dv = 16 * tc + cl;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * tr + g4 + r;
            const bool resp = c0 + i < n && c0 + i >= P;
            sm.out[1][i][dv] = io_traits<IO>::from_f(resp ? scale * acc[r] : 0.f);
          }
        }
    }
    prev_noisy = has_noisy;
  }
  if (nchunks > 0) {
    lds_barrier();
    store_outputs(nchunks - 1, prev_noisy);
  }
  if (a.h_final)
    write_state_global(a.h_final + ((size_t)(a.state_slot ? a.state_slot[doc] : doc) * H + h) * D * D);
}

template <typename IO, int D>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t st) {
  using Cfg = FwdCfg<IO, D>;
  const int pairs = a.num_docs * a.H;
  const int groups = (pairs + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * Cfg::NTILE));
  TimedLaunch tl(K_FWD, st);
  hipLaunchKernelGGL((gdn_dual_fwd_kernel<IO, D>), grid, dim3(Cfg::NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gdn_fwd(const FwdArgs &a_in, hipStream_t st, const FwdPlan *plan) {
  if (a_in.num_docs == 0) return hipSuccess;
  FwdArgs a = a_in;
  if (a.workspace) {
    // bf16, d = 128: per pass (the whole batch, or one window of chunks of
    // every document) the chunk matrices and the scan hand-over in one
    // parallel pass (gdn_fwd_prep.hip),
    // the state recurrence (chunk-start states -> the checkpoints or the
    // workspace; strided checkpoints besides), then the outputs in parallel;
    // with the q/k L2 flag first the per-row factors the kernels fold in
    // (gdn_l2.hip)
    FwdPlan p{};
    if (plan) {
      p = *plan;
    } else {  // one pass over the workspace in its one-pass layout
      p.slots = a.T / kChunk + a.num_docs;
      const size_t per = (size_t)p.slots * a.H;
      p.cmat = a.workspace;
      p.pack = p.cmat + per * 6 * kChunk * kChunk;
      p.states = a.ckpt && a.ckpt_stride == 1 ? nullptr : p.pack + per * kScanPackFloats;
      const size_t per_bytes = per * (6 * kChunk * kChunk + kScanPackFloats + (size_t)a.D * a.D) * 4;
      p.l2f = reinterpret_cast<float4 *>(reinterpret_cast<char *>(a.workspace) + ((per_bytes + 255) & ~(size_t)255));
    }
    if (a.flags & 1) {
      if (a.cw == 0) {  // with the conv loads the preparation pass forms them
        hipError_t e = launch_l2_factors(a, p.l2f, st);
        if (e != hipSuccess) return e;
      }
      a.l2f = p.l2f;
    }
    float *const states = p.states ? p.states : a.ckpt;
    const bool ckpt_apart = a.ckpt && states != a.ckpt;  // checkpoints written besides the states
    const int nwin = p.win > 0 ? max(1, (p.max_chunks + p.win - 1) / p.win) : 1;
    for (int w = 0; w < nwin; ++w) {
      FwdArgs aw = a;
      aw.win_lo = p.win > 0 ? w * p.win : 0;
      aw.win_len = p.win;
      {
        TimedLaunch tl(K_FWD_PREP, st);
        hipError_t e = launch_fwd_prep_d128(aw, p.cmat, p.pack, st, p.slots);
        if (e != hipSuccess) return e;
      }
      {
        ScanArgs sa{};
        sa.num_docs = a.num_docs;
        sa.H = a.H;
        sa.cu = a.cu;
        sa.pack = p.pack;
        sa.init = w == 0 ? a.h0 : p.carry;
        sa.final_out = w == nwin - 1 ? a.h_final : p.carry;
        sa.slot = a.state_slot;
        sa.states = states;
        if (ckpt_apart) {
          sa.ckpt = a.ckpt;
          sa.ckpt_stride = a.ckpt_stride;
        }
        TimedLaunch tl(K_FWD_SCAN, st);
        hipError_t e;
        if (p.win > 0) {
          sa.win_lo = aw.win_lo;
          sa.win_len = p.win;
          sa.units = a.num_docs;
          e = launch_scan_d128(sa, false, st);
        } else {
          e = scan_d128_runs(sa, false, a.scan_span, a.scan_units, a.scan_ws, st);
        }
        if (e != hipSuccess) return e;
      }
      TimedLaunch tl(K_FWD, st);
      hipError_t e = launch_fwd_out_d128(aw, p.cmat, states, st, p.slots);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // fp32 io is instantiated at d = 16 only (the fp32 tiles at d = 128 exceed the LDS budget)
  if (a.bf16) return a.D == 128 ? launch_fwd_t<u16, 128>(a, st) : launch_fwd_t<u16, 16>(a, st);
  return a.D == 16 ? launch_fwd_t<float, 16>(a, st) : hipErrorInvalidValue;
}

}  // namespace flare
