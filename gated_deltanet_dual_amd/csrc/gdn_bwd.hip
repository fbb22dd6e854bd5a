// gdn_bwd.hip -- reverse mode of the fused dual-stream Gated DeltaNet forward.
//
// Method ("FLARE: Diffusion for Hybrid Language Model", papernotes.org notes,
// Key designs items 2 and 3): the gradient of every noisy block flows into the
// clean causal chain at the block's boundary, documents are independent, and
// only strided clean checkpoints are kept from the forward.
//
// Chunk algebra (per chunk of C tokens, start state S_c, end-state adjoint dS'):
//   forward  rhs = V - diag(G) K S_c,  U = T rhs,  o = s (diag(G) Q S_c + Mo U),
//            r_q = G_p q~ S_c + Mq U,  r_k = G_p k~ S_c + Mk U,
//            rhs~ = v~ - diag(G~) r_k,  u~ = T~ rhs~,  o~ = s (diag(G~_e) r_q + M~ u~),
//            S'  = G_C S_c + K^T diag(D) U
//   reverse  dr_q = s diag(G~_e) do~,  du~ = s M~^T do~,  drhs~ = T~^T du~,
//            dr_k = -diag(G~) drhs~,
//            dU = diag(D) K dS' + s Mo^T do + Mq^T dr_q + Mk^T dr_k,  drhs = T^T dU,
//            dS_c = G_C dS' + s Q^T diag(G) do + q~^T diag(G_p) dr_q
//                   + k~^T diag(G_p) dr_k - K^T diag(G) drhs,
//   and for every masked Gram M = G o E o w (E decay/mask, w the write
//   strengths) with dM accumulated from the products it enters,
//   dG = dM o E o w, d(rows) += dG Y, d(cols) += dG^T X, and the gate
//   gradients follow from d log-decay = reverse cumulative sums.
// (The identical algebra is checked against the oracle's token-level reverse
// mode in the CPU tests.)
//
// Two kernels:
//   pass 1, gdn_bwd_scan_kernel: one workgroup per (document, head, 32-column
//     d_v tile) marches the chunks in reverse carrying dS' (column-separable)
//     and stores each chunk's end-state adjoint into the workspace, in the
//     checkpoint slot layout; dh0 is the adjoint left after chunk 0.
//   pass 2, gdn_bwd_chunk_kernel: one workgroup per (chunk, head), fully
//     parallel: rebuilds the chunk from its checkpoint S_c and its dS', loops
//     over 16-column d_v tiles accumulating the C x C Gram adjoints and the
//     d_k-side gradients in registers, then emits dq, dk, dv, dalpha, dbeta and
//     their noisy twins with no cross-workgroup reduction (deterministic).
#include <type_traits>

#include "chunk_common.h"
#include "device_common.h"
#include "bwd_common.h"
#include "gemm_lds.h"
#include "host_plan.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

template <typename IO, int D> struct BwdCfg {
  static constexpr bool BF = std::is_same<IO, u16>::value;
  static constexpr int C = 32, NW = 4, NT = 256;
  static constexpr int DV = D >= 32 ? 32 : D;  // pass-1 d_v tile
  static constexpr int NTILE = D / DV;
  static constexpr int CT = DV / 16;
  static constexpr int LDX = D + 8, LDM = C + 4, LDV = DV + 4;
  static constexpr int ES = sizeof(IO);
  static constexpr int NST = (D / 16) * CT;
  static constexpr int SPW = (NST + NW - 1) / NW;
  static constexpr int XL = BF ? RowU16 : RowF32;   // layout tag of the q/k tiles
  static constexpr int XLT = BF ? ColU16 : ColF32;  // the same tiles read transposed
  static constexpr int DVT = 16;                    // pass-2 d_v tile
  static constexpr int LV = DVT + 4;
};

// Loads the chunk's q, k, q~, k~ rows (noisy prompt rows and rows past the
// document end as zeros) straight into LDS.
template <typename IO, int D, int LDX>
__device__ __forceinline__ void load_x_tiles(IO (*x)[32][LDX], const FwdArgs &f, int64_t t0g, int c0, int n,
                                             int P, int h) {
  constexpr int C = 32, NT = 256, ES = sizeof(IO);
  constexpr int RU = D * ES / 16, PU = C * RU;
  const IO *const pq = reinterpret_cast<const IO *>(f.q), *const pk = reinterpret_cast<const IO *>(f.k);
  const IO *const pqn = reinterpret_cast<const IO *>(f.qn), *const pkn = reinterpret_cast<const IO *>(f.kn);
  for (int u = threadIdx.x; u < 4 * PU; u += NT) {
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    const int tpos = c0 + row;
    bool ok = tpos < n;
    if (m >= 2) ok = ok && tpos >= P;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    const IO *src = m == 0 ? pq : m == 1 ? pk : m == 2 ? pqn : pkn;
    if (ok) val = *reinterpret_cast<const uint4 *>(src + ((t0g + tpos) * f.H + h) * D + cu16 * (16 / ES));
    *reinterpret_cast<uint4 *>(&x[m][row][cu16 * (16 / ES)]) = val;
  }
}

// Loads columns [dv0, dv0 + W) of a [T, H, D] io tensor for the chunk's rows
// into an fp32 LDS tile [C][LD] (rows that do not exist, or that are noisy
// prompt rows when noisy, as zeros).
template <typename IO, int D, int W, int LD>
__device__ __forceinline__ void load_cols_f32(float (*dst)[LD], const void *src_v, int H, int64_t t0g, int c0,
                                              int n, int P, bool noisy, int h, int dv0) {
  const IO *src = reinterpret_cast<const IO *>(src_v);
  for (int e = threadIdx.x; e < 32 * W; e += 256) {
    const int row = e / W, col = e % W;
    const int tpos = c0 + row;
    const bool ok = tpos < n && (!noisy || tpos >= P);
    dst[row][col] = ok ? io_traits<IO>::to_f(src[((t0g + tpos) * H + h) * D + dv0 + col]) : 0.f;
  }
}

// =============================================================== pass 1
template <typename IO, int D> struct ScanSmem {
  using Cfg = BwdCfg<IO, D>;
  static constexpr int C = Cfg::C, DV = Cfg::DV, LDX = Cfg::LDX, LDM = Cfg::LDM, LDV = Cfg::LDV;
  alignas(16) IO x[4][C][LDX];       // q, k, q~, k~
  alignas(16) IO dst[2][DV][LDX];    // dS'^T (bf16 hi, lo; fp32 io: value in [0])
  alignas(16) float dob[2][C][LDV];  // do, do~ tile
  alignas(16) float cc[8][C][LDM];
  alignas(16) float vec[8][C][LDV];  // DRQ, DUN, DRK, DU, Y1, Y2, Y3, Y4
  alignas(16) float tmp[2][16][17];
  alignas(16) float lg[C], beta[C], lgn[C], betan[C];
};
enum { V_DRQ = 0, V_DUN, V_DRK, V_DU, V_Y1, V_Y2, V_Y3, V_Y4 };

template <typename IO, int D>
__global__ __launch_bounds__(256) void gdn_bwd_scan_kernel(BwdArgs a) {
  using Cfg = BwdCfg<IO, D>;
  using Sm = ScanSmem<IO, D>;
  constexpr bool BF = Cfg::BF;
  constexpr int C = Cfg::C, NT = Cfg::NT, DV = Cfg::DV, NTILE = Cfg::NTILE, CT = Cfg::CT;
  constexpr int LDX = Cfg::LDX, LDM = Cfg::LDM, LDV = Cfg::LDV, SPW = Cfg::SPW, NST = Cfg::NST;
  constexpr int XLT = Cfg::XLT;
  __shared__ Sm sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;

  const int L = blockIdx.x;
  const int grp = L / (8 * NTILE), rem = L % (8 * NTILE);
  const int tile = rem / 8;
  const int pair = grp * 8 + (rem % 8);
  if (pair >= f.num_docs * f.H) return;
  const int doc = pair / f.H, h = pair % f.H;
  const int H = f.H;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int P = f.plen[doc];
  const int B = f.B;  // a power of two up to 32 (checked by the host): i % B = i & (B - 1)
  const int nchunks = (n + C - 1) / C;
  const int dv0 = tile * DV;
  const float s = f.scale;
  float *ws = reinterpret_cast<float *>(a.workspace);
  const int64_t ck_base = (int64_t)(t0g / C) + doc;

  for (int e = tid; e < 8 * C * LDM; e += NT) (&sm.cc[0][0][0])[e] = 0.f;

  // dS' tiles owned by this wave (same layout as the forward's state tiles)
  floatx4 dS[SPW];
#pragma unroll
  for (int e = 0; e < SPW; ++e) {
    const int q = wave * SPW + e;
    dS[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (q < NST && a.dh_final) {
      const int rt = q / CT, ct = q % CT;
      const float *src = a.dh_final + ((size_t)doc * H + h) * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) dS[e][r] = src[(size_t)(16 * rt + g4 + r) * D + dv0 + 16 * ct + cl];
    }
  }
  auto store_dS_global = [&](float *dst) {
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int q = wave * SPW + e;
      if (q < NST) {
        const int rt = q / CT, ct = q % CT;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(16 * rt + g4 + r) * D + dv0 + 16 * ct + cl] = dS[e][r];
      }
    }
  };

  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * C;
    const bool has_noisy = (c0 + C > P) && (P < n);
    // ------------------------------------------------------------- [A] inputs
    lds_barrier();
    load_x_tiles<IO, D, LDX>(sm.x, f, t0g, c0, n, P, h);
    load_cols_f32<IO, D, DV, LDV>(sm.dob[0], a.d_o, H, t0g, c0, n, P, false, h, dv0);
    load_cols_f32<IO, D, DV, LDV>(sm.dob[1], a.d_on, H, t0g, c0, n, P, true, h, dv0);
    load_gates(f, t0g, c0, n, P, h, B, sm.lg, sm.beta, sm.lgn, sm.betan);
    // the adjoint of this chunk's end state, for pass 2
    store_dS_global(ws + ((ck_base + c) * H + h) * (size_t)D * D);
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int q = wave * SPW + e;
      if (q < NST) {
        const int rt = q / CT, ct = q % CT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = dS[e][r];
          if constexpr (BF) {
            const u16 hi = f2bf(v);
            sm.dst[0][16 * ct + cl][16 * rt + g4 + r] = hi;
            sm.dst[1][16 * ct + cl][16 * rt + g4 + r] = f2bf(v - bf2f(hi));
          } else {
            sm.dst[0][16 * ct + cl][16 * rt + g4 + r] = v;
          }
        }
      }
    }
    lds_barrier();
    // ------------------------------------------------------------- [C] Grams, solves, elementwise
    chunk_grams<BF, D, LDX, LDM>(sm.x, sm.cc, sm.lg, sm.beta, sm.lgn, sm.betan, c0, n, P, B, has_noisy, true);
    const float lgC = sm.lg[C - 1];
    if (wave == 0) {
      solve_unit_lower<LDM>(&sm.cc[CC_AT][0][0], &sm.cc[CC_T][0][0], &sm.tmp[0][0][0], true);
      // dU starts as diag(D) K dS'
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          gemm_tile<BF, D, Cfg::XL, Cfg::XL>(acc, &sm.x[1][0][0], LDX, 16 * tr, &sm.dst[0][0][0], LDX, 16 * tc);
          if constexpr (BF)
            gemm_tile<BF, D, Cfg::XL, Cfg::XL>(acc, &sm.x[1][0][0], LDX, 16 * tr, &sm.dst[1][0][0], LDX, 16 * tc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * tr + g4 + r;
            sm.vec[V_DU][i][16 * tc + cl] = acc[r] * sm.beta[i] * __expf(lgC - sm.lg[i]);
          }
        }
    } else if (wave == 1) {
      for (int e = lane; e < C * DV; e += 64) {
        const int i = e / DV, col = e % DV;
        sm.vec[V_Y1][i][col] = s * __expf(sm.lg[i]) * sm.dob[0][i][col];
      }
    } else if (wave == 2 && has_noisy) {
      for (int e = lane; e < C * DV; e += 64) {
        const int i = e / DV, col = e % DV;
        const int pi = (i & -B);
        const float drq = s * __expf(sm.lgn[pi + B - 1]) * sm.dob[1][i][col];
        sm.vec[V_DRQ][i][col] = drq;
        sm.vec[V_Y2][i][col] = (pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f) * drq;
      }
    } else if (wave == 3 && has_noisy) {
      solve_unit_lower<LDM>(&sm.cc[CC_ANT][0][0], &sm.cc[CC_TN][0][0], &sm.tmp[1][0][0], B > 16);
    }
    lds_barrier();
    // ------------------------------------------------------------- [D] noisy chain: du~ -> drhs~ -> dr_k
    if (wave == 2 && has_noisy) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_MN][0][0], LDM, 16 * tr, &sm.dob[1][0][0], LDV, 16 * tc);
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.vec[V_DUN][16 * tr + g4 + r][16 * tc + cl] = s * acc[r];
        }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_TN][0][0], LDM, 16 * tr, &sm.vec[V_DUN][0][0], LDV, 16 * tc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * tr + g4 + r;
            const int pi = (i & -B);
            const float drk = -__expf(sm.lgn[i]) * acc[r];
            sm.vec[V_DRK][i][16 * tc + cl] = drk;
            sm.vec[V_Y3][i][16 * tc + cl] = (pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f) * drk;
          }
        }
    }
    lds_barrier();
    // ------------------------------------------------------------- [E] dU
    for (int job = wave; job < 2 * CT; job += 4) {
      const int tr = job / CT, tc = job % CT;
      floatx4 acc, t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sm.vec[V_DU][16 * tr + g4 + r][16 * tc + cl];
      gemm_tile<BF, C, ColF32, ColF32>(t2, &sm.cc[CC_MO][0][0], LDM, 16 * tr, &sm.dob[0][0][0], LDV, 16 * tc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += s * t2[r];
      if (has_noisy) {
        gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_MQ][0][0], LDM, 16 * tr, &sm.vec[V_DRQ][0][0], LDV, 16 * tc);
        gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_MK][0][0], LDM, 16 * tr, &sm.vec[V_DRK][0][0], LDV, 16 * tc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.vec[V_DU][16 * tr + g4 + r][16 * tc + cl] = acc[r];
    }
    lds_barrier();
    // ------------------------------------------------------------- [F] drhs = T^T dU ; Y4 = -G drhs
    for (int job = wave; job < 2 * CT; job += 4) {
      const int tr = job / CT, tc = job % CT;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_T][0][0], LDM, 16 * tr, &sm.vec[V_DU][0][0], LDV, 16 * tc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * tr + g4 + r;
        sm.vec[V_Y4][i][16 * tc + cl] = -__expf(sm.lg[i]) * acc[r];
      }
    }
    lds_barrier();
    // ------------------------------------------------------------- [G] dS_c
    const float gC = __expf(lgC);
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int q = wave * SPW + e;
      if (q < NST) {
        const int rt = q / CT, ct = q % CT;
#pragma unroll
        for (int r = 0; r < 4; ++r) dS[e][r] *= gC;
        gemm_tile<BF, C, XLT, ColF32>(dS[e], &sm.x[0][0][0], LDX, 16 * rt, &sm.vec[V_Y1][0][0], LDV, 16 * ct);
        gemm_tile<BF, C, XLT, ColF32>(dS[e], &sm.x[1][0][0], LDX, 16 * rt, &sm.vec[V_Y4][0][0], LDV, 16 * ct);
        if (has_noisy) {
          gemm_tile<BF, C, XLT, ColF32>(dS[e], &sm.x[2][0][0], LDX, 16 * rt, &sm.vec[V_Y2][0][0], LDV, 16 * ct);
          gemm_tile<BF, C, XLT, ColF32>(dS[e], &sm.x[3][0][0], LDX, 16 * rt, &sm.vec[V_Y3][0][0], LDV, 16 * ct);
        }
      }
    }
  }
  if (a.dh0) store_dS_global(a.dh0 + ((size_t)doc * H + h) * D * D);
}

// =============================================================== pass 2
template <typename IO, int D> struct ChunkSmem {
  using Cfg = BwdCfg<IO, D>;
  static constexpr int C = Cfg::C, LDX = Cfg::LDX, LDM = Cfg::LDM, DVT = Cfg::DVT, LV = Cfg::LV;
  alignas(16) IO x[4][C][LDX];          // q, k, q~, k~ ; reused to stage the d_k-side gradients
  alignas(16) float cc[8][C][LDM];      // Aw^T, T, Mwo, Mwq, Mwk, A~w^T, T~, Mw~ ; later the Gram adjoints
  alignas(16) float sf[D][DVT + 4];     // S_c tile   [d_k][16]
  alignas(16) float df[D][DVT + 4];     // dS' tile   [d_k][16]
  alignas(16) float vec[19][C][LV];
  alignas(16) float tmp[2][16][17];
  alignas(16) float lg[C], beta[C], lgn[C], betan[C];
  // per-wave gate-gradient partials, each lane writing only rows/columns it
  // owns: pg / pgn go to d gamma_i / d gamma~_i directly; pgp[i] to
  // d gamma[p(i) - 1], pge[i] to d gamma~[end of i's block], pc[i] to d gamma[C-1]
  alignas(16) float pg[4][C], pgn[4][C], pb[4][C], pbn[4][C], pgp[4][C], pge[4][C], pc[4][C];
  alignas(16) float plgc[4];
};
enum {
  W_V = 0, W_KS, W_U, W_BU, W_DUV, W_VN, W_RQ0, W_RK0, W_RQ, W_RK, W_UN, W_BUN, W_DO, W_DON, W_DRQ, W_DUN,
  W_DU, W_DRHS, W_Y4
};
// W_V holds v then rhs; W_VN holds v~, then rhs~, then drhs~ (= dv~); W_DUN holds du~ then dr_k.

template <typename IO, int D>
__global__ __launch_bounds__(256) void gdn_bwd_chunk_kernel(BwdArgs a) {
  using Cfg = BwdCfg<IO, D>;
  using Sm = ChunkSmem<IO, D>;
  constexpr bool BF = Cfg::BF;
  constexpr int C = Cfg::C, NT = Cfg::NT, LDX = Cfg::LDX, LDM = Cfg::LDM, DVT = Cfg::DVT, LV = Cfg::LV;
  constexpr int XL = Cfg::XL, XLT = Cfg::XLT;
  constexpr int KT = D / 16;  // d_k tiles
  __shared__ Sm sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  const int H = f.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;

  // slot -> (document, chunk): slots of document i start at floor(cu_i / C) + i
  int lo = 0, hi = f.num_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)f.cu[mid] / C + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int doc = lo;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int c = slot - (int)(t0g / C) - doc;
  if (c < 0 || c * C >= n) return;
  const int P = f.plen[doc];
  const int B = f.B;  // a power of two up to 32 (checked by the host): i % B = i & (B - 1)
  const int c0 = c * C;
  const bool has_noisy = (c0 + C > P) && (P < n);
  const float s = f.scale;
  const float *Sc = a.ckpt_in + ((int64_t)slot * H + h) * (size_t)D * D;
  const float *dSn = reinterpret_cast<const float *>(a.workspace) + ((int64_t)slot * H + h) * (size_t)D * D;

  for (int e = tid; e < 8 * C * LDM; e += NT) (&sm.cc[0][0][0])[e] = 0.f;
  for (int e = tid; e < 7 * 4 * C; e += NT) (&sm.pg[0][0])[e] = 0.f;
  if (tid < 4) sm.plgc[tid] = 0.f;
  load_x_tiles<IO, D, LDX>(sm.x, f, t0g, c0, n, P, h);
  load_gates(f, t0g, c0, n, P, h, B, sm.lg, sm.beta, sm.lgn, sm.betan);
  lds_barrier();
  chunk_grams<BF, D, LDX, LDM>(sm.x, sm.cc, sm.lg, sm.beta, sm.lgn, sm.betan, c0, n, P, B, has_noisy, false);
  lds_barrier();
  if (wave == 0) solve_unit_lower<LDM>(&sm.cc[CC_AT][0][0], &sm.cc[CC_T][0][0], &sm.tmp[0][0][0], true, sm.beta);
  if (wave == 3 && has_noisy)
    solve_unit_lower<LDM>(&sm.cc[CC_ANT][0][0], &sm.cc[CC_TN][0][0], &sm.tmp[1][0][0], B > 16, sm.betan);

  const float lgC = sm.lg[C - 1];
  auto Gp = [&](int i) { const int pi = (i & -B); return pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f; };
  auto Ge = [&](int i) { const int pi = (i & -B); return __expf(sm.lgn[pi + B - 1]); };
  auto Dd = [&](int i) { return sm.beta[i] * __expf(lgC - sm.lg[i]); };
  auto resp_row = [&](int i) { return c0 + i < n && c0 + i >= P; };

  // Gram adjoints: wave w owns tile w = (w >> 1, w & 1) of each of the six
  floatx4 dM[6];
#pragma unroll
  for (int m = 0; m < 6; ++m) dM[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  enum { DM_O = 0, DM_Q, DM_K, DM_N, DM_A, DM_AN };
  const int mti = wave >> 1, mtj = wave & 1;
  // d_k-side gradients: wave 0 dq, 1 dk, 2 dq~, 3 dk~; tiles (row tile, d_k tile)
  floatx4 dX[2][KT];
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) dX[tr][kt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int dv0 = 0; dv0 < D; dv0 += DVT) {
    lds_barrier();
    // ---- tile inputs: S_c and dS' columns, v, v~, do, do~
    for (int e = tid; e < D * DVT; e += NT) {
      const int r = e / DVT, col = e % DVT;
      sm.sf[r][col] = Sc[(size_t)r * D + dv0 + col];
      sm.df[r][col] = dSn[(size_t)r * D + dv0 + col];
    }
    load_cols_f32<IO, D, DVT, LV>(sm.vec[W_V], f.v, H, t0g, c0, n, P, false, h, dv0);
    load_cols_f32<IO, D, DVT, LV>(sm.vec[W_VN], f.vn, H, t0g, c0, n, P, true, h, dv0);
    load_cols_f32<IO, D, DVT, LV>(sm.vec[W_DO], a.d_o, H, t0g, c0, n, P, false, h, dv0);
    load_cols_f32<IO, D, DVT, LV>(sm.vec[W_DON], a.d_on, H, t0g, c0, n, P, true, h, dv0);
    lds_barrier();
    // ---- [1] X S_c products
    if (wave == 0) {
      // KS, rhs = v - G KS, U = T rhs, b U, D U
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, D, XL, ColF32>(acc, &sm.x[1][0][0], LDX, 16 * tr, &sm.sf[0][0], DVT + 4, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[W_KS][i][cl] = acc[r];
          sm.vec[W_V][i][cl] -= __expf(sm.lg[i]) * acc[r];
        }
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, C, RowF32, ColF32>(acc, &sm.cc[CC_T][0][0], LDM, 16 * tr, &sm.vec[W_V][0][0], LV, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[W_U][i][cl] = acc[r];
          sm.vec[W_BU][i][cl] = sm.beta[i] * acc[r];
          sm.vec[W_DUV][i][cl] = Dd(i) * acc[r];
        }
      }
    } else if (wave == 1) {
      // QS only enters the gate gradient: d gamma_i += s G_i do_i . (q_i S_c)
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, D, XL, ColF32>(acc, &sm.x[0][0][0], LDX, 16 * tr, &sm.sf[0][0], DVT + 4, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          const float t = sum16(acc[r] * sm.vec[W_DO][i][cl]);
          if (cl == 0) sm.pg[1][i] += s * __expf(sm.lg[i]) * t;
        }
      }
    } else if (has_noisy) {
      const int xm = wave == 2 ? 2 : 3, dst = wave == 2 ? W_RQ0 : W_RK0;
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, D, XL, ColF32>(acc, &sm.x[xm][0][0], LDX, 16 * tr, &sm.sf[0][0], DVT + 4, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[dst][i][cl] = Gp(i) * acc[r];
        }
      }
    }
    lds_barrier();
    // ---- [2] r_q, r_k -> u~ (waves 2, 3); K dS' -> D K dS', dD (wave 1); dMo (all)
    floatx4 kd[2];
    if (wave == 1) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        kd[tr] = floatx4{0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, D, XL, ColF32>(kd[tr], &sm.x[1][0][0], LDX, 16 * tr, &sm.df[0][0], DVT + 4, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          const float t = sum16(kd[tr][r] * sm.vec[W_U][i][cl]);  // dD_i partial
          if (cl == 0) {
            const float Di = Dd(i);
            sm.pb[1][i] += t * __expf(lgC - sm.lg[i]);
            sm.pg[1][i] -= t * Di;
            sm.pc[1][i] += t * Di;
          }
          sm.vec[W_DU][i][cl] = Dd(i) * kd[tr][r];
        }
      }
    } else if (wave == 2 && has_noisy) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sm.vec[W_RQ0][16 * tr + g4 + r][cl];
        gemm_tile<BF, C, RowF32, ColF32>(acc, &sm.cc[CC_MQ][0][0], LDM, 16 * tr, &sm.vec[W_BU][0][0], LV, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.vec[W_RQ][16 * tr + g4 + r][cl] = acc[r];
      }
    } else if (wave == 3 && has_noisy) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sm.vec[W_RK0][16 * tr + g4 + r][cl];
        gemm_tile<BF, C, RowF32, ColF32>(acc, &sm.cc[CC_MK][0][0], LDM, 16 * tr, &sm.vec[W_BU][0][0], LV, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[W_RK][i][cl] = acc[r];
          sm.vec[W_VN][i][cl] -= __expf(sm.lgn[i]) * acc[r];  // rhs~
        }
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, C, RowF32, ColF32>(acc, &sm.cc[CC_TN][0][0], LDM, 16 * tr, &sm.vec[W_VN][0][0], LV, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[W_UN][i][cl] = acc[r];
          sm.vec[W_BUN][i][cl] = sm.betan[i] * acc[r];
        }
      }
    }
    // dMo += s do U^T (tile of this wave)
    {
      floatx4 t2 = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, DVT, RowF32, RowF32>(t2, &sm.vec[W_DO][0][0], LV, 16 * mti, &sm.vec[W_U][0][0], LV, 16 * mtj);
#pragma unroll
      for (int r = 0; r < 4; ++r) dM[DM_O][r] += s * t2[r];
    }
    lds_barrier();
    // ---- [3] noisy backward chain (wave 2): dr_q, du~, drhs~, dr_k
    if (wave == 2 && has_noisy) {
      for (int e = lane; e < C * DVT; e += 64) {
        const int i = e / DVT, col = e % DVT;
        sm.vec[W_DRQ][i][col] = s * Ge(i) * sm.vec[W_DON][i][col];
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {  // du~ = s diag(b~) Mw~^T do~
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_MN][0][0], LDM, 16 * tr, &sm.vec[W_DON][0][0], LV, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[W_DUN][i][cl] = s * sm.betan[i] * acc[r];
          // d gamma~ at the block end: s G~_e do~_i . r_q,i
          const float t = sum16(sm.vec[W_DON][i][cl] * sm.vec[W_RQ][i][cl]);
          if (cl == 0 && resp_row(i)) sm.pge[2][i] += s * Ge(i) * t;
        }
      }
      floatx4 dr[2];
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {  // drhs~ = T~^T du~
        dr[tr] = floatx4{0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, C, ColF32, ColF32>(dr[tr], &sm.cc[CC_TN][0][0], LDM, 16 * tr, &sm.vec[W_DUN][0][0], LV, 0);
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          const float drn = resp_row(i) ? dr[tr][r] : 0.f;
          const float t = sum16(drn * sm.vec[W_RK][i][cl]);
          if (cl == 0) sm.pgn[2][i] -= __expf(sm.lgn[i]) * t;
          sm.vec[W_VN][i][cl] = drn;                         // dv~
          sm.vec[W_DUN][i][cl] = -__expf(sm.lgn[i]) * drn;   // dr_k
          const float t2 = sum16(sm.vec[W_DRQ][i][cl] * sm.vec[W_RQ0][i][cl] +
                                 sm.vec[W_DUN][i][cl] * sm.vec[W_RK0][i][cl]);
          if (cl == 0) sm.pgp[2][i] += t2;
        }
    }
    lds_barrier();
    // ---- [4] dU = D K dS' + diag(b) (s Mwo^T do + Mwq^T dr_q + Mwk^T dr_k)  (waves 0, 1)
    if (wave < 2) {
      const int tr = wave;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f}, t2 = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, C, ColF32, ColF32>(t2, &sm.cc[CC_MO][0][0], LDM, 16 * tr, &sm.vec[W_DO][0][0], LV, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = s * t2[r];
      if (has_noisy) {
        gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_MQ][0][0], LDM, 16 * tr, &sm.vec[W_DRQ][0][0], LV, 0);
        gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_MK][0][0], LDM, 16 * tr, &sm.vec[W_DUN][0][0], LV, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * tr + g4 + r;
        sm.vec[W_DU][i][cl] += sm.beta[i] * acc[r];
      }
    } else if (wave == 2 && has_noisy) {
      // dv~ rows of this tile -> global (prompt rows are written as zero elsewhere)
      IO *gdvn = reinterpret_cast<IO *>(a.dvn);
      for (int e = lane; e < C * DVT; e += 64) {
        const int i = e / DVT, col = e % DVT;
        if (resp_row(i))
          gdvn[((t0g + c0 + i) * H + h) * D + dv0 + col] = io_traits<IO>::from_f(sm.vec[W_VN][i][col]);
      }
    }
    lds_barrier();
    // ---- [5] drhs = T^T dU (wave 0) ; Y4 = -G drhs ; dv
    if (wave == 0) {
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, C, ColF32, ColF32>(acc, &sm.cc[CC_T][0][0], LDM, 16 * tr, &sm.vec[W_DU][0][0], LV, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tr + g4 + r;
          sm.vec[W_DRHS][i][cl] = acc[r];
          sm.vec[W_Y4][i][cl] = -__expf(sm.lg[i]) * acc[r];
          const float t = sum16(acc[r] * sm.vec[W_KS][i][cl]);
          if (cl == 0) sm.pg[0][i] -= __expf(sm.lg[i]) * t;
        }
      }
    } else if (wave == 1) {
      // Gamma_C <dS', S_c> over this tile
      float part = 0.f;
      for (int e = lane; e < D * DVT; e += 64) part += sm.df[e / DVT][e % DVT] * sm.sf[e / DVT][e % DVT];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
      if (lane == 0) sm.plgc[1] += __expf(lgC) * part;
    }
    lds_barrier();
    // ---- [6] dv out, Gram adjoints, d_k-side products
    {
      IO *gdv = reinterpret_cast<IO *>(a.dv);
      for (int e = tid; e < C * DVT; e += NT) {
        const int i = e / DVT, col = e % DVT;
        if (c0 + i < n) gdv[((t0g + c0 + i) * H + h) * D + dv0 + col] = io_traits<IO>::from_f(sm.vec[W_DRHS][i][col]);
      }
    }
    {
      floatx4 t2 = {0.f, 0.f, 0.f, 0.f};
      gemm_tile<BF, DVT, RowF32, RowF32>(t2, &sm.vec[W_DRHS][0][0], LV, 16 * mti, &sm.vec[W_U][0][0], LV, 16 * mtj);
#pragma unroll
      for (int r = 0; r < 4; ++r) dM[DM_A][r] -= t2[r];
      if (has_noisy) {
        gemm_tile<BF, DVT, RowF32, RowF32>(dM[DM_Q], &sm.vec[W_DRQ][0][0], LV, 16 * mti, &sm.vec[W_U][0][0], LV, 16 * mtj);
        gemm_tile<BF, DVT, RowF32, RowF32>(dM[DM_K], &sm.vec[W_DUN][0][0], LV, 16 * mti, &sm.vec[W_U][0][0], LV, 16 * mtj);
        floatx4 t3 = {0.f, 0.f, 0.f, 0.f}, t4 = {0.f, 0.f, 0.f, 0.f};
        gemm_tile<BF, DVT, RowF32, RowF32>(t3, &sm.vec[W_DON][0][0], LV, 16 * mti, &sm.vec[W_UN][0][0], LV, 16 * mtj);
        gemm_tile<BF, DVT, RowF32, RowF32>(t4, &sm.vec[W_VN][0][0], LV, 16 * mti, &sm.vec[W_UN][0][0], LV, 16 * mtj);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dM[DM_N][r] += s * t3[r];
          dM[DM_AN][r] -= t4[r];
        }
      }
    }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (wave == 0) {
          gemm_tile<BF, DVT, RowF32, RowF32>(dX[tr][kt], &sm.vec[W_DO][0][0], LV, 16 * tr, &sm.sf[0][0], DVT + 4, 16 * kt);
        } else if (wave == 1) {
          gemm_tile<BF, DVT, RowF32, RowF32>(dX[tr][kt], &sm.vec[W_Y4][0][0], LV, 16 * tr, &sm.sf[0][0], DVT + 4, 16 * kt);
          gemm_tile<BF, DVT, RowF32, RowF32>(dX[tr][kt], &sm.vec[W_DUV][0][0], LV, 16 * tr, &sm.df[0][0], DVT + 4, 16 * kt);
        } else if (has_noisy) {
          gemm_tile<BF, DVT, RowF32, RowF32>(dX[tr][kt], &sm.vec[wave == 2 ? W_DRQ : W_DUN][0][0], LV, 16 * tr,
                                              &sm.sf[0][0], DVT + 4, 16 * kt);
        }
      }
  }
  lds_barrier();

  // ---- row scales of the S_c products: dq rows by s G, dq~/dk~ rows by G_p
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * tr + g4 + r;
      const float sc = wave == 0 ? s * __expf(sm.lg[i]) : wave == 1 ? 1.f : Gp(i);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) dX[tr][kt][r] *= sc;
    }

  // ---- Gram adjoints -> dG (in place over the unweighted Grams) + gate partials
  {
    const int i0 = 16 * mti + g4, j = 16 * mtj + cl;
    // Mo : w = b, e = lg_i, f = lg_j, mask j <= i
    // Mq/Mk : w = b, e = lg[p_i - 1], mask j < p_i (resp)
    // M~ : w = b~, e = lgn[end(i)], f = lgn_j, mask same block (resp)
    // A^T / A~^T stored transposed: element [j][i]
#pragma unroll
    for (int m = 0; m < 6; ++m) {
      if (!has_noisy && (m == DM_Q || m == DM_K || m == DM_N || m == DM_AN)) continue;
      const int ccm = m == DM_O ? CC_MO : m == DM_Q ? CC_MQ : m == DM_K ? CC_MK : m == DM_N ? CC_MN
                    : m == DM_A ? CC_AT : CC_ANT;
      const bool tr_store = (m == DM_A || m == DM_AN);
      const bool noisyw = (m == DM_N || m == DM_AN);
      const float wj = noisyw ? sm.betan[j] : sm.beta[j];
      const float fj = noisyw ? sm.lgn[j] : sm.lg[j];
      float colw = 0.f, colf = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        float *cell = tr_store ? &sm.cc[ccm][j][i] : &sm.cc[ccm][i][j];
        const float mw = *cell;  // unweighted masked Gram, already zero outside the mask
        float ei;
        bool mask;
        if (m == DM_O) { ei = sm.lg[i]; mask = j <= i; }
        else if (m == DM_A) { ei = sm.lg[i]; mask = j < i; }
        else if (m == DM_Q || m == DM_K) {
          const int pi = (i & -B);
          ei = pi > 0 ? sm.lg[pi - 1] : 0.f;
          mask = resp_row(i) && j < pi;
        } else if (m == DM_N) {
          const int pi = (i & -B);
          ei = sm.lgn[pi + B - 1];
          mask = resp_row(i) && j >= pi && j < pi + B;
        } else {
          const int pi = (i & -B);
          ei = sm.lgn[i];
          mask = resp_row(i) && j < i && j >= pi;
        }
        const float dm = dM[m][r];
        const float E = mask ? __expf(ei - fj) : 0.f;
        const float mfull = mw * wj;
        *cell = dm * E * wj;  // dG
        const float dd = dm * mfull;
        // row part d e_i
        const float rs = sum16(dd);
        if (cl == 0) {
          if (m == DM_O || m == DM_A) sm.pg[wave][i] += rs;
          else if (m == DM_Q || m == DM_K) sm.pgp[wave][i] += rs;
          else if (m == DM_N) sm.pge[wave][i] += rs;
          else sm.pgn[wave][i] += rs;
        }
        colf += dd;
        colw += dm * mw;
      }
      // column parts: over the 4 row groups of the tile
      colf += __shfl_xor(colf, 16, 64);
      colf += __shfl_xor(colf, 32, 64);
      colw += __shfl_xor(colw, 16, 64);
      colw += __shfl_xor(colw, 32, 64);
      if (lane < 16) {
        if (noisyw) {
          sm.pgn[wave][j] -= colf;
          sm.pbn[wave][j] += colw;
        } else {
          sm.pg[wave][j] -= colf;
          sm.pb[wave][j] += colw;
        }
      }
    }
  }
  lds_barrier();

  // ---- d_k-side Gram products (contraction over the chunk)
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      floatx4 &acc = dX[tr][kt];
      const int ra = 16 * tr, rb = 16 * kt;
      if (wave == 0) {  // dq += dGo k
        gemm_tile<BF, C, RowF32, XLT>(acc, &sm.cc[CC_MO][0][0], LDM, ra, &sm.x[1][0][0], LDX, rb);
      } else if (wave == 1) {  // dk += dGo^T q + dGA k + dGA^T k + dGq^T q~ + dGk^T k~
        gemm_tile<BF, C, ColF32, XLT>(acc, &sm.cc[CC_MO][0][0], LDM, ra, &sm.x[0][0][0], LDX, rb);
        gemm_tile<BF, C, ColF32, XLT>(acc, &sm.cc[CC_AT][0][0], LDM, ra, &sm.x[1][0][0], LDX, rb);
        gemm_tile<BF, C, RowF32, XLT>(acc, &sm.cc[CC_AT][0][0], LDM, ra, &sm.x[1][0][0], LDX, rb);
        if (has_noisy) {
          gemm_tile<BF, C, ColF32, XLT>(acc, &sm.cc[CC_MQ][0][0], LDM, ra, &sm.x[2][0][0], LDX, rb);
          gemm_tile<BF, C, ColF32, XLT>(acc, &sm.cc[CC_MK][0][0], LDM, ra, &sm.x[3][0][0], LDX, rb);
        }
      } else if (wave == 2 && has_noisy) {  // dq~ += dGq k + dG~ k~
        gemm_tile<BF, C, RowF32, XLT>(acc, &sm.cc[CC_MQ][0][0], LDM, ra, &sm.x[1][0][0], LDX, rb);
        gemm_tile<BF, C, RowF32, XLT>(acc, &sm.cc[CC_MN][0][0], LDM, ra, &sm.x[3][0][0], LDX, rb);
      } else if (wave == 3 && has_noisy) {  // dk~ += dGk k + dGA~ k~ + dGA~^T k~ + dG~^T q~
        gemm_tile<BF, C, RowF32, XLT>(acc, &sm.cc[CC_MK][0][0], LDM, ra, &sm.x[1][0][0], LDX, rb);
        gemm_tile<BF, C, ColF32, XLT>(acc, &sm.cc[CC_ANT][0][0], LDM, ra, &sm.x[3][0][0], LDX, rb);
        gemm_tile<BF, C, RowF32, XLT>(acc, &sm.cc[CC_ANT][0][0], LDM, ra, &sm.x[3][0][0], LDX, rb);
        gemm_tile<BF, C, ColF32, XLT>(acc, &sm.cc[CC_MN][0][0], LDM, ra, &sm.x[2][0][0], LDX, rb);
      }
    }
  lds_barrier();
  // ---- stage the four d_k-side gradients in the (now free) q/k tiles and store rows
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * tr + g4 + r;
        float v = dX[tr][kt][r];
        if (wave >= 2 && !resp_row(i)) v = 0.f;
        sm.x[wave][i][16 * kt + cl] = io_traits<IO>::from_f(v);
      }
  lds_barrier();
  {
    constexpr int ES = sizeof(IO), RU = D * ES / 16;
    IO *outp[4] = {reinterpret_cast<IO *>(a.dq), reinterpret_cast<IO *>(a.dk), reinterpret_cast<IO *>(a.dqn),
                   reinterpret_cast<IO *>(a.dkn)};
    for (int u = tid; u < 4 * C * RU; u += NT) {
      const int m = u / (C * RU), rr = u % (C * RU), row = rr / RU, cu16 = rr % RU;
      if (c0 + row >= n) continue;
      IO *dst = m == 0 ? outp[0] : m == 1 ? outp[1] : m == 2 ? outp[2] : outp[3];
      *reinterpret_cast<uint4 *>(dst + ((t0g + c0 + row) * H + h) * D + cu16 * (16 / ES)) =
          *reinterpret_cast<const uint4 *>(&sm.x[m][row][cu16 * (16 / ES)]);
    }
  }
  // ---- gates: scatter the per-row partials to the positions they belong to
  // (one thread, fixed order: deterministic), then d log a = reverse cumulative
  // sum of d gamma and d a = d log a / a
  if (tid == 0) {
    for (int i = 0; i < C; ++i) {
      const int pi = (i & -B);
      for (int w = 0; w < 4; ++w) {
        if (pi > 0) sm.pg[0][pi - 1] += sm.pgp[w][i];
        sm.pgn[0][pi + B - 1] += sm.pge[w][i];
        sm.pg[0][C - 1] += sm.pc[w][i];
      }
    }
  }
  lds_barrier();
  if (tid < 64) {
    const int i = tid & 31;
    const bool noisy = tid >= 32;
    float dg = 0.f, db = 0.f;
    if (!noisy) {
      for (int m = i; m < C; ++m) {
        float v = sm.pg[0][m] + sm.pg[1][m] + sm.pg[2][m] + sm.pg[3][m];
        if (m == C - 1) v += sm.plgc[0] + sm.plgc[1] + sm.plgc[2] + sm.plgc[3];
        dg += v;
      }
      db = sm.pb[0][i] + sm.pb[1][i] + sm.pb[2][i] + sm.pb[3][i];
    } else {
      const int end = (i & -B) + B;
      for (int m = i; m < end; ++m) dg += sm.pgn[0][m] + sm.pgn[1][m] + sm.pgn[2][m] + sm.pgn[3][m];
      db = sm.pbn[0][i] + sm.pbn[1][i] + sm.pbn[2][i] + sm.pbn[3][i];
    }
    const int64_t gi = (t0g + c0 + i) * H + h;
    if (c0 + i < n) {
      if (!noisy) {
        a.dalpha[gi] = dg / f.alpha[gi];
        a.dbeta[gi] = db;
      } else {
        const bool rsp = c0 + i >= P;
        a.dalpha_n[gi] = rsp ? dg / f.alpha_n[gi] : 0.f;
        a.dbeta_n[gi] = rsp ? db : 0.f;
      }
    }
  }
  // noisy prompt rows of dv~ (and the whole noisy tile of a prompt-only chunk)
  if (!has_noisy || c0 < P) {
    IO *gdvn = reinterpret_cast<IO *>(a.dvn);
    for (int e = tid; e < C * D; e += NT) {
      const int i = e / D, col = e % D;
      if (c0 + i < n && c0 + i < P) gdvn[((t0g + c0 + i) * H + h) * D + col] = io_traits<IO>::from_f(0.f);
    }
  }
}

// The chunked backward (bf16 io, d = 128), per pass (the whole batch, or one
// window of chunks of every document, last window first): the chunk matrices
// (or the forward's), the chunk-start states rebuilt from strided checkpoints
// when only every stride-th one was kept (the forward's hand-over, then runs
// of a multiple of the stride from checkpoints, all in parallel), the reverse scan's
// hand-over, the reverse scan (carried between windows), the per-chunk pass.
static hipError_t launch_bwd_chunked(const BwdArgs &a_in, hipStream_t st, const BwdPlan *plan) {
  BwdArgs a = a_in;
  constexpr int C = kChunk, D = 128;
  BwdPlan p{};
  if (plan) {
    p = *plan;
  } else {  // one pass over the workspace in its one-pass layout, stride-1 checkpoints
    p.slots = a.T / C + a.f.num_docs;
    const size_t per = (size_t)p.slots * a.f.H;
    p.adj = reinterpret_cast<float *>(a.workspace);
    p.tri = p.adj + per * D * D;
    p.pack = p.tri + per * 6 * C * C;
    const size_t per_bytes = per * ((size_t)D * D + 6 * C * C + kScanPackFloats) * 4;
    p.l2f = reinterpret_cast<float4 *>(reinterpret_cast<char *>(a.workspace) + ((per_bytes + 255) & ~(size_t)255));
    p.stride = 1;
  }
  if (a.f.flags & 1) {  // the q/k L2 flag: per-row factors (gdn_l2.hip)
    hipError_t e0 = launch_l2_factors(a.f, p.l2f, st);
    if (e0 != hipSuccess) return e0;
    a.f.l2f = p.l2f;
  }
  const int nwin = p.win > 0 ? max(1, (p.max_chunks + p.win - 1) / p.win) : 1;
  for (int j = 0; j < nwin; ++j) {
    const int w = nwin - 1 - j;
    BwdArgs aw = a;
    aw.f.win_lo = p.win > 0 ? w * p.win : 0;
    aw.f.win_len = p.win;
    aw.workspace = p.adj;
    aw.tri = p.tri;
    aw.pack = p.pack;
    const bool own_cm = !(a.fwd_cm && p.win == 0);
    if (!own_cm) aw.tri = const_cast<float *>(a.fwd_cm);  // read only from here on
    aw.kpack = own_cm ? nullptr : a.fwd_pack;  // the forward's K fragment sets, when its hand-over is there
    if (p.stride > 1) {
      // the forward's hand-over for the rebuild (with the chunk matrices,
      // when they are not the forward's)
      if (own_cm) {
        TimedLaunch tl(K_FWD_PREP, st);
        hipError_t e0 = launch_fwd_prep_d128(aw.f, aw.tri, p.pack, st, p.slots);
        if (e0 != hipSuccess) return e0;
      } else {
        TimedLaunch tl(K_FWD_PRE, st);
        hipError_t e0 = launch_fwd_pre_d128(aw.f, aw.tri, p.pack, st, p.slots);
        if (e0 != hipSuccess) return e0;
      }
      ScanArgs rb{};
      rb.num_docs = a.f.num_docs;
      rb.H = a.f.H;
      rb.cu = a.f.cu;
      rb.pack = p.pack;
      rb.states = p.states;
      rb.seg_span = p.rebuild_span;
      rb.seg_init = a.ckpt_in;
      rb.seg_init_stride = p.stride;
      rb.seg_init_all = 1;
      rb.win_lo = aw.f.win_lo;
      rb.win_len = p.win;
      rb.units = p.win > 0 ? (int64_t)a.f.num_docs * (p.win / p.rebuild_span) : p.rebuild_units;
      TimedLaunch tl(K_FWD_SCAN, st);
      hipError_t e0 = launch_scan_d128(rb, false, st);
      if (e0 != hipSuccess) return e0;
      aw.ckpt_in = p.states;
      aw.ckpt_global = 0;
    } else {
      if (own_cm) {
        TimedLaunch tl(K_TRI, st);
        hipError_t e0 = launch_tri_d128(aw, st, p.slots);
        if (e0 != hipSuccess) return e0;
      }
      aw.ckpt_global = p.win > 0;
    }
    {
      TimedLaunch tl(K_BWD_PRE, st);
      hipError_t e0 = launch_bwd_pre_d128(aw, st, p.slots);
      if (e0 != hipSuccess) return e0;
    }
    {
      ScanArgs sa{};
      sa.num_docs = a.f.num_docs;
      sa.H = a.f.H;
      sa.cu = a.f.cu;
      sa.pack = p.pack;
      sa.init = j == 0 ? a.dh_final : p.carry;
      sa.final_out = j == nwin - 1 ? a.dh0 : p.carry;
      sa.states = p.adj;
      sa.kx = p.pack;  // K dS' per chunk, for the per-chunk pass
      sa.kpack = aw.kpack;
      TimedLaunch tl(K_BWD_SCAN, st);
      hipError_t e1;
      if (p.win > 0) {
        sa.win_lo = aw.f.win_lo;
        sa.win_len = p.win;
        sa.units = a.f.num_docs;
        e1 = launch_scan_d128(sa, true, st);
      } else {
        e1 = scan_d128_runs(sa, true, a.f.scan_span, a.f.scan_units, a.f.scan_ws, st, own_cm ? nullptr : a.fwd_maps);
      }
      if (e1 != hipSuccess) return e1;
    }
    TimedLaunch tl(K_BWD_CHUNK, st);
    hipError_t e2 = launch_bwd_chunk_d128(aw, st, p.slots);
    if (e2 != hipSuccess) return e2;
  }
  return hipSuccess;
}

template <typename IO, int D>
static hipError_t launch_bwd_t(const BwdArgs &a_in, hipStream_t st) {
  using Cfg = BwdCfg<IO, D>;
  BwdArgs a = a_in;
  const FwdArgs &f = a.f;
  const int pairs = f.num_docs * f.H;
  const int groups = (pairs + 7) / 8;
  const int64_t slots = a.T / Cfg::C + f.num_docs;
  a.tri = reinterpret_cast<float *>(a.workspace) + (size_t)slots * f.H * D * D;
  {
    TimedLaunch tl(K_BWD_SCAN, st);
    hipLaunchKernelGGL((gdn_bwd_scan_kernel<IO, D>), dim3((unsigned)(groups * 8 * Cfg::NTILE)), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (slots > 0) {
    TimedLaunch tl(K_BWD_CHUNK, st);
    hipLaunchKernelGGL((gdn_bwd_chunk_kernel<IO, D>), dim3((unsigned)(slots * f.H)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_bwd(const BwdArgs &a, hipStream_t st, const BwdPlan *plan) {
  if (a.f.num_docs == 0) return hipSuccess;
  if (a.f.bf16 && a.f.D == 128) return launch_bwd_chunked(a, st, plan);
  if (a.f.bf16) return launch_bwd_t<u16, 16>(a, st);
  return a.f.D == 16 ? launch_bwd_t<float, 16>(a, st) : hipErrorInvalidValue;
}

}  // namespace flare
