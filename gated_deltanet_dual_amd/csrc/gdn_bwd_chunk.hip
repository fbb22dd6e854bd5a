// gdn_bwd_chunk.hip -- per-chunk gradient kernel of the dual-stream backward
// for bf16 io at d_k = d_v = 128 (the other shapes use the generic kernel in
// gdn_bwd.hip).  The algebra is the one written out at the top of gdn_bwd.hip;
// only the schedule differs.
//
// One workgroup of 8 waves per (chunk slot, head), fully parallel over chunks.
//   phase 0  q, k, q~, k~ rows, gates and the chunk matrices of the
//            chunk-matrix pass (T, T~ and the weighted masked Grams Mwo, Mwq,
//            Mwk, Mw~, gdn_tri.hip) -> LDS.
//   phase 1  wave w owns d_v columns [16w, 16w + 16).  Every C x 16 quantity of
//            the chunk -- K S_c, U, the noisy reads r_q, r_k, u~, the noisy
//            adjoints, dU, drhs -- is computed in MFMA accumulator registers and
//            fed straight back into the next product (slab.h), so the whole
//            column-separable chain runs without LDS round trips or barriers.
//            S_c columns come straight from global memory as B fragments
//            (its rows for phase 2 are read in the same phase, so they come
//            from L2); K dS' is the reverse scan's own product, stored by it
//            in the hand-over; v, v~, do, do~ rows are staged through LDS.
//   phase 2  the products that reduce over d_v: wave w takes up to two of the
//            16 x 16 tiles of the six Gram adjoints that the masks leave
//            non-zero (at most 16 of the 24) and the 16-column d_k tile w of
//            dq, dk, dq~, dk~, with U, u~, drhs, drhs~ shared through LDS.
//   phase 3  Gram adjoints -> Gram-weight gradients (each wave recomputes the
//            raw q/k products of its tiles with MFMA, instead of keeping
//            six unweighted Gram matrices in LDS), their contractions with the
//            q/k rows, gate gradients, stores.
// Nothing is reduced across workgroups, so the result is deterministic.
//
// L2 (the q/k L2 flag, folded into per-row factors as gdn_l2.hip describes):
// the same kernel on the transformed problem -- folded write strengths from
// the gate load, v' = v / r_k, the output gradient r_q do -- then the
// gradients mapped back: dv = dv' / r_k, db = db' r_k^2,
// dq = dq' - r_q^2 q (q . dq'), dk = dk' + r_k^2 k (dv' . v' - 2 b' db'),
// and the same for the noisy stream.
#include "bwd_common.h"
#include "chunk_common.h"
#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"
#include "slab.h"
#include "timing.h"

namespace flare {

namespace {

constexpr int kC = 32, kD = 128, kNW = 8, kNT = 64 * kNW;
constexpr int kLDX = kD + 8, kLDP = kD + 8, kLDG = kC + 8, kLDQ = kC + 4;
enum { P_G = 0, P_GN, P_B, P_BN, P_GP, P_GE, P_C, P_DV, P_DVN, P_NUM };
enum { A_U = 0, A_UN, A_DRHS, A_DRN };
// the chunk matrices (T, T~, Mwo, Mwq, Mwk, Mw~) as bf16 hi / lo planes in the
// orientation each product reads them (_N as stored, _T transposed)
enum { Q_T_N = 0, Q_T_T, Q_TN_N, Q_TN_T, Q_MWO_T, Q_MWQ_N, Q_MWQ_T, Q_MWK_N, Q_MWK_T, Q_MWN_T, Q_NUM };
// per-row gate factors, formed once per chunk:
//   GF_M = G_i, GF_P = G_{p_i - 1} (1 at p_i = 0), GF_E = G~ at the end of i's
//   block, GF_C = G_C / G_i, GF_D = b_i G_C / G_i, GF_N = G~_i
enum { GF_M = 0, GF_P, GF_E, GF_C, GF_D, GF_N, GF_NUM };
static_assert(6 * 2 * 2 * kC * kLDG <= 4 * 2 * kC * kLDP, "dG planes must fit in the d_v arrays");

struct Chunk2Smem {
  alignas(16) u16 x[4][kC][kLDX];       // q, k, q~, k~ ; at the end the staging of dq, dk, dq~, dk~
  alignas(16) u16 cq[Q_NUM][2][kC][kLDQ];  // T, T~ and the weighted masked Grams, bf16 hi / lo planes
  // U, u~, drhs, drhs~ for the d_v reductions as bf16 hi / lo planes (each
  // value split once, by the wave that computed it); after those reductions
  // the same bytes hold the Gram-weight gradients dG, [6][orientation][hi, lo][kC][kLDG]
  alignas(16) u16 arrp[4][2][kC][kLDP];
  alignas(16) float lg[kC], beta[kC], lgn[kC], betan[kC];
  alignas(16) float part[kNW][P_NUM][kC];  // per-wave gate-gradient partials
  alignas(16) float plgc[kNW];
  alignas(16) float gsum[2][kC];
  alignas(16) float gf[GF_NUM][kC];
  alignas(16) float alpha[2][kC];        // a, a~ of the chunk's rows (1 past the end / in the prompt)
  alignas(16) float tot[P_NUM][kC];      // the per-wave gate partials summed over the waves
  alignas(16) float fac[4][kC];          // L2: r_q, r_k, r_q~, r_k~ of the chunk's rows
  alignas(16) float vsc[2][kC];          // L2: 1 / r_k, 1 / r_k~
};
// L2, after phase 1 (in the bytes of the chunk-matrix planes, dead by then):
// per-wave row partials of q . dq' and q~ . dq~', and the per-row dk terms
struct L2Late {
  float qdot[kNW][2][kC];
  float ck[2][kC];
};
static_assert(sizeof(L2Late) <= sizeof(((Chunk2Smem *)nullptr)->cq), "L2 scratch must fit in the plane bytes");

// 16-byte row fragment of a [T, H, D] bf16 tensor straight from global memory:
// rows c0 + row0 + (l & 15), columns k0 + 8 (l >> 4) .. +7.  The load is
// unconditional, from a row clamped into the document, and its value is left
// untouched (no wait); frag_mask zeroes rows past the document end (and noisy
// prompt rows when noisy) when it is consumed.
__device__ __forceinline__ uint4 gfrag_raw(const u16 *src, int H, int h, int64_t t0g, int c0, int n, int row0,
                                          int k0) {
  const int l = lane_id();
  const int tpos = c0 + row0 + (l & 15);
  return *reinterpret_cast<const uint4 *>(src + ((t0g + min(tpos, n - 1)) * H + h) * kD + k0 + 8 * (l >> 4));
}
// The same for a noisy-stream tensor: a prompt row (masked by frag_mask) is
// read from the clean twin's same row, which the same lane loads too.
__device__ __forceinline__ uint4 gfrag_raw_noisy(const u16 *src, const u16 *clean, int H, int h, int64_t t0g, int c0,
                                                int n, int P, int row0, int k0) {
  const int l = lane_id();
  const int tpos = c0 + row0 + (l & 15);
  return *reinterpret_cast<const uint4 *>((tpos < P ? clean : src) + ((t0g + min(tpos, n - 1)) * H + h) * kD + k0 +
                                          8 * (l >> 4));
}
__device__ __forceinline__ bf16x8 frag_mask(const uint4 &v, int c0, int n, int P, bool noisy, int row0) {
  const int tpos = c0 + row0 + (lane_id() & 15);
  const bool ok = tpos < n && (!noisy || tpos >= P);
  return __builtin_bit_cast(bf16x8, ok ? v : make_uint4(0u, 0u, 0u, 0u));
}

// The Gram tiles some position of the chunk's masks lets through, bit t for
// tile (m = t / 4, rows 16 ((t >> 1) & 1) .., columns 16 (t & 1) ..) of the
// six Gram adjoints, in the order Mo, Mq, Mk, M~, A, A~ (B the block size, a
// power of two up to 32; p_i = i & -B the start of row i's block):
//   Mo (j <= i), A (j < i): all but the upper right tile
//   Mq, Mk (j < p_i): tile (ti, tj) iff 16 tj < max p_i over its rows
//   M~ (j in i's block): the diagonal tiles, all four when B = 32
//   A~ (j < i in i's block): none when B = 1, else as M~ but not upper right
// Without noisy rows only Mo and A.
__device__ __forceinline__ uint32_t gram_live_tiles(int B, bool has_noisy) {
  uint32_t live = 0;
#pragma unroll
  for (int t = 0; t < 24; ++t) {
    const int m = t >> 2, ti = (t >> 1) & 1, tj = t & 1;
    bool on;
    if (m == 0 || m == 4) on = !(ti == 0 && tj == 1);
    else if (!has_noisy) on = false;
    else if (m == 1 || m == 2) on = 16 * tj < ((16 * ti + 15) & -B);
    else if (m == 3) on = B == 32 || ti == tj;
    else on = B > 1 && (ti == tj || (B == 32 && ti == 1));
    live |= on ? 1u << t : 0u;
  }
  return live;
}
// Index of the n-th (from 0) set bit of x, or -1 (x and n wave-uniform).
__device__ __forceinline__ int nth_set_bit(uint32_t x, int n) {
  for (int k = 0; k < n && x; ++k) x &= x - 1;
  return x ? __builtin_ctz(x) : -1;
}

}  // namespace

template <bool L2>
__global__ __launch_bounds__(kNT) void gdn_bwd_chunk_d128_kernel(BwdArgs a) {
  constexpr int C = kC, D = kD, NT = kNT, LDX = kLDX, LDP = kLDP, LDG = kLDG, LDQ = kLDQ;
  __shared__ Chunk2Smem sm;
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
  const int64_t sslot = a.ckpt_global ? (int64_t)(f.cu[doc] / C) + doc + c : slot;
  const float *Sc = a.ckpt_in + (sslot * H + h) * (size_t)D * D;
  const float *dSn = reinterpret_cast<const float *>(a.workspace) + ((int64_t)slot * H + h) * (size_t)D * D;
  const u16 *const pq = reinterpret_cast<const u16 *>(f.q), *const pk = reinterpret_cast<const u16 *>(f.k);
  const u16 *const pqn = reinterpret_cast<const u16 *>(f.qn), *const pkn = reinterpret_cast<const u16 *>(f.kn);
  const u16 *const pv = reinterpret_cast<const u16 *>(f.v), *const pvn = reinterpret_cast<const u16 *>(f.vn);
  const u16 *const pdo = reinterpret_cast<const u16 *>(a.d_o), *const pdon = reinterpret_cast<const u16 *>(a.d_on);
  const int col0 = 16 * wave;  // this wave's d_v slab (phase 1) and d_k tile (phase 2)

  // ================================================================ phase 0
  // every global load of the phase first, so they are all in flight together:
  // q, k, q~, k~ rows and v, v~, do, do~ rows (4 + 4 16-byte units per
  // thread), gates, T and T~ (one float4 per thread), S_c and dS' columns.
  constexpr int RU = D / 8, PU = C * RU, UX = 4 * PU / NT;
  uint4 xr[UX];
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    const int tpos = c0 + row;
    const bool ok = tpos < n && (m < 2 || tpos >= P);
    // a noisy prompt row (zeroed here) is read from the clean twin this thread loads too
    const u16 *src = m == 0 || (m == 2 && tpos < P) ? pq : m == 1 || (m == 3 && tpos < P) ? pk : m == 2 ? pqn : pkn;
    const uint4 v = *reinterpret_cast<const uint4 *>(src + ((t0g + min(tpos, n - 1)) * H + h) * D + cu16 * 8);
    xr[e] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  // the gate value raw (no use yet, so no wait on the loads issued before it)
  const float graw = tid < 4 * C ? gate_load_raw(f, t0g, c0, n, h, tid) : 0.f;
  float l2r = 1.f;  // L2, thread tid < 128: factor tid / 32 of row tid % 32
  if (L2 && tid < 4 * C) {
    const float *fr = reinterpret_cast<const float *>(f.l2f + (t0g + min(c0 + (tid & (C - 1)), n - 1)) * H + h);
    l2r = fr[tid / C];
  }
  // the six chunk matrices: thread tid takes 4 consecutive entries of a row
  // (8 threads per row, the matrix the same across a wave), read once, only
  // the parts that can be non-zero (exec-masked loads; the rest is zero)
  float4 tri4[3];
  const float *const trec = a.tri + ((size_t)slot * H + h) * 6 * C * C;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int u = j * NT + tid, mtx = __builtin_amdgcn_readfirstlane(u >> 8);
    const int row = (u & 255) >> 3, col = 4 * (u & 7);
    tri4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cm_half_live(mtx, row, col & 16, B, has_noisy)) tri4[j] = ld_nt_f4(trec + 4 * cm_f4_index(mtx, row, col));
  }
  // v, v~, do, do~ rows: staged through LDS (the bytes of the d_v arrays, which
  // phase 1 fills only after every wave has taken its slab from them)
  uint4 vr[UX];
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    // (a noisy prompt row, zeroed when staged, is read from the clean twin this thread loads too)
    const bool pr = c0 + row < P;
    const u16 *src = m == 0 || (m == 1 && pr) ? pv : m == 1 ? pvn : m == 2 || pr ? pdo : pdon;
    vr[e] = *reinterpret_cast<const uint4 *>(src + ((t0g + min(c0 + row, n - 1)) * H + h) * D + cu16 * 8);
  }
  u16 (*const vst)[C][LDX] = reinterpret_cast<u16 (*)[C][LDX]>(&sm.arrp[0][0][0][0]);
  // S_c columns of the slab (k = 32 ks + 8 g + e over d_k), converted to
  // B fragments after the Gram phase
  float xs[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[ks][e] = Sc[(size_t)(32 * ks + 2 * g4 + e) * D + col0 + cl];
  // rows [16 wave, 16 wave + 16) of S_c for the d_k tile of dq..dk~ (raw fp32,
  // held to phase 2): read while the workgroup's column reads of the same
  // state are in flight, so they come from L2
  float4 rsc[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const size_t off = (size_t)(col0 + cl) * D + 32 * ks + 2 * g4;
    rsc[ks][0] = *reinterpret_cast<const float4 *>(Sc + off);
    rsc[ks][1] = *reinterpret_cast<const float4 *>(Sc + off + 4);
  }
  // K dS' of the slab, as the reverse scan formed it in its step (slab layout)
  Slab KD;
  {
    const floatx4 *kxp = reinterpret_cast<const floatx4 *>(a.pack + ((size_t)slot * H + h) * kPackWords + kPackR) +
                         wave * (8 * 64);
    KD.t[0] = __builtin_nontemporal_load(&kxp[lane]);  // read once
    KD.t[1] = __builtin_nontemporal_load(&kxp[64 + lane]);
  }
  // LDS: zero the partials, then the loaded rows, the chunk matrices, gates
  for (int e = tid; e < kNW * P_NUM * C; e += NT) (&sm.part[0][0][0])[e] = 0.f;
  lds_barrier();
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    *reinterpret_cast<uint4 *>(&sm.x[m][row][cu16 * 8]) = xr[e];
    // v, v~, do, do~: rows past the document end, and the noisy ones' prompt rows, read 0
    const int tpos = c0 + row;
    const bool ok = tpos < n && ((m & 1) == 0 || tpos >= P);
    *reinterpret_cast<uint4 *>(&vst[m][row][cu16 * 8]) = ok ? vr[e] : make_uint4(0u, 0u, 0u, 0u);
  }
  // the chunk matrices -> hi / lo planes: 4 consecutive entries of a row per
  // thread, one 8-byte write per plane as stored, four 2-byte writes per plane
  // transposed (the matrix index is the same across a wave)
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int u = j * NT + tid, which = u / (C * C / 4);
    const int row = (u & 255) >> 3, col = 4 * (u & 7);
    const float x4[4] = {tri4[j].x, tri4[j].y, tri4[j].z, tri4[j].w};
    u16 hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hb[e] = f2bf(x4[e]);
      lb[e] = f2bf(x4[e] - bf2f(hb[e]));
    }
    const int qn = which == 0 ? Q_T_N : which == 1 ? Q_TN_N : which == 3 ? Q_MWQ_N : which == 4 ? Q_MWK_N : -1;
    const int qt = which == 0 ? Q_T_T : which == 1 ? Q_TN_T : which == 2 ? Q_MWO_T : which == 3 ? Q_MWQ_T
                 : which == 4 ? Q_MWK_T : Q_MWN_T;
    if (qn >= 0) {
      *reinterpret_cast<uint2 *>(&sm.cq[qn][0][row][col]) =
          make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
      *reinterpret_cast<uint2 *>(&sm.cq[qn][1][row][col]) =
          make_uint2(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.cq[qt][0][col + e][row] = hb[e];
      sm.cq[qt][1][col + e][row] = lb[e];
    }
  }
  const float gval = gate_fix(graw, c0, n, P, tid);
  if (tid < 4 * C) gate_scan(gval, B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  if (tid < C) sm.alpha[0][tid] = gval;
  else if (tid >= 2 * C && tid < 3 * C) sm.alpha[1][tid - 2 * C] = gval;
  if (L2 && tid < 4 * C) {
    sm.fac[tid / C][tid & (C - 1)] = l2r;
    if ((tid / C) & 1) sm.vsc[tid / (2 * C)][tid & (C - 1)] = l2r > 0.f ? 1.f / l2r : 0.f;
  }
  lds_barrier();

  const float lgC = sm.lg[C - 1];
  if (tid < C) {  // the gate factor table, visible after the next barrier
    const int i = tid, pi = (i & -B);
    const float ec = __expf(lgC - sm.lg[i]);
    sm.gf[GF_M][i] = __expf(sm.lg[i]);
    sm.gf[GF_P][i] = pi > 0 ? __expf(sm.lg[pi - 1]) : 1.f;
    sm.gf[GF_E][i] = __expf(sm.lgn[pi + B - 1]);
    sm.gf[GF_C][i] = ec;
    sm.gf[GF_D][i] = sm.beta[i] * ec;
    sm.gf[GF_N][i] = __expf(sm.lgn[i]);
  }
  auto Gm = [&](int i) { return sm.gf[GF_M][i]; };
  auto Gp = [&](int i) { return sm.gf[GF_P][i]; };
  auto Ge = [&](int i) { return sm.gf[GF_E][i]; };
  auto Dd = [&](int i) { return sm.gf[GF_D][i]; };
  auto Gn = [&](int i) { return sm.gf[GF_N][i]; };
  auto resp_row = [&](int i) { return c0 + i < n && c0 + i >= P; };

  bf16x8 sbh[4], sbl[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) split8(xs[ks], sbh[ks], sbl[ks]);

  // ---- X S_c products
  Slab KS = slab_zero(), QS = slab_zero(), QNS = slab_zero(), KNS = slab_zero();
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 ak = frag_bf16(&sm.x[1][0][0], LDX, 16 * tr, 32 * ks);
      const bf16x8 aq = frag_bf16(&sm.x[0][0][0], LDX, 16 * tr, 32 * ks);
      mma_bf16(KS.t[tr], ak, sbh[ks]);
      mma_bf16(KS.t[tr], ak, sbl[ks]);
      mma_bf16(QS.t[tr], aq, sbh[ks]);
      if (has_noisy) {
        const bf16x8 aqn = frag_bf16(&sm.x[2][0][0], LDX, 16 * tr, 32 * ks);
        const bf16x8 akn = frag_bf16(&sm.x[3][0][0], LDX, 16 * tr, 32 * ks);
        mma_bf16(QNS.t[tr], aqn, sbh[ks]);
        mma_bf16(QNS.t[tr], aqn, sbl[ks]);
        mma_bf16(KNS.t[tr], akn, sbh[ks]);
        mma_bf16(KNS.t[tr], akn, sbl[ks]);
      }
    }
  // this wave's v, v~, do, do~ slabs (taken before the barrier: after it, waves
  // write the d_v arrays over the staged rows)
  auto slab_of = [&](int m) {
    Slab sl;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) sl.t[tr][r] = bf2f(vst[m][slab_row(tr, r)][col0 + cl]);
    return sl;
  };
  Slab V = slab_of(0), VN = slab_of(1), DO = slab_of(2), DON = slab_of(3);
  if constexpr (L2) {  // v' = v / r_k and the output gradient r_q do (both streams)
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        V.t[tr][r] *= sm.vsc[0][i];
        VN.t[tr][r] *= sm.vsc[1][i];
        DO.t[tr][r] *= sm.fac[0][i];
        DON.t[tr][r] *= sm.fac[2][i];
      }
  }
  lds_barrier();  // the Gram matrices visible

  // ================================================================ phase 1
  float pg[2][4], pgn[2][4], pb[2][4], pgp[2][4], pge[2][4], pc[2][4];
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) pg[tr][r] = pgn[tr][r] = pb[tr][r] = pgp[tr][r] = pge[tr][r] = pc[tr][r] = 0.f;

  // rhs = v - G K S_c ; U = T rhs
  Slab rhs;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = slab_row(tr, r);
      rhs.t[tr][r] = V.t[tr][r] - Gm(i) * KS.t[tr][r];
      pg[tr][r] += s * Gm(i) * row_sum16(QS.t[tr][r] * DO.t[tr][r]);  // d gamma_i from o_i = s G_i q_i S_c
    }
  Slab U = slab_zero();
  cc_mul_planes<3>(U, &sm.cq[Q_T_N][0][0][0], &sm.cq[Q_T_N][1][0][0], LDQ, rhs);

  // noisy reads and block: r_q, r_k, u~ ; noisy adjoints dr_q, du~, drhs~, dr_k
  Slab UN = slab_zero(), DRQ = slab_zero(), DRN = slab_zero(), DUN = slab_zero();
  if (has_noisy) {
    Slab RQ, RK, RQ0, RK0;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        RQ0.t[tr][r] = Gp(i) * QNS.t[tr][r];
        RK0.t[tr][r] = Gp(i) * KNS.t[tr][r];
      }
    RQ = RQ0;
    RK = RK0;
    cc_mul_planes<3>(RQ, &sm.cq[Q_MWQ_N][0][0][0], &sm.cq[Q_MWQ_N][1][0][0], LDQ, U);  // + Mq diag(b) U
    cc_mul_planes<3>(RK, &sm.cq[Q_MWK_N][0][0][0], &sm.cq[Q_MWK_N][1][0][0], LDQ, U);
    Slab rhsn;
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) rhsn.t[tr][r] = VN.t[tr][r] - Gn(slab_row(tr, r)) * RK.t[tr][r];
    cc_mul_planes<3>(UN, &sm.cq[Q_TN_N][0][0][0], &sm.cq[Q_TN_N][1][0][0], LDQ, rhsn);
    // du~ = s diag(b~) M~^T do~ = s Mw~^T do~
    Slab dun = slab_zero();
    cc_mul_planes<L2 ? 3 : 2>(dun, &sm.cq[Q_MWN_T][0][0][0], &sm.cq[Q_MWN_T][1][0][0], LDQ, DON);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        dun.t[tr][r] *= s;
        DRQ.t[tr][r] = s * Ge(i) * DON.t[tr][r];
        const float t = row_sum16(DON.t[tr][r] * RQ.t[tr][r]);
        if (resp_row(i)) pge[tr][r] += s * Ge(i) * t;  // d gamma~ at the block end
      }
    // drhs~ = T~^T du~ (response rows only); dr_k = -G~ drhs~
    cc_mul_planes<3>(DRN, &sm.cq[Q_TN_T][0][0][0], &sm.cq[Q_TN_T][1][0][0], LDQ, dun);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        const float drn = resp_row(i) ? DRN.t[tr][r] : 0.f;
        DRN.t[tr][r] = drn;
        const float gn = Gn(i);
        pgn[tr][r] -= gn * row_sum16(drn * RK.t[tr][r]);
        DUN.t[tr][r] = -gn * drn;
        pgp[tr][r] += row_sum16(DRQ.t[tr][r] * RQ0.t[tr][r] + DUN.t[tr][r] * RK0.t[tr][r]);
      }
  }

  // dU = D K dS' + diag(b) (s Mo^T do + Mq^T dr_q + Mk^T dr_k)
  //    = D K dS' + s Mwo^T do + Mwq^T dr_q + Mwk^T dr_k
  Slab dU = slab_zero();
  cc_mul_planes<L2 ? 3 : 2>(dU, &sm.cq[Q_MWO_T][0][0][0], &sm.cq[Q_MWO_T][1][0][0], LDQ, DO);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) dU.t[tr] *= s;
  if (has_noisy) {
    cc_mul_planes<3>(dU, &sm.cq[Q_MWQ_T][0][0][0], &sm.cq[Q_MWQ_T][1][0][0], LDQ, DRQ);
    cc_mul_planes<3>(dU, &sm.cq[Q_MWK_T][0][0][0], &sm.cq[Q_MWK_T][1][0][0], LDQ, DUN);
  }
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = slab_row(tr, r);
      const float Di = Dd(i);
      const float t = row_sum16(KD.t[tr][r] * U.t[tr][r]);  // d D_i
      pb[tr][r] += t * sm.gf[GF_C][i];
      pg[tr][r] -= t * Di;
      pc[tr][r] += t * Di;
      dU.t[tr][r] = Di * KD.t[tr][r] + dU.t[tr][r];
    }
  // drhs = T^T dU (= dv)
  Slab DRHS = slab_zero();
  cc_mul_planes<3>(DRHS, &sm.cq[Q_T_T][0][0][0], &sm.cq[Q_T_T][1][0][0], LDQ, dU);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = slab_row(tr, r);
      pg[tr][r] -= Gm(i) * row_sum16(DRHS.t[tr][r] * KS.t[tr][r]);
    }
  float pdv[2][4], pdvn[2][4];  // L2: row partials of dv' . v' and dv~' . v~'
  if constexpr (L2) {
    u16 *const gdv = reinterpret_cast<u16 *>(a.dv), *const gdvn = reinterpret_cast<u16 *>(a.dvn);
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        pdv[tr][r] = row_sum16(DRHS.t[tr][r] * V.t[tr][r]);
        pdvn[tr][r] = row_sum16(DRN.t[tr][r] * VN.t[tr][r]);
        // dv = dv' / r_k, dv~ = dv~' / r_k~ (drhs~ is zero outside the response rows)
        if (c0 + i < n) {
          const int64_t off = ((t0g + c0 + i) * H + h) * D + col0 + cl;
          gdv[off] = f2bf(DRHS.t[tr][r] * sm.vsc[0][i]);
          gdvn[off] = f2bf(DRN.t[tr][r] * sm.vsc[1][i]);
        }
      }
  }

  // ---- the four shared C x d_v arrays -> LDS as bf16 hi / lo planes; the hi
  // planes of drhs and drhs~ are dv and dv~ rounded to bf16, stored from there
  // as 16-byte rows once every wave has written its slab
  {
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        const float vals[4] = {U.t[tr][r], UN.t[tr][r], DRHS.t[tr][r], DRN.t[tr][r]};
#pragma unroll
        for (int ai = 0; ai < 4; ++ai) {
          const u16 hb = f2bf(vals[ai]);
          sm.arrp[ai][0][i][col0 + cl] = hb;
          sm.arrp[ai][1][i][col0 + cl] = f2bf(vals[ai] - bf2f(hb));
        }
      }
  }
  // per-row gate partials of this wave (lanes of column 0 own the row sums)
  if (cl == 0) {
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = slab_row(tr, r);
        sm.part[wave][P_G][i] = pg[tr][r];
        sm.part[wave][P_GN][i] = pgn[tr][r];
        sm.part[wave][P_B][i] = pb[tr][r];
        sm.part[wave][P_GP][i] = pgp[tr][r];
        sm.part[wave][P_GE][i] = pge[tr][r];
        sm.part[wave][P_C][i] = pc[tr][r];
        if constexpr (L2) {
          sm.part[wave][P_DV][i] = pdv[tr][r];
          sm.part[wave][P_DVN][i] = pdvn[tr][r];
        }
      }
  }
  // ---- phase 2's do, do~ row fragments (rows 16 tr .., k-step ks over d_v),
  // issued after the phase-1 values are stored, so they arrive during the barrier
  uint4 rfdo[2][4], rfdon[2][4];
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      rfdo[tr][ks] = gfrag_raw(pdo, H, h, t0g, c0, n, 16 * tr, 32 * ks);
      rfdon[tr][ks] = gfrag_raw_noisy(pdon, pdo, H, h, t0g, c0, n, P, 16 * tr, 32 * ks);
    }

  // rows [16 wave, 16 wave + 16) of dS' for the d_k tile of dk, raw fp32, in
  // flight during the Gram adjoints
  float4 rds[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const size_t off = (size_t)(col0 + cl) * D + 32 * ks + 2 * g4;
    rds[ks][0] = *reinterpret_cast<const float4 *>(dSn + off);
    rds[ks][1] = *reinterpret_cast<const float4 *>(dSn + off + 4);
  }
  lds_barrier();
  // ================================================================ phase 2
  {  // <dS', S_c> over rows [16 wave, 16 wave + 16), fp32
    float plg = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        plg += rsc[ks][j].x * rds[ks][j].x + rsc[ks][j].y * rds[ks][j].y + rsc[ks][j].z * rds[ks][j].z +
               rsc[ks][j].w * rds[ks][j].w;
    const float t = xsum32(xsum16(dpp_sum16(plg)));
    if (lane == 0) sm.plgc[wave] = __expf(lgC) * t;
  }
  bf16x8 fdo[2][4], fdon[2][4];
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      fdo[tr][ks] = frag_mask(rfdo[tr][ks], c0, n, P, false, 16 * tr);
      fdon[tr][ks] = frag_mask(rfdon[tr][ks], c0, n, P, true, 16 * tr);
    }
  // Gram adjoints: 6 matrices x 4 tiles, tile t -> (m = t / 4, ti, tj).  Only
  // the tiles the masks leave non-zero are formed (at most 16 of the 24: the
  // masks are lower triangular, and the noisy ones confined to blocks), dealt
  // to the waves in order: wave w takes the (w + 8 jt)-th live tile.
  enum { DM_O = 0, DM_Q, DM_K, DM_N, DM_A, DM_AN };
  const uint32_t live = gram_live_tiles(B, has_noisy);
  const int tl[2] = {nth_set_bit(live, wave), nth_set_bit(live, wave + 8)};
  floatx4 dM[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int t = tl[jt];
    const int m = t >> 2, ti = (t >> 1) & 1, tj = t & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (t >= 0) {
      const int right = (m == DM_N || m == DM_AN) ? A_UN : A_U;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 bh = frag_bf16(&sm.arrp[right][0][0][0], LDP, 16 * tj, 32 * ks);
        const bf16x8 bl = frag_bf16(&sm.arrp[right][1][0][0], LDP, 16 * tj, 32 * ks);
        if (m == DM_O || m == DM_Q || m == DM_N) {  // left operand do / do~ (exact bf16)
          // ti is wave-dependent: select between registers, never index them
          const bf16x8 a0 = m == DM_O ? fdo[0][ks] : fdon[0][ks];
          const bf16x8 a1 = m == DM_O ? fdo[1][ks] : fdon[1][ks];
          const bf16x8 ah = ti == 0 ? a0 : a1;
          mma_bf16(acc, ah, bh);
          mma_bf16(acc, ah, bl);
        } else {
          const int left = m == DM_A ? A_DRHS : A_DRN;
          const bf16x8 ah = frag_bf16(&sm.arrp[left][0][0][0], LDP, 16 * ti, 32 * ks);
          const bf16x8 al = frag_bf16(&sm.arrp[left][1][0][0], LDP, 16 * ti, 32 * ks);
          mma_bf16(acc, ah, bh);
          mma_bf16(acc, ah, bl);
          mma_bf16(acc, al, bh);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + g4 + r;
        float sc = 1.f;
        if (m == DM_O || m == DM_N) sc = s;
        else if (m == DM_Q) sc = s * Ge(i);
        else if (m == DM_K) sc = -Gn(i);
        else sc = -1.f;
        if constexpr (L2) {  // the products with the raw do / do~ rows: r_q do
          if (m == DM_O) sc *= sm.fac[0][i];
          else if (m == DM_Q || m == DM_N) sc *= sm.fac[2][i];
        }
        acc[r] *= sc;
      }
    }
    dM[jt] = acc;
  }

  // d_k tile `wave` of dq, dk, dq~, dk~: the d_v contractions with S_c, dS'
  floatx4 dq[2], dk[2], dqn[2], dkn[2];
  {
    floatx4 a_dq[2], a_dk1[2], a_dk2[2], a_dqn[2], a_dkn[2];
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
      a_dq[tr] = a_dk1[tr] = a_dk2[tr] = a_dqn[tr] = a_dkn[tr] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 sh, sl, dh, dl;
      {
        const float x0[8] = {rsc[ks][0].x, rsc[ks][0].y, rsc[ks][0].z, rsc[ks][0].w,
                             rsc[ks][1].x, rsc[ks][1].y, rsc[ks][1].z, rsc[ks][1].w};
        const float x1[8] = {rds[ks][0].x, rds[ks][0].y, rds[ks][0].z, rds[ks][0].w,
                             rds[ks][1].x, rds[ks][1].y, rds[ks][1].z, rds[ks][1].w};
        split8(x0, sh, sl);
        split8(x1, dh, dl);
      }
#pragma unroll
      for (int tr = 0; tr < 2; ++tr) {
        const bf16x8 ado = fdo[tr][ks];
        mma_bf16(a_dq[tr], ado, sh);
        mma_bf16(a_dq[tr], ado, sl);
        bf16x8 ah = frag_bf16(&sm.arrp[A_DRHS][0][0][0], LDP, 16 * tr, 32 * ks);
        bf16x8 al = frag_bf16(&sm.arrp[A_DRHS][1][0][0], LDP, 16 * tr, 32 * ks);
        mma_bf16(a_dk1[tr], ah, sh);
        mma_bf16(a_dk1[tr], ah, sl);
        mma_bf16(a_dk1[tr], al, sh);
        ah = frag_bf16(&sm.arrp[A_U][0][0][0], LDP, 16 * tr, 32 * ks);
        al = frag_bf16(&sm.arrp[A_U][1][0][0], LDP, 16 * tr, 32 * ks);
        mma_bf16(a_dk2[tr], ah, dh);
        mma_bf16(a_dk2[tr], ah, dl);
        mma_bf16(a_dk2[tr], al, dh);
        if (has_noisy) {
          const bf16x8 adon = fdon[tr][ks];
          mma_bf16(a_dqn[tr], adon, sh);
          mma_bf16(a_dqn[tr], adon, sl);
          ah = frag_bf16(&sm.arrp[A_DRN][0][0][0], LDP, 16 * tr, 32 * ks);
          al = frag_bf16(&sm.arrp[A_DRN][1][0][0], LDP, 16 * tr, 32 * ks);
          mma_bf16(a_dkn[tr], ah, sh);
          mma_bf16(a_dkn[tr], ah, sl);
          mma_bf16(a_dkn[tr], al, sh);
        }
      }
    }
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * tr + g4 + r;
        dq[tr][r] = s * Gm(i) * a_dq[tr][r];
        dk[tr][r] = -Gm(i) * a_dk1[tr][r] + Dd(i) * a_dk2[tr][r];
        dqn[tr][r] = Gp(i) * s * Ge(i) * a_dqn[tr][r];
        if constexpr (L2) {
          dq[tr][r] *= sm.fac[0][i];
          dqn[tr][r] *= sm.fac[2][i];
        }
        dkn[tr][r] = -Gp(i) * Gn(i) * a_dkn[tr][r];
      }
  }

  // dv, dv~ rows from the hi planes (drhs~ is zero outside the response rows),
  // before phase 3 reuses the planes' bytes (L2: stored from registers above)
  if constexpr (!L2) {
    u16 *const gdv = reinterpret_cast<u16 *>(a.dv), *const gdvn = reinterpret_cast<u16 *>(a.dvn);
#pragma unroll
    for (int e = 0; e < 2 * PU / NT; ++e) {
      const int u = e * NT + tid;
      const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
      if (c0 + row < n)
        st_nt_u4((m == 0 ? gdv : gdvn) + ((t0g + c0 + row) * H + h) * D + cu16 * 8,
                 *reinterpret_cast<const uint4 *>(&sm.arrp[m == 0 ? A_DRHS : A_DRN][0][row][cu16 * 8]));
    }
  }

  // ================================================================ phase 3
  // Gram adjoints -> dG as bf16 hi / lo planes in both orientations (in the
  // bytes of the d_v arrays, which every wave is done with) + gate partials
  lds_barrier();
  auto dgp = [&](int mtx, int orient, int plane) {  // [32][LDG] u16
    return reinterpret_cast<u16 *>(&sm.arrp[0][0][0][0]) + (((size_t)mtx * 2 + orient) * 2 + plane) * C * LDG;
  };
  {  // the tiles no mask lets through read as zero (both orientations, both
     // planes); without noisy rows only Mo and A are read
    const uint32_t dead = ~live & (has_noisy ? 0xFFFFFFu : 0xF000Fu);
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) {
      const int t = nth_set_bit(dead, wave + 8 * jt);
      if (t < 0) break;
      const int m = t >> 2, ti = (t >> 1) & 1, tj = t & 1;
      const int rr = lane >> 2, c4 = 4 * (lane & 3);
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        *reinterpret_cast<uint2 *>(dgp(m, 0, pl) + (16 * ti + rr) * LDG + 16 * tj + c4) = make_uint2(0u, 0u);
        *reinterpret_cast<uint2 *>(dgp(m, 1, pl) + (16 * tj + rr) * LDG + 16 * ti + c4) = make_uint2(0u, 0u);
      }
    }
  }
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int t = tl[jt];
    if (t < 0) continue;
    const int m = t >> 2, ti = (t >> 1) & 1, tj = t & 1;
    const int i0 = 16 * ti + g4, j = 16 * tj + cl;
    // the raw products x_i . y_j of this tile (bf16 rows, exact products):
    //   Mo: q.k   Mq: q~.k   Mk: k~.k   M~: q~.k~   A: k.k   A~: k~.k~
    // gated and masked below:
    //   Mo : w = b, e = lg_i, f = lg_j, mask j <= i
    //   Mq/Mk : w = b, e = lg[p_i - 1], mask j < p_i (resp)
    //   M~ : w = b~, e = lgn[end(i)], f = lgn_j, mask same block (resp)
    //   A : e = lg_i, mask j < i ;  A~ : e = lgn_i, mask j < i in the block of i (resp)
    const int xl = m == DM_O ? 0 : m == DM_Q || m == DM_N ? 2 : m == DM_A ? 1 : 3;
    const int xr_ = m == DM_O || m == DM_Q || m == DM_K || m == DM_A ? 1 : 3;
    floatx4 raw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      mma_bf16(raw, frag_bf16(&sm.x[xl][0][0], LDX, 16 * ti, 32 * ks), frag_bf16(&sm.x[xr_][0][0], LDX, 16 * tj, 32 * ks));
    const bool noisyw = (m == DM_N || m == DM_AN);
    const float wj = noisyw ? sm.betan[j] : sm.beta[j];
    const float fj = noisyw ? sm.lgn[j] : sm.lg[j];
    float colw = 0.f, colf = 0.f;
    float dgv[4], rsum[4];
    const int pbase = (m == DM_O || m == DM_A) ? P_G : (m == DM_Q || m == DM_K) ? P_GP : m == DM_N ? P_GE : P_GN;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r;
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
      const float dm = dM[jt][r];
      const float E = mask ? __expf(ei - fj) : 0.f;
      const float mw = raw[r] * E;  // the unweighted masked Gram
      const float mfull = mw * wj;
      dgv[r] = dm * E * wj;  // dG[i][j]
      const float dd = dm * mfull;
      rsum[r] = row_sum16(dd);  // row part d e_i
      colf += dd;
      colw += dm * mw;
    }
    // dG[i0 .. i0+3][j]: orientation 0 rows i (scalar halves), orientation 1
    // rows j (the four i are adjacent: one 8-byte write per plane)
    {
      uint32_t hw[2], lw[2];
      u16 hb[4], lb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hb[r] = f2bf(dgv[r]);
        lb[r] = f2bf(dgv[r] - bf2f(hb[r]));
        dgp(m, 0, 0)[(i0 + r) * LDG + j] = hb[r];
        dgp(m, 0, 1)[(i0 + r) * LDG + j] = lb[r];
      }
      hw[0] = hb[0] | ((uint32_t)hb[1] << 16); hw[1] = hb[2] | ((uint32_t)hb[3] << 16);
      lw[0] = lb[0] | ((uint32_t)lb[1] << 16); lw[1] = lb[2] | ((uint32_t)lb[3] << 16);
      *reinterpret_cast<uint2 *>(dgp(m, 1, 0) + j * LDG + i0) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2 *>(dgp(m, 1, 1) + j * LDG + i0) = make_uint2(lw[0], lw[1]);
    }
    // row parts of the tile's 4 rows of this lane group, one read-modify-write
    if (cl == 0) {
      float4 *pp = reinterpret_cast<float4 *>(&sm.part[wave][pbase][i0]);
      const float4 o = *pp;
      *pp = make_float4(o.x + rsum[0], o.y + rsum[1], o.z + rsum[2], o.w + rsum[3]);
    }
    // column parts: over the 4 row groups of the tile
    colf = xsum32(xsum16(colf));
    colw = xsum32(xsum16(colw));
    if (lane < 16) {
      if (noisyw) {
        sm.part[wave][P_GN][j] -= colf;
        sm.part[wave][P_BN][j] += colw;
      } else {
        sm.part[wave][P_G][j] -= colf;
        sm.part[wave][P_B][j] += colw;
      }
    }
  }
  lds_barrier();
  L2Late *const late = reinterpret_cast<L2Late *>(&sm.cq[0][0][0][0]);
  if (L2 && tid < 2 * C) {
    // the per-row dk terms r_k^2 (dv' . v' - 2 b' db'), read after the next barrier
    const int i = tid & (C - 1), ns = tid / C;
    float dvv = 0.f, dbb = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      dvv += sm.part[w][ns ? P_DVN : P_DV][i];
      dbb += sm.part[w][ns ? P_BN : P_B][i];
    }
    const float rk = sm.fac[ns ? 3 : 1][i];
    late->ck[ns][i] = rk * rk * (dvv - 2.f * (ns ? sm.betan[i] : sm.beta[i]) * dbb);
  }

  // Gram contractions for d_k tile `wave`: B fragments are columns of q, k, q~, k~
  {
    const bf16x8 bq = frag_bf16_T(&sm.x[0][0][0], LDX, col0, 0);
    const bf16x8 bk = frag_bf16_T(&sm.x[1][0][0], LDX, col0, 0);
    const bf16x8 bqn = frag_bf16_T(&sm.x[2][0][0], LDX, col0, 0);
    const bf16x8 bkn = frag_bf16_T(&sm.x[3][0][0], LDX, col0, 0);
    // A = dG (orientation 0) or dG^T (orientation 1) rows ra .. ra + 15
    auto gmul = [&](floatx4 &acc, int mtx, int orient, int ra, const bf16x8 &b) {
      const bf16x8 ah = frag_bf16(dgp(mtx, orient, 0), LDG, ra, 0);
      const bf16x8 al = frag_bf16(dgp(mtx, orient, 1), LDG, ra, 0);
      mma_bf16(acc, ah, b);
      mma_bf16(acc, al, b);
    };
#pragma unroll
    for (int tr = 0; tr < 2; ++tr) {
      const int ra = 16 * tr;
      gmul(dq[tr], DM_O, 0, ra, bk);   // dq += dGo k
      gmul(dk[tr], DM_O, 1, ra, bq);   // dk += dGo^T q + dGA k + dGA^T k
      gmul(dk[tr], DM_A, 0, ra, bk);
      gmul(dk[tr], DM_A, 1, ra, bk);
      if (has_noisy) {
        gmul(dk[tr], DM_Q, 1, ra, bqn);   // + dGq^T q~ + dGk^T k~
        gmul(dk[tr], DM_K, 1, ra, bkn);
        gmul(dqn[tr], DM_Q, 0, ra, bk);   // dq~ += dGq k + dG~ k~
        gmul(dqn[tr], DM_N, 0, ra, bkn);
        gmul(dkn[tr], DM_K, 0, ra, bk);   // dk~ += dGk k + dGA~ k~ + dGA~^T k~ + dG~^T q~
        gmul(dkn[tr], DM_AN, 0, ra, bkn);
        gmul(dkn[tr], DM_AN, 1, ra, bkn);
        gmul(dkn[tr], DM_N, 1, ra, bqn);
      }
    }
  }
  if constexpr (L2) {  // row partials of q . dq' and q~ . dq~' over this d_k tile
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * tr + g4 + r;
        const float pq = row_sum16(bf2f(sm.x[0][i][col0 + cl]) * dq[tr][r]);
        const float pqn = row_sum16(bf2f(sm.x[2][i][col0 + cl]) * dqn[tr][r]);
        if (cl == 0) {
          late->qdot[wave][0][i] = pq;
          late->qdot[wave][1][i] = pqn;
        }
      }
  }
  lds_barrier();
  // ---- stage the four d_k-side gradients in the (now free) q/k tiles, then store rows
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * tr + g4 + r;
      const bool rs = resp_row(i);
      if constexpr (L2) {
        // dq = dq' - r_q^2 q (q . dq'), dk = dk' + k r_k^2 (dv' . v' - 2 b' db'), both streams
        float qd = 0.f, qnd = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
          qd += late->qdot[w][0][i];
          qnd += late->qdot[w][1][i];
        }
        const float rq = sm.fac[0][i], rqn = sm.fac[2][i];
        dq[tr][r] -= rq * rq * bf2f(sm.x[0][i][col0 + cl]) * qd;
        dk[tr][r] += bf2f(sm.x[1][i][col0 + cl]) * late->ck[0][i];
        dqn[tr][r] -= rqn * rqn * bf2f(sm.x[2][i][col0 + cl]) * qnd;
        dkn[tr][r] += bf2f(sm.x[3][i][col0 + cl]) * late->ck[1][i];
      }
      sm.x[0][i][col0 + cl] = f2bf(dq[tr][r]);
      sm.x[1][i][col0 + cl] = f2bf(dk[tr][r]);
      sm.x[2][i][col0 + cl] = f2bf(rs ? dqn[tr][r] : 0.f);
      sm.x[3][i][col0 + cl] = f2bf(rs ? dkn[tr][r] : 0.f);
    }
  // ---- gates, step 1: each partial summed over the waves, in wave order
  if (tid < P_NUM * C) {
    const int t = tid / C, i = tid % C;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) v += sm.part[w][t][i];
    sm.tot[t][i] = v;
  }
  lds_barrier();
  {
    constexpr int RU = D / 8;
    u16 *outp[4] = {reinterpret_cast<u16 *>(a.dq), reinterpret_cast<u16 *>(a.dk), reinterpret_cast<u16 *>(a.dqn),
                    reinterpret_cast<u16 *>(a.dkn)};
    for (int u = tid; u < 4 * C * RU; u += NT) {
      const int m = u / (C * RU), rr = u % (C * RU), row = rr / RU, cu16 = rr % RU;
      if (c0 + row >= n) continue;
      u16 *dst = m == 0 ? outp[0] : m == 1 ? outp[1] : m == 2 ? outp[2] : outp[3];
      st_nt_u4(dst + ((t0g + c0 + row) * H + h) * D + cu16 * 8, *reinterpret_cast<const uint4 *>(&sm.x[m][row][cu16 * 8]));
    }
  }
  // ---- gates, step 2 (wave 0; lanes 0-31 the clean rows i, lanes 32-63 the
  // noisy rows): move the boundary terms to the rows they belong to, then
  // d alpha_i = sum over m >= i of d gamma_m (clean: to the chunk end; noisy:
  // to the end of i's block) over alpha_i.  Sums over lanes run as fixed
  // shuffle trees, so the result is the same on every run.
  if (wave == 0) {
    const int i = lane & (C - 1);
    const bool noisy = lane >= C;
    const int ib = i & (B - 1);
    // per-block sums of the block-start reads (clean) / block-end reads (noisy):
    // segmented inclusive prefix over the rows of each block, total at its last row
    float bs = noisy ? sm.tot[P_GE][i] : sm.tot[P_GP][i];
    for (int off = 1; off < B; off <<= 1) {
      const float y = __shfl_up(bs, off, B);
      if (ib >= off) bs += y;
    }
    float v = noisy ? sm.tot[P_GN][i] : sm.tot[P_G][i];
    // clean: the block starting at p = i + 1 reads S_p, whose gates end at row i
    const float next_block = __shfl_down(bs, B, C);
    if (!noisy && ib == B - 1 && i + B < C) v += next_block;
    if (noisy && ib == B - 1) v += bs;
    // clean, last row: the chunk-end terms (<dS', S_c> and the decay of the write strengths)
    float pc = noisy ? 0.f : sm.tot[P_C][i];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) pc += __shfl_xor(pc, off, C);
    if (!noisy && i == C - 1) {
      float pl = 0.f;
      for (int w = 0; w < kNW; ++w) pl += sm.plgc[w];
      v += pl + pc;
    }
    // suffix sums: to the chunk end (clean), to the end of the block (noisy)
    const int seg = noisy ? B : C, is = noisy ? ib : i;
    for (int off = 1; off < C; off <<= 1) {
      const float y = __shfl_down(v, off, C);
      if (is + off < seg) v += y;
    }
    const float db = noisy ? sm.tot[P_BN][i] : sm.tot[P_B][i];
    const int64_t gi = (t0g + c0 + i) * H + h;
    if (c0 + i < n) {
      if (!noisy) {
        a.dalpha[gi] = v / sm.alpha[0][i];
        a.dbeta[gi] = L2 ? db * sm.fac[1][i] * sm.fac[1][i] : db;
      } else {
        const bool rsp = c0 + i >= P;
        a.dalpha_n[gi] = rsp ? v / sm.alpha[1][i] : 0.f;
        a.dbeta_n[gi] = rsp ? (L2 ? db * sm.fac[3][i] * sm.fac[3][i] : db) : 0.f;
      }
    }
  }
}

hipError_t launch_bwd_chunk_d128(const BwdArgs &a, hipStream_t st, int64_t slots) {
  if (a.f.l2f)
    hipLaunchKernelGGL(gdn_bwd_chunk_d128_kernel<true>, dim3((unsigned)(slots * a.f.H)), dim3(kNT), 0, st, a);
  else
    hipLaunchKernelGGL(gdn_bwd_chunk_d128_kernel<false>, dim3((unsigned)(slots * a.f.H)), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
