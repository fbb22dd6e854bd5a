// block_step.hip -- serving block step over a pool of recurrent states.
//
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
// designs item 4: a denoising forward reads the global causal state pool but
// never writes it (EVAL); once the block is fixed, a causal replay of the block
// writes the final state into the pool (COMMIT).  The per-token update is the
// gated delta rule of Key designs item 2.
//
// One workgroup per (request, head) -- two for 32-token blocks, each owning
// half of the state's columns.  The workgroup's part of the d x d fp32 state is
// read once with 16-byte loads and kept in registers: the threads of one
// 4-column quad are adjacent lanes, each holding every NRG-th row, so the sums
// over rows are DPP reductions across those lanes with no LDS partials.  The
// small B x B work (dot products, the unit-triangular solve) runs while the
// state is still arriving.  The B updates are applied in their
// chunked (UT) form so the state is touched by exactly one reduction pass:
//   w_j = S^T k_j, r_l = S^T q_l                      (one pass over S)
//   A_ij = (G_i/G_j) b_j k_i.k_j (j < i), T = (I + A)^-1
//   U = T (V - diag(G) W)
//   EVAL:   o_l = s (G_e r_l + sum_j (G_e/G_j) b_j (q_l.k_j) u_j)   for every l
//   COMMIT: o_t = s (G_t r_t + sum_{j<=t} (G_t/G_j) b_j (q_t.k_j) u_j),
//           S  <- G_e S + sum_j (G_e/G_j) b_j k_j u_j^T            (written back)
//   VERIFY (AR-Trust, Key designs item 4): COMMIT's outputs for K drafted
//           tokens, and the state after every token, S_t = a_t S_{t-1} +
//           b_t k_t u_t^T, written to a candidate buffer; the pool is not
//           written.  A later scatter copies candidate r into the pool once r
//           tokens are accepted.  The same rollback by replay: EVAL with
//           causal reads (COMMIT's outputs, nothing written), then a COMMIT
//           of each request's accepted prefix (per-request token counts).
//   BOUNDARIES (the chunk-then-refine forward): from a chunk-start state, the
//           per-token recurrence over a window of clean tokens, writing the
//           state at every block start it passes.
// with G_i = prod_{m<=i} a_m taken as exp of a cumulative sum of log a.
// Everything is fp32 on the VALU: the step moves ~4 flop per byte of state, far
// below the MI355X fp32 ridge, so the kernel is bound by HBM bandwidth.
#include "device_common.h"
#include "kernels.h"
#include "serving.h"
#include "slab.h"
#include "timing.h"

namespace flare {

// DV: the state columns (d_v) one workgroup owns; D / DV workgroups share a
// (request, head), each with the whole k and q rows and its own columns of v,
// the state and the outputs
template <int D, int DV> struct StepCfg {
  static constexpr int NT = D >= 128 ? 256 : 64;  // threads
  static constexpr int NCQ = DV / 4;              // column quads
  static constexpr int NRG = NT / NCQ;            // row groups: adjacent lanes of one quad
  static constexpr int RPG = D / NRG;             // rows per group (rows rg * RPG + i)
  static constexpr int G = D >= 128 ? 2 : 8;      // vectors per pass (few: registers, occupancy)
  static_assert(NRG == 8 || NRG == 16, "row groups are reduced over 8 or 16 lanes");
  static_assert(D % DV == 0 && NT % DV == 0, "whole column splits");
};

// Sum over the NRG adjacent lanes of a row group (a DPP row or half-row).
template <int NRG>
__device__ __forceinline__ float rowgroup_sum(float x) {
  x += dpp_f32<0xB1>(x);   // xor 1
  x += dpp_f32<0x4E>(x);   // xor 2
  x += dpp_f32<0x141>(x);  // the other quad of the half-row
  if constexpr (NRG == 16) x += dpp_f32<0x140>(x);  // the other half-row
  return x;
}

// CONV: the block inputs are raw projections that go through the serving
// ShortConv first (the request's W - 1 clean history rows, then the block;
// SiLU; q/k L2 norm) -- see BlockStepArgs
// KIND: 0 = EVAL, 1 = COMMIT, 2 = the token-wise state writers (VERIFY and
// BOUNDARIES); the readers carry no state-update registers
// CW: 0 for the plain step, else the widest ShortConv it is built for (its LDS
// staging holds CW - 1 history rows and CW taps per channel)
template <typename IO, int D, int DV, int BMAX, int CW, int KIND>
__global__ __launch_bounds__((StepCfg<D, DV>::NT)) void block_step_kernel(BlockStepArgs a) {
  using Cfg = StepCfg<D, DV>;
  constexpr bool CONV = CW > 0;
  static_assert(!CONV || DV == D, "the ShortConv step keeps whole rows");
  constexpr int NT = Cfg::NT, NRG = Cfg::NRG, RPG = Cfg::RPG, G = Cfg::G;
  constexpr int NSPLIT = D / DV;         // workgroups per (request, head)
  constexpr int NV = 2 * BMAX;           // k vectors then q vectors
  constexpr int EPU = 16 / sizeof(IO);   // io elements per 16 bytes
  constexpr int UPR = D / EPU;           // 16-byte units per row
  constexpr int UPRV = DV / EPU;         // 16-byte units of this workgroup's columns per row
  constexpr int WM1 = CONV ? CW - 1 : 0;  // most history rows
  constexpr int NRAW = CONV ? WM1 + BMAX : 1;
  const int req = blockIdx.x / (a.H * NSPLIT), h = (blockIdx.x / NSPLIT) % a.H;
  const int col0 = (blockIdx.x % NSPLIT) * DV;  // this workgroup's first state / value column
  // table mode: the request's number of real tokens; a BOUNDARIES window
  // runs over exactly the tokens before its last block start (possibly none)
  const int cnt = a.count ? min(max(a.count[req], 0), a.B) : a.B;
  const int B = KIND == 2 && a.mode == 3 ? cnt : a.B;
  // EVAL and COMMIT: B is the block size, a power of two up to 32 (checked by
  // the host), so dividing by it is a shift; the token-wise writers' window
  // counts are arbitrary
  const int lgB = 31 - __clz(B > 0 ? B : 1);
  auto divB = [&](int x) { return KIND == 2 ? x / B : x >> lgB; };
  auto modB = [&](int x) { return KIND == 2 ? x % B : x & (B - 1); };
  if (KIND == 1 && cnt == 0) return;  // a COMMIT of no token leaves the state as it is
  const int t = threadIdx.x;
  const int rg = t % NRG, cq = t / NRG;

  // k_0..k_{B-1} at 0.., q_0..q_{B-1} at BMAX..; rows padded by 4 floats so the
  // 16 rows of a matrix-core fragment fall in different LDS banks
  constexpr int LDXS = D + 4;
  __shared__ __align__(16) float sX[NV][LDXS];
  __shared__ __align__(16) float sV[BMAX][DV];
  __shared__ __align__(16) float sW[NV][DV];   // S^T x for every x in sX (this workgroup's columns)
  __shared__ __align__(16) float sU[BMAX][DV];
  // B x B coefficients, rows 16-byte aligned for broadcast reads: k.k then the
  // UT system A, q.k then the output weights P, the inverse T
  __shared__ __align__(16) float sKK[BMAX][BMAX], sQK[BMAX][BMAX], sT[BMAX][BMAX];
  __shared__ float sG[BMAX], sBeta[BMAX];
  // CONV: the raw rows of q, k, v (history, then the block) as fp32, and the
  // head's conv weights [projection][channel * W + tap]
  __shared__ __align__(16) float sRaw[CONV ? 3 : 1][NRAW][CONV ? D : 4];
  __shared__ __align__(16) float sCW[CONV ? 3 : 1][CONV ? D * (WM1 + 1) : 4];

  const IO *const pk = reinterpret_cast<const IO *>(a.k), *const pq = reinterpret_cast<const IO *>(a.q);
  const IO *const pv = reinterpret_cast<const IO *>(a.v);
  const float *const pal = a.alpha, *const pbe = a.beta;

  const int slot = a.slot_idx ? a.slot_idx[req] : req;
  float *S = a.pool + ((size_t)slot * a.H + h) * D * D + col0;  // row r of the columns at S + r D
  // table mode: the request's first token row
  const int64_t rbase = a.row0 ? (int64_t)a.row0[req] : (int64_t)req * B;
  auto trow = [&](int r) { return rbase + (r < cnt ? r : max(cnt - 1, 0)); };  // loads stay on real rows
  // MF (bf16 io, 32-token blocks, half-row workgroups): the state's pass runs
  // on the matrix cores and the state is held in their operand layout -- wave
  // w's lane (n, g) holds column 16 w + n of its part, rows 32 ks + 8 g + e
  // (ks, e < 4, 8); otherwise the (rg, cq) layout below
  constexpr bool MF = sizeof(IO) == 2 && BMAX == 32 && D == 128 && DV == 64;
  float4 s4[MF ? 1 : RPG];
  float sf[MF ? 4 : 1][8];
  const int wvs = __builtin_amdgcn_readfirstlane(t >> 6), n16 = t & 15, kg = (t & 63) >> 4;
  {
    // 0. the block inputs first (16-byte loads into registers), then the
    //    state: vector-memory results return in issue order, so the small B x B
    //    work below waits only for the inputs while the state is in flight
    constexpr int IU = ((CONV ? 3 * NRAW * UPR : BMAX * (2 * UPR + UPRV)) + NT - 1) / NT;  // input units per thread
    uint4 in_raw[IU];
    const int W1 = CONV ? a.W - 1 : 0;  // history rows
    const int NR = W1 + B;              // raw rows per projection (CONV)
    const size_t C = (size_t)a.H * D;
    const IO *const hist = reinterpret_cast<const IO *>(a.cache);
#pragma unroll
    for (int e = 0; e < IU; ++e) {
      const int u = e * NT + t;
      in_raw[e] = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (CONV) {
        // projection-major [q, k, v][history rows, block rows][16-byte units]
        if (u < 3 * NR * UPR) {
          const int sec = u / (NR * UPR), row = (u / UPR) % NR, cu = u % UPR;
          const IO *src = row < W1 ? hist + (((size_t)slot * W1 + row) * 3 + sec) * C + (size_t)h * D
                                   : (sec == 0 ? pq : sec == 1 ? pk : pv) +
                                         (((size_t)req * B + (row - W1)) * a.H + h) * D;
          in_raw[e] = *reinterpret_cast<const uint4 *>(src + cu * EPU);
        }
      } else if (u < 2 * B * UPR) {  // k and q rows, whole
        const int which = divB(u / UPR), r = modB(u / UPR), cu = u % UPR;
        in_raw[e] = *reinterpret_cast<const uint4 *>((which == 0 ? pk : pq) + ((size_t)trow(r) * a.H + h) * D +
                                                     cu * EPU);
      } else if (u < B * (2 * UPR + UPRV)) {  // v rows, this workgroup's columns
        const int uv = u - 2 * B * UPR, r = uv / UPRV, cu = uv % UPRV;
        in_raw[e] = *reinterpret_cast<const uint4 *>(pv + ((size_t)trow(r) * a.H + h) * D + col0 + cu * EPU);
      }
    }
    // CONV: the head's weights, loaded with the inputs (float4 units)
    constexpr int WUMAX = CONV ? (3 * D * (WM1 + 1) / 4 + NT - 1) / NT : 1;
    float4 cw4[WUMAX];
    if constexpr (CONV) {
      const int per = D * a.W / 4;  // float4 units per projection
#pragma unroll
      for (int e = 0; e < WUMAX; ++e) {
        const int u = e * NT + t;
        cw4[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (u < 3 * per) {
          const int sec = u / per, off = u % per;
          cw4[e] = *reinterpret_cast<const float4 *>(a.cw[sec] + (size_t)h * D * a.W + 4 * off);
        }
      }
    }
    float la = 0.f, be = 0.f;
    if (t < B && t < cnt) {  // tokens past the count: alpha = 1, beta = 0 (identity)
      const size_t gi = (size_t)trow(t) * a.H + h;
      la = __logf(pal[gi]);
      be = pbe[gi];
    }
    // the state: thread (rg, cq) holds rows rg * RPG .. + RPG - 1, columns
    // 4 cq .. 4 cq + 3 (a wave reads whole 128-byte row segments); nothing
    // waits for it until the reduction.  Each state is read once per call,
    // so the loads are non-temporal (they do not displace other lines from
    // the caches)
    if constexpr (MF) {
      const float *Sw = S + 16 * wvs + n16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[ks][e] = Sw[(size_t)(32 * ks + 8 * kg + e) * D];
    } else {
#pragma unroll
      for (int i = 0; i < RPG; ++i)
      {
        const floatx4 v =
            __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(S + (size_t)(rg * RPG + i) * D + 4 * cq));
        s4[i] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }

    // 1. block inputs -> LDS as fp32 (CONV: the raw rows, convolved below)
#pragma unroll
    for (int e = 0; e < IU; ++e) {
      const int u = e * NT + t;
      if (u < (CONV ? 3 * NR * UPR : B * (2 * UPR + UPRV))) {
        float *dst;
        if constexpr (CONV) {
          const int sec = u / (NR * UPR), row = (u / UPR) % NR, cu = u % UPR;
          dst = &sRaw[sec][row][cu * EPU];
        } else if (u < 2 * B * UPR) {
          const int which = divB(u / UPR), r = modB(u / UPR), cu = u % UPR;
          dst = which == 0 ? &sX[r][cu * EPU] : &sX[BMAX + r][cu * EPU];
        } else {
          const int uv = u - 2 * B * UPR;
          dst = &sV[uv / UPRV][(uv % UPRV) * EPU];
        }
        const uint4 raw = in_raw[e];
        if constexpr (sizeof(IO) == 2) {
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
          float4 lo, hi;
          lo.x = __uint_as_float(w[0] << 16); lo.y = __uint_as_float(w[0] & 0xffff0000u);
          lo.z = __uint_as_float(w[1] << 16); lo.w = __uint_as_float(w[1] & 0xffff0000u);
          hi.x = __uint_as_float(w[2] << 16); hi.y = __uint_as_float(w[2] & 0xffff0000u);
          hi.z = __uint_as_float(w[3] << 16); hi.w = __uint_as_float(w[3] & 0xffff0000u);
          reinterpret_cast<float4 *>(dst)[0] = lo;
          reinterpret_cast<float4 *>(dst)[1] = hi;
        } else {
          *reinterpret_cast<uint4 *>(dst) = raw;
        }
      }
    }
    if constexpr (CONV) {
      const int per = D * a.W / 4;
#pragma unroll
      for (int e = 0; e < WUMAX; ++e) {
        const int u = e * NT + t;
        if (u < 3 * per) *reinterpret_cast<float4 *>(&sCW[u / per][4 * (u % per)]) = cw4[e];
      }
    }
    if (t < 64) {
      // gates: inclusive scan of log(alpha) over the block (one wave)
      const int j = t;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off, 64);
        if (j >= off) la += y;
      }
      if (j < B) {
        sG[j] = la;
        sBeta[j] = be;
      }
    }
    __syncthreads();

    if constexpr (CONV) {
      // COMMIT: the new clean history is the last W - 1 raw rows
      if constexpr (KIND == 1) {
        IO *const hw = reinterpret_cast<IO *>(a.cache);
        for (int u = t; u < 3 * W1 * UPR; u += NT) {
          const int sec = u / (W1 * UPR), row = (u / UPR) % W1, cu = u % UPR;
          const float *src = &sRaw[sec][B + row][cu * EPU];
          IO *dst = hw + (((size_t)slot * W1 + row) * 3 + sec) * C + (size_t)h * D + cu * EPU;
          if constexpr (sizeof(IO) == 2) {
            *reinterpret_cast<uint4 *>(dst) = make_uint4(pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]),
                                                         pack_bf16x2(src[4], src[5]), pack_bf16x2(src[6], src[7]));
          } else {
            *reinterpret_cast<float4 *>(dst) = *reinterpret_cast<const float4 *>(src);
          }
        }
      }
      // the convolution: block row j, tap i reads raw row j + i (history first)
      for (int e = t; e < 3 * B * D; e += NT) {
        const int sec = divB(e / D), j = modB(e / D), c = e % D;
        const float *w = &sCW[sec][c * a.W];
        float y = 0.f;
        for (int i = 0; i < a.W; ++i) y = fmaf(w[i], sRaw[sec][j + i][c], y);
        if (a.act) y = y / (1.f + __expf(-y));
        float *dst = sec == 0 ? &sX[BMAX + j][c] : sec == 1 ? &sX[j][c] : &sV[j][c];
        *dst = y;
      }
      __syncthreads();
      if (a.l2) {
        // q and k rows divided by sqrt(sum y^2 + 1e-6), 16 lanes per row
        constexpr int GROUPS = NT / 16, PER = D / 16;
        const int grp = t / 16, sub = t % 16;
        for (int r0 = 0; r0 < 2 * B; r0 += GROUPS) {  // uniform trip count: every lane joins the DPP sums
          const int rr = r0 + grp;
          const bool valid = rr < 2 * B;
          float *row = sX[valid ? (rr < B ? rr : BMAX + rr - B) : 0];
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < PER; ++e) ss = fmaf(row[sub * PER + e], row[sub * PER + e], ss);
          const float sc = rsqrtf(dpp_sum16(ss) + 1e-6f);
          if (valid) {
#pragma unroll
            for (int e = 0; e < PER; ++e) row[sub * PER + e] *= sc;
          }
        }
        __syncthreads();
      }
    }

    // 2. B x B dot products k_i.k_j and q_l.k_j while the state is still in
    //    flight: for bf16 io and blocks of up to 32 tokens on the matrix cores
    //    (the rows are exact in bf16; 16 x 16 tiles of KK^T and QK^T, two per
    //    wave), otherwise 16 lanes per dot (a DPP row)
    constexpr bool MFMA_DOTS = sizeof(IO) == 2 && BMAX >= 16 && D % 32 == 0;
    if constexpr (MFMA_DOTS) {
      const int nt = (B + 15) / 16;  // tiles in use per side
      const int wv = __builtin_amdgcn_readfirstlane(t >> 6), ln = t & 63;
      for (int tt = wv; tt < 8; tt += NT / 64) {  // tile tt: which (KK^T, QK^T), ti, tj
        const int which = tt >> 2, ti = (tt >> 1) & 1, tj = tt & 1;
        if (ti >= nt || tj >= nt) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          mma_bf16(acc, frag_f32_hi(&sX[which ? BMAX : 0][0], LDXS, 16 * ti, 32 * ks),
                   frag_f32_hi(&sX[0][0], LDXS, 16 * tj, 32 * ks));
        // accumulator lane layout: rows 4 (lane / 16) + r, column lane % 16
        float (*dst)[BMAX] = which ? sQK : sKK;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[16 * ti + 4 * (ln >> 4) + r][16 * tj + (ln & 15)] = acc[r];
      }
    } else {
      constexpr int GROUPS = NT / 16, PER = D / 16;
      const int grp = t / 16, sub = t % 16;
      const int ndots = 2 * B * B;
      for (int d0 = 0; d0 < ndots; d0 += GROUPS) {  // uniform trip count: every lane joins the DPP sums
        const int dd = d0 + grp;
        const bool valid = dd < ndots;
        const int which = valid ? divB(divB(dd)) : 0, ij = valid ? dd - which * B * B : 0;
        const int i = divB(ij), j = modB(ij);
        const float *x = sX[which ? BMAX + i : i];
        const float *y = sX[j];
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) p += x[sub * PER + e] * y[sub * PER + e];
        p = dpp_sum16(p);
        if (valid && sub == 0) {
          if (which) sQK[i][j] = p; else sKK[i][j] = p;
        }
      }
    }
    __syncthreads();

    // 2b. the coefficients, in place and zero outside the block:
    //     A[i][m] = (G_i / G_m) b_m k_i.k_m for m < i (the UT system) and
    //     P[l][j] = (G_e / G_j) b_j q_l.k_j for j <= e, e the row the output
    //     reads (the block end for EVAL, l otherwise)
    for (int e = t; e < BMAX * BMAX; e += NT) {
      const int i = e / BMAX, m = e % BMAX;
      float A = 0.f, P = 0.f;
      if (i < B && m < B) {
        const float bm = sBeta[m];
        if (m < i) A = __expf(sG[i] - sG[m]) * bm * sKK[i][m];
        const int end = KIND == 0 && !a.causal ? B - 1 : i;
        if (m <= end) P = __expf(sG[end] - sG[m]) * bm * sQK[i][m];
      }
      sKK[i][m] = A;
      sQK[i][m] = P;
    }
    __syncthreads();

    // 3. T = (I + A)^-1 by forward substitution, one lane per column, the
    //    column in registers (T[m][c] = 0 for m < c, so every row sums over all
    //    earlier m); columns past the block come out as unit vectors.  The
    //    other threads go on to the reduction.
    if (t < BMAX) {
      const int c = t;
      float tc[BMAX];
#pragma unroll
      for (int i = 0; i < BMAX; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc += sKK[i][m] * tc[m];
        tc[i] = i == c ? 1.f : (i > c ? -acc : 0.f);
        sT[i][c] = tc[i];
      }
    }

    // 4. one pass over the state: W[x] = S^T x for the 2B vectors.  MF: as
    //    16 x 16 x 32 bf16 tiles, the k / q rows exact in bf16, S split hi + lo,
    //    wave w the 16 columns it holds.  Otherwise G vectors at a time, the
    //    row-group partials summed across adjacent lanes (DPP).
    if constexpr (MF) {
      bf16x8 sh[4], sl[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) split8(sf[ks], sh[ks], sl[ks]);
      const int nt = (B + 15) / 16;  // row tiles in use per half (k, q)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {  // rows 16 mt of sX / sW: k tiles 0, 1, q tiles 2, 3
        if ((mt & 1) >= nt) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 ax = frag_f32_hi(&sX[0][0], LDXS, 16 * mt, 32 * ks);
          mma_bf16(acc, ax, sh[ks]);
          mma_bf16(acc, ax, sl[ks]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sW[16 * mt + 4 * kg + r][16 * wvs + n16] = acc[r];
      }
    }
    if constexpr (!MF)
    for (int v0 = 0; v0 < 2 * B; v0 += G) {
      float4 acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int vi = v0 + g;
        const int src = vi < B ? vi : BMAX + min(vi - B, BMAX - 1);
        const bool live = vi < 2 * B;
        if constexpr (RPG % 4 == 0) {
#pragma unroll
          for (int i4 = 0; i4 < RPG; i4 += 4) {  // four rows of x per 16-byte LDS read
            float4 x4 = *reinterpret_cast<const float4 *>(&sX[src][rg * RPG + i4]);
            if (!live) x4 = make_float4(0.f, 0.f, 0.f, 0.f);
            const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              acc[g].x += xs[ii] * s4[i4 + ii].x;
              acc[g].y += xs[ii] * s4[i4 + ii].y;
              acc[g].z += xs[ii] * s4[i4 + ii].z;
              acc[g].w += xs[ii] * s4[i4 + ii].w;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < RPG; ++i) {
            const float x = live ? sX[src][rg * RPG + i] : 0.f;
            acc[g].x += x * s4[i].x;
            acc[g].y += x * s4[i].y;
            acc[g].z += x * s4[i].z;
            acc[g].w += x * s4[i].w;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float4 r4;
        r4.x = rowgroup_sum<NRG>(acc[g].x);
        r4.y = rowgroup_sum<NRG>(acc[g].y);
        r4.z = rowgroup_sum<NRG>(acc[g].z);
        r4.w = rowgroup_sum<NRG>(acc[g].w);
        const int vi = v0 + g;
        if (rg == 0 && vi < 2 * B) {
          const int dst = vi < B ? vi : BMAX + (vi - B);
          *reinterpret_cast<float4 *>(&sW[dst][4 * cq]) = r4;
        }
      }
    }
    __syncthreads();

    // 5. U = T (V - diag(G) W_k): first Y = V - diag(G) W_k in place of V,
    //    then every NPC-th row of U per thread (T is lower triangular)
    for (int e = t; e < B * DV; e += NT) {
      const int m = e / DV, c = e % DV;
      sV[m][c] -= __expf(sG[m]) * sW[m][c];
    }
    __syncthreads();
    {
      constexpr int NPC = NT / DV;  // threads per column
      const int c = t % DV;
      for (int i = t / DV; i < B; i += NPC) {
        float u = 0.f;
#pragma unroll 4
        for (int m = 0; m <= i; ++m) u += sT[i][m] * sV[m][c];
        sU[i][c] = u;
      }
    }
    __syncthreads();

    const float s = a.scale;
    const int last = B - 1;

    // 6. the new state (first: the state registers are free for the outputs),
    //    token by token or as one rank-B update, for the modes
    //    that write states; thread (rg, cq) owns rows rg * RPG .. + RPG - 1,
    //    columns 4 cq .. 4 cq + 3 (the layout it read)
    //    VERIFY (2): S_t = a_t S_{t-1} + b_t k_t u_t^T after every token, to
    //      the candidate buffer;
    //    BOUNDARIES (3): the same recurrence over the window's first count
    //      tokens; the state before local token q for q = lo, lo + bB, ...
    //      <= count goes to pool_out[g0 + (q - lo) / bB];
    //    COMMIT (1): S <- G_e S + sum_j (G_e / G_j) b_j k_j u_j^T, written back
    //      (or to pool_out)
    const int toff = rg * RPG * D + 4 * cq;  // the thread's first state element; rows follow at D
    // states are written once and not read back by this call: non-temporal
    auto store = [&](float *base, const float4 *n) {
      float *const p = base + toff;
#pragma unroll
      for (int i = 0; i < RPG; ++i)
        __builtin_nontemporal_store(floatx4{n[i].x, n[i].y, n[i].z, n[i].w}, reinterpret_cast<floatx4 *>(p + i * D));
    };
    // MF layout: one token's update n = a n + (b k_j) u_j^T and the stores
    auto mf_step = [&](float (*nn)[8], int j, float aj, float wk) {
      const float u = sU[j][16 * wvs + n16];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 k0 = *reinterpret_cast<const float4 *>(&sX[j][32 * ks + 8 * kg]);
        const float4 k1 = *reinterpret_cast<const float4 *>(&sX[j][32 * ks + 8 * kg + 4]);
        const float kr[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) nn[ks][e] = aj * nn[ks][e] + (kr[e] * wk) * u;
      }
    };
    auto mf_store = [&](float *base, const float (*nn)[8]) {
      float *const p = base + 16 * wvs + n16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[(size_t)(32 * ks + 8 * kg + e) * D] = nn[ks][e];
    };
    if constexpr (MF && KIND == 1) {
      const float ge = __expf(sG[last]);
      float nn[4][8];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) nn[ks][e] = ge * sf[ks][e];
      for (int j = 0; j < B; ++j) mf_step(nn, j, 1.f, __expf(sG[last] - sG[j]) * sBeta[j]);
      mf_store(a.pool_out ? a.pool_out + ((size_t)req * a.H + h) * D * D + col0 : S, nn);
    } else if constexpr (MF && KIND == 2) {
      const bool bounds = a.mode == 3;
      const int lo = bounds ? a.blo[req] : 0, g0 = bounds ? a.bg0[req] : 0, bB = bounds ? a.bB : 1;
      const size_t tstride = (size_t)a.H * D * D;
      float *const cand = bounds ? nullptr : a.cand + ((size_t)req * B * a.H + h) * D * D + col0;
      auto bnd = [&](int q) { return a.pool_out + ((size_t)(g0 + (q - lo) / bB) * a.H + h) * D * D + col0; };
      float nn[4][8];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) nn[ks][e] = sf[ks][e];
      if (bounds && lo == 0) mf_store(bnd(0), nn);
      for (int j = 0; j < B; ++j) {
        mf_step(nn, j, __expf(sG[j] - (j > 0 ? sG[j - 1] : 0.f)), sBeta[j]);
        if (!bounds) {
          mf_store(cand + j * tstride, nn);
        } else {
          const int q = j + 1;
          if (q >= lo && (q - lo) % bB == 0) mf_store(bnd(q), nn);
        }
      }
    } else if constexpr (KIND == 1) {
      const float ge = __expf(sG[last]);
      float4 n[RPG];
#pragma unroll
      for (int i = 0; i < RPG; ++i) n[i] = make_float4(ge * s4[i].x, ge * s4[i].y, ge * s4[i].z, ge * s4[i].w);
      for (int j = 0; j < B; ++j) {
        const float wk = __expf(sG[last] - sG[j]) * sBeta[j];
        const float4 u = *reinterpret_cast<const float4 *>(&sU[j][4 * cq]);
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          const float kk = sX[j][rg * RPG + i] * wk;
          n[i].x += kk * u.x; n[i].y += kk * u.y; n[i].z += kk * u.z; n[i].w += kk * u.w;
        }
      }
      store(a.pool_out ? a.pool_out + ((size_t)req * a.H + h) * D * D + col0 : S, n);
    } else if constexpr (KIND == 2) {
      const bool bounds = a.mode == 3;
      const int lo = bounds ? a.blo[req] : 0, g0 = bounds ? a.bg0[req] : 0, bB = bounds ? a.bB : 1;
      const size_t tstride = (size_t)a.H * D * D;
      float *const cand = bounds ? nullptr : a.cand + ((size_t)req * B * a.H + h) * D * D + col0;
      auto bnd = [&](int q) { return a.pool_out + ((size_t)(g0 + (q - lo) / bB) * a.H + h) * D * D + col0; };
      float4 n[RPG];
#pragma unroll
      for (int i = 0; i < RPG; ++i) n[i] = s4[i];
      if (bounds && lo == 0) store(bnd(0), n);
      // VERIFY: every token of the block; BOUNDARIES: every token before the
      // window's last block start
      for (int j = 0; j < B; ++j) {
        const float aj = __expf(sG[j] - (j > 0 ? sG[j - 1] : 0.f)), wk = sBeta[j];
        const float4 u = *reinterpret_cast<const float4 *>(&sU[j][4 * cq]);
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          const float kk = sX[j][rg * RPG + i] * wk;
          n[i].x = aj * n[i].x + kk * u.x;
          n[i].y = aj * n[i].y + kk * u.y;
          n[i].z = aj * n[i].z + kk * u.z;
          n[i].w = aj * n[i].w + kk * u.w;
        }
        if (!bounds) {
          store(cand + j * tstride, n);
        } else {
          const int q = j + 1;
          if (q >= lo && (q - lo) % bB == 0) store(bnd(q), n);
        }
      }
    }

    // 7. outputs, EPU consecutive columns per work item (one 16-byte store)
    if (a.o) {
      IO *o = reinterpret_cast<IO *>(a.o);
      for (int e = t; e < B * UPRV; e += NT) {
        const int l = e / UPRV, c0 = (e % UPRV) * EPU;
        if (l >= cnt) continue;                  // no output for identity tokens
        const int end = KIND == 0 && !a.causal ? last : l;  // EVAL reads the block end
        const float ge = __expf(sG[end]);
        float acc[EPU];
#pragma unroll
        for (int c = 0; c < EPU; ++c) acc[c] = ge * sW[BMAX + l][c0 + c];
#pragma unroll 4
        for (int j = 0; j <= end; ++j) {
          const float wq = sQK[l][j];
#pragma unroll
          for (int c = 0; c < EPU; ++c) acc[c] += wq * sU[j][c0 + c];
        }
        IO *dst = o + ((size_t)trow(l) * a.H + h) * D + col0 + c0;
        if constexpr (sizeof(IO) == 2) {
          uint4 w;
          w.x = pack_bf16x2(s * acc[0], s * acc[1]);
          w.y = pack_bf16x2(s * acc[2], s * acc[3]);
          w.z = pack_bf16x2(s * acc[4], s * acc[5]);
          w.w = pack_bf16x2(s * acc[6], s * acc[7]);
          *reinterpret_cast<uint4 *>(dst) = w;
        } else {
          *reinterpret_cast<float4 *>(dst) = make_float4(s * acc[0], s * acc[1], s * acc[2], s * acc[3]);
        }
      }
    }
  }
}

template <typename IO, int D, int DV, int BMAX, int CW>
static void launch_kind(const BlockStepArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)(a.num_req * a.H * (D / DV)));
  const dim3 block(StepCfg<D, DV>::NT);
  if (a.mode == 0)
    hipLaunchKernelGGL((block_step_kernel<IO, D, DV, BMAX, CW, 0>), grid, block, 0, st, a);
  else if (a.mode == 1)
    hipLaunchKernelGGL((block_step_kernel<IO, D, DV, BMAX, CW, 1>), grid, block, 0, st, a);
  else if constexpr (CW == 0)
    hipLaunchKernelGGL((block_step_kernel<IO, D, DV, BMAX, CW, 2>), grid, block, 0, st, a);
}

template <typename IO, int D>
static hipError_t launch_step_d(const BlockStepArgs &a, hipStream_t st) {
  // the 32-token step splits a d = 128 state's columns over two workgroups
  // (its LDS then allows two workgroups per CU instead of one); the short
  // blocks keep whole rows, whose stores cover full 128-byte row segments per
  // wave (half rows measured slower there)
  constexpr int DV32 = D >= 128 ? D / 2 : D;
  if (a.conv && a.mode > 1) return hipErrorInvalidValue;  // the ShortConv step evaluates or commits
  TimedLaunch tl(K_BLOCK_STEP, st);
  if (a.conv) {
    // the serving ShortConv is built for blocks of up to 8 tokens and widths
    // up to 8; widths up to 4 take the smaller LDS staging (one more
    // workgroup per CU)
    if (a.B > 8 || a.W > 8) return hipErrorInvalidValue;
    if (a.W <= 4) {
      if (a.B <= 4) launch_kind<IO, D, D, 4, 4>(a, st);
      else launch_kind<IO, D, D, 8, 4>(a, st);
    } else {
      if (a.B <= 4) launch_kind<IO, D, D, 4, 8>(a, st);
      else launch_kind<IO, D, D, 8, 8>(a, st);
    }
  } else if (a.B <= 4) {
    launch_kind<IO, D, D, 4, 0>(a, st);
  } else if (a.B <= 8) {
    launch_kind<IO, D, D, 8, 0>(a, st);
  } else {
    launch_kind<IO, D, DV32, 32, 0>(a, st);
  }
  return hipGetLastError();
}

// One workgroup per (document, history row, projection): the row W - 1 - j
// before the document end, or zeros before its start, into the slot.
template <typename IO>
__global__ __launch_bounds__(256) void conv_cache_fill_kernel(ConvCacheArgs a) {
  const int W1 = a.W - 1;
  const int doc = blockIdx.x / (W1 * 3), j = (blockIdx.x / 3) % W1, sec = blockIdx.x % 3;
  const int s = a.cu[doc], e = a.cu[doc + 1];
  const int t = e - W1 + j;
  constexpr int EPU = 16 / sizeof(IO);
  const IO *src = reinterpret_cast<const IO *>(a.x[sec]) + (size_t)max(t, 0) * a.C;
  IO *dst = reinterpret_cast<IO *>(a.cache) + (((size_t)a.slot[doc] * W1 + j) * 3 + sec) * a.C;
  for (int u = threadIdx.x; u < a.C / EPU; u += 256) {
    const uint4 v = t >= s ? reinterpret_cast<const uint4 *>(src)[u] : make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4 *>(dst)[u] = v;
  }
}

hipError_t launch_conv_cache_fill(const ConvCacheArgs &a, hipStream_t st) {
  if (a.num_docs == 0 || a.W <= 1) return hipSuccess;
  const dim3 grid((unsigned)(a.num_docs * (a.W - 1) * 3));
  if (a.bf16)
    hipLaunchKernelGGL(conv_cache_fill_kernel<u16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(conv_cache_fill_kernel<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// One workgroup per (request, head): the accepted candidate's d x d state into
// the request's pool slot, 16-byte loads and stores.  The count is clamped to
// [0, K]; 0 leaves the slot as it was.
template <int D>
__global__ __launch_bounds__(256) void gdn_scatter_kernel(ScatterArgs a, const int32_t *__restrict__ accepted,
                                                          const int32_t *__restrict__ slot_idx) {
  const int req = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int r = min(max(accepted[req], 0), a.K);
  if (r == 0) return;
  // the candidate buffer and the pool never overlap (restrict), so the
  // unrolled copy issues its loads ahead of its stores
  typedef float v4f __attribute__((ext_vector_type(4)));  // a native vector: stays in registers
  const v4f *__restrict__ src =
      reinterpret_cast<const v4f *>(a.cand + (((size_t)req * a.K + (r - 1)) * a.H + h) * D * D);
  v4f *__restrict__ dst = reinterpret_cast<v4f *>(a.pool + ((size_t)slot_idx[req] * a.H + h) * D * D);
  constexpr int NV = D * D / 4;
  if constexpr (NV >= 256) {
    // all sixteen 16-byte loads of a thread in flight, then their stores
    constexpr int PER = NV / 256, GRP = PER < 16 ? PER : 16;
    static_assert(PER % GRP == 0, "whole groups");
#pragma unroll
    for (int e0 = 0; e0 < PER; e0 += GRP) {
      v4f v[GRP];
#pragma unroll
      for (int e = 0; e < GRP; ++e) v[e] = __builtin_nontemporal_load(&src[(e0 + e) * 256 + threadIdx.x]);
#pragma unroll
      for (int e = 0; e < GRP; ++e) __builtin_nontemporal_store(v[e], &dst[(e0 + e) * 256 + threadIdx.x]);
    }
  } else {
    if ((int)threadIdx.x < NV) dst[threadIdx.x] = src[threadIdx.x];
  }
}

hipError_t launch_gdn_scatter(const ScatterArgs &a, hipStream_t st) {
  if (a.num_req == 0) return hipSuccess;
  TimedLaunch tl(K_SCATTER, st);
  const dim3 grid((unsigned)(a.num_req * a.H));
  if (a.D == 128)
    hipLaunchKernelGGL(gdn_scatter_kernel<128>, grid, dim3(256), 0, st, a, a.accepted, a.slot_idx);
  else
    hipLaunchKernelGGL(gdn_scatter_kernel<16>, grid, dim3(256), 0, st, a, a.accepted, a.slot_idx);
  return hipGetLastError();
}

hipError_t launch_block_step(const BlockStepArgs &a, hipStream_t st) {
  if (a.num_req == 0) return hipSuccess;
  if (a.bf16) return a.D == 128 ? launch_step_d<u16, 128>(a, st) : launch_step_d<u16, 16>(a, st);
  return a.D == 128 ? launch_step_d<float, 128>(a, st) : launch_step_d<float, 16>(a, st);
}

}  // namespace flare
