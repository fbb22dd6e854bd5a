// gdn_fwd_pre.hip -- the state-independent part of the forward's chunk step
// (bf16 io, d_k = d_v = 128, no flags), fully in parallel over (chunk, head),
// ahead of the forward scan.
//
// Method ("FLARE: Diffusion for Hybrid Language Model", papernotes.org notes,
// Key designs item 2; Overall framework): the clean stream follows the gated
// delta rule.  Per chunk of C = 32 tokens with start state S_c and the chunk
// matrices from the chunk-matrix pass (gdn_tri.hip),
//   U    = T (V - diag(G) K S_c),   S_{c+1} = G_C S_c + K^T diag(D) U,
// D_i = b_i G_C / G_i.  Only K S_c carries the state, so
//   S_{c+1} = G_C S_c + K^T (Z + W (K S_c)),
//   Z = diag(D) T V,   W = -diag(D) T diag(G),
// the backward's reverse step with its right-hand side R = K^T Z.  This
// kernel forms Z, W, G_C and the two fragment sets of K in the order the scan
// consumes them (bwd_common.h; Z in the R area as [slab 8][tile 2][lane 64][4]).
//
// One workgroup of 8 waves per (chunk slot, head); wave w owns d_v columns
// [16 w, 16 w + 16) of Z (a register slab, slab.h) and one fragment set.
// L2: the q/k L2 flag folded into per-row factors (gdn_l2.hip): the write
// strengths arrive folded from the gate load, the v rows are divided by r_k.
#include "bwd_common.h"
#include "chunk_common.h"
#include "device_common.h"
#include "kernels.h"
#include "slab.h"

namespace flare {

namespace {

constexpr int fC = 32, fD = 128, fNW = 8, fNT = 64 * fNW;
constexpr int fLDT = fC + 4, fLDM = fC + 4;

struct FwdPreSmem {
  alignas(16) u16 kt[fD][fLDT];    // k transposed ([d_k][chunk row])
  alignas(16) float tm[fC][fLDM];  // T
  alignas(16) float lg[fC], beta[fC], lgn[fC], betan[fC];
  alignas(16) float vsc[fC];  // L2: 1 / r_k of the chunk's rows
};

}  // namespace

template <bool L2>
__global__ __launch_bounds__(fNT) void gdn_fwd_pre_d128_kernel(FwdArgs f, const float *cmat, float *pack_all) {
  constexpr int C = fC, D = fD, LDM = fLDM;
  __shared__ FwdPreSmem sm;
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
  const int col0 = 16 * wave;
  const u16 *const pk = reinterpret_cast<const u16 *>(f.k), *const pv = reinterpret_cast<const u16 *>(f.v);
  float *const pack = pack_all + ((size_t)slot * H + h) * kPackWords;

  // ---- every global load first (unconditional, rows clamped into the document)
  // k rows: four consecutive rows 4 (t % 8) .. +3 of the 16-byte unit
  // (t / 8) % 16, so the transposed writes are 8 bytes; threads 128 and up
  // load copies (cache hits) and do not write them, so no load is conditional
  const int prow = 4 * (tid & 7), pu = (tid >> 3) & 15;
  uint4 xv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    xv[rr] = *reinterpret_cast<const uint4 *>(pk + ((t0g + min(c0 + prow + rr, n - 1)) * H + h) * D + 8 * pu);
  const float4 tv = cm_load_f4<false>(cmat + ((size_t)slot * H + h) * 6 * C * C, tid & 255, B, false);  // T
  const float graw = tid < 4 * C ? gate_load_raw(f, t0g, c0, n, h, tid) : 0.f;
  u16 rv[2][4];
  gslab_raw<D>(rv, pv, H, h, t0g, c0, n, col0);
  // this wave's K fragment (ks, tr) = (wave / 2, wave % 2)
  const int ka_row = 16 * (wave & 1) + cl, ka_col = 32 * (wave >> 1) + g4;
  const u16 *ka_src = pk + ((t0g + min(c0 + ka_row, n - 1)) * H + h) * D;
  const uint2 ka0 = *reinterpret_cast<const uint2 *>(ka_src + ka_col);
  const uint2 ka1 = *reinterpret_cast<const uint2 *>(ka_src + ka_col + 16);
  float rkl = 1.f;
  if (L2 && tid < C) rkl = f.l2f[(t0g + min(c0 + tid, n - 1)) * H + h].y;

  // ---- LDS: k transposed (rows past the document end zero), T, gates
  if (tid < 128) {
    uint4 w4[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) w4[rr] = c0 + prow + rr < n ? xv[rr] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4][4] = {{w4[0].x, w4[0].y, w4[0].z, w4[0].w},
                              {w4[1].x, w4[1].y, w4[1].z, w4[1].w},
                              {w4[2].x, w4[2].y, w4[2].z, w4[2].w},
                              {w4[3].x, w4[3].y, w4[3].z, w4[3].w}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xffffu, v1 = (w[1][e >> 1] >> sh) & 0xffffu;
      const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xffffu, v3 = (w[3][e >> 1] >> sh) & 0xffffu;
      *reinterpret_cast<uint2 *>(&sm.kt[8 * pu + e][prow]) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
  if (tid < C * C / 4) *reinterpret_cast<float4 *>(&sm.tm[cm_row(tid)][cm_col(tid)]) = tv;
  if (tid < 4 * C) gate_scan(gate_fix(graw, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  if (L2 && tid < C) sm.vsc[tid] = rkl > 0.f ? 1.f / rkl : 0.f;
  lds_barrier();

  const float lgC = sm.lg[C - 1];
  auto Dd = [&](int i) { return sm.beta[i] * __expf(lgC - sm.lg[i]); };
  // ---- the fragment sets (one per wave)
  {
    const bool ok = c0 + ka_row < n;
    reinterpret_cast<uint4 *>(pack + kPackKA)[wave * 64 + lane] =
        ok ? make_uint4(ka0.x, ka0.y, ka1.x, ka1.y) : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    const u16 *col = &sm.kt[16 * wave + cl][0];
    const uint2 lo4 = *reinterpret_cast<const uint2 *>(col + g4);
    const uint2 hi4 = *reinterpret_cast<const uint2 *>(col + 16 + g4);
    reinterpret_cast<uint4 *>(pack + kPackKT)[wave * 64 + lane] = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
  }
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
      x[e] = ok ? di * sm.tm[i][j] * __expf(sm.lg[j]) : 0.f;
    }
    bf16x8 wh, wl;
    split8(x, wh, wl);
    uint4 *dst = reinterpret_cast<uint4 *>(pack + kPackW);
    dst[(2 * tr) * 64 + lane] = __builtin_bit_cast(uint4, wh);
    dst[(2 * tr + 1) * 64 + lane] = __builtin_bit_cast(uint4, wl);
  }
  if (tid == 0) pack[kPackG] = __expf(lgC);

  // ---- Z = diag(D) T V for this wave's slab (R = K^T Z: the scan adds Z to
  // W (K S_c) ahead of its K^T product), stored as [slab][tile][lane][4]
  Slab V = slab_mask(rv, c0, n, P, false);
  Slab Z = slab_zero();
  if constexpr (L2) {  // v' = v / r_k is no longer exact in bf16: both operands split
#pragma unroll
    for (int tr = 0; tr < 2; ++tr)
#pragma unroll
      for (int r = 0; r < 4; ++r) V.t[tr][r] *= sm.vsc[slab_row(tr, r)];
    cc_mul<3, false>(Z, &sm.tm[0][0], LDM, V);
  } else {
    cc_mul<2, false>(Z, &sm.tm[0][0], LDM, V);
  }
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) Z.t[tr][r] *= Dd(slab_row(tr, r));
  float4 *zdst = reinterpret_cast<float4 *>(pack + kPackR) + (size_t)wave * 2 * 64;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) zdst[tr * 64 + lane] = make_float4(Z.t[tr][0], Z.t[tr][1], Z.t[tr][2], Z.t[tr][3]);
}

hipError_t launch_fwd_pre_d128(const FwdArgs &a, const float *cmat, float *pack, hipStream_t st, int64_t slots) {
  if (a.l2f)
    hipLaunchKernelGGL(gdn_fwd_pre_d128_kernel<true>, dim3((unsigned)(slots * a.H)), dim3(fNT), 0, st, a, cmat, pack);
  else
    hipLaunchKernelGGL(gdn_fwd_pre_d128_kernel<false>, dim3((unsigned)(slots * a.H)), dim3(fNT), 0, st, a, cmat,
                       pack);
  return hipGetLastError();
}

}  // namespace flare
