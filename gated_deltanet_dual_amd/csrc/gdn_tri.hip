// gdn_tri.hip -- the chunk matrices of the backward that do not depend on the
// state (bf16 io, d = 128): the unit-lower-triangular inverses T = (I + A)^-1,
// A_ij = b_j exp(lg_i - lg_j) k_i . k_j (j < i), of the clean stream and T~ of
// the noisy blocks, and the four weighted masked Gram matrices Mwo, Mwq, Mwk,
// Mw~ (bwd_common.h).  They depend only on q, k, q~, k~ and the gates, so they
// are formed here once, fully in parallel over (chunk, head), instead of on
// the sequential reverse scan's critical path.  One workgroup of 4 waves per
// (chunk slot, head), all four in parallel: wave 0 solves T, wave 1 T~,
// wave 2 forms Mwo and Mwq, wave 3 Mwk and Mw~.  Output per (slot, head):
// [T, T~, Mwo, Mwq, Mwk, Mw~], each 32 x 32 fp32 row-major.
#include "bwd_common.h"
#include "chunk_common.h"
#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"

namespace flare {

namespace {
constexpr int tC = 32, tD = 128, tNT = 256, tLDX = tD + 8, tLDM = tC + 4;
struct TriSmem {
  alignas(16) u16 x[4][tC][tLDX];     // q, k, q~, k~
  alignas(16) float at[2][tC][tLDM];  // A^T, A~^T (gated, without b)
  alignas(16) float tm[6][tC][tLDM];  // T, T~, Mwo, Mwq, Mwk, Mw~
  alignas(16) float tmp[2][16][17];
  alignas(16) float lg[tC], beta[tC], lgn[tC], betan[tC];
};
}  // namespace

__global__ __launch_bounds__(tNT) void gdn_tri_d128_kernel(BwdArgs a) {
  constexpr int C = tC, D = tD, NT = tNT, LDX = tLDX, LDM = tLDM;
  __shared__ TriSmem sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // all global loads first (unconditional, rows clamped into the document):
  // gates and the q, k, q~, k~ rows (8 16-byte units per thread)
  const float graw = tid < 4 * C ? gate_load_raw(f, t0g, c0, n, h, tid) : 0.f;
  constexpr int RU = D / 8, PU = C * RU, UX = 4 * PU / NT;
  uint4 xr[UX];
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    xr[e] = *reinterpret_cast<const uint4 *>(px[m] + ((t0g + min(c0 + row, n - 1)) * H + h) * D + cu16 * 8);
  }
  for (int e = tid; e < 8 * C * LDM; e += NT) (&sm.at[0][0][0])[e] = 0.f;  // at and tm
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    const int tpos = c0 + row;
    const bool ok = tpos < n && (m < 2 || tpos >= P);
    *reinterpret_cast<uint4 *>(&sm.x[m][row][cu16 * 8]) = ok ? xr[e] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid < 4 * C) gate_scan(gate_fix(graw, c0, n, P, tid), B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  lds_barrier();

  // each wave forms and stores only matrices it wrote itself (ordered per wave)
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
  float *dst = a.tri + ((size_t)slot * H + h) * 6 * C * C;
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

hipError_t launch_tri_d128(const BwdArgs &a, hipStream_t st, int64_t slots) {
  hipLaunchKernelGGL(gdn_tri_d128_kernel, dim3((unsigned)(slots * a.f.H)), dim3(tNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
