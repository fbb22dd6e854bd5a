// gdn_tri.hip -- the unit-lower-triangular inverses of every chunk for the
// backward (bf16 io, d = 128): T = (I + A)^-1 with A_ij = b_j exp(lg_i - lg_j)
// k_i . k_j (j < i) of the clean stream, and T~ of the noisy blocks.  They
// depend only on k and the gates, so they are solved here once, fully in
// parallel over (chunk, head), instead of on the sequential reverse scan and
// the per-chunk kernel's critical path.  One workgroup of 2 waves per (chunk
// slot, head): wave 0 solves T, wave 1 T~; the small footprint lets several
// workgroups share a CU and hide each other's latency.
#include "bwd_common.h"
#include "chunk_common.h"
#include "device_common.h"
#include "gemm_lds.h"
#include "kernels.h"

namespace flare {

namespace {
constexpr int tC = 32, tD = 128, tNT = 128, tLDX = tD + 8, tLDM = tC + 4;
struct TriSmem {
  alignas(16) u16 x[2][tC][tLDX];     // k, k~
  alignas(16) float at[2][tC][tLDM];  // A^T, A~^T (gated, without b)
  alignas(16) float tm[2][tC][tLDM];  // T, T~
  alignas(16) float tmp[2][16][17];
  alignas(16) float lg[tC], beta[tC], lgn[tC], betan[tC];
};
}  // namespace

__global__ __launch_bounds__(tNT) void gdn_tri_d128_kernel(BwdArgs a) {
  constexpr int C = tC, D = tD, NT = tNT, LDX = tLDX, LDM = tLDM;
  __shared__ TriSmem sm;
  const FwdArgs &f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = f.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  int doc, c;
  if (!slot_to_chunk(f, slot, doc, c)) return;
  const int64_t t0g = f.cu[doc];
  const int n = f.cu[doc + 1] - f.cu[doc];
  const int P = f.plen[doc];
  const int B = f.B;
  const int c0 = c * C;
  const bool has_noisy = (c0 + C > P) && (P < n);
  const u16 *const pk = reinterpret_cast<const u16 *>(f.k), *const pkn = reinterpret_cast<const u16 *>(f.kn);

  // all global loads first: gates and the k, k~ rows (8 16-byte units per thread)
  const float gval = gate_load(f, t0g, c0, n, P, h, tid);
  constexpr int RU = D / 8, PU = C * RU, UX = 2 * PU / NT;
  uint4 xr[UX];
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    const int tpos = c0 + row;
    const bool ok = tpos < n && (m == 0 || tpos >= P);
    const uint4 v =
        *reinterpret_cast<const uint4 *>((m == 0 ? pk : pkn) + ((t0g + min(tpos, n - 1)) * H + h) * D + cu16 * 8);
    xr[e] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int e = tid; e < 4 * C * LDM; e += NT) (&sm.at[0][0][0])[e] = 0.f;  // at and tm
#pragma unroll
  for (int e = 0; e < UX; ++e) {
    const int u = e * NT + tid;
    const int m = u / PU, r = u % PU, row = r / RU, cu16 = r % RU;
    *reinterpret_cast<uint4 *>(&sm.x[m][row][cu16 * 8]) = xr[e];
  }
  gate_scan(gval, B, tid, sm.lg, sm.beta, sm.lgn, sm.betan);
  lds_barrier();

  // each wave's Gram, solve and store touch only its own LDS (ordered per wave)
  if (wave == 0) {
    gram_at<D, LDX, LDM>(sm.x[0], sm.at[0], sm.lg);
    solve_unit_lower<LDM>(&sm.at[0][0][0], &sm.tm[0][0][0], &sm.tmp[0][0][0], true, sm.beta);
  } else if (has_noisy) {
    gram_ant<D, LDX, LDM>(sm.x[1], sm.at[1], sm.lgn, c0, n, P, B);
    solve_unit_lower<LDM>(&sm.at[1][0][0], &sm.tm[1][0][0], &sm.tmp[1][0][0], B > 16, sm.betan);
  }
  float *dst = a.tri + ((size_t)slot * H + h) * 2 * C * C + (size_t)wave * C * C;
#pragma unroll
  for (int e = 0; e < C * C / 4 / 64; ++e) {
    const int u = e * 64 + lane, row = u / (C / 4), c4 = u % (C / 4);
    *reinterpret_cast<float4 *>(dst + row * C + 4 * c4) = *reinterpret_cast<const float4 *>(&sm.tm[wave][row][4 * c4]);
  }
}

hipError_t launch_tri_d128(const BwdArgs &a, hipStream_t st, int64_t slots) {
  hipLaunchKernelGGL(gdn_tri_d128_kernel, dim3((unsigned)(slots * a.f.H)), dim3(tNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace flare
