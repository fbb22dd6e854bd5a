// chunk_common.h -- the unit-lower-triangular chunk solve shared by the
// forward and backward kernels.
#pragma once

#include "device_common.h"

namespace flare {

// T = (I + A)^-1 for a 32 x 32 unit-lower-triangular system given as A^T
// (strictly lower A; A^T row j holds column j of A), written row-major to Tm.
// With colscale, A^T row j is multiplied by colscale[j] on the fly (the column
// scale of A, e.g. the write strengths b_j kept out of the stored Gram).
// One wave: lanes 0..31 solve the two diagonal 16 x 16 blocks, one column per
// lane, by right-looking substitution kept in registers; the off-diagonal block
// T_10 = -T_11 A_10 T_00 then runs on fp32 MFMA in the same wave (the wave's
// LDS operations complete in order, so no barrier is needed).
template <int LDM>
__device__ __forceinline__ void solve_unit_lower(const float *At, float *Tm, float *tmp, bool offdiag,
                                                 const float *colscale = nullptr) {
  const int lane = lane_id();
  if (lane < 32) {
    const int r0 = 16 * (lane >> 4), cl = lane & 15;
    // rows of A^T are fetched four substitution steps ahead (independent of
    // x), so the substitution rarely waits on LDS; about five rows are live
    float at[16][16];
    auto fetch_row = [&](int ii) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 v4 = *reinterpret_cast<const float4 *>(At + (r0 + ii) * LDM + r0 + 4 * q4);
        if (colscale) {
          const float cs = colscale[r0 + ii];
          v4.x *= cs; v4.y *= cs; v4.z *= cs; v4.w *= cs;
        }
        at[ii][4 * q4] = v4.x; at[ii][4 * q4 + 1] = v4.y; at[ii][4 * q4 + 2] = v4.z; at[ii][4 * q4 + 3] = v4.w;
      }
    };
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) fetch_row(ii);
    float x[16];
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) x[ii] = ii == cl ? 1.f : 0.f;
#pragma unroll
    for (int ii = 0; ii < 15; ++ii) {
      if (ii + 4 < 15) fetch_row(ii + 4);
      const float xi = x[ii];
#pragma unroll
      for (int jj = ii + 1; jj < 16; ++jj) x[jj] -= at[ii][jj] * xi;  // at[ii][jj] = A[r0+jj][r0+ii]
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) Tm[(r0 + ii) * LDM + r0 + cl] = x[ii];
  }
  if (offdiag) {
    floatx4 xa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)  // X = A_10 T_00, A_10[i][k] = A^T[k][16 + i]
      mma_f32(xa, frag1_f32_T(At, LDM, 16, k0) * (colscale ? colscale[k0 + (lane >> 4)] : 1.f),
              frag1_f32_T(Tm, LDM, 0, k0));
#pragma unroll
    for (int r = 0; r < 4; ++r) tmp[acc_row(r) * 17 + acc_col()] = xa[r];
    floatx4 ta = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)  // T_10 = -T_11 X
      mma_f32(ta, frag1_f32(Tm + 16 * LDM + 16, LDM, 0, k0), frag1_f32_T(tmp, 17, 0, k0));
#pragma unroll
    for (int r = 0; r < 4; ++r) Tm[(16 + acc_row(r)) * LDM + acc_col()] = -ta[r];
  }
}

}  // namespace flare
