// chunk_common.h -- the unit-lower-triangular chunk solve shared by the
// forward and backward kernels, and the rule for which parts of a stored
// chunk-matrix record can be non-zero (the record's writer and readers
// touch only those).
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

namespace flare {

// Whether the half-row starting at column lo (0 or 16; 64 bytes of fp32) of
// row `row` of chunk matrix `mtx` can hold a non-zero entry.  The order is
// the chunk-matrix pass's: T, T~, Mwo, Mwq, Mwk, Mw~.  B is the block size (a
// power of two dividing the 32-token chunk), p = row & -B the start of the
// row's noisy block and p + B - 1 its end.  From the masks that define them:
//   T = (I + A)^-1, A strictly lower    -> j <= i
//   T~, inverse of the in-block system  -> p <= j <= i
//   Mwo (masked clean Gram, j <= i)     -> j <= i
//   Mwq, Mwk (reads before the block)   -> j < p
//   Mw~ (the block-end read)            -> p <= j <= p + B - 1
// and the four noisy ones are not formed in a chunk without response rows.
// The passes that form them store only live parts; every reader loads only
// those and takes the others as zero, which they are.  mtx, lo, B and
// has_noisy are wave-uniform, so the choice of rule is a scalar branch.
__device__ __forceinline__ bool cm_half_live(int mtx, int row, int lo, int B, bool has_noisy) {
  const int p = row & -B;
  if (mtx == 0 || mtx == 2) return lo <= row;
  if (!has_noisy) return false;
  if (mtx == 1) return lo <= row && lo + 15 >= p;
  if (mtx == 5) return lo <= p + B - 1 && lo + 15 >= p;
  return lo < p;
}

// A chunk-matrix record in memory: the six 32 x 32 fp32 matrices, each stored
// tile-major as four 16 x 16 tiles (tile (ti, tj) at 2 ti + tj, rows of 64
// bytes), so that a dead tile is whole 128-byte lines.  Float4 u (0 .. 1535)
// holds row cm_row(u), columns cm_col(u) .. + 3 of matrix u >> 8; the 64
// float4s of a tile are one wave's share when a wave takes 64 consecutive u.
__device__ __forceinline__ int cm_row(int u) { return 16 * ((u >> 7) & 1) + ((u >> 2) & 15); }
__device__ __forceinline__ int cm_col(int u) { return 16 * ((u >> 6) & 1) + 4 * (u & 3); }
// The float4 of matrix mtx holding row `row`, columns col .. col + 3 (col a multiple of 4).
__device__ __forceinline__ int cm_f4_index(int mtx, int row, int col) {
  return 256 * mtx + 64 * (2 * (row >> 4) + (col >> 4)) + 4 * (row & 15) + ((col & 15) >> 2);
}
// Whether float4 u of a record is live.  The wave's lanes must hold 64
// consecutive u starting at a multiple of 64 (one tile), so that the matrix
// and the tile are the wave's.
__device__ __forceinline__ bool cm_f4_live(int u, int B, bool has_noisy) {
  const int t = __builtin_amdgcn_readfirstlane(u >> 6);  // matrix 4 t / 16 .., tile t & 3
  return cm_half_live(t >> 2, 16 * ((t >> 1) & 1) + ((u >> 2) & 15), 16 * (t & 1), B, has_noisy);
}

// Load float4 u of a chunk-matrix record (lanes as for cm_f4_live), or zero
// when it is not live.  The load is always issued (no load sits under a
// branch): a dead one is aimed at the record's first float4 (live in every
// chunk: T's diagonal starts there), which the same launch reads anyway, so
// it costs no HBM traffic.
template <bool NT>
__device__ __forceinline__ float4 cm_load_f4(const float *rec, int u, int B, bool has_noisy) {
  const bool live = cm_f4_live(u, B, has_noisy);
  const float *src = rec + 4 * (live ? u : 0);
  const float4 v = NT ? ld_nt_f4(src) : *reinterpret_cast<const float4 *>(src);
  return live ? v : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace flare
