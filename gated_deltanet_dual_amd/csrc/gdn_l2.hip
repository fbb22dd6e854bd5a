// gdn_l2.hip -- the optional q/k L2 normalisation of the chunked bf16 d = 128
// path, folded into per-row factors (a reading: the FLARE notes do not state
// it; it is the usual normalisation in front of a gated delta rule, dividing
// each (token, head) row of q and k by sqrt(sum x^2 + 1e-6)).
//
// With k^ = r_k k (r_k = 1 / sqrt(|k|^2 + 1e-6)) the gated delta rule of
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes, Key
// designs item 2) reads
//   S_t = a_t (S - b_t k^ k^^T S) + b_t k^ v^T
//       = a_t (S - b'_t k k^T S) + b'_t k v'^T,   b' = b r_k^2,  v' = v / r_k,
// and o_t = s S_t^T q^ = r_q s S_t^T q.  So the chunked kernels run on the raw
// bf16 rows of q and k (exact MFMA operands, no rounding of normalised rows)
// with b', v' and the output rows scaled by r_q; the noisy stream the same
// with its own factors.  The reverse mode runs the same transformed problem
// with the output gradient r_q do, then maps its gradients back:
//   dv = dv' / r_k,  db = db' r_k^2,
//   dq = dq' - r_q^2 q (q . dq'),
//   dk = dk' + r_k^2 k (dv' . v' - 2 b' db')
// (the last two terms: the dependence of v' and b' on |k|).
//
// This file holds the factor pass: per (token, head) of the packed batch,
// {r_q, r_k, r_q~, r_k~} into a float4, one 16-lane group per row and array.
#include "conv_load.h"
#include "device_common.h"
#include "kernels.h"

namespace flare {

__global__ __launch_bounds__(256) void gdn_l2_factors_kernel(FwdArgs f, float4 *out, int64_t rows) {
  // group of 16 lanes = (row = t * H + h, array m); 16 groups per workgroup
  const int lane = threadIdx.x & 15;
  const int64_t grp = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int64_t row = grp >> 2;
  const int m = (int)(grp & 3);
  const u16 *src = reinterpret_cast<const u16 *>(m == 0 ? f.q : m == 1 ? f.k : m == 2 ? f.qn : f.kn);
  const int64_t r = row < rows ? row : rows - 1;
  const uint4 v = *reinterpret_cast<const uint4 *>(src + r * 128 + lane * 8);
  const float rf = l2_factor(l2_rowsum16(v));
  if (lane == 0 && row < rows) reinterpret_cast<float *>(out + row)[m] = rf;
}

hipError_t launch_l2_factors(const FwdArgs &a, float4 *out, hipStream_t st) {
  const int64_t rows = a.T * a.H;
  if (rows == 0) return hipSuccess;
  const int64_t groups = rows * 4;
  hipLaunchKernelGGL(gdn_l2_factors_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, st, a, out, rows);
  return hipGetLastError();
}

}  // namespace flare
