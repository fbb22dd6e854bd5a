// block_step.hip -- serving block step over a pool of recurrent states.
//
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
// designs item 4: a denoising forward reads the global causal state pool but
// never writes it (EVAL); once the block is fixed, a causal replay of the block
// writes the final state into the pool (COMMIT).  The per-token update is the
// gated delta rule of Key designs item 2.
//
// One workgroup per (request, head).  The whole d x d fp32 state of the pair is
// read once with 16-byte loads and kept in registers: thread t owns columns
// 4*(t % (D/4)) .. +3 of a group of rows.  The B updates are applied in their
// chunked (UT) form so the state is touched by exactly one reduction pass:
//   w_j = S^T k_j, r_l = S^T q_l                      (one pass over S)
//   A_ij = (G_i/G_j) b_j k_i.k_j (j < i), T = (I + A)^-1
//   U = T (V - diag(G) W)
//   EVAL:   o_l = s (G_e r_l + sum_j (G_e/G_j) b_j (q_l.k_j) u_j)   for every l
//   COMMIT: o_t = s (G_t r_t + sum_{j<=t} (G_t/G_j) b_j (q_t.k_j) u_j),
//           S  <- G_e S + sum_j (G_e/G_j) b_j k_j u_j^T            (written back)
// with G_i = prod_{m<=i} a_m taken as exp of a cumulative sum of log a.
// Everything is fp32 on the VALU: the step moves ~4 flop per byte of state, far
// below the MI355X fp32 ridge, so the kernel is bound by HBM bandwidth.
#include "device_common.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

template <int D> struct StepCfg {
  static constexpr int NT = D >= 128 ? 256 : 64;  // threads
  static constexpr int NCQ = D / 4;               // column quads
  static constexpr int NRG = NT / NCQ;            // row groups
  static constexpr int RPG = D / NRG;             // rows per group
  static constexpr int G = 8;                     // vectors reduced per pass
};

template <typename IO, int D, int BMAX>
__global__ __launch_bounds__(StepCfg<D>::NT) void block_step_kernel(BlockStepArgs a) {
  using Cfg = StepCfg<D>;
  constexpr int NT = Cfg::NT, NCQ = Cfg::NCQ, NRG = Cfg::NRG, RPG = Cfg::RPG, G = Cfg::G;
  constexpr int NV = 2 * BMAX;  // k vectors then q vectors
  const int B = a.B;
  const int t = threadIdx.x;
  const int req = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int cq = t % NCQ, rg = t / NCQ;

  __shared__ float sX[NV][D];          // k_0..k_{B-1}, q_0..q_{B-1} (fp32)
  __shared__ float sVv[BMAX][D];       // values
  __shared__ float sW[NV][D];          // S^T x for every x in sX
  __shared__ __align__(16) float sPart[NRG][G][D];
  __shared__ float sU[BMAX][D];
  __shared__ float sKK[BMAX][BMAX], sQK[BMAX][BMAX], sT[BMAX][BMAX];
  __shared__ float sG[BMAX], sBeta[BMAX];

  const int slot = a.slot_idx[req];
  float *S = a.pool + ((size_t)slot * a.H + h) * D * D;

  // 1. stream the state into registers (16-byte loads, all issued up front)
  float4 s4[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i)
    s4[i] = *reinterpret_cast<const float4 *>(S + (size_t)(rg * RPG + i) * D + 4 * cq);

  // 2. block inputs -> LDS as fp32
  const IO *q = reinterpret_cast<const IO *>(a.q);
  const IO *k = reinterpret_cast<const IO *>(a.k);
  const IO *v = reinterpret_cast<const IO *>(a.v);
  for (int e = t; e < B * D; e += NT) {
    const int j = e / D, c = e % D;
    const size_t row = (((size_t)req * B + j) * a.H + h) * D + c;
    sX[j][c] = io_traits<IO>::to_f(k[row]);
    sX[BMAX + j][c] = io_traits<IO>::to_f(q[row]);
    sVv[j][c] = io_traits<IO>::to_f(v[row]);
  }
  if (t < 64) {
    // gates: inclusive scan of log(alpha) over the block (one wave)
    const int j = t;
    float la = 0.f, be = 0.f;
    if (j < B) {
      const size_t gi = ((size_t)req * B + j) * a.H + h;
      la = __logf(a.alpha[gi]);
      be = a.beta[gi];
    }
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

  // 3. one reduction pass: W[x] = S^T x for the 2B vectors, G at a time
  for (int v0 = 0; v0 < 2 * B; v0 += G) {
    float4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int row = rg * RPG + i;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int vi = v0 + g;
        const int src = min(vi < B ? vi : BMAX + (vi - B), NV - 1);
        const float x = (vi < 2 * B) ? sX[src][row] : 0.f;
        acc[g].x += x * s4[i].x;
        acc[g].y += x * s4[i].y;
        acc[g].z += x * s4[i].z;
        acc[g].w += x * s4[i].w;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) *reinterpret_cast<float4 *>(&sPart[rg][g][4 * cq]) = acc[g];
    __syncthreads();
    for (int e = t; e < G * NCQ; e += NT) {
      const int g = e / NCQ, c4 = e % NCQ;
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
      for (int r = 0; r < NRG; ++r) {
        const float4 p = *reinterpret_cast<const float4 *>(&sPart[r][g][4 * c4]);
        sum.x += p.x; sum.y += p.y; sum.z += p.z; sum.w += p.w;
      }
      const int vi = v0 + g;
      if (vi < 2 * B) {
        const int dst = vi < B ? vi : BMAX + (vi - B);
        *reinterpret_cast<float4 *>(&sW[dst][4 * c4]) = sum;
      }
    }
    __syncthreads();
  }

  // 4. B x B dot products k_i.k_j and q_l.k_j
  for (int e = t; e < 2 * B * B; e += NT) {
    const int which = e / (B * B), ij = e % (B * B);
    const int i = ij / B, j = ij % B;
    const float *x = sX[which ? BMAX + i : i];
    const float *y = sX[j];
    float d = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) d += x[c] * y[c];
    if (which) sQK[i][j] = d; else sKK[i][j] = d;
  }
  __syncthreads();

  // 5. T = (I + A)^-1 by forward substitution, one lane per column; the
  //    column lives in sT and is read back only by the thread that wrote it.
  if (t < B) {
    const int c = t;
    for (int i = 0; i < B; ++i) {
      float x = 0.f;
      if (i == c) {
        x = 1.f;
      } else if (i > c) {
        float acc = 0.f;
        for (int m = c; m < i; ++m) acc += __expf(sG[i] - sG[m]) * sBeta[m] * sKK[i][m] * sT[m][c];
        x = -acc;
      }
      sT[i][c] = x;
    }
  }
  __syncthreads();

  // 6. U = T (V - diag(G) W_k)
  for (int e = t; e < B * D; e += NT) {
    const int i = e / D, c = e % D;
    float u = 0.f;
    for (int m = 0; m <= i; ++m) u += sT[i][m] * (sVv[m][c] - __expf(sG[m]) * sW[m][c]);
    sU[i][c] = u;
  }
  __syncthreads();

  // 7. outputs
  const float s = a.scale;
  const int last = B - 1;
  if (a.o) {
    IO *o = reinterpret_cast<IO *>(a.o);
    for (int e = t; e < B * D; e += NT) {
      const int l = e / D, c = e % D;
      const int end = a.mode == 0 ? last : l;  // EVAL reads the block end
      float acc = __expf(sG[end]) * sW[BMAX + l][c];
      for (int j = 0; j <= end; ++j) acc += __expf(sG[end] - sG[j]) * sBeta[j] * sQK[l][j] * sU[j][c];
      o[(((size_t)req * B + l) * a.H + h) * D + c] = io_traits<IO>::from_f(s * acc);
    }
  }

  // 8. COMMIT: rank-B update of the register-resident state, written back
  if (a.mode == 1) {
    const float ge = __expf(sG[last]);
    float wj[BMAX];
#pragma unroll
    for (int j = 0; j < BMAX; ++j) wj[j] = j < B ? __expf(sG[last] - sG[j]) * sBeta[j] : 0.f;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int row = rg * RPG + i;
      float4 n = make_float4(ge * s4[i].x, ge * s4[i].y, ge * s4[i].z, ge * s4[i].w);
#pragma unroll
      for (int j = 0; j < BMAX; ++j) {
        if (j >= B) break;
        const float kk = sX[j][row] * wj[j];
        const float4 u = *reinterpret_cast<const float4 *>(&sU[j][4 * cq]);
        n.x += kk * u.x; n.y += kk * u.y; n.z += kk * u.z; n.w += kk * u.w;
      }
      *reinterpret_cast<float4 *>(S + (size_t)row * D + 4 * cq) = n;
    }
  }
}

template <typename IO, int D>
static hipError_t launch_step_d(const BlockStepArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)(a.num_req * a.H));
  const dim3 block(StepCfg<D>::NT);
  TimedLaunch tl(K_BLOCK_STEP, st);
  if (a.B <= 4)
    hipLaunchKernelGGL((block_step_kernel<IO, D, 4>), grid, block, 0, st, a);
  else if (a.B <= 8)
    hipLaunchKernelGGL((block_step_kernel<IO, D, 8>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((block_step_kernel<IO, D, 32>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_block_step(const BlockStepArgs &a, hipStream_t st) {
  if (a.num_req == 0) return hipSuccess;
  if (a.bf16) return a.D == 128 ? launch_step_d<u16, 128>(a, st) : launch_step_d<u16, 16>(a, st);
  return a.D == 128 ? launch_step_d<float, 128>(a, st) : launch_step_d<float, 16>(a, st);
}

}  // namespace flare
