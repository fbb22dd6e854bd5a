// route1.hip -- the "chunk-then-refine" route for the noisy stream, an
// alternative to the masked boundary reads of the chunked forward.
//
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
// designs item 2: the noisy block b of a document starts from the clean state
// at its boundary e(b-1) = P + (b-1) B and every position of the block reads
// the block-end state.  The pages describe two ways to get there: keep every
// block-boundary state (memory O(L/B) states; the route that runs out of
// memory at small B on their hardware and wins with dense products at large
// B) or rebuild the boundary states on chip from strided chunk states (the
// route the chunked forward of this library takes).  This file is the first:
//   1. the clean stream alone (every row taken as clean) with its chunk-start
//      states saved -- the chunked forward;
//   2. "chunk": every block-boundary state S_p materialised in memory, from
//      the start state of p's chunk and the clean tokens before p in it (the
//      serving step's COMMIT over that window, tokens past p made identity);
//   3. "refine": every noisy block from its S_p (the serving step's EVAL).
// The per-block tables come from the documents' layout on the device.
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "timing.h"

namespace flare {

namespace {


// Per-document block offsets (exclusive scan of the response block counts)
// and the clean-only prompt lengths, in one workgroup.
__global__ __launch_bounds__(256) void route1_offsets_kernel(const int32_t *cu, const int32_t *plen, int N, int B,
                                                             int32_t *boff, int32_t *plen_all) {
  __shared__ int32_t sc[256];
  __shared__ int32_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 256) {
    const int i = base + t;
    int nb = 0;
    if (i < N) {
      const int n = cu[i + 1] - cu[i], P = plen[i];
      nb = n > P ? (n - P + B - 1) / B : 0;
      plen_all[i] = n;
    }
    sc[t] = nb;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = t >= off ? sc[t - off] : 0;
      __syncthreads();
      sc[t] += v;
      __syncthreads();
    }
    if (i < N) boff[i] = carry + sc[t] - nb;
    __syncthreads();
    if (t == 255) carry += sc[255];
    __syncthreads();
  }
}

// One workgroup per document: the chunk window and the refine window of each
// of its response blocks.
__global__ __launch_bounds__(256) void route1_blocks_kernel(const int32_t *cu, const int32_t *plen, int B,
                                                            const int32_t *boff, int32_t *r0m, int32_t *cm,
                                                            int32_t *slm, int32_t *r0r, int32_t *cr) {
  const int i = blockIdx.x;
  const int s = cu[i], n = cu[i + 1] - s, P = plen[i];
  const int nb = n > P ? (n - P + B - 1) / B : 0;
  for (int j = threadIdx.x; j < nb; j += 256) {
    const int g = boff[i] + j;
    const int p = P + j * B;   // document-local start of the block
    const int c = p / kChunk;  // its chunk
    r0m[g] = s + c * kChunk;   // the chunk's clean tokens before p
    cm[g] = p - c * kChunk;
    slm[g] = s / kChunk + i + c;  // the chunk's checkpoint slot
    r0r[g] = s + p;               // the noisy block
    cr[g] = min(B, n - p);
  }
}

}  // namespace

hipError_t launch_route1(const FwdArgs &f, const Route1Plan &pl, hipStream_t st) {
  const int N = f.num_docs;
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(route1_offsets_kernel, dim3(1), dim3(256), 0, st, f.cu, f.plen, N, f.B, pl.boff, pl.plen_all);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.n_blocks > 0) {
    hipLaunchKernelGGL(route1_blocks_kernel, dim3((unsigned)N), dim3(256), 0, st, f.cu, f.plen, f.B, pl.boff,
                       pl.r0m, pl.cm, pl.slm, pl.r0r, pl.cr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 1. the clean stream with its chunk-start states (every row taken as clean:
  //    the noisy outputs come out zero and are refined below)
  FwdArgs clean = f;
  clean.plen = pl.plen_all;
  if ((e = launch_gdn_fwd(clean, st)) != hipSuccess) return e;
  if (pl.n_blocks == 0) return hipSuccess;
  BlockStepArgs b{};
  b.num_req = (int)pl.n_blocks;
  b.H = f.H;
  b.D = f.D;
  b.bf16 = f.bf16;
  b.scale = f.scale;
  // 2. chunk: S_p from the chunk-start state and the clean tokens before p
  b.B = kChunk;
  b.mode = 1;
  b.slot_idx = pl.slm;
  b.pool = f.ckpt;
  b.q = f.q; b.k = f.k; b.v = f.v; b.alpha = f.alpha; b.beta = f.beta;
  b.o = nullptr;
  b.row0 = pl.r0m;
  b.count = pl.cm;
  b.pool_out = pl.bstates;
  if ((e = launch_block_step(b, st)) != hipSuccess) return e;
  // 3. refine: every noisy block from its boundary state, read at its end
  b.B = f.B;
  b.mode = 0;
  b.slot_idx = nullptr;
  b.pool = pl.bstates;
  b.q = f.qn; b.k = f.kn; b.v = f.vn; b.alpha = f.alpha_n; b.beta = f.beta_n;
  b.o = f.on;
  b.row0 = pl.r0r;
  b.count = pl.cr;
  b.pool_out = nullptr;
  return launch_block_step(b, st);
}

}  // namespace flare
