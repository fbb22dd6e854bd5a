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
//   2. "chunk": every block-boundary state S_p materialised in memory, one
//      workgroup per (chunk, head) that holds a block start: it reads the
//      chunk-start state once and writes the state at each block start in
//      the chunk, by the per-token recurrence over the chunk's clean tokens;
//   3. "refine": every noisy block from its S_p (the serving step's EVAL).
// The per-block tables come from the documents' layout on the device.
#include "device_common.h"
#include "host_plan.h"
#include "kernels.h"
#include "serving.h"
#include "timing.h"

namespace flare {

namespace {


// Per-document offsets of the response blocks and of the chunk windows
// (exclusive scans of their counts), and the clean-only prompt lengths, in
// one workgroup.
__global__ __launch_bounds__(256) void route1_offsets_kernel(const int32_t *cu, const int32_t *plen, int N, int B,
                                                             int32_t *boff, int32_t *woff, int32_t *plen_all) {
  __shared__ int32_t sb[256], sw[256];
  __shared__ int32_t carry_b, carry_w;
  const int t = threadIdx.x;
  if (t == 0) carry_b = carry_w = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 256) {
    const int i = base + t;
    int nb = 0, nw = 0;
    if (i < N) {
      const int n = cu[i + 1] - cu[i], P = plen[i];
      if (n > P) {
        nb = (n - P + B - 1) / B;
        nw = (n + kChunk - 1) / kChunk - P / kChunk;
      }
      plen_all[i] = n;
    }
    sb[t] = nb;
    sw[t] = nw;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int vb = t >= off ? sb[t - off] : 0, vw = t >= off ? sw[t - off] : 0;
      __syncthreads();
      sb[t] += vb;
      sw[t] += vw;
      __syncthreads();
    }
    if (i < N) {
      boff[i] = carry_b + sb[t] - nb;
      woff[i] = carry_w + sw[t] - nw;
    }
    __syncthreads();
    if (t == 255) {
      carry_b += sb[255];
      carry_w += sw[255];
    }
    __syncthreads();
  }
}

// One workgroup per document: its chunk windows (every chunk from the one
// holding the prompt end to the last; each holds at least one block start)
// and the refine window of each response block.
__global__ __launch_bounds__(256) void route1_tables_kernel(const int32_t *cu, const int32_t *plen, int B,
                                                            const int32_t *boff, const int32_t *woff,
                                                            int32_t *wrow, int32_t *wcnt, int32_t *wslot,
                                                            int32_t *wlo, int32_t *wg0, int32_t *r0r,
                                                            int32_t *cr) {
  const int i = blockIdx.x;
  const int s = cu[i], n = cu[i + 1] - s, P = plen[i];
  if (n <= P) return;
  const int nb = (n - P + B - 1) / B;
  const int c0 = P / kChunk, nw = (n + kChunk - 1) / kChunk - c0;
  for (int j = threadIdx.x; j < nw; j += 256) {
    const int w = woff[i] + j, c = c0 + j;
    const int first = max(P, c * kChunk);  // the window's first block start
    wrow[w] = s + c * kChunk;
    const int span = min(kChunk, n - c * kChunk);  // the chunk's tokens in the document
    const int lo = first - c * kChunk;
    wcnt[w] = lo + (span - 1 - lo) / B * B;  // its last block start: the tokens the window runs over
    wslot[w] = s / kChunk + i + c;  // the chunk's start-state slot
    wlo[w] = lo;
    wg0[w] = boff[i] + (first - P) / B;
  }
  for (int j = threadIdx.x; j < nb; j += 256) {
    const int g = boff[i] + j, p = P + j * B;
    r0r[g] = s + p;
    cr[g] = min(B, n - p);
  }
}

}  // namespace

hipError_t launch_route1(const FwdArgs &f, const Route1Plan &pl, hipStream_t st) {
  const int N = f.num_docs;
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(route1_offsets_kernel, dim3(1), dim3(256), 0, st, f.cu, f.plen, N, f.B, pl.boff, pl.woff,
                     pl.plen_all);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.n_blocks > 0) {
    hipLaunchKernelGGL(route1_tables_kernel, dim3((unsigned)N), dim3(256), 0, st, f.cu, f.plen, f.B, pl.boff,
                       pl.woff, pl.wrow, pl.wcnt, pl.wslot, pl.wlo, pl.wg0, pl.r0r, pl.cr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 1. the clean stream with its chunk-start states (every row taken as clean:
  //    the noisy outputs come out zero and are refined below)
  FwdArgs clean = f;
  clean.plen = pl.plen_all;
  if ((e = launch_gdn_fwd(clean, st)) != hipSuccess) return e;
  if (pl.n_blocks == 0) return hipSuccess;
  BlockStepArgs b{};
  b.H = f.H;
  b.D = f.D;
  b.bf16 = f.bf16;
  b.scale = f.scale;
  // 2. chunk: the block-start states of every chunk window from its start state
  b.num_req = (int)pl.n_windows;
  b.B = kChunk;
  b.mode = 3;
  b.slot_idx = pl.wslot;
  b.pool = f.ckpt;
  b.q = f.q; b.k = f.k; b.v = f.v; b.alpha = f.alpha; b.beta = f.beta;
  b.o = nullptr;
  b.row0 = pl.wrow;
  b.count = pl.wcnt;
  b.blo = pl.wlo;
  b.bg0 = pl.wg0;
  b.bB = f.B;
  b.pool_out = pl.bstates;
  if ((e = launch_block_step(b, st)) != hipSuccess) return e;
  // 3. refine: every noisy block from its boundary state, read at its end
  b.num_req = (int)pl.n_blocks;
  b.B = f.B;
  b.mode = 0;
  b.slot_idx = nullptr;
  b.pool = pl.bstates;
  b.q = f.qn; b.k = f.kn; b.v = f.vn; b.alpha = f.alpha_n; b.beta = f.beta_n;
  b.o = f.on;
  b.row0 = pl.r0r;
  b.count = pl.cr;
  b.blo = b.bg0 = nullptr;
  b.pool_out = nullptr;
  return launch_block_step(b, st);
}

}  // namespace flare
