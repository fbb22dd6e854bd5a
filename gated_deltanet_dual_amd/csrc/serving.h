// serving.h -- argument blocks and launchers of the serving-step kernels and
// of the chunk-then-refine forward (internal).
#pragma once

#include "kernels.h"

namespace flare {

// mode 0 EVAL, 1 COMMIT, 2 VERIFY (COMMIT's outputs; the state after every
// token written to cand [num_req][B][H][D][D] instead of the last to the
// pool), 3 BOUNDARIES (table mode only, see below)
struct BlockStepArgs {
  int num_req, H, D, B, mode, bf16;
  float scale;
  const int32_t *slot_idx;
  float *pool;
  const void *q, *k, *v;
  const float *alpha, *beta;
  void *o;
  float *cand;
  // conv != 0: q, k, v are the raw projections; each goes through the
  // width-W ShortConv whose W - 1 earlier rows come from the request's clean
  // history cache [n_slots][W - 1][3][H * D] (io), then SiLU (act) and, for q
  // and k, the per-row L2 norm (l2); COMMIT keeps the last W - 1 raw rows as
  // the new history
  int conv, W, act, l2;
  void *cache;
  const float *cw[3];  // [H * D][W] per projection (q, k, v)
  // table mode (not with conv), all optional: request r's tokens are the rows
  // row0[r] .. row0[r] + B - 1 of token-major [T, H, D] inputs (gates
  // [T, H]); only the first count[r] (clamped to [0, B]) are real (the rest
  // are identity updates, their outputs not written; a COMMIT with none
  // leaves the state untouched); slot_idx NULL reads state r; COMMIT writes
  // the new state to pool_out[r] instead of in place
  const int32_t *row0, *count;
  float *pool_out;
  // mode 3 (table mode): no outputs; request r's window runs over its first
  // count[r] tokens (count[r] is its last block start, local) and the state
  // before its local token q, for q = blo[r], blo[r] + bB, ... <= count[r],
  // goes to pool_out[bg0[r] + (q - blo[r]) / bB]
  const int32_t *blo, *bg0;
  int bB;
  // mode 0 only: causal reads (o_t reads the state after token t, as COMMIT)
  // instead of block-end reads
  int causal;
};
hipError_t launch_block_step(const BlockStepArgs &a, hipStream_t st);

// the clean history of each document after a prefill: cache[slot_i][j][s] =
// x_s[end_i - (W - 1) + j] (zero before the document start)
struct ConvCacheArgs {
  int num_docs, C, W, bf16;
  const int32_t *cu, *slot;
  const void *x[3];
  void *cache;
};
hipError_t launch_conv_cache_fill(const ConvCacheArgs &a, hipStream_t st);

// AR-Trust rollback: pool[slot[r]] = cand[r][accepted[r] - 1] for accepted
// counts clamped to [0, K] (0 leaves the slot)
struct ScatterArgs {
  int num_req, H, D, K;
  const int32_t *slot_idx, *accepted;
  const float *cand;
  float *pool;
};
hipError_t launch_gdn_scatter(const ScatterArgs &a, hipStream_t st);

// the chunk-then-refine route (route1.hip): f as for launch_gdn_fwd with the
// chunk-start states f.ckpt required; the plan's arrays live in the workspace
struct Route1Plan {
  int64_t n_blocks;   // response blocks over all documents
  int64_t n_windows;  // chunks holding at least one block start
  float *bstates;     // [n_blocks, H, D, D] the block-boundary states
  int32_t *boff, *woff, *plen_all;          // [N]
  int32_t *wrow, *wcnt, *wslot, *wlo, *wg0;  // [n_windows] per chunk window
  int32_t *r0r, *cr;                         // [n_blocks] per noisy block
};
hipError_t launch_route1(const FwdArgs &f, const Route1Plan &pl, hipStream_t st);

}  // namespace flare
