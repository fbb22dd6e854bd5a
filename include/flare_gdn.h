/*
 * flare_gdn.h -- C ABI of the MI355X (gfx950) dual-stream Gated DeltaNet
 * library: the clean causal stream, the block-wise noisy stream, their reverse
 * mode, the serving block step and the dual-source causal ShortConv.
 *
 * Source of the method: "FLARE: Diffusion for Hybrid Language Model"
 * (papernotes.org notes on arXiv 2606.01774):
 *   - Overall framework: the prompt is clean causal context only; the response
 *     is cut into consecutive blocks of B tokens (default 4).
 *   - Key designs, item 2: gated delta rule
 *       S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,
 *     the noisy block b starts from the clean boundary state S_{e(b-1)} and
 *     every position of the block reads the block-end state, scaled by
 *     1/sqrt(d_k); only strided clean checkpoints are kept, and the block
 *     gradients flow into the causal chain.
 *   - Key designs, item 3: ShortConv of width W before the GDN layer, whose
 *     taps before the block start read the clean input; cu_seqlens guards and
 *     block-aligned document boundaries, per-document state reset.
 *   - Key designs, item 4: denoising forwards read the global causal state pool
 *     but never write it; a causal replay writes it once the block is fixed.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued on it; no compute entry point synchronises,
 *     allocates or frees device memory (the measurement aid
 *     flare_timing_avg_ms, outside this contract, waits on its own events).
 *   - The caller owns every buffer.  Host arrays are read during the call only.
 *   - Outputs are fully overwritten (rows that are zero by definition are
 *     written as zeros); nothing is accumulated into.  Outputs must not alias
 *     inputs.
 *   - All arguments are validated on the host before anything is launched; a
 *     non-OK status means nothing was enqueued.  flare_last_error() returns a
 *     thread-local message for the last non-OK status of the calling thread.
 *   - Layouts are row-major with the last dimension contiguous.  T is the total
 *     number of packed tokens (cu_seqlens_host[num_docs]), H the head count.
 *   - io dtype (q, k, v, outputs and their gradients): FLARE_F32 or FLARE_BF16.
 *     Gates (alpha, beta), states and checkpoints are always fp32.
 */
#ifndef FLARE_GDN_H
#define FLARE_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLARE_OK = 0,
  FLARE_ERR_NULL = 1,        /* a required pointer is NULL                      */
  FLARE_ERR_SHAPE = 2,       /* inconsistent sizes / lengths / indices          */
  FLARE_ERR_ALIGN = 3,       /* prompt length or block size not aligned         */
  FLARE_ERR_UNSUPPORTED = 4, /* a size or dtype this build does not instantiate */
  FLARE_ERR_WORKSPACE = 5,   /* workspace too small or misaligned              */
  FLARE_ERR_HIP = 6          /* the HIP runtime reported an error               */
} flare_status;

enum { FLARE_F32 = 0, FLARE_BF16 = 1 };
enum { FLARE_BLOCK_EVAL = 0, FLARE_BLOCK_COMMIT = 1 };
/* shape.flags: divide q, k (and the noisy q~, k~) by sqrt(sum x^2 + 1e-6)
 * over d_k per (token, head) before use. */
#define FLARE_QK_L2NORM 1

/* Packed variable-length batch (the cu_seqlens guard of Key designs item 3).
 * Documents lie back to back; document i covers tokens
 * [cu_seqlens[i], cu_seqlens[i+1]) and its first prompt_lens[i] tokens are the
 * clean-only prompt.  Both arrays must be given on the device (read by the
 * kernels) and on the host (validated and planned before launch), with equal
 * contents.  Requirements: cu_seqlens[0] == 0, non-decreasing;
 * 0 <= prompt_lens[i] <= n_i; prompt_lens[i] % block_size == 0. */
typedef struct {
  int32_t num_docs;
  const int32_t *cu_seqlens;       /* device [num_docs+1] */
  const int32_t *cu_seqlens_host;  /* host   [num_docs+1] */
  const int32_t *prompt_lens;      /* device [num_docs]   */
  const int32_t *prompt_lens_host; /* host   [num_docs]   */
} flare_varlen;

/* Layer shape.  This build instantiates d_k == d_v in {16, 128} and
 * block_size in {1, 2, 4, 8, 16, 32}.  scale <= 0 selects 1/sqrt(d_k). */
typedef struct {
  int32_t num_heads;
  int32_t d_k;
  int32_t d_v;
  int32_t block_size;
  int32_t io_dtype; /* FLARE_F32 or FLARE_BF16 */
  int32_t flags;    /* 0 or FLARE_QK_L2NORM     */
  float scale;
} flare_gdn_shape;

/* Tokens per chunk of the chunk-parallel scan (documents are chunked locally,
 * from their own first token). */
int32_t flare_gdn_chunk_size(void);

/* Bytes of device workspace flare_gdn_dual_fwd (for_bwd = 0) or
 * flare_gdn_dual_bwd (for_bwd = 1) needs for this batch; 0 when the
 * configuration needs none (the forward needs workspace only for bf16 io at
 * d = 128 without flags) and on invalid arguments.  The workspace holds, per
 * chunk slot (checkpoint slot layout, stride 1) and head, six 32 x 32 fp32
 * chunk matrices first; for the backward also the chunk's end-state adjoint;
 * at bf16 io and d = 128 also the hand-over between a chunk pre-pass and the
 * sequential scan (86272 bytes), and for the forward room for the chunk-start
 * state (used when no checkpoints are asked for). */
size_t flare_gdn_dual_workspace_size(const flare_varlen *varlen,
                                     const flare_gdn_shape *shape, int for_bwd);

/* Strided checkpoints and chunk windows (Key designs item 2: keep only every
 * s-th clean state and rebuild the rest when they are needed).  Bytes of
 * workspace the chunked path (bf16 io, d = 128) needs when flare_gdn_dual_bwd
 * reads checkpoints of stride ckpt_stride_chunks (for_bwd = 1; the forward's
 * workspace does not depend on the stride) and when it runs in windows of
 * window_chunks chunks of every document (0: one pass over the whole batch).
 * A window keeps the per-chunk buffers of that many chunks of every document
 * only, so the workspace no longer grows with the sequence length; the chain
 * of states (and of their adjoints) is carried from window to window.  The
 * backward needs window_chunks to be a multiple of the stride; with a stride
 * above 1 it rebuilds the chunk-start states of each window from the
 * checkpoints, as parallel runs of stride chunks each.  Returns 0 on invalid
 * arguments and for shapes without the chunked path (there only stride 1,
 * window 0 and flare_gdn_dual_workspace_size apply).
 *
 * flare_gdn_dual_fwd and flare_gdn_dual_bwd choose the window from the
 * workspace_bytes they are given: one pass when it holds the one-pass layout
 * (flare_gdn_dual_workspace_size_window(..., 0)), else the largest window
 * (multiple of the stride for the backward) whose layout fits, else
 * FLARE_ERR_WORKSPACE.  Results do not depend on the window or on the stride
 * (the same arithmetic runs in the same order), except where the one-pass
 * scan of a long document runs in parallel runs (flare_gdn_dual_fwd's state
 * scan in runs then differs by rounding). */
size_t flare_gdn_dual_workspace_size_window(const flare_varlen *varlen,
                                            const flare_gdn_shape *shape,
                                            int for_bwd,
                                            int32_t ckpt_stride_chunks,
                                            int32_t window_chunks);

/* Checkpoints.  With C = flare_gdn_chunk_size() and stride s (in chunks), the
 * checkpoint of document i, local chunk c (c % s == 0) is the clean state at
 * the start of that chunk, fp32 [H, d_k, d_v], stored at slot
 *     floor(cu_seqlens[i] / (C*s)) + i + c / s
 * of a buffer [num_slots, H, d_k, d_v] with num_slots = floor(T / (C*s)) + N.
 * The slots of different documents never overlap.  Any s >= 1 may be written
 * by flare_gdn_dual_fwd; flare_gdn_dual_bwd reads s > 1 on the chunked path
 * (bf16 io, d = 128) only.  flare_gdn_dual_ckpt_size returns the buffer size
 * in bytes (0 on invalid arguments); flare_gdn_ckpt_slot is the slot formula
 * above. */
size_t flare_gdn_dual_ckpt_size(const flare_varlen *varlen,
                                const flare_gdn_shape *shape,
                                int32_t ckpt_stride_chunks);
int64_t flare_gdn_ckpt_slot(int32_t cu_seqlens_i, int32_t doc_index,
                            int32_t chunk_index, int32_t ckpt_stride_chunks);

/* Dual-stream forward (Key designs item 2; Overall framework).
 *   q, k       [T, H, d_k] io      clean queries / keys
 *   v          [T, H, d_v] io      clean values
 *   alpha,beta [T, H] fp32         clean gates, 0 < alpha <= 1
 *   qn,kn,vn,alpha_n,beta_n        noisy stream, same shapes; prompt rows are
 *                                  never read
 *   h0         [N, H, d_k, d_v] fp32 initial state per document, NULL = 0
 *   o          [T, H, d_v] io      clean outputs o_t = s S_t^T q_t
 *   on         [T, H, d_v] io      noisy outputs: every response position of a
 *                                  block reads the block-end noisy state; prompt
 *                                  rows are written 0
 *   h_final    [N, H, d_k, d_v] fp32 clean state after each document, or NULL
 *   ckpt       chunk-start clean states for the backward (see
 *              flare_gdn_dual_ckpt_size), or NULL for inference
 *   workspace  device scratch of flare_gdn_dual_workspace_size(..., 0) bytes
 *              (one pass), or of flare_gdn_dual_workspace_size_window(..., 0,
 *              s, w) bytes for windows of w chunks; 256-byte aligned; may be
 *              NULL when that size is 0
 * The clean block-boundary states are never written to memory. */
flare_status flare_gdn_dual_fwd(const flare_varlen *varlen,
                                const flare_gdn_shape *shape, const void *q,
                                const void *k, const void *v,
                                const float *alpha, const float *beta,
                                const void *qn, const void *kn, const void *vn,
                                const float *alpha_n, const float *beta_n,
                                const float *h0, void *o, void *on,
                                float *h_final, float *ckpt,
                                int32_t ckpt_stride_chunks, void *workspace,
                                size_t workspace_bytes, void *stream);

/* The same forward with the layer's ShortConv in its loads (Key designs items
 * 2 and 3: the dual ShortConv in front of the GDN layer, fused): q, k, v and
 * their noisy twins are never read or written.  Every row is formed, where the
 * chunked kernels load it, from the raw projections by the dual ShortConv of
 * flare_qkv_prologue (a noisy tap before the start of its block reads the
 * clean projection, taps before the document start read zero, noisy prompt
 * rows are zero), then SiLU when activation = 1, then rounded to bf16.
 *   width       1..4
 *   weight[3]   fp32 [H * d, width] for q, k, v (tap width - 1 on the current
 *               token), no bias
 *   x[3], xn[3] bf16 [T, H * d] clean and noisy projections of q, k, v
 *               (prompt rows of xn never read)
 * shape->flags = FLARE_QK_L2NORM normalises the q and k rows after the
 * convolution.  The result equals flare_qkv_prologue(..., qk_l2norm = 0)
 * followed by flare_gdn_dual_fwd with the same shape, bit for bit.  bf16 io at
 * d = 128 only (FLARE_ERR_UNSUPPORTED otherwise).  All other arguments,
 * checkpoints and the workspace (one pass or windows) as flare_gdn_dual_fwd. */
flare_status flare_gdn_dual_fwd_conv(const flare_varlen *varlen,
                                     const flare_gdn_shape *shape, int32_t width,
                                     const float *const weight[3],
                                     int32_t activation, const void *const x[3],
                                     const void *const xn[3], const float *alpha,
                                     const float *beta, const float *alpha_n,
                                     const float *beta_n, const float *h0,
                                     void *o, void *on, float *h_final,
                                     float *ckpt, int32_t ckpt_stride_chunks,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/* The chunk-then-refine route for the same forward (Key designs item 2 and
 * the pages' comparison of the two ways to give every noisy block its clean
 * boundary state): the clean stream with its chunk-start states (ckpt,
 * required, flare_gdn_dual_ckpt_size(..., 1) bytes), then every block-boundary
 * state materialised in the workspace, then every noisy block refined from its
 * state.  Same results as flare_gdn_dual_fwd (o, on, h_final) at O(L / B)
 * states of memory; built for comparing the two routes.  Requirements as
 * flare_gdn_dual_fwd, plus d_k = d_v in {16, 128} and no flags; the
 * workspace is flare_gdn_route1_workspace_size bytes, 256-byte aligned. */
size_t flare_gdn_route1_workspace_size(const flare_varlen *varlen,
                                       const flare_gdn_shape *shape);
flare_status flare_gdn_dual_fwd_route1(const flare_varlen *varlen,
                                       const flare_gdn_shape *shape,
                                       const void *q, const void *k,
                                       const void *v, const float *alpha,
                                       const float *beta, const void *qn,
                                       const void *kn, const void *vn,
                                       const float *alpha_n,
                                       const float *beta_n, const float *h0,
                                       void *o, void *on, float *h_final,
                                       float *ckpt, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Prefill into the serving pool (Key designs item 4: the serving pool holds
 * one causal state per request): flare_gdn_dual_fwd with every document's
 * state kept in a pool slot instead of the h0 / h_final arrays.
 *   doc_slot       device int32 [N]: the pool slot of each document
 *   doc_slot_host  optional host copy, checked for range and duplicates
 *                  (FLARE_ERR_SHAPE) as in flare_gdn_block_step
 *   state_pool     fp32 [num_slots, H, d_k, d_v]; document i's final clean
 *                  state is written to state_pool[doc_slot[i]], every other
 *                  slot is untouched
 *   read_initial   1: document i starts from state_pool[doc_slot[i]] (read
 *                  before it is overwritten); 0: from zero
 * All other arguments, requirements and the workspace are those of
 * flare_gdn_dual_fwd.  The pool can then be served by flare_gdn_block_step
 * and flare_gdn_verify without a copy. */
flare_status flare_gdn_dual_fwd_pool(const flare_varlen *varlen,
                                     const flare_gdn_shape *shape,
                                     const void *q, const void *k, const void *v,
                                     const float *alpha, const float *beta,
                                     const void *qn, const void *kn,
                                     const void *vn, const float *alpha_n,
                                     const float *beta_n,
                                     const int32_t *doc_slot,
                                     const int32_t *doc_slot_host,
                                     float *state_pool, int32_t num_slots,
                                     int32_t read_initial, void *o, void *on,
                                     float *ckpt, int32_t ckpt_stride_chunks,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Reverse mode of flare_gdn_dual_fwd (Key designs items 2 and 3): the adjoint
 * reaching each noisy block start is added to the clean adjoint at that block's
 * boundary, the adjoint is reset per document, and nothing crosses documents.
 * Inputs: the forward's inputs, its checkpoints (same stride), the output
 * gradients d_o, d_on [T, H, d_v] io (prompt rows of d_on ignored) and
 * dh_final [N, H, d_k, d_v] fp32 or NULL.
 * Outputs (written, not accumulated): dq, dk [T,H,d_k], dv [T,H,d_v] io;
 * dalpha, dbeta [T,H] fp32; the same five for the noisy stream (prompt rows 0);
 * dh0 [N,H,d_k,d_v] fp32 or NULL.  workspace: see
 * flare_gdn_dual_workspace_size(..., 1) (one pass, stride 1) and
 * flare_gdn_dual_workspace_size_window, 256-byte aligned.
 * fwd_workspace: NULL, or the workspace of the flare_gdn_dual_fwd call that
 * produced ckpt, when that call ran in one pass, still holding what it wrote
 * there (same inputs, shape and batch): its chunk matrices are then read
 * instead of formed again when this call runs in one pass too (a windowed
 * call forms its own).  The result is the same either way. */
flare_status flare_gdn_dual_bwd(
    const flare_varlen *varlen, const flare_gdn_shape *shape, const void *q,
    const void *k, const void *v, const float *alpha, const float *beta,
    const void *qn, const void *kn, const void *vn, const float *alpha_n,
    const float *beta_n, const float *h0, const float *ckpt,
    int32_t ckpt_stride_chunks, const void *fwd_workspace, const void *d_o, const void *d_on,
    const float *dh_final, void *dq, void *dk, void *dv, float *dalpha,
    float *dbeta, void *dqn, void *dkn, void *dvn, float *dalpha_n,
    float *dbeta_n, float *dh0, void *workspace, size_t workspace_bytes,
    void *stream);

/* Serving block step over a pool of per-request recurrent states (Key designs
 * item 4).
 *   slot_idx      [num_req] int32 device: pool slot of each request; slots must
 *                 be distinct and in [0, num_slots).  Checked only when
 *                 slot_idx_host (same contents) is given; otherwise duplicate or
 *                 out-of-range slots are undefined behaviour.
 *   state_pool    [num_slots, H, d_k, d_v] fp32
 *   q, k          [num_req, B, H, d_k] io;  v [num_req, B, H, d_v] io
 *   alpha, beta   [num_req, B, H] fp32, B = shape->block_size
 *   o             [num_req, B, H, d_v] io
 * FLARE_BLOCK_EVAL: a denoising read.  The B noisy updates are applied to a
 *   private copy of the pooled state and every position reads the block-end
 *   state.  The pool is not written.
 * FLARE_BLOCK_COMMIT: causal replay of the committed block.  The B clean
 *   updates are applied in order, o_t reads the state after token t (o may be
 *   NULL to skip the outputs), and the final state is written to the pool. */
flare_status flare_gdn_block_step(int32_t num_req, const int32_t *slot_idx,
                                  const int32_t *slot_idx_host,
                                  float *state_pool, int32_t num_slots,
                                  const flare_gdn_shape *shape, const void *q,
                                  const void *k, const void *v,
                                  const float *alpha, const float *beta,
                                  void *o, int32_t mode, void *stream);

/* The serving step with the ShortConv in front (Key designs item 3 for the
 * convolution, item 4 for the pool): flare_gdn_block_step whose q, k, v are
 * the raw projections xq, xk, xv [num_req, B, H, d] io.  Each request keeps
 * its clean history -- the last width-1 clean projection rows -- in
 *   conv_cache   io [num_slots, width-1, 3 (q, k, v), H * d], slot slot_idx[r]
 *                (may be NULL when width = 1)
 * so the block's taps before its start read that clean history and the taps
 * inside read the block itself (EVAL: the noisy draft; COMMIT: the fixed
 * block), then SiLU (activation = 1) and, with qk_l2norm, q and k divided per
 * (token, head) by sqrt(sum x^2 + 1e-6).  COMMIT also replaces the history
 * with the last width-1 raw rows of history + block; EVAL writes neither the
 * state pool nor the cache.
 *   weight[3]    fp32 [H * d, width] per projection, tap width-1 on the
 *                current token (as flare_shortconv_dual); no bias
 * Requirements: as flare_gdn_block_step, shape->flags = 0, width in [1, 8],
 * block_size <= 8 (FLARE_ERR_UNSUPPORTED otherwise). */
flare_status flare_gdn_block_step_conv(int32_t num_req, const int32_t *slot_idx,
                                       const int32_t *slot_idx_host,
                                       float *state_pool, void *conv_cache,
                                       int32_t num_slots,
                                       const flare_gdn_shape *shape,
                                       int32_t width,
                                       const float *const weight[3],
                                       int32_t activation, int32_t qk_l2norm,
                                       const void *xq, const void *xk,
                                       const void *xv, const float *alpha,
                                       const float *beta, void *o, int32_t mode,
                                       void *stream);

/* After a prefill (flare_gdn_dual_fwd_pool): each document's clean history,
 * conv_cache[doc_slot[i]][j][s] = x[s][end_i - (width-1) + j], zero for rows
 * before the document start.  x[3]: the clean q, k, v projections
 * [T, heads * head_dim] io of the prefilled batch; doc_slot: device int32
 * [N]; doc_slot_host optional (range and duplicates checked).  Nothing to do
 * for width = 1. */
flare_status flare_conv_cache_fill(const flare_varlen *varlen, int32_t heads,
                                   int32_t head_dim, int32_t width,
                                   int32_t io_dtype, const void *const x[3],
                                   const int32_t *doc_slot,
                                   const int32_t *doc_slot_host,
                                   void *conv_cache, int32_t num_slots,
                                   void *stream);

/* AR-Trust (Key designs item 4: the noisy stream drafts K tokens, the clean
 * stream verifies them in one parallel pass, and a partial acceptance of the
 * first r < K tokens is rolled back without recomputation by keeping the K
 * intermediate states and scattering the accepted one).
 *
 * flare_gdn_verify: for each request r and head, from S = pool[slot_idx[r]]
 * (read only), the K = shape->block_size clean causal updates of the drafted
 * tokens with per-token outputs o_t = s S_t^T q_t (as COMMIT), and the state
 * after every token written to
 *   cand   [num_req, K, H, d_k, d_v] fp32, cand[r][t] = state after token t+1
 * Arguments as flare_gdn_block_step (q, k, v, alpha, beta, o: [num_req, K, H, .]);
 * o and cand are required.  The pool is not written.
 *
 * flare_gdn_scatter: for each request r, with a = accepted[r] (device int32,
 * clamped to [0, K]), a >= 1 copies cand[r][a-1] into pool[slot_idx[r]] and
 * a = 0 leaves the slot as it was.  cand as written by flare_gdn_verify with
 * the same shape; slot_idx_host (optional) as for flare_gdn_block_step.  The
 * accepted counts stay on the device: the caller's acceptance test never
 * round-trips through the host. */
flare_status flare_gdn_verify(int32_t num_req, const int32_t *slot_idx,
                              const int32_t *slot_idx_host,
                              const float *state_pool, int32_t num_slots,
                              const flare_gdn_shape *shape, const void *q,
                              const void *k, const void *v, const float *alpha,
                              const float *beta, void *o, float *cand,
                              void *stream);
flare_status flare_gdn_scatter(int32_t num_req, const int32_t *slot_idx,
                               const int32_t *slot_idx_host,
                               const int32_t *accepted, const float *cand,
                               float *state_pool, int32_t num_slots,
                               const flare_gdn_shape *shape, void *stream);


/* AR-Trust without the candidate buffer (Key designs item 4 names the
 * rollback; this pair reaches the same pool state by replaying the accepted
 * prefix instead of keeping every intermediate state).  Per (request, head) it
 * reads the pooled state twice and writes it once, where verify + scatter
 * write K candidates and copy one.
 *
 * flare_gdn_verify_outputs: the per-token causal outputs of flare_gdn_verify
 * (o_t = s S_t^T q_t after drafted token t), without the candidates.  Arguments
 * as flare_gdn_verify without cand; o is required; the pool is not written.
 *
 * flare_gdn_commit_prefix: for each request r, with a = accepted[r] (device
 * int32, clamped to [0, K], K = shape->block_size), the COMMIT of the first a
 * drafted tokens: their clean updates are applied to pool[slot_idx[r]] in
 * order and the state is written back; a = 0 leaves the slot untouched.  The
 * resulting slot equals what flare_gdn_scatter writes after flare_gdn_verify
 * (up to rounding).  q, k, v, alpha, beta [num_req, K, H, .] as for
 * flare_gdn_verify; o (optional, [num_req, K, H, d_v]) receives the causal
 * outputs of the first a tokens (rows past a are not written).  Other
 * arguments and errors as flare_gdn_block_step. */
flare_status flare_gdn_verify_outputs(int32_t num_req, const int32_t *slot_idx,
                                      const int32_t *slot_idx_host,
                                      const float *state_pool,
                                      int32_t num_slots,
                                      const flare_gdn_shape *shape,
                                      const void *q, const void *k,
                                      const void *v, const float *alpha,
                                      const float *beta, void *o,
                                      void *stream);
flare_status flare_gdn_commit_prefix(int32_t num_req, const int32_t *slot_idx,
                                     const int32_t *slot_idx_host,
                                     float *state_pool, int32_t num_slots,
                                     const flare_gdn_shape *shape,
                                     const void *q, const void *k,
                                     const void *v, const float *alpha,
                                     const float *beta,
                                     const int32_t *accepted, void *o,
                                     void *stream);

/* Dual-source depthwise causal ShortConv (Key designs item 3).
 *   x, xn   [T, channels] io        clean / noisy inputs (xn prompt rows unread)
 *   weight  [channels, width] fp32  weight[c, width-1] multiplies the current
 *                                   token
 *   bias    [channels] fp32 or NULL
 *   activation 0 = none, 1 = SiLU (applied after the bias)
 *   y       [T, channels] io  y[t] = sum_j weight[c,j] x[t-(width-1)+j], taps
 *                             before the document start read 0
 *   yn      [T, channels] io  same taps, but a tap that lies before the start
 *                             of t's noisy block reads x (clean history) and a
 *                             tap inside the block reads xn; prompt rows 0
 * Requirements: 1 <= width <= 8, channels % 8 == 0 for bf16 (% 4 for f32). */
flare_status flare_shortconv_dual(const flare_varlen *varlen,
                                  int32_t block_size, int32_t channels,
                                  int32_t width, int32_t io_dtype,
                                  const void *x, const void *xn,
                                  const float *weight, const float *bias,
                                  int32_t activation, void *y, void *yn,
                                  void *stream);

/* Reverse mode of flare_shortconv_dual (Key designs item 3: the gradient of a
 * noisy output reaches the clean input through its taps before the block start
 * and the noisy input through its taps inside the block).  Same varlen,
 * block_size, channels, width, io_dtype, x, xn, weight, bias and activation as
 * the forward call, plus
 *   dy, dyn  [T, channels] io   gradients of y and yn (dyn prompt rows ignored)
 *   dx, dxn  [T, channels] io   written: gradients of x and xn (dxn prompt rows 0)
 *   dweight  [channels, width] fp32  written
 *   dbias    [channels] fp32 or NULL  written when given (the sum of the
 *            pre-activation gradients, whether or not the forward had a bias)
 *   workspace  flare_shortconv_dual_bwd_workspace_size bytes, 256-byte aligned
 *            (per-run partial sums of dweight and dbias, reduced in a fixed
 *            order: the result is run-to-run identical)
 * Requirements as for the forward. */
size_t flare_shortconv_dual_bwd_workspace_size(const flare_varlen *varlen,
                                               int32_t block_size, int32_t channels,
                                               int32_t width);
flare_status flare_shortconv_dual_bwd(const flare_varlen *varlen,
                                      int32_t block_size, int32_t channels,
                                      int32_t width, int32_t io_dtype,
                                      const void *x, const void *xn,
                                      const float *weight, const float *bias,
                                      int32_t activation, const void *dy,
                                      const void *dyn, void *dx, void *dxn,
                                      float *dweight, float *dbias,
                                      void *workspace, size_t workspace_bytes,
                                      void *stream);

/* The GDN layer's input prologue, fused: the dual-source ShortConv of
 * flare_shortconv_dual (Key designs item 3) on each of the q, k, v projections
 * of both streams in one launch, an optional SiLU, and -- with qk_l2norm -- q
 * and k divided per (token, head) by sqrt(sum x^2 + 1e-6) (not on the pages:
 * the usual q/k normalisation in front of a gated delta rule, the same
 * reading as FLARE_QK_L2NORM).  The outputs are ready for flare_gdn_dual_fwd
 * without flags.
 *   heads, head_dim   each projection is [T, heads * head_dim] io, channels
 *                     contiguous (the [T, H, d] layout of q, k, v)
 *   x[3], xn[3]       clean / noisy projections (q, k, v); noisy prompt rows
 *                     are never read
 *   weight[3]         fp32 [heads * head_dim, width] per projection, tap
 *                     width-1 on the current token; no bias
 *   y[3], yn[3]       written: the prologue outputs (noisy prompt rows 0)
 * Requirements as for flare_shortconv_dual per projection, plus with qk_l2norm
 * head_dim / (8 / sizeof(io) channels, 4 / sizeof(io) for width > 4) a power of
 * two of at most 64 (FLARE_ERR_UNSUPPORTED otherwise).  The arrays are host
 * arrays of device pointers, read during the call. */
flare_status flare_qkv_prologue(const flare_varlen *varlen, int32_t block_size,
                                int32_t heads, int32_t head_dim, int32_t width,
                                int32_t io_dtype, const void *const x[3],
                                const void *const xn[3],
                                const float *const weight[3],
                                int32_t activation, int32_t qk_l2norm,
                                void *const y[3], void *const yn[3],
                                void *stream);

/* Reverse mode of flare_qkv_prologue: the same inputs, plus
 *   dy[3], dyn[3]     gradients of y, yn (dyn prompt rows ignored)
 *   dx[3], dxn[3]     written: gradients of the projections (dxn prompt rows 0)
 *   dweight[3]        written: fp32 [heads * head_dim, width]
 *   workspace         flare_qkv_prologue_bwd_workspace_size bytes, 256-byte
 *                     aligned (per-block weight partials, reduced in a fixed
 *                     order: results are run-to-run identical)
 * The L2 step's gradient is taken inside the kernel from the recomputed
 * convolution outputs. */
size_t flare_qkv_prologue_bwd_workspace_size(const flare_varlen *varlen,
                                             int32_t block_size, int32_t heads,
                                             int32_t head_dim, int32_t width);
flare_status flare_qkv_prologue_bwd(const flare_varlen *varlen,
                                    int32_t block_size, int32_t heads,
                                    int32_t head_dim, int32_t width,
                                    int32_t io_dtype, const void *const x[3],
                                    const void *const xn[3],
                                    const float *const weight[3],
                                    int32_t activation, int32_t qk_l2norm,
                                    const void *const dy[3],
                                    const void *const dyn[3], void *const dx[3],
                                    void *const dxn[3], float *const dweight[3],
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/* flare_qkv_prologue_bwd without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight training
 * or serving loops, harnesses that forbid allocation.  The weight-gradient
 * partials go to a static device array of the library instead,
 * flare_noalloc_scratch_bytes() = 64 MiB on every GPU the library runs on,
 * held until the process ends.  The call allocates and frees nothing.
 * Arguments, results and the other errors as flare_qkv_prologue_bwd.
 * Errors: FLARE_ERR_WORKSPACE when the batch would need more partials than
 * the array holds (flare_qkv_prologue_bwd_workspace_size() > 64 MiB, e.g.
 * more than 3 x 32768 tokens x 4096 channels at width 4).
 * The first call on a device (with that device current) looks the array's
 * device address up with hipGetSymbolAddress: make that first call outside a
 * graph capture.  All calls on one GPU share its array: calls that overlap
 * in time on one GPU (two streams, two host threads) race; calls ordered on
 * one stream do not (the partials are fully written before they are read, so
 * nothing carries over from the previous call). */
size_t flare_noalloc_scratch_bytes(void);
flare_status flare_qkv_prologue_bwd_noalloc(const flare_varlen *varlen,
                                            int32_t block_size, int32_t heads,
                                            int32_t head_dim, int32_t width,
                                            int32_t io_dtype,
                                            const void *const x[3],
                                            const void *const xn[3],
                                            const float *const weight[3],
                                            int32_t activation,
                                            int32_t qk_l2norm,
                                            const void *const dy[3],
                                            const void *const dyn[3],
                                            void *const dx[3],
                                            void *const dxn[3],
                                            float *const dweight[3],
                                            void *stream);

/* Thread-local message for the last non-OK status; "" if none. */
const char *flare_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t flare_version(void);

/* ---- per-launch timing (measurement aid; no passage of the method) -------
 * While enabled, every kernel launch made by the entry points above is
 * bracketed by two HIP events recorded on the launch's own stream, so the
 * duration of each kernel is known even when one entry point launches several
 * (the backward launches the reverse scan, then the per-chunk kernel).
 * Kernel names: "gdn_dual_fwd_kernel", "gdn_bwd_scan_kernel",
 * "gdn_bwd_chunk_kernel", "block_step_kernel", "shortconv_dual_kernel",
 * "shortconv_dual_bwd_kernel" (both kernels of flare_shortconv_dual_bwd;
 * flare_qkv_prologue and its reverse mode are timed under the ShortConv names;
 * flare_gdn_verify under "block_step_kernel"), "gdn_scatter_kernel",
 * and, for bf16 io at d = 128, the chunked passes: "gdn_fwd_prep_kernel"
 * (the forward's chunk matrices and scan hand-over in one pass; also the
 * backward's re-formed hand-over when it rebuilds states from strided
 * checkpoints), "gdn_tri_kernel" (the chunk matrices alone, for a backward
 * that does not take the forward's), "gdn_fwd_pre_kernel" (the hand-over
 * from given chunk matrices) and "gdn_bwd_pre_kernel" (the state-independent
 * parts of the reverse chunk step),
 * "gdn_fwd_scan_kernel" (the forward state recurrence; "gdn_dual_fwd_kernel"
 * then names the forward's output pass) and "gdn_bwd_scan_kernel" (the
 * reverse recurrence).
 * flare_timing_enable(1) turns it on (events are created lazily, host side
 * only; no device memory is allocated), (0) off.  Returns the previous state.
 * flare_timing_avg_ms() blocks until the recorded launches of that kernel
 * have finished and returns their mean duration in ms (-1 if none), writing
 * the launch count to *launches when non-NULL.  flare_timing_reset() drops
 * every record.  Process-wide, guarded by a mutex. */
int32_t flare_timing_enable(int32_t on);
double flare_timing_avg_ms(const char *kernel, int64_t *launches);
void flare_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* FLARE_GDN_H */
