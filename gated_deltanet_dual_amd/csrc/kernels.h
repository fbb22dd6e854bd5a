// kernels.h -- argument blocks and launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flare {

// ShortConv over up to three sections of channels sharing one document
// layout (the q, k, v projections of the GDN layer's input prologue; one
// section for a plain ShortConv).  Each section is [T, C] with its own
// tensors and weights; the first nnorm sections are L2-normalised after the
// convolution (and activation) per group of hd consecutive channels (a head).
struct ShortConvArgs {
  int num_docs, B, C, W, activation, bf16;
  int nsec, nnorm, hd;
  int64_t T;
  const int32_t *cu, *plen;
  const void *x[3], *xn[3];
  const float *w[3], *bias;  // bias: plain ShortConv (one section) only
  void *y[3], *yn[3];
};
hipError_t launch_shortconv(const ShortConvArgs &a, hipStream_t st);

// reverse mode of the ShortConv (shortconv_bwd.hip)
struct ShortConvBwdArgs {
  int num_docs, B, C, W, activation, bf16;
  int nsec, nnorm, hd;
  int64_t T;
  const int32_t *cu, *plen;
  const void *x[3], *xn[3], *dy[3], *dyn[3];
  const float *w[3], *bias;
  void *dx[3], *dxn[3];
  float *dw[3], *dbias;
  // workspace: per section [ceil(T / 256)][C][W + 1] block partials of
  // dweight and dbias
  float *part;
};
hipError_t launch_shortconv_bwd(const ShortConvBwdArgs &a, hipStream_t st);

struct FwdArgs {
  int num_docs, H, D, B, flags, bf16, ckpt_stride;
  // 0, or S when every document has S chunk slots (equal lengths, a multiple
  // of the chunk, one pass): the output pass then visits the slots chunk-major
  // from the last chunks down, the states the scan wrote last first
  int slot_order;
  float scale;
  const int32_t *cu, *plen;
  const void *q, *k, *v, *qn, *kn, *vn;
  const float *alpha, *beta, *alpha_n, *beta_n, *h0;
  void *o, *on;
  float *h_final, *ckpt;
  float *workspace;  // the forward's chunk matrices (bf16, d = 128, no flags)
  int64_t T;
  // NULL, or per document the index of its state in h0 / h_final (a state
  // pool): document i starts from h0[state_slot[i]] and ends in
  // h_final[state_slot[i]]
  const int32_t *state_slot;
  // The chunked bf16 d = 128 kernels with the q/k L2 flag: per (token, head)
  // {r_q, r_k, r_q~, r_k~}, r = 1 / sqrt(sum x^2 + 1e-6) of that row (NULL
  // without the flag).  The kernels never form the normalised rows: with
  // k^ = r_k k the step is the plain one on (k, b r_k^2, v / r_k), and
  // o = r_q s S^T q (gdn_l2.hip).
  const float4 *l2f;
  // the state scan in parallel runs of scan_span chunks (0: one chain per
  // document and head), scan_units runs, their buffers at scan_ws (gdn_scan.hip)
  int scan_span;
  int64_t scan_units;
  float *scan_ws;
  // Chunk windows (win_len > 0): a launch covers chunks [win_lo, win_lo +
  // win_len) of every document, and the per-chunk workspace arrays hold only
  // those, at slot doc * win_len + (c - win_lo); win_len = 0: every chunk, at
  // its checkpoint slot of stride 1.
  int win_lo, win_len;
  // The ShortConv in the loads (cw > 0; chunked forward only): q, k, v and
  // their noisy twins are not read; every row is formed from the raw
  // projections cx / cxn ([T, H * 128] bf16: q, k, v) by the dual ShortConv
  // of width cw with weights cwt ([H * 128, cw] fp32) and SiLU when cact
  // (conv_load.h); with the q/k L2 flag the preparation pass forms the L2
  // factors from those rows into l2f.
  const void *cx[3], *cxn[3];
  const float *cwt[3];
  int cw, cact;
};
// Where the chunked forward (bf16 io, d = 128) keeps its per-chunk buffers
// and how it walks the chunks: one pass (win = 0) or windows of win chunks of
// every document, the chain carried between them in carry.
struct FwdPlan {
  float *cmat, *pack;
  float *states;  // chunk-start states per slot; NULL: the stride-1 checkpoints (one pass)
  float4 *l2f;    // q/k L2 factors, when the flag is set
  float *carry;   // windows: [N, H, 128, 128]
  int win, max_chunks;
  int64_t slots;  // per-chunk slots of one pass (window)
};
// a.workspace set: the chunked passes, with `plan` (NULL: one pass over the
// whole workspace in its one-pass layout); else the per-(document, head) kernel
hipError_t launch_gdn_fwd(const FwdArgs &a, hipStream_t st, const FwdPlan *plan = nullptr);
// the per-row L2 factors of q, k, q~, k~ into a.l2f (gdn_l2.hip)
hipError_t launch_l2_factors(const FwdArgs &a, float4 *out, hipStream_t st);

// bf16 io at d = 128 without flags: the forward's pre-pass (chunk matrices
// `cmat` -> scan hand-over `pack`, gdn_fwd_pre.hip) and its output pass
// (chunk-start states -> o, o~, gdn_fwd_out.hip)
hipError_t launch_fwd_pre_d128(const FwdArgs &a, const float *cmat, float *pack, hipStream_t st, int64_t slots);
// both in one pass: the chunk matrices into `cmat` and the hand-over into
// `pack` from one load of the chunk (gdn_fwd_prep.hip)
hipError_t launch_fwd_prep_d128(const FwdArgs &a, float *cmat, float *pack, hipStream_t st, int64_t slots);
hipError_t launch_fwd_out_d128(const FwdArgs &a, const float *cmat, const float *states, hipStream_t st,
                               int64_t slots);

// The sequential chunk recurrence X <- g_C X + R + K^T (W (K X)) over the chunks
// of each document (gdn_scan.hip), forward or in reverse.
//
// Runs: with seg_span > 0 each document's chunks are cut into runs of
// seg_span chunks, scanned in parallel; run (document i, index g) is unit
// ckpt_slot(cu_i, i, g * seg_span, seg_span) (host_plan.h), units in all
// ckpt_num_slots(T, N, seg_span).  A document's first run in scan order starts
// from init (or zero), every other run from seg_init[unit] (or zero when
// seg_init is NULL); with identity_init every run starts from the identity
// instead, and with homog the step drops its right-hand side, so the run
// computes its transfer map X -> M X.  seg_final[unit] receives X after the
// run's last step.  seg_span = 0: one run per document (unit = document).
struct ScanArgs {
  int num_docs, H;
  const int32_t *cu;
  const float *pack;   // per (chunk slot, head): the pre-pass's hand-over
  const float *init;   // [N, H, 128, 128] X before the first step, or NULL (zero)
  float *final_out;    // [N, H, 128, 128] X after the last step, or NULL
  float *states;       // [slots, H, 128, 128]: X before the step of chunk c, at chunk c's slot (or NULL)
  const int32_t *slot; // NULL, or per document the index of its init / final_out state
  int states_stride;   // 0 or 1: every chunk; S > 1: chunks c % S == 0 only, at ckpt_slot(cu_i, i, c, S)
  int seg_span;        // chunks per run (0: whole documents)
  int64_t units;       // number of units (runs), seg_span > 0
  const float *seg_init;
  float *seg_final;
  int identity_init, homog;
  // every run starts from seg_init, a document's first one too (the runs
  // rebuilding the chunk-start states from strided checkpoints)
  int seg_init_all;
  // > 0: seg_init is indexed by the run's checkpoint slot of this stride (a
  // divisor of seg_span) instead of seg_span's
  int seg_init_stride;
  // Chunk windows (win_len > 0, states_stride 1): each document's chain covers
  // chunks [win_lo, win_lo + win_len) only, from init to final_out (a chain
  // with no chunk there copies init to final_out); pack and states are
  // indexed by the window slot doc * win_len + (c - win_lo).  With seg_span
  // > 0 as well (win_lo and win_len multiples of it) the units are the runs
  // inside the window, numbered doc * (win_len / seg_span) + g, and
  // seg_init / seg_final are indexed by the run's checkpoint slot of stride
  // seg_span (so the strided checkpoints are the runs' start values).
  int win_lo, win_len;
  // Strided checkpoints besides states: X before the step of chunk c,
  // c % ckpt_stride == 0, at ckpt_slot(cu_i, i, c, ckpt_stride) (or NULL).
  float *ckpt;
  int ckpt_stride;
  // Reverse scan only: K X of every chunk, the product its step forms anyway
  // (for the per-chunk backward kernel, which would otherwise form K dS' from
  // dS' itself), as slabs [slab 8][tile 2][lane 64][4] at the start of the
  // chunk's R area in the hand-over (kx = pack): each wave writes only over
  // its own R slab, after its step has consumed it.  NULL: not written.
  float *kx;
  // NULL, or a hand-over of the same slot layout whose K fragment units (the
  // A operands of K X and K^T Y, identical in every hand-over of the chunk)
  // the reverse scan reads instead of pack's (the forward's hand-over; the
  // forward scan ignores this field).
  const float *kpack;
};
hipError_t launch_scan_d128(const ScanArgs &a, bool reverse, hipStream_t st);
// The runs' start states from their transfer maps M (identity-init, homog
// runs) and offsets N (zero-init runs): in scan order X_0 = init (or zero),
// seg_out[unit_g] = X_g, X_{g+1} = M_g X_g + N_g (gdn_scan.hip).
hipError_t launch_scan_compose_d128(const ScanArgs &a, const float *M, const float *Nb, float *seg_out, bool reverse,
                                    hipStream_t st, bool m_transposed = false);
// The scan of a, in one chain per (document, head) when span == 0, else in
// parallel runs of span chunks joined by their transfer maps: the maps, the
// offsets, the composition, then every run from its start value (ws holds
// 3 x units x H x 128 x 128 fp32).
// maps_t: the runs' transfer maps given transposed (the reverse scan taking
// the forward's), so that their scan pass is skipped; NULL: formed here.
hipError_t scan_d128_runs(const ScanArgs &a, bool reverse, int span, int64_t units, float *ws, hipStream_t st,
                          const float *maps_t = nullptr);

struct BwdArgs {
  FwdArgs f;
  const float *ckpt_in;
  const void *d_o, *d_on;
  const float *dh_final;
  void *dq, *dk, *dv, *dqn, *dkn, *dvn;
  float *dalpha, *dbeta, *dalpha_n, *dbeta_n, *dh0;
  void *workspace;       // end-state adjoints [slots][H][D][D], then `tri`
  size_t workspace_bytes;
  int64_t T;
  float *tri;            // per slot and head [slots][H][6][32][32] (each matrix tile-major, chunk_common.h): T, T~, Mwo, Mwq, Mwk, Mw~ (set by the launcher)
  const float *fwd_cm;   // the same matrices from the forward's workspace, or NULL
  const float *fwd_pack; // the forward's scan hand-over in the same workspace, or NULL
  // the hand-over whose K fragment sets the reverse scan reads (the forward's,
  // when its chunk matrices are reused); the pre-pass then does not write
  // its own (set by the launcher)
  const float *kpack;
  // the forward's runs' transfer maps (long documents, one pass), or NULL: the
  // reverse scan's map of a run is the transpose of the forward's (its chain
  // matrix is the forward's transposed), so it composes with those
  const float *fwd_maps;
  float *pack;           // bf16, d = 128: the pre-pass's hand-over to the scan, per slot and head (set by the launcher)
  // ckpt_in holds every chunk-start state at the chunk's checkpoint slot of
  // stride 1 (a checkpoint buffer) rather than at the (window) slot
  int ckpt_global;
};
// The backward's per-chunk buffers on the chunked path (bf16 io, d = 128):
// as for the forward, plus the rebuilt chunk-start states when the
// checkpoints hold only every stride-th one.
struct BwdPlan {
  float *adj, *tri, *pack;
  float *states;  // rebuilt chunk-start states per slot (stride > 1), else NULL
  float4 *l2f;
  float *carry;   // windows: [N, H, 128, 128]
  int win, max_chunks, stride;
  int64_t slots;
  // the rebuild's runs: rebuild_span chunks each (a multiple of the stride,
  // dividing the window), rebuild_units of them in one pass
  int rebuild_span;
  int64_t rebuild_units;
};
hipError_t launch_gdn_bwd(const BwdArgs &a, hipStream_t st, const BwdPlan *plan = nullptr);
// per-chunk backward kernel for bf16 io at d = 128 (gdn_bwd_chunk.hip)
hipError_t launch_bwd_chunk_d128(const BwdArgs &a, hipStream_t st, int64_t slots);
// the chunk solves T, T~ into a.tri for bf16 io at d = 128 (gdn_tri.hip)
hipError_t launch_tri_d128(const BwdArgs &a, hipStream_t st, int64_t slots);
// the state-independent part of the reverse scan's chunk step into a.pack
// (gdn_bwd_pre.hip)
hipError_t launch_bwd_pre_d128(const BwdArgs &a, hipStream_t st, int64_t slots);

}  // namespace flare
