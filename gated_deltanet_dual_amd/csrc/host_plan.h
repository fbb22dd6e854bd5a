// host_plan.h -- host-side validation and launch planning for the flare_gdn
// C ABI.  Pure C++ (no HIP types) so it is unit-testable on a machine without a
// GPU; the HIP entry points call these before enqueuing anything.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/flare_gdn.h"

namespace flare {

constexpr int kChunk = 32;          // tokens per chunk of the chunk-parallel scan
constexpr int kConvBwdRun = 256;  // tokens per row of the ShortConv reverse-mode partials
constexpr int kVersion = 100;       // 0.1.0
// fp32 words per (chunk slot, head) of the backward's hand-over from its
// state-independent pre-pass to its reverse scan (bf16 io, d = 128): the
// 128 x 128 right-hand side, the 32 x 32 chain matrix as hi / lo bf16
// fragments, the chunk's k rows as two sets of bf16 fragments, the chunk decay
constexpr int kScanPackFloats = 16384 + 1024 + 2048 + 2048 + 64;

// Records a message for flare_last_error() and returns the status.
flare_status fail(flare_status st, const char *fmt, ...);
void clear_error();
const char *last_error();

// Summary of a validated packed batch.
struct VarlenInfo {
  int32_t num_docs = 0;
  int64_t total_tokens = 0;
  int32_t max_len = 0;
  int64_t total_chunks = 0;  // sum over documents of ceil(n_i / kChunk)
  int32_t uniform_len = -1;  // the documents' common length, or -1 when they differ (or there are none)
};

// Checks a flare_varlen: non-NULL host and device arrays (device arrays may be
// NULL only when num_docs == 0 and nothing is launched), cu[0] == 0,
// non-decreasing, 0 <= P_i <= n_i and P_i % block_size == 0.
flare_status check_varlen(const flare_varlen *v, int32_t block_size, VarlenInfo *out);

// Checks a flare_gdn_shape for the GDN entry points: heads > 0, d_k == d_v in
// {16, 128}, block_size in {1,2,4,8,16,32} (divides kChunk), io dtype, flags.
flare_status check_gdn_shape(const flare_gdn_shape *s);

float resolve_scale(const flare_gdn_shape *s);

int64_t ckpt_slot(int32_t cu_i, int32_t doc, int32_t chunk, int32_t stride);
int64_t ckpt_num_slots(const VarlenInfo &vi, int32_t stride);

// Bytes of bwd workspace: per chunk slot and head, the end-state adjoint and
// six chunk matrices (checkpoint slot layout), and for bf16 io at d = 128 the
// scan hand-over (kScanPackFloats).
size_t bwd_workspace_bytes(const VarlenInfo &vi, const flare_gdn_shape *s);
bool bwd_uses_scan_pack(const flare_gdn_shape *s);
// Byte offsets of the q/k L2 factors (float4 per token and head) in the
// backward's and the forward's workspace, when the flag is set.
size_t bwd_l2_offset(const VarlenInfo &vi, const flare_gdn_shape *s);
size_t fwd_l2_offset(const VarlenInfo &vi, const flare_gdn_shape *s);
// The state scans of the chunked path (bf16 io, d = 128) run each document's
// chunks as one chain per head unless too few chains fill the chip: then each
// document is cut into runs of scan_seg_span() chunks, scanned in parallel
// and joined by their affine transfer maps (0: no runs).  The run buffers sit
// at these offsets of the forward's / backward's workspace.
constexpr int kScanWorkgroupTarget = 256;  // workgroups that fill the chip (one per CU)
constexpr int kScanMinRun = 32;            // shortest run worth its transfer map
int scan_seg_span(const VarlenInfo &vi, int32_t heads);
size_t fwd_seg_offset(const VarlenInfo &vi, const flare_gdn_shape *s);
size_t bwd_seg_offset(const VarlenInfo &vi, const flare_gdn_shape *s);

// Byte layout of the chunked path's workspace (bf16 io, d = 128), as offsets
// into the caller's buffer; a region of size 0 is absent.  One pass (win = 0)
// keeps every chunk's buffers at its checkpoint slot of stride 1; chunk
// windows (win > 0) keep only one window of chunks of every document, at slot
// doc * win + (c - window start), and carry the state (or its adjoint) from
// window to window in `carry`.
struct ChunkLayout {
  int win = 0;
  int64_t slots = 0;                     // per-chunk slots of one pass
  size_t adj = 0, adj_bytes = 0;         // bwd: end-state adjoints [slots][H][D][D]
  size_t cmat = 0, cmat_bytes = 0;       // six chunk matrices [slots][H][6][32][32], each tile-major (chunk_common.h)
  size_t pack = 0, pack_bytes = 0;       // scan hand-over [slots][H][kScanPackFloats]
  size_t states = 0, states_bytes = 0;   // chunk-start states [slots][H][D][D]
  size_t l2f = 0, l2f_bytes = 0;         // q/k L2 factors [T][H][4]
  size_t seg = 0, seg_bytes = 0;         // one pass: the scan's run buffers
  size_t carry = 0, carry_bytes = 0;     // windows: the carried chain [N][H][D][D]
  size_t total = 0;
};
// The forward's layout (fwd_uses_chunk_matrices only): chunk matrices,
// hand-over, chunk-start states (used unless stride-1 checkpoints are
// written), L2 factors, then the run buffers or the carry.
ChunkLayout fwd_layout(const VarlenInfo &vi, const flare_gdn_shape *s, int win);
// The backward's layout: adjoints, chunk matrices, and on the chunked path
// the hand-over, the rebuilt chunk-start states (checkpoint stride > 1),
// L2 factors, then the run buffers or the carry.  Windows need the chunked
// path and a multiple of the stride.
ChunkLayout bwd_layout(const VarlenInfo &vi, const flare_gdn_shape *s, int win, int stride);
// Chunks of the longest document.
int max_chunks(const VarlenInfo &vi);
// Chunks per run when the backward rebuilds the chunk-start states from
// checkpoints of stride `stride`: the largest multiple of the stride of at
// most kRebuildRun chunks (the stride itself when larger) that divides the
// window (win > 0).  Short runs leave the scan waiting on its loads; runs of
// a few dozen chunks reach the throughput of whole chains.
constexpr int kRebuildRun = 32;
int rebuild_span(int stride, int win);
// The window an entry point runs at with a workspace of `bytes`: 0 (one pass)
// when the one-pass layout fits, else the largest multiple of `unit` chunks
// whose windowed layout fits, -1 when none does.
int pick_window(const VarlenInfo &vi, const flare_gdn_shape *s, bool bwd, int stride, int unit, size_t bytes);

// Bytes of fwd workspace when the forward runs its chunked passes (bf16 io,
// d = 128; the q/k L2 flag allowed), else 0: per chunk slot and head the six
// chunk matrices, the scan hand-over and a chunk-start state, then the L2
// factors when flagged.
size_t fwd_workspace_bytes(const VarlenInfo &vi, const flare_gdn_shape *s);
bool fwd_uses_chunk_matrices(const flare_gdn_shape *s);

// The chunk-then-refine route: the number of response blocks (from the host
// copies of the document layout) and its workspace, laid out as the forward's
// workspace, the block-boundary states, then the int32 plan arrays.
int64_t route1_num_blocks(const flare_varlen *v, int32_t block_size);
// chunks holding at least one response block start, over all documents
int64_t route1_num_windows(const flare_varlen *v);
size_t route1_workspace_bytes(const VarlenInfo &vi, const flare_gdn_shape *s, int64_t n_blocks);

// Slots distinct and in [0, num_slots) (no check when slot_host is NULL).
flare_status check_slots_host(int32_t n, const int32_t *slot_host, int32_t num_slots);

// Serving step: slots distinct and in range when the host copy is given.
flare_status check_block_step(int32_t num_req, const int32_t *slot_idx,
                              const int32_t *slot_idx_host, const float *pool,
                              int32_t num_slots, const flare_gdn_shape *s,
                              const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, const void *o,
                              int32_t mode);

// Bytes of ShortConv-backward workspace: per section, the per-block partials
// of the weight and bias gradients, ceil(T / 256) blocks x channels x
// (width + 1) fp32.
size_t shortconv_bwd_workspace_bytes(const VarlenInfo &vi, int32_t channels, int32_t width, int32_t sections = 1);

// Channels a lane of the ShortConv kernels holds (8 bytes of a row, 4 bytes
// for widths above 4).
inline int conv_lane_channels(int32_t io_dtype, int32_t width) {
  return (width <= 4 ? 8 : 4) / (io_dtype == FLARE_BF16 ? 2 : 4);
}

// The QKV prologue: each of the three sections is a ShortConv over
// heads * head_dim channels; with qk_l2norm the head rows of q and k are
// normalised inside the kernel, which needs head_dim / conv_lane_channels to
// be a power of two of at most 64 lanes.
flare_status check_qkv_prologue(const flare_varlen *v, int32_t block_size, int32_t heads, int32_t head_dim,
                                int32_t width, int32_t io_dtype, const void *const x[3], const void *const xn[3],
                                const float *const w[3], int32_t activation, int32_t qk_l2norm,
                                const void *const y[3], const void *const yn[3], VarlenInfo *out);

flare_status check_shortconv(const flare_varlen *v, int32_t block_size, int32_t channels,
                             int32_t width, int32_t io_dtype, const void *x, const void *xn,
                             const float *w, int32_t activation, const void *y, const void *yn,
                             VarlenInfo *out);

}  // namespace flare
