// api.hip -- extern "C" entry points of libflare_gdn.so.  Every call validates
// its arguments on the host (host_plan.cpp) before enqueuing anything on the
// caller's stream; the library never allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include "host_plan.h"
#include "kernels.h"
#include "serving.h"

using namespace flare;

static flare_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return FLARE_OK;
  return fail(FLARE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static flare_status check_fwd_common(const flare_varlen *varlen, const flare_gdn_shape *shape,
                                     VarlenInfo *vi) {
  flare_status st = check_gdn_shape(shape);
  if (st != FLARE_OK) return st;
  if (shape->io_dtype == FLARE_F32 && shape->d_k != 16)
    return fail(FLARE_ERR_UNSUPPORTED, "fp32 io is instantiated for d = 16 only");
  return check_varlen(varlen, shape->block_size, vi);
}

extern "C" {

int32_t flare_gdn_chunk_size(void) { return kChunk; }

int32_t flare_version(void) { return kVersion; }

const char *flare_last_error(void) { return last_error(); }

size_t flare_gdn_dual_workspace_size(const flare_varlen *varlen, const flare_gdn_shape *shape,
                                     int for_bwd) {
  VarlenInfo vi;
  if (check_fwd_common(varlen, shape, &vi) != FLARE_OK) return 0;
  return for_bwd ? bwd_workspace_bytes(vi, shape) : fwd_workspace_bytes(vi, shape);
}

size_t flare_gdn_dual_workspace_size_window(const flare_varlen *varlen, const flare_gdn_shape *shape, int for_bwd,
                                            int32_t ckpt_stride_chunks, int32_t window_chunks) {
  VarlenInfo vi;
  if (check_fwd_common(varlen, shape, &vi) != FLARE_OK) return 0;
  if (ckpt_stride_chunks < 1 || window_chunks < 0) return 0;
  if (for_bwd) {
    if (!bwd_uses_scan_pack(shape)) {
      return ckpt_stride_chunks == 1 && window_chunks == 0 ? bwd_workspace_bytes(vi, shape) : 0;
    }
    if (window_chunks % ckpt_stride_chunks != 0) return 0;
    return bwd_layout(vi, shape, window_chunks, ckpt_stride_chunks).total;
  }
  if (!fwd_uses_chunk_matrices(shape)) return 0;
  return fwd_layout(vi, shape, window_chunks).total;
}

size_t flare_gdn_dual_ckpt_size(const flare_varlen *varlen, const flare_gdn_shape *shape,
                                int32_t ckpt_stride_chunks) {
  VarlenInfo vi;
  if (ckpt_stride_chunks < 1) return 0;
  if (check_fwd_common(varlen, shape, &vi) != FLARE_OK) return 0;
  return (size_t)ckpt_num_slots(vi, ckpt_stride_chunks) * shape->num_heads * shape->d_k *
         shape->d_v * sizeof(float);
}

int64_t flare_gdn_ckpt_slot(int32_t cu_seqlens_i, int32_t doc_index, int32_t chunk_index,
                            int32_t ckpt_stride_chunks) {
  if (ckpt_stride_chunks <= 0) return -1;
  return ckpt_slot(cu_seqlens_i, doc_index, chunk_index, ckpt_stride_chunks);
}

// The forward's argument block from the validated call (the workspace and the
// pool slots are set by the caller).
static FwdArgs fwd_args(const flare_varlen *varlen, const flare_gdn_shape *shape, const VarlenInfo &vi,
                        const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                        const void *qn, const void *kn, const void *vn, const float *alpha_n, const float *beta_n,
                        const float *h0, void *o, void *on, float *h_final, float *ckpt, int32_t ckpt_stride) {
  FwdArgs a{};
  a.num_docs = varlen->num_docs;
  a.H = shape->num_heads;
  a.D = shape->d_k;
  a.B = shape->block_size;
  a.flags = shape->flags;
  a.bf16 = shape->io_dtype == FLARE_BF16;
  a.ckpt_stride = ckpt ? ckpt_stride : 1;
  a.scale = resolve_scale(shape);
  a.cu = varlen->cu_seqlens;
  a.plen = varlen->prompt_lens;
  a.q = q; a.k = k; a.v = v; a.qn = qn; a.kn = kn; a.vn = vn;
  a.alpha = alpha; a.beta = beta; a.alpha_n = alpha_n; a.beta_n = beta_n;
  a.h0 = h0; a.o = o; a.on = on; a.h_final = h_final; a.ckpt = ckpt;
  a.T = vi.total_tokens;
  return a;
}

// The ShortConv the forward forms its q, k, v rows with (flare_gdn_dual_fwd_conv).
struct ConvSpec {
  int width, activation;
  const void *const *x, *const *xn;
  const float *const *w;
};

static flare_status fwd_impl(const flare_varlen *varlen, const flare_gdn_shape *shape, const void *q, const void *k,
                             const void *v, const float *alpha, const float *beta, const void *qn, const void *kn,
                             const void *vn, const float *alpha_n, const float *beta_n, const float *h0, void *o,
                             void *on, float *h_final, const int32_t *state_slot, float *ckpt,
                             int32_t ckpt_stride_chunks, void *workspace, size_t workspace_bytes, void *stream,
                             const ConvSpec *conv = nullptr) {
  VarlenInfo vi;
  flare_status st = check_fwd_common(varlen, shape, &vi);
  if (st != FLARE_OK) return st;
  if (ckpt && ckpt_stride_chunks < 1)
    return fail(FLARE_ERR_SHAPE, "checkpoint stride %d (at least 1)", ckpt_stride_chunks);
  if (conv) {
    if (!fwd_uses_chunk_matrices(shape))
      return fail(FLARE_ERR_UNSUPPORTED, "gdn_dual_fwd_conv: bf16 io at d = 128 only");
    if (conv->width < 1 || conv->width > 4)
      return fail(FLARE_ERR_UNSUPPORTED, "gdn_dual_fwd_conv: width %d not in [1, 4]", conv->width);
    if (conv->activation != 0 && conv->activation != 1)
      return fail(FLARE_ERR_UNSUPPORTED, "activation %d unknown", conv->activation);
    if (vi.total_tokens > 0) {
      if (!conv->x || !conv->xn || !conv->w) return fail(FLARE_ERR_NULL, "gdn_dual_fwd_conv: a pointer array is NULL");
      for (int i = 0; i < 3; ++i)
        if (!conv->x[i] || !conv->xn[i] || !conv->w[i])
          return fail(FLARE_ERR_NULL, "gdn_dual_fwd_conv: projection or weight %d is NULL", i);
      if (!alpha || !beta || !alpha_n || !beta_n || !o || !on)
        return fail(FLARE_ERR_NULL, "gdn_dual_fwd_conv: a required pointer is NULL");
    }
  } else if (vi.total_tokens > 0 &&
             (!q || !k || !v || !alpha || !beta || !qn || !kn || !vn || !alpha_n || !beta_n || !o || !on)) {
    return fail(FLARE_ERR_NULL, "gdn_dual_fwd: a required pointer is NULL");
  }
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(FLARE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  FwdArgs a = fwd_args(varlen, shape, vi, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0, o, on, h_final,
                       ckpt, ckpt_stride_chunks);
  a.state_slot = state_slot;
  if (conv && vi.total_tokens > 0) {
    for (int i = 0; i < 3; ++i) {
      a.cx[i] = conv->x[i];
      a.cxn[i] = conv->xn[i];
      a.cwt[i] = conv->w[i];
    }
    a.cw = conv->width;
    a.cact = conv->activation;
  }
  if (!fwd_uses_chunk_matrices(shape)) {  // the per-(document, head) kernel
    a.workspace = nullptr;
    return hip_status(launch_gdn_fwd(a, (hipStream_t)stream), "gdn_dual_fwd launch");
  }
  // the chunked passes (also for a batch of empty documents: h_final = h0
  // through the scan): in one pass when the workspace holds every chunk's
  // buffers, else in windows of as many chunks as it holds
  const int win = workspace ? pick_window(vi, shape, false, 1, 1, workspace_bytes) : -1;
  if (win < 0)
    return fail(FLARE_ERR_WORKSPACE, "workspace of %zu bytes: %zu needed (%zu for windows of one chunk)",
                workspace_bytes, fwd_layout(vi, shape, 0).total, fwd_layout(vi, shape, 1).total);
  if (win > 0 && state_slot)
    return fail(FLARE_ERR_WORKSPACE, "the pool forward runs in one pass: workspace of %zu bytes, %zu needed",
                workspace_bytes, fwd_layout(vi, shape, 0).total);
  const ChunkLayout L = fwd_layout(vi, shape, win);
  char *const w = reinterpret_cast<char *>(workspace);
  a.workspace = reinterpret_cast<float *>(workspace);
  if (win == 0 && vi.uniform_len > 0 && vi.uniform_len % kChunk == 0 && vi.num_docs > 1)
    a.slot_order = vi.uniform_len / kChunk + 1;
  FwdPlan p{};
  p.win = win;
  p.max_chunks = max_chunks(vi);
  p.slots = L.slots;
  p.cmat = reinterpret_cast<float *>(w + L.cmat);
  p.pack = reinterpret_cast<float *>(w + L.pack);
  // one pass with stride-1 checkpoints: the checkpoints are the states
  p.states = (win == 0 && ckpt && ckpt_stride_chunks == 1) ? nullptr : reinterpret_cast<float *>(w + L.states);
  p.l2f = reinterpret_cast<float4 *>(w + L.l2f);
  p.carry = win > 0 ? reinterpret_cast<float *>(w + L.carry) : nullptr;
  if (win == 0) {  // the state scan in parallel runs for long documents
    a.scan_span = scan_seg_span(vi, shape->num_heads);
    a.scan_units = a.scan_span > 0 ? ckpt_num_slots(vi, a.scan_span) : 0;
    a.scan_ws = reinterpret_cast<float *>(w + L.seg);
  }
  return hip_status(launch_gdn_fwd(a, (hipStream_t)stream, &p), "gdn_dual_fwd launch");
}

flare_status flare_gdn_dual_fwd(const flare_varlen *varlen, const flare_gdn_shape *shape,
                                const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, const void *qn, const void *kn, const void *vn,
                                const float *alpha_n, const float *beta_n, const float *h0,
                                void *o, void *on, float *h_final, float *ckpt,
                                int32_t ckpt_stride_chunks, void *workspace, size_t workspace_bytes,
                                void *stream) {
  clear_error();
  return fwd_impl(varlen, shape, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0, o, on, h_final, nullptr,
                  ckpt, ckpt_stride_chunks, workspace, workspace_bytes, stream);
}

flare_status flare_gdn_dual_fwd_conv(const flare_varlen *varlen, const flare_gdn_shape *shape, int32_t width,
                                     const float *const weight[3], int32_t activation, const void *const x[3],
                                     const void *const xn[3], const float *alpha, const float *beta,
                                     const float *alpha_n, const float *beta_n, const float *h0, void *o, void *on,
                                     float *h_final, float *ckpt, int32_t ckpt_stride_chunks, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  clear_error();
  const ConvSpec cs{width, activation, x, xn, weight};
  return fwd_impl(varlen, shape, nullptr, nullptr, nullptr, alpha, beta, nullptr, nullptr, nullptr, alpha_n, beta_n,
                  h0, o, on, h_final, nullptr, ckpt, ckpt_stride_chunks, workspace, workspace_bytes, stream, &cs);
}

size_t flare_gdn_route1_workspace_size(const flare_varlen *varlen, const flare_gdn_shape *shape) {
  VarlenInfo vi;
  if (check_fwd_common(varlen, shape, &vi) != FLARE_OK) return 0;
  if (shape->d_k != shape->d_v || (shape->d_k != 16 && shape->d_k != 128) || shape->flags != 0) return 0;
  return route1_workspace_bytes(vi, shape, route1_num_blocks(varlen, shape->block_size));
}

flare_status flare_gdn_dual_fwd_route1(const flare_varlen *varlen, const flare_gdn_shape *shape, const void *q,
                                       const void *k, const void *v, const float *alpha, const float *beta,
                                       const void *qn, const void *kn, const void *vn, const float *alpha_n,
                                       const float *beta_n, const float *h0, void *o, void *on, float *h_final,
                                       float *ckpt, void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_fwd_common(varlen, shape, &vi);
  if (st != FLARE_OK) return st;
  if (shape->flags != 0) return fail(FLARE_ERR_UNSUPPORTED, "route1: no flags (normalise q, k beforehand)");
  if (shape->d_k != shape->d_v || (shape->d_k != 16 && shape->d_k != 128))
    return fail(FLARE_ERR_UNSUPPORTED, "route1: d_k = d_v in {16, 128}");
  if (vi.total_tokens > 0 &&
      (!q || !k || !v || !alpha || !beta || !qn || !kn || !vn || !alpha_n || !beta_n || !o || !on || !ckpt))
    return fail(FLARE_ERR_NULL, "gdn_dual_fwd_route1: a required pointer is NULL (the chunk-start states too)");
  const int64_t nblk = route1_num_blocks(varlen, shape->block_size);
  const size_t need = route1_workspace_bytes(vi, shape, nblk);
  if (vi.total_tokens > 0 && (!workspace || workspace_bytes < need))
    return fail(FLARE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(FLARE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  FwdArgs a = fwd_args(varlen, shape, vi, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0, o, on, h_final,
                       ckpt, 1);
  if (vi.total_tokens == 0) {
    // only empty documents: no block, no window; the forward writes h_final
    a.workspace = nullptr;
    return hip_status(launch_gdn_fwd(a, (hipStream_t)stream), "gdn_dual_fwd_route1 launch");
  }
  // workspace: the forward's, the boundary states, the plan arrays
  char *w = reinterpret_cast<char *>(workspace);
  const size_t fwd = fwd_workspace_bytes(vi, shape);
  a.workspace = fwd > 0 ? reinterpret_cast<float *>(w) : nullptr;
  w += (fwd + 255) & ~(size_t)255;
  Route1Plan pl{};
  pl.n_blocks = nblk;
  pl.n_windows = route1_num_windows(varlen);  // at most one per block
  pl.bstates = reinterpret_cast<float *>(w);
  w += ((size_t)nblk * a.H * a.D * a.D * 4 + 255) & ~(size_t)255;
  int32_t *ip = reinterpret_cast<int32_t *>(w);
  pl.boff = ip; ip += a.num_docs;
  pl.woff = ip; ip += a.num_docs;
  pl.plen_all = ip; ip += a.num_docs;
  pl.wrow = ip; ip += nblk;
  pl.wcnt = ip; ip += nblk;
  pl.wslot = ip; ip += nblk;
  pl.wlo = ip; ip += nblk;
  pl.wg0 = ip; ip += nblk;
  pl.r0r = ip; ip += nblk;
  pl.cr = ip;
  return hip_status(launch_route1(a, pl, (hipStream_t)stream), "gdn_dual_fwd_route1 launch");
}

flare_status flare_gdn_dual_fwd_pool(const flare_varlen *varlen, const flare_gdn_shape *shape, const void *q,
                                     const void *k, const void *v, const float *alpha, const float *beta,
                                     const void *qn, const void *kn, const void *vn, const float *alpha_n,
                                     const float *beta_n, const int32_t *doc_slot, const int32_t *doc_slot_host,
                                     float *state_pool, int32_t num_slots, int32_t read_initial, void *o, void *on,
                                     float *ckpt, int32_t ckpt_stride_chunks, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  clear_error();
  if (!varlen) return fail(FLARE_ERR_NULL, "varlen is NULL");
  if (read_initial != 0 && read_initial != 1) return fail(FLARE_ERR_SHAPE, "read_initial %d is not 0 or 1", read_initial);
  if (varlen->num_docs > 0) {
    if (!doc_slot || !state_pool) return fail(FLARE_ERR_NULL, "gdn_dual_fwd_pool: doc_slot or state_pool is NULL");
    if (varlen->num_docs > num_slots)
      return fail(FLARE_ERR_SHAPE, "%d documents > %d pool slots", varlen->num_docs, num_slots);
    const flare_status st = check_slots_host(varlen->num_docs, doc_slot_host, num_slots);
    if (st != FLARE_OK) return st;
  }
  return fwd_impl(varlen, shape, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n,
                  read_initial ? state_pool : nullptr, o, on, state_pool, doc_slot, ckpt, ckpt_stride_chunks,
                  workspace, workspace_bytes, stream);
}

flare_status flare_gdn_dual_bwd(const flare_varlen *varlen, const flare_gdn_shape *shape,
                                const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, const void *qn, const void *kn, const void *vn,
                                const float *alpha_n, const float *beta_n, const float *h0,
                                const float *ckpt, int32_t ckpt_stride_chunks, const void *fwd_workspace,
                                const void *d_o,
                                const void *d_on, const float *dh_final, void *dq, void *dk,
                                void *dv, float *dalpha, float *dbeta, void *dqn, void *dkn,
                                void *dvn, float *dalpha_n, float *dbeta_n, float *dh0,
                                void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_fwd_common(varlen, shape, &vi);
  if (st != FLARE_OK) return st;
  if (ckpt_stride_chunks < 1)
    return fail(FLARE_ERR_SHAPE, "checkpoint stride %d (at least 1)", ckpt_stride_chunks);
  if (ckpt_stride_chunks > 1 && !bwd_uses_scan_pack(shape))
    return fail(FLARE_ERR_UNSUPPORTED, "checkpoint stride %d: the rebuild is built for bf16 io at d = 128",
                ckpt_stride_chunks);
  if ((shape->flags & FLARE_QK_L2NORM) && !bwd_uses_scan_pack(shape))
    return fail(FLARE_ERR_UNSUPPORTED,
                "the backward takes the q/k L2 flag for bf16 io at d = 128 only (normalise q, k beforehand)");
  if (vi.total_tokens > 0 &&
      (!q || !k || !v || !alpha || !beta || !qn || !kn || !vn || !alpha_n || !beta_n || !ckpt ||
       !d_o || !d_on || !dq || !dk || !dv || !dalpha || !dbeta || !dqn || !dkn || !dvn ||
       !dalpha_n || !dbeta_n))
    return fail(FLARE_ERR_NULL, "gdn_dual_bwd: a required pointer is NULL");
  const bool chunked = bwd_uses_scan_pack(shape);
  // the chunked path runs in one pass when the workspace holds every chunk's
  // buffers, else in windows of a multiple of the stride
  int win = 0;
  if (vi.total_tokens > 0 || chunked) {  // the chunked path scans empty documents too (dh0 = dh_final)
    win = workspace ? (chunked ? pick_window(vi, shape, true, ckpt_stride_chunks, ckpt_stride_chunks, workspace_bytes)
                               : (workspace_bytes >= bwd_workspace_bytes(vi, shape) ? 0 : -1))
                    : -1;
    if (win < 0)
      return fail(FLARE_ERR_WORKSPACE, "workspace of %zu bytes: %zu needed (%zu for windows of %d chunks)",
                  workspace_bytes, chunked ? bwd_layout(vi, shape, 0, ckpt_stride_chunks).total
                                           : bwd_workspace_bytes(vi, shape),
                  chunked ? bwd_layout(vi, shape, ckpt_stride_chunks, ckpt_stride_chunks).total
                          : bwd_workspace_bytes(vi, shape),
                  ckpt_stride_chunks);
  }
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(FLARE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  BwdArgs a{};
  a.f.num_docs = varlen->num_docs;
  a.f.H = shape->num_heads;
  a.f.D = shape->d_k;
  a.f.B = shape->block_size;
  a.f.flags = shape->flags;
  a.f.bf16 = shape->io_dtype == FLARE_BF16;
  a.f.ckpt_stride = ckpt_stride_chunks;
  a.f.scale = resolve_scale(shape);
  a.f.cu = varlen->cu_seqlens;
  a.f.plen = varlen->prompt_lens;
  a.f.q = q; a.f.k = k; a.f.v = v; a.f.qn = qn; a.f.kn = kn; a.f.vn = vn;
  a.f.alpha = alpha; a.f.beta = beta; a.f.alpha_n = alpha_n; a.f.beta_n = beta_n;
  a.f.h0 = h0;
  a.f.T = vi.total_tokens;
  a.ckpt_in = ckpt;
  // the forward's chunk matrices, when its workspace held them
  a.fwd_cm = (fwd_workspace && fwd_workspace_bytes(vi, shape) > 0) ? reinterpret_cast<const float *>(fwd_workspace)
                                                                      : nullptr;
  // and its scan hand-over, whose K fragment sets the reverse scan reuses
  a.fwd_pack = a.fwd_cm ? reinterpret_cast<const float *>(reinterpret_cast<const char *>(fwd_workspace) +
                                                          fwd_layout(vi, shape, 0).pack)
                        : nullptr;
  a.d_o = d_o; a.d_on = d_on; a.dh_final = dh_final;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dqn = dqn; a.dkn = dkn; a.dvn = dvn;
  a.dalpha = dalpha; a.dbeta = dbeta; a.dalpha_n = dalpha_n; a.dbeta_n = dbeta_n; a.dh0 = dh0;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.T = vi.total_tokens;
  if (!chunked) return hip_status(launch_gdn_bwd(a, (hipStream_t)stream), "gdn_dual_bwd launch");
  const ChunkLayout L = bwd_layout(vi, shape, win, ckpt_stride_chunks);
  char *const w = reinterpret_cast<char *>(workspace);
  BwdPlan p{};
  p.win = win;
  p.max_chunks = max_chunks(vi);
  p.stride = ckpt_stride_chunks;
  p.slots = L.slots;
  p.rebuild_span = rebuild_span(ckpt_stride_chunks, win);
  p.rebuild_units = ckpt_num_slots(vi, p.rebuild_span);
  p.adj = reinterpret_cast<float *>(w + L.adj);
  p.tri = reinterpret_cast<float *>(w + L.cmat);
  p.pack = reinterpret_cast<float *>(w + L.pack);
  p.states = L.states_bytes ? reinterpret_cast<float *>(w + L.states) : nullptr;
  p.l2f = reinterpret_cast<float4 *>(w + L.l2f);
  p.carry = win > 0 ? reinterpret_cast<float *>(w + L.carry) : nullptr;
  if (win == 0) {  // the reverse scan in parallel runs for long documents
    a.f.scan_span = scan_seg_span(vi, shape->num_heads);
    a.f.scan_units = a.f.scan_span > 0 ? ckpt_num_slots(vi, a.f.scan_span) : 0;
    a.f.scan_ws = reinterpret_cast<float *>(w + L.seg);
    // the forward's runs' transfer maps, at the start of its run buffers
    if (a.fwd_cm && a.f.scan_span > 0)
      a.fwd_maps = reinterpret_cast<const float *>(reinterpret_cast<const char *>(fwd_workspace) +
                                                   fwd_seg_offset(vi, shape));
  }
  return hip_status(launch_gdn_bwd(a, (hipStream_t)stream, &p), "gdn_dual_bwd launch");
}

// The serving step's argument block for num_req requests of shape's blocks.
static BlockStepArgs step_args(int32_t num_req, const flare_gdn_shape *shape, int32_t mode,
                               const int32_t *slot_idx, const float *pool, const void *q, const void *k,
                               const void *v, const float *alpha, const float *beta, void *o) {
  BlockStepArgs a{};
  a.num_req = num_req;
  a.H = shape->num_heads;
  a.D = shape->d_k;
  a.B = shape->block_size;
  a.mode = mode;
  a.bf16 = shape->io_dtype == FLARE_BF16;
  a.scale = resolve_scale(shape);
  a.slot_idx = slot_idx;
  a.pool = const_cast<float *>(pool);  // written only by the modes that commit
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.o = o;
  return a;
}

flare_status flare_gdn_block_step(int32_t num_req, const int32_t *slot_idx,
                                  const int32_t *slot_idx_host, float *state_pool,
                                  int32_t num_slots, const flare_gdn_shape *shape, const void *q,
                                  const void *k, const void *v, const float *alpha,
                                  const float *beta, void *o, int32_t mode, void *stream) {
  clear_error();
  flare_status st = check_block_step(num_req, slot_idx, slot_idx_host, state_pool, num_slots, shape,
                                     q, k, v, alpha, beta, o, mode);
  if (st != FLARE_OK) return st;
  BlockStepArgs a = step_args(num_req, shape, mode, slot_idx, state_pool, q, k, v, alpha, beta, o);
  return hip_status(launch_block_step(a, (hipStream_t)stream), "gdn_block_step launch");
}

flare_status flare_gdn_block_step_conv(int32_t num_req, const int32_t *slot_idx, const int32_t *slot_idx_host,
                                       float *state_pool, void *conv_cache, int32_t num_slots,
                                       const flare_gdn_shape *shape, int32_t width, const float *const weight[3],
                                       int32_t activation, int32_t qk_l2norm, const void *xq, const void *xk,
                                       const void *xv, const float *alpha, const float *beta, void *o, int32_t mode,
                                       void *stream) {
  clear_error();
  flare_status st = check_block_step(num_req, slot_idx, slot_idx_host, state_pool, num_slots, shape, xq, xk, xv,
                                     alpha, beta, o, mode);
  if (st != FLARE_OK) return st;
  if (shape->flags != 0) return fail(FLARE_ERR_UNSUPPORTED, "block_step_conv: the L2 step is its own argument");
  if (width < 1 || width > 8) return fail(FLARE_ERR_UNSUPPORTED, "width %d not in [1, 8]", width);
  if (shape->block_size > 8)
    return fail(FLARE_ERR_UNSUPPORTED, "block_step_conv is built for blocks of up to 8 tokens (got %d)",
                shape->block_size);
  if (activation != 0 && activation != 1) return fail(FLARE_ERR_UNSUPPORTED, "activation %d unknown", activation);
  if (qk_l2norm != 0 && qk_l2norm != 1) return fail(FLARE_ERR_UNSUPPORTED, "qk_l2norm %d unknown", qk_l2norm);
  if (num_req > 0) {
    if (!weight || !weight[0] || !weight[1] || !weight[2])
      return fail(FLARE_ERR_NULL, "block_step_conv: a weight pointer is NULL");
    if (width > 1 && !conv_cache) return fail(FLARE_ERR_NULL, "block_step_conv: conv_cache is NULL");
  }
  BlockStepArgs a = step_args(num_req, shape, mode, slot_idx, state_pool, xq, xk, xv, alpha, beta, o);
  a.conv = 1;
  a.W = width;
  a.act = activation;
  a.l2 = qk_l2norm;
  a.cache = conv_cache;
  for (int s = 0; s < 3; ++s) a.cw[s] = num_req > 0 ? weight[s] : nullptr;
  return hip_status(launch_block_step(a, (hipStream_t)stream), "gdn_block_step_conv launch");
}

flare_status flare_conv_cache_fill(const flare_varlen *varlen, int32_t heads, int32_t head_dim, int32_t width,
                                   int32_t io_dtype, const void *const x[3], const int32_t *doc_slot,
                                   const int32_t *doc_slot_host, void *conv_cache, int32_t num_slots,
                                   void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_varlen(varlen, 1, &vi);
  if (st != FLARE_OK) return st;
  if (heads <= 0 || head_dim <= 0 || (int64_t)heads * head_dim > INT32_MAX)
    return fail(FLARE_ERR_SHAPE, "heads and head_dim must be positive");
  if (width < 1 || width > 8) return fail(FLARE_ERR_UNSUPPORTED, "width %d not in [1, 8]", width);
  if (io_dtype != FLARE_F32 && io_dtype != FLARE_BF16) return fail(FLARE_ERR_UNSUPPORTED, "io_dtype %d unknown", io_dtype);
  const int C = heads * head_dim;
  if (C % (io_dtype == FLARE_BF16 ? 8 : 4) != 0)
    return fail(FLARE_ERR_ALIGN, "heads * head_dim = %d must be a multiple of 16 bytes", C);
  const int N = varlen->num_docs;
  if (N == 0 || width == 1) return FLARE_OK;
  if (N > num_slots) return fail(FLARE_ERR_SHAPE, "%d documents > %d slots", N, num_slots);
  if (!x || !x[0] || !x[1] || !x[2] || !doc_slot || !conv_cache)
    return fail(FLARE_ERR_NULL, "conv_cache_fill: a required pointer is NULL");
  st = check_slots_host(N, doc_slot_host, num_slots);
  if (st != FLARE_OK) return st;
  ConvCacheArgs a{};
  a.num_docs = N;
  a.C = C;
  a.W = width;
  a.bf16 = io_dtype == FLARE_BF16;
  a.cu = varlen->cu_seqlens;
  a.slot = doc_slot;
  for (int s = 0; s < 3; ++s) a.x[s] = x[s];
  a.cache = conv_cache;
  return hip_status(launch_conv_cache_fill(a, (hipStream_t)stream), "conv_cache_fill launch");
}

flare_status flare_gdn_verify(int32_t num_req, const int32_t *slot_idx, const int32_t *slot_idx_host,
                              const float *state_pool, int32_t num_slots, const flare_gdn_shape *shape,
                              const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                              void *o, float *cand, void *stream) {
  clear_error();
  // the same inputs as a COMMIT of the K = block_size drafted tokens
  flare_status st = check_block_step(num_req, slot_idx, slot_idx_host, state_pool, num_slots, shape, q, k, v,
                                     alpha, beta, o, FLARE_BLOCK_COMMIT);
  if (st != FLARE_OK) return st;
  if (num_req > 0 && (!o || !cand)) return fail(FLARE_ERR_NULL, "verify needs the outputs and the candidate buffer");
  BlockStepArgs a = step_args(num_req, shape, 2, slot_idx, state_pool, q, k, v, alpha, beta, o);
  a.cand = cand;
  return hip_status(launch_block_step(a, (hipStream_t)stream), "gdn_verify launch");
}

flare_status flare_gdn_scatter(int32_t num_req, const int32_t *slot_idx, const int32_t *slot_idx_host,
                               const int32_t *accepted, const float *cand, float *state_pool, int32_t num_slots,
                               const flare_gdn_shape *shape, void *stream) {
  clear_error();
  flare_status st = check_gdn_shape(shape);
  if (st != FLARE_OK) return st;
  if (num_req < 0 || num_slots < 0) return fail(FLARE_ERR_SHAPE, "negative count");
  if (num_req == 0) return FLARE_OK;
  if (num_req > num_slots) return fail(FLARE_ERR_SHAPE, "num_req %d > num_slots %d", num_req, num_slots);
  if (!slot_idx || !accepted || !cand || !state_pool) return fail(FLARE_ERR_NULL, "scatter: a required pointer is NULL");
  st = check_slots_host(num_req, slot_idx_host, num_slots);
  if (st != FLARE_OK) return st;
  ScatterArgs a{};
  a.num_req = num_req;
  a.H = shape->num_heads;
  a.D = shape->d_k;
  a.K = shape->block_size;
  a.slot_idx = slot_idx;
  a.accepted = accepted;
  a.cand = cand;
  a.pool = state_pool;
  return hip_status(launch_gdn_scatter(a, (hipStream_t)stream), "gdn_scatter launch");
}

flare_status flare_gdn_verify_outputs(int32_t num_req, const int32_t *slot_idx, const int32_t *slot_idx_host,
                                      const float *state_pool, int32_t num_slots, const flare_gdn_shape *shape,
                                      const void *q, const void *k, const void *v, const float *alpha,
                                      const float *beta, void *o, void *stream) {
  clear_error();
  flare_status st = check_block_step(num_req, slot_idx, slot_idx_host, state_pool, num_slots, shape, q, k, v,
                                     alpha, beta, o, FLARE_BLOCK_EVAL);
  if (st != FLARE_OK) return st;
  BlockStepArgs a = step_args(num_req, shape, 0, slot_idx, state_pool, q, k, v, alpha, beta, o);
  a.causal = 1;
  return hip_status(launch_block_step(a, (hipStream_t)stream), "gdn_verify_outputs launch");
}

flare_status flare_gdn_commit_prefix(int32_t num_req, const int32_t *slot_idx, const int32_t *slot_idx_host,
                                     float *state_pool, int32_t num_slots, const flare_gdn_shape *shape,
                                     const void *q, const void *k, const void *v, const float *alpha,
                                     const float *beta, const int32_t *accepted, void *o, void *stream) {
  clear_error();
  flare_status st = check_block_step(num_req, slot_idx, slot_idx_host, state_pool, num_slots, shape, q, k, v,
                                     alpha, beta, o, FLARE_BLOCK_COMMIT);
  if (st != FLARE_OK) return st;
  if (num_req > 0 && !accepted) return fail(FLARE_ERR_NULL, "commit_prefix needs the accepted counts");
  BlockStepArgs a = step_args(num_req, shape, 1, slot_idx, state_pool, q, k, v, alpha, beta, o);
  a.count = accepted;  // the first accepted[r] tokens are replayed, the rest are identity
  return hip_status(launch_block_step(a, (hipStream_t)stream), "gdn_commit_prefix launch");
}

flare_status flare_shortconv_dual(const flare_varlen *varlen, int32_t block_size, int32_t channels,
                                  int32_t width, int32_t io_dtype, const void *x, const void *xn,
                                  const float *weight, const float *bias, int32_t activation,
                                  void *y, void *yn, void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_shortconv(varlen, block_size, channels, width, io_dtype, x, xn, weight,
                                    activation, y, yn, &vi);
  if (st != FLARE_OK) return st;
  ShortConvArgs a{};
  a.num_docs = varlen->num_docs;
  a.B = block_size;
  a.C = channels;
  a.W = width;
  a.activation = activation;
  a.bf16 = io_dtype == FLARE_BF16;
  a.nsec = 1;
  a.T = vi.total_tokens;
  a.cu = varlen->cu_seqlens;
  a.plen = varlen->prompt_lens;
  a.x[0] = x; a.xn[0] = xn; a.w[0] = weight; a.bias = bias; a.y[0] = y; a.yn[0] = yn;
  return hip_status(launch_shortconv(a, (hipStream_t)stream), "shortconv_dual launch");
}

size_t flare_shortconv_dual_bwd_workspace_size(const flare_varlen *varlen, int32_t block_size,
                                               int32_t channels, int32_t width) {
  VarlenInfo vi;
  if (check_varlen(varlen, block_size, &vi) != FLARE_OK || channels <= 0 || width < 1 || width > 8) return 0;
  return shortconv_bwd_workspace_bytes(vi, channels, width);
}

flare_status flare_shortconv_dual_bwd(const flare_varlen *varlen, int32_t block_size, int32_t channels,
                                      int32_t width, int32_t io_dtype, const void *x, const void *xn,
                                      const float *weight, const float *bias, int32_t activation,
                                      const void *dy, const void *dyn, void *dx, void *dxn,
                                      float *dweight, float *dbias, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_shortconv(varlen, block_size, channels, width, io_dtype, x, xn, weight,
                                    activation, dx, dxn, &vi);
  if (st != FLARE_OK) return st;
  if (!dweight) return fail(FLARE_ERR_NULL, "shortconv_dual_bwd: dweight is NULL");
  if (vi.total_tokens > 0 && (!dy || !dyn))
    return fail(FLARE_ERR_NULL, "shortconv_dual_bwd: dy or dyn is NULL");
  const size_t need = shortconv_bwd_workspace_bytes(vi, channels, width);
  if (vi.total_tokens > 0 && (!workspace || workspace_bytes < need))
    return fail(FLARE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(FLARE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  ShortConvBwdArgs a{};
  a.num_docs = varlen->num_docs;
  a.B = block_size;
  a.C = channels;
  a.W = width;
  a.activation = activation;
  a.bf16 = io_dtype == FLARE_BF16;
  a.nsec = 1;
  a.T = vi.total_tokens;
  a.cu = varlen->cu_seqlens;
  a.plen = varlen->prompt_lens;
  a.x[0] = x; a.xn[0] = xn; a.dy[0] = dy; a.dyn[0] = dyn; a.w[0] = weight; a.bias = bias;
  a.dx[0] = dx; a.dxn[0] = dxn; a.dw[0] = dweight; a.dbias = dbias;
  a.part = reinterpret_cast<float *>(workspace);
  return hip_status(launch_shortconv_bwd(a, (hipStream_t)stream), "shortconv_dual_bwd launch");
}

flare_status flare_qkv_prologue(const flare_varlen *varlen, int32_t block_size, int32_t heads, int32_t head_dim,
                                int32_t width, int32_t io_dtype, const void *const x[3], const void *const xn[3],
                                const float *const weight[3], int32_t activation, int32_t qk_l2norm,
                                void *const y[3], void *const yn[3], void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_qkv_prologue(varlen, block_size, heads, head_dim, width, io_dtype, x, xn, weight,
                                       activation, qk_l2norm, (const void *const *)y, (const void *const *)yn, &vi);
  if (st != FLARE_OK) return st;
  ShortConvArgs a{};
  a.num_docs = varlen->num_docs;
  a.B = block_size;
  a.C = heads * head_dim;
  a.W = width;
  a.activation = activation;
  a.bf16 = io_dtype == FLARE_BF16;
  a.nsec = 3;
  a.nnorm = qk_l2norm ? 2 : 0;
  a.hd = head_dim;
  a.T = vi.total_tokens;
  a.cu = varlen->cu_seqlens;
  a.plen = varlen->prompt_lens;
  for (int s = 0; s < 3; ++s) {
    a.x[s] = x[s]; a.xn[s] = xn[s]; a.w[s] = weight[s]; a.y[s] = y[s]; a.yn[s] = yn[s];
  }
  return hip_status(launch_shortconv(a, (hipStream_t)stream), "qkv_prologue launch");
}

size_t flare_qkv_prologue_bwd_workspace_size(const flare_varlen *varlen, int32_t block_size, int32_t heads,
                                             int32_t head_dim, int32_t width) {
  VarlenInfo vi;
  if (check_varlen(varlen, block_size, &vi) != FLARE_OK || heads <= 0 || head_dim <= 0 || width < 1 || width > 8 ||
      (int64_t)heads * head_dim > INT32_MAX)
    return 0;
  return shortconv_bwd_workspace_bytes(vi, heads * head_dim, width, 3);
}

flare_status flare_qkv_prologue_bwd(const flare_varlen *varlen, int32_t block_size, int32_t heads, int32_t head_dim,
                                    int32_t width, int32_t io_dtype, const void *const x[3],
                                    const void *const xn[3], const float *const weight[3], int32_t activation,
                                    int32_t qk_l2norm, const void *const dy[3], const void *const dyn[3],
                                    void *const dx[3], void *const dxn[3], float *const dweight[3], void *workspace,
                                    size_t workspace_bytes, void *stream) {
  clear_error();
  VarlenInfo vi;
  flare_status st = check_qkv_prologue(varlen, block_size, heads, head_dim, width, io_dtype, x, xn, weight,
                                       activation, qk_l2norm, (const void *const *)dx, (const void *const *)dxn, &vi);
  if (st != FLARE_OK) return st;
  if (!dy || !dyn || !dweight) return fail(FLARE_ERR_NULL, "qkv_prologue_bwd: a pointer array is NULL");
  for (int s = 0; s < 3; ++s) {
    if (!dweight[s]) return fail(FLARE_ERR_NULL, "qkv_prologue_bwd: dweight[%d] is NULL", s);
    if (vi.total_tokens > 0 && (!dy[s] || !dyn[s]))
      return fail(FLARE_ERR_NULL, "qkv_prologue_bwd: dy[%d] or dyn[%d] is NULL", s, s);
  }
  const int C = heads * head_dim;
  const size_t need = shortconv_bwd_workspace_bytes(vi, C, width, 3);
  if (vi.total_tokens > 0 && (!workspace || workspace_bytes < need))
    return fail(FLARE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(FLARE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  ShortConvBwdArgs a{};
  a.num_docs = varlen->num_docs;
  a.B = block_size;
  a.C = C;
  a.W = width;
  a.activation = activation;
  a.bf16 = io_dtype == FLARE_BF16;
  a.nsec = 3;
  a.nnorm = qk_l2norm ? 2 : 0;
  a.hd = head_dim;
  a.T = vi.total_tokens;
  a.cu = varlen->cu_seqlens;
  a.plen = varlen->prompt_lens;
  for (int s = 0; s < 3; ++s) {
    a.x[s] = x[s]; a.xn[s] = xn[s]; a.dy[s] = dy[s]; a.dyn[s] = dyn[s]; a.w[s] = weight[s];
    a.dx[s] = dx[s]; a.dxn[s] = dxn[s]; a.dw[s] = dweight[s];
  }
  a.part = reinterpret_cast<float *>(workspace);
  return hip_status(launch_shortconv_bwd(a, (hipStream_t)stream), "qkv_prologue_bwd launch");
}

}  // extern "C"
