// host_plan.cpp -- validation of the packed-batch description and shapes before
// any launch (the cu_seqlens guard and block alignment of "FLARE: Diffusion for
// Hybrid Language Model", papernotes.org notes, Key designs item 3), plus the
// checkpoint-slot and workspace arithmetic.
#include "host_plan.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace flare {

namespace {
thread_local char g_msg[512] = "";
}

flare_status fail(flare_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_msg[0] = '\0'; }
const char *last_error() { return g_msg; }

static bool pow2_le32(int32_t b) {
  return b == 1 || b == 2 || b == 4 || b == 8 || b == 16 || b == 32;
}

flare_status check_varlen(const flare_varlen *v, int32_t block_size, VarlenInfo *out) {
  if (!v) return fail(FLARE_ERR_NULL, "varlen is NULL");
  if (v->num_docs < 0) return fail(FLARE_ERR_SHAPE, "num_docs < 0 (%d)", v->num_docs);
  if (!v->cu_seqlens_host || !v->prompt_lens_host)
    return fail(FLARE_ERR_NULL, "cu_seqlens_host / prompt_lens_host must be given");
  if (v->num_docs > 0 && (!v->cu_seqlens || !v->prompt_lens))
    return fail(FLARE_ERR_NULL, "device cu_seqlens / prompt_lens must be given");
  if (block_size <= 0) return fail(FLARE_ERR_SHAPE, "block_size must be positive");
  const int32_t *cu = v->cu_seqlens_host;
  const int32_t *pl = v->prompt_lens_host;
  if (cu[0] != 0) return fail(FLARE_ERR_SHAPE, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  VarlenInfo vi;
  vi.num_docs = v->num_docs;
  for (int32_t i = 0; i < v->num_docs; ++i) {
    const int64_t n = (int64_t)cu[i + 1] - cu[i];
    if (n < 0) return fail(FLARE_ERR_SHAPE, "cu_seqlens decreases at document %d", i);
    if (pl[i] < 0 || pl[i] > n)
      return fail(FLARE_ERR_SHAPE, "prompt_lens[%d] = %d outside [0, %lld]", i, pl[i], (long long)n);
    if (pl[i] % block_size != 0)
      return fail(FLARE_ERR_ALIGN, "prompt_lens[%d] = %d is not a multiple of block_size %d", i,
                  pl[i], block_size);
    if (n > vi.max_len) vi.max_len = (int32_t)n;
    vi.uniform_len = i == 0 ? (int32_t)n : (vi.uniform_len == (int32_t)n ? vi.uniform_len : -1);
    vi.total_chunks += (n + kChunk - 1) / kChunk;
  }
  vi.total_tokens = cu[v->num_docs];
  if (out) *out = vi;
  return FLARE_OK;
}

flare_status check_gdn_shape(const flare_gdn_shape *s) {
  if (!s) return fail(FLARE_ERR_NULL, "shape is NULL");
  if (s->num_heads <= 0) return fail(FLARE_ERR_SHAPE, "num_heads must be positive");
  if (s->d_k != s->d_v)
    return fail(FLARE_ERR_UNSUPPORTED, "d_k (%d) != d_v (%d) is not instantiated", s->d_k, s->d_v);
  if (s->d_k != 16 && s->d_k != 128)
    return fail(FLARE_ERR_UNSUPPORTED, "head dim %d not instantiated (16, 128)", s->d_k);
  if (!pow2_le32(s->block_size))
    return fail(FLARE_ERR_UNSUPPORTED, "block_size %d not in {1,2,4,8,16,32}", s->block_size);
  if (kChunk % s->block_size != 0)
    return fail(FLARE_ERR_ALIGN, "block_size %d does not divide the chunk %d", s->block_size, kChunk);
  if (s->io_dtype != FLARE_F32 && s->io_dtype != FLARE_BF16)
    return fail(FLARE_ERR_UNSUPPORTED, "io_dtype %d unknown", s->io_dtype);
  if (s->flags & ~FLARE_QK_L2NORM) return fail(FLARE_ERR_UNSUPPORTED, "unknown flags 0x%x", s->flags);
  return FLARE_OK;
}

float resolve_scale(const flare_gdn_shape *s) {
  if (s->scale > 0.0f) return s->scale;
  return 1.0f / __builtin_sqrtf((float)s->d_k);
}

int64_t ckpt_slot(int32_t cu_i, int32_t doc, int32_t chunk, int32_t stride) {
  const int64_t span = (int64_t)kChunk * stride;
  return (int64_t)cu_i / span + doc + chunk / stride;
}

int64_t ckpt_num_slots(const VarlenInfo &vi, int32_t stride) {
  const int64_t span = (int64_t)kChunk * stride;
  return vi.total_tokens / span + vi.num_docs;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t l2_factor_bytes(const VarlenInfo &vi, const flare_gdn_shape *s) {
  return (s->flags & FLARE_QK_L2NORM) ? (size_t)vi.total_tokens * s->num_heads * 4 * sizeof(float) : 0;
}

int scan_seg_span(const VarlenInfo &vi, int32_t heads) {
  // one chain per (document, head) and four workgroups per chain: cut the
  // documents into runs when the chains cannot fill the chip, aiming at about
  // twice kScanWorkgroupTarget workgroups, and only for runs of at least
  // kScanMinRun chunks (shorter ones cost more in the transfer maps than the
  // parallel runs save)
  const int64_t chains = (int64_t)vi.num_docs * heads * 4;
  if (chains <= 0 || chains >= kScanWorkgroupTarget) return 0;
  const int64_t runs = (2 * kScanWorkgroupTarget + chains - 1) / chains;
  const int64_t max_chunks = ((int64_t)vi.max_len + kChunk - 1) / kChunk;
  const int64_t span = (max_chunks + runs - 1) / runs;
  return span >= kScanMinRun ? (int)span : 0;
}

static size_t seg_bytes(const VarlenInfo &vi, const flare_gdn_shape *s) {
  const int span = scan_seg_span(vi, s->num_heads);
  if (span == 0) return 0;
  // the runs' transfer maps, offsets and start values
  return 3 * (size_t)ckpt_num_slots(vi, span) * s->num_heads * s->d_k * s->d_v * sizeof(float);
}

size_t bwd_l2_offset(const VarlenInfo &vi, const flare_gdn_shape *s) { return bwd_layout(vi, s, 0, 1).l2f; }

size_t bwd_seg_offset(const VarlenInfo &vi, const flare_gdn_shape *s) { return bwd_layout(vi, s, 0, 1).seg; }

size_t bwd_workspace_bytes(const VarlenInfo &vi, const flare_gdn_shape *s) {
  // per chunk slot and head, fp32, in the checkpoint slot layout (stride 1):
  // the chunk's end-state adjoint (d_k x d_v), written by the reverse scan and
  // read by the per-chunk pass, then six kChunk x kChunk chunk matrices (the
  // triangular inverses T, T~ and four weighted Gram matrices), written by the
  // chunk-matrix pass and read by both; for bf16 io at d = 128 then the
  // pre-pass's hand-over to the reverse scan; with the q/k L2 flag then the
  // per-(token, head) factors {r_q, r_k, r_q~, r_k~}; when the scan runs in
  // parallel runs (long documents, bf16 io at d = 128), the runs' transfer
  // maps, offsets and start values
  return bwd_layout(vi, s, 0, 1).total;
}

bool bwd_uses_scan_pack(const flare_gdn_shape *s) {
  return s->io_dtype == FLARE_BF16 && s->d_k == 128 && s->d_v == 128;
}

bool fwd_uses_chunk_matrices(const flare_gdn_shape *s) {
  return s->io_dtype == FLARE_BF16 && s->d_k == 128 && s->d_v == 128 && (s->flags & ~FLARE_QK_L2NORM) == 0;
}

size_t fwd_l2_offset(const VarlenInfo &vi, const flare_gdn_shape *s) { return fwd_layout(vi, s, 0).l2f; }

size_t fwd_seg_offset(const VarlenInfo &vi, const flare_gdn_shape *s) { return fwd_layout(vi, s, 0).seg; }

size_t fwd_workspace_bytes(const VarlenInfo &vi, const flare_gdn_shape *s) {
  if (!fwd_uses_chunk_matrices(s)) return 0;
  // per chunk slot and head, fp32: the six chunk matrices, the scan hand-over,
  // and room for the chunk-start state when no checkpoints are asked for; with
  // the q/k L2 flag then the per-(token, head) factors {r_q, r_k, r_q~, r_k~};
  // then the scan's run buffers when it runs in parallel runs
  return fwd_layout(vi, s, 0).total;
}

int max_chunks(const VarlenInfo &vi) { return (int)(((int64_t)vi.max_len + kChunk - 1) / kChunk); }

int rebuild_span(int stride, int win) {
  int best = stride;
  for (int span = 2 * stride; span <= kRebuildRun; span += stride)
    if (win == 0 || win % span == 0) best = span;
  return best;
}

ChunkLayout fwd_layout(const VarlenInfo &vi, const flare_gdn_shape *s, int win) {
  ChunkLayout L;
  L.win = win;
  L.slots = win > 0 ? (int64_t)vi.num_docs * win : ckpt_num_slots(vi, 1);
  const size_t per = (size_t)L.slots * s->num_heads;
  const size_t dd = (size_t)s->d_k * s->d_v * sizeof(float);
  L.cmat = 0;
  L.cmat_bytes = per * 6 * kChunk * kChunk * sizeof(float);
  L.pack = L.cmat + L.cmat_bytes;
  L.pack_bytes = per * kScanPackFloats * sizeof(float);
  L.states = L.pack + L.pack_bytes;
  L.states_bytes = per * dd;
  L.l2f = round256(L.states + L.states_bytes);
  L.l2f_bytes = l2_factor_bytes(vi, s);
  const size_t tail = round256(L.l2f + L.l2f_bytes);
  if (win > 0) {
    L.carry = tail;
    L.carry_bytes = (size_t)vi.num_docs * s->num_heads * dd;
    L.total = L.carry + L.carry_bytes + 256;
  } else {
    L.seg = tail;
    L.seg_bytes = seg_bytes(vi, s);
    L.total = L.seg + L.seg_bytes + 256;
  }
  return L;
}

ChunkLayout bwd_layout(const VarlenInfo &vi, const flare_gdn_shape *s, int win, int stride) {
  ChunkLayout L;
  const bool chunked = bwd_uses_scan_pack(s);
  L.win = win;
  L.slots = win > 0 ? (int64_t)vi.num_docs * win : ckpt_num_slots(vi, 1);
  const size_t per = (size_t)L.slots * s->num_heads;
  const size_t dd = (size_t)s->d_k * s->d_v * sizeof(float);
  L.adj = 0;
  L.adj_bytes = per * dd;
  L.cmat = L.adj + L.adj_bytes;
  L.cmat_bytes = per * 6 * kChunk * kChunk * sizeof(float);
  L.pack = L.cmat + L.cmat_bytes;
  L.pack_bytes = chunked ? per * kScanPackFloats * sizeof(float) : 0;
  L.states = L.pack + L.pack_bytes;
  L.states_bytes = chunked && stride > 1 ? per * dd : 0;
  L.l2f = round256(L.states + L.states_bytes);
  L.l2f_bytes = l2_factor_bytes(vi, s);
  const size_t tail = round256(L.l2f + L.l2f_bytes);
  if (win > 0) {
    L.carry = tail;
    L.carry_bytes = (size_t)vi.num_docs * s->num_heads * dd;
    L.total = L.carry + L.carry_bytes + 256;
  } else {
    L.seg = tail;
    L.seg_bytes = chunked ? seg_bytes(vi, s) : 0;
    L.total = L.seg + L.seg_bytes + 256;
  }
  return L;
}

int pick_window(const VarlenInfo &vi, const flare_gdn_shape *s, bool bwd, int stride, int unit, size_t bytes) {
  auto total = [&](int win) { return bwd ? bwd_layout(vi, s, win, stride).total : fwd_layout(vi, s, win).total; };
  if (total(0) <= bytes) return 0;
  if (unit < 1 || vi.num_docs == 0) return -1;
  // the windowed total grows with the window: the largest k with total(k unit) <= bytes
  int64_t lo = 0, hi = ((int64_t)max_chunks(vi) + unit - 1) / unit;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (total((int)(mid * unit)) <= bytes) lo = mid; else hi = mid - 1;
  }
  return lo > 0 ? (int)(lo * unit) : -1;
}

int64_t route1_num_blocks(const flare_varlen *v, int32_t block_size) {
  int64_t nb = 0;
  for (int32_t i = 0; i < v->num_docs; ++i) {
    const int64_t n = (int64_t)v->cu_seqlens_host[i + 1] - v->cu_seqlens_host[i];
    const int64_t P = v->prompt_lens_host[i];
    if (n > P) nb += (n - P + block_size - 1) / block_size;
  }
  return nb;
}

int64_t route1_num_windows(const flare_varlen *v) {
  int64_t nw = 0;
  for (int32_t i = 0; i < v->num_docs; ++i) {
    const int64_t n = (int64_t)v->cu_seqlens_host[i + 1] - v->cu_seqlens_host[i];
    const int64_t P = v->prompt_lens_host[i];
    if (n > P) nw += (n + kChunk - 1) / kChunk - P / kChunk;
  }
  return nw;
}

size_t route1_workspace_bytes(const VarlenInfo &vi, const flare_gdn_shape *s, int64_t n_blocks) {
  return round256(fwd_workspace_bytes(vi, s)) + round256((size_t)n_blocks * s->num_heads * s->d_k * s->d_v * 4) +
         round256((size_t)(3 * vi.num_docs + 7 * n_blocks) * sizeof(int32_t)) + 256;
}

flare_status check_block_step(int32_t num_req, const int32_t *slot_idx,
                              const int32_t *slot_idx_host, const float *pool,
                              int32_t num_slots, const flare_gdn_shape *s,
                              const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, const void *o,
                              int32_t mode) {
  flare_status st = check_gdn_shape(s);
  if (st != FLARE_OK) return st;
  if (num_req < 0) return fail(FLARE_ERR_SHAPE, "num_req < 0");
  if (num_slots < 0) return fail(FLARE_ERR_SHAPE, "num_slots < 0");
  if (mode != FLARE_BLOCK_EVAL && mode != FLARE_BLOCK_COMMIT)
    return fail(FLARE_ERR_SHAPE, "mode %d is neither EVAL nor COMMIT", mode);
  if (num_req == 0) return FLARE_OK;
  if (num_req > num_slots) return fail(FLARE_ERR_SHAPE, "num_req %d > num_slots %d", num_req, num_slots);
  if (!slot_idx || !pool || !q || !k || !v || !alpha || !beta)
    return fail(FLARE_ERR_NULL, "block_step: a required pointer is NULL");
  if (mode == FLARE_BLOCK_EVAL && !o) return fail(FLARE_ERR_NULL, "EVAL needs an output buffer");
  return check_slots_host(num_req, slot_idx_host, num_slots);
}

flare_status check_slots_host(int32_t n, const int32_t *slot_host, int32_t num_slots) {
  if (!slot_host) return FLARE_OK;
  // distinct and in range: counting sort over the slot range
  if (num_slots > (1 << 26)) return fail(FLARE_ERR_SHAPE, "num_slots too large to check");
  unsigned char *seen = new unsigned char[(size_t)num_slots]();
  for (int32_t r = 0; r < n; ++r) {
    const int32_t sl = slot_host[r];
    if (sl < 0 || sl >= num_slots) {
      delete[] seen;
      return fail(FLARE_ERR_SHAPE, "slot_idx[%d] = %d outside [0, %d)", r, sl, num_slots);
    }
    if (seen[sl]) {
      delete[] seen;
      return fail(FLARE_ERR_SHAPE, "slot %d used by two requests", sl);
    }
    seen[sl] = 1;
  }
  delete[] seen;
  return FLARE_OK;
}

size_t shortconv_bwd_workspace_bytes(const VarlenInfo &vi, int32_t channels, int32_t width, int32_t sections) {
  const int64_t blocks = (vi.total_tokens + kConvBwdRun - 1) / kConvBwdRun;
  return (size_t)sections * blocks * channels * (width + 1) * sizeof(float) + 256;
}

flare_status check_qkv_prologue(const flare_varlen *v, int32_t block_size, int32_t heads, int32_t head_dim,
                                int32_t width, int32_t io_dtype, const void *const x[3], const void *const xn[3],
                                const float *const w[3], int32_t activation, int32_t qk_l2norm,
                                const void *const y[3], const void *const yn[3], VarlenInfo *out) {
  if (heads <= 0 || head_dim <= 0) return fail(FLARE_ERR_SHAPE, "heads and head_dim must be positive");
  if ((int64_t)heads * head_dim > INT32_MAX) return fail(FLARE_ERR_SHAPE, "heads * head_dim too large");
  if (qk_l2norm != 0 && qk_l2norm != 1) return fail(FLARE_ERR_UNSUPPORTED, "qk_l2norm %d unknown", qk_l2norm);
  if (!x || !xn || !w || !y || !yn) return fail(FLARE_ERR_NULL, "qkv prologue: a pointer array is NULL");
  for (int s = 0; s < 3; ++s) {
    const flare_status st = check_shortconv(v, block_size, heads * head_dim, width, io_dtype, x[s], xn[s], w[s],
                                            activation, y[s], yn[s], out);
    if (st != FLARE_OK) return st;
  }
  if (qk_l2norm) {
    const int n = conv_lane_channels(io_dtype, width);
    const int g = head_dim / n;
    if (head_dim % n != 0 || g > 64 || (g & (g - 1)) != 0)
      return fail(FLARE_ERR_UNSUPPORTED, "qk_l2norm needs head_dim / %d to be a power of two <= 64 (head_dim %d)", n,
                  head_dim);
  }
  return FLARE_OK;
}

flare_status check_shortconv(const flare_varlen *v, int32_t block_size, int32_t channels,
                             int32_t width, int32_t io_dtype, const void *x, const void *xn,
                             const float *w, int32_t activation, const void *y, const void *yn,
                             VarlenInfo *out) {
  flare_status st = check_varlen(v, block_size, out);
  if (st != FLARE_OK) return st;
  if (channels <= 0) return fail(FLARE_ERR_SHAPE, "channels must be positive");
  if (width < 1 || width > 8) return fail(FLARE_ERR_UNSUPPORTED, "width %d not in [1, 8]", width);
  if (io_dtype != FLARE_F32 && io_dtype != FLARE_BF16)
    return fail(FLARE_ERR_UNSUPPORTED, "io_dtype %d unknown", io_dtype);
  const int vec = io_dtype == FLARE_BF16 ? 8 : 4;
  if (channels % vec != 0)
    return fail(FLARE_ERR_ALIGN, "channels %d must be a multiple of %d", channels, vec);
  if (activation != 0 && activation != 1)
    return fail(FLARE_ERR_UNSUPPORTED, "activation %d unknown", activation);
  if (out->total_tokens > 0 && (!x || !xn || !w || !y || !yn))
    return fail(FLARE_ERR_NULL, "shortconv: a required pointer is NULL");
  // token positions are 32-bit in the kernels, with room for a run past the end
  if (out->total_tokens > INT32_MAX - 4096)
    return fail(FLARE_ERR_UNSUPPORTED, "shortconv: %lld tokens, at most 2^31 - 4097",
                (long long)out->total_tokens);
  return FLARE_OK;
}

}  // namespace flare
