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
};
hipError_t launch_gdn_fwd(const FwdArgs &a, hipStream_t st);

// bf16 io at d = 128 without flags: the forward's pre-pass (chunk matrices
// `cmat` -> scan hand-over `pack`, gdn_fwd_pre.hip) and its output pass
// (chunk-start states -> o, o~, gdn_fwd_out.hip)
hipError_t launch_fwd_pre_d128(const FwdArgs &a, const float *cmat, float *pack, hipStream_t st, int64_t slots);
hipError_t launch_fwd_out_d128(const FwdArgs &a, const float *cmat, const float *states, hipStream_t st,
                               int64_t slots);

// The sequential chunk recurrence X <- g_C X + R + K^T (W (K X)) over the chunks
// of each document (gdn_scan.hip), forward or in reverse.
struct ScanArgs {
  int num_docs, H;
  const int32_t *cu;
  const float *pack;   // per (chunk slot, head): the pre-pass's hand-over
  const float *init;   // [N, H, 128, 128] X before the first step, or NULL (zero)
  float *final_out;    // [N, H, 128, 128] X after the last step, or NULL
  float *states;       // [slots, H, 128, 128]: X before the step of chunk c, at chunk c's slot
  const int32_t *slot; // NULL, or per document the index of its init / final_out state
};
hipError_t launch_scan_d128(const ScanArgs &a, bool reverse, hipStream_t st);

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
  float *tri;            // per slot and head [slots][H][6][32][32]: T, T~, Mwo, Mwq, Mwk, Mw~ (set by the launcher)
  const float *fwd_cm;   // the same matrices from the forward's workspace, or NULL
  float *pack;           // bf16, d = 128: the pre-pass's hand-over to the scan, per slot and head (set by the launcher)
};
hipError_t launch_gdn_bwd(const BwdArgs &a, hipStream_t st);
// per-chunk backward kernel for bf16 io at d = 128 (gdn_bwd_chunk.hip)
hipError_t launch_bwd_chunk_d128(const BwdArgs &a, hipStream_t st, int64_t slots);
// the chunk solves T, T~ into a.tri for bf16 io at d = 128 (gdn_tri.hip)
hipError_t launch_tri_d128(const BwdArgs &a, hipStream_t st, int64_t slots);
// the state-independent part of the reverse scan's chunk step into a.pack
// (gdn_bwd_pre.hip)
hipError_t launch_bwd_pre_d128(const BwdArgs &a, hipStream_t st, int64_t slots);

}  // namespace flare
