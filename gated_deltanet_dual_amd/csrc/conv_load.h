// conv_load.h -- the layer's dual ShortConv computed where the chunked
// forward loads its q, k, v rows (bf16 io, d = 128), so the convolution's
// outputs never go to memory.
//
// "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
// designs item 3: a depthwise causal ShortConv of width W sits in front of the
// GDN layer; a noisy output's tap that lies before the start of its block
// reads the clean input, a tap inside the block the noisy input; taps before
// the document start read zero; noisy prompt rows are zero.  The arithmetic
// is the one of the standalone ShortConv kernel (shortconv.hip): taps in lag
// order, fused multiply-adds from zero, then SiLU when asked, then rounding
// to bf16 -- so the rows the GDN kernels see are the very rows that kernel
// would have stored.
//
// Blocks never straddle a chunk boundary in the response (chunk starts are
// multiples of 32, blocks start at P + jB with B | 32 and B | P), so a noisy
// tap inside its block never reaches before the chunk start.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace flare {

// A thread's R consecutive chunk rows [r0, r0 + R) of 8 channels
// [8 cu16, 8 cu16 + 8) of head h in section sec (0 q, 1 k, 2 v), for the
// clean stream and, when `noisy`, the noisy one: the input windows (rows
// r0 - (W - 1) .. r0 + R - 1 of x and x~, as 16-byte units) and the weights
// by lag, loaded first; the outputs formed later by `rows`.
template <int W, int R>
struct ConvRows {
  static constexpr int NWIN = W + R - 1;
  uint4 cw[NWIN], nw[NWIN];
  float4 wraw[2 * W];  // the 8 W weights of the 8 channels, as stored ([channel][tap])

  __device__ __forceinline__ void load(const FwdArgs &f, int sec, int64_t t0g, int c0, int r0, int n, int h,
                                       int cu16, bool noisy) {
    const int64_t C = (int64_t)f.H * 128;
    const int64_t ch = (int64_t)h * 128 + 8 * cu16;
    // the section's pointers by selection (an indexed read of the argument
    // block's arrays would copy the block to scratch)
    const void *const x0 = f.cx[0], *const x1 = f.cx[1], *const x2 = f.cx[2];
    const void *const n0 = f.cxn[0], *const n1 = f.cxn[1], *const n2 = f.cxn[2];
    const float *const w0 = f.cwt[0], *const w1 = f.cwt[1], *const w2 = f.cwt[2];
    const u16 *const x = reinterpret_cast<const u16 *>(sec == 0 ? x0 : sec == 1 ? x1 : x2);
    const u16 *const xn = reinterpret_cast<const u16 *>(sec == 0 ? n0 : sec == 1 ? n1 : n2);
    const float *const wsec = sec == 0 ? w0 : sec == 1 ? w1 : w2;
#pragma unroll
    for (int j = 0; j < NWIN; ++j) {
      const int tp = min(max(c0 + r0 - (W - 1) + j, 0), n - 1);  // clamped into the document
      const int64_t off = (t0g + tp) * C + ch;
      cw[j] = *reinterpret_cast<const uint4 *>(x + off);
      nw[j] = noisy ? *reinterpret_cast<const uint4 *>(xn + off) : make_uint4(0u, 0u, 0u, 0u);
    }
    const float4 *w = reinterpret_cast<const float4 *>(wsec + ch * W);
#pragma unroll
    for (int j = 0; j < 2 * W; ++j) wraw[j] = w[j];
  }

  // y[i], yn[i]: chunk row r0 + i of the clean and the noisy output, bf16
  __device__ __forceinline__ void rows(int c0, int r0, int P, int B, bool act, uint4 (&y)[R], uint4 (&yn)[R]) const {
    float wl[W][8];  // wl[L][c] multiplies the input L tokens back
#pragma unroll
    for (int j = 0; j < 2 * W; ++j) {
      const float v4[4] = {wraw[j].x, wraw[j].y, wraw[j].z, wraw[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * j + e, c = idx / W, tap = idx % W;
        wl[W - 1 - tap][c] = v4[e];
      }
    }
    auto unpack = [](const uint4 &u, float (&o)[8]) {
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __uint_as_float(w4[e] << 16);
        o[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
      }
    };
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int tp = c0 + r0 + i;
      const int nb = min(tp + 1, W);  // taps inside the document
      const bool resp = tp >= P;
      const int na = resp ? min((tp - P) % B + 1, W) : 0;  // taps inside the block
      float yc[8], ynv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) yc[c] = ynv[c] = 0.f;
#pragma unroll
      for (int L = 0; L < W; ++L) {
        float hx[8], hn[8];
        unpack(cw[W - 1 + i - L], hx);
        unpack(nw[W - 1 + i - L], hn);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float hxu = L < nb ? hx[c] : 0.f;
          yc[c] = fmaf(wl[L][c], hxu, yc[c]);
          ynv[c] = fmaf(wl[L][c], L < na ? hn[c] : hxu, ynv[c]);
        }
      }
      if (act) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          yc[c] = yc[c] / (1.f + __expf(-yc[c]));
          ynv[c] = ynv[c] / (1.f + __expf(-ynv[c]));
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) ynv[c] = resp ? ynv[c] : 0.f;  // noisy prompt rows are zero
      y[i] = make_uint4(pack_bf16x2(yc[0], yc[1]), pack_bf16x2(yc[2], yc[3]), pack_bf16x2(yc[4], yc[5]),
                        pack_bf16x2(yc[6], yc[7]));
      yn[i] = make_uint4(pack_bf16x2(ynv[0], ynv[1]), pack_bf16x2(ynv[2], ynv[3]), pack_bf16x2(ynv[4], ynv[5]),
                         pack_bf16x2(ynv[6], ynv[7]));
    }
  }
};

// a if c else b, per component (a select of whole vectors can end up as a
// select among copies in scratch memory)
__device__ __forceinline__ uint4 sel4(bool c, const uint4 &a, const uint4 &b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// sum of squares of a 128-channel bf16 row held as 16-byte units by 16
// consecutive lanes (lane l: channels 8 l .. 8 l + 7), on every lane of the
// group; the q/k L2 factor pass (gdn_l2.hip) and the forward's conv loads
// both use it, so their factors agree bit for bit
__device__ __forceinline__ float l2_rowsum16(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xffff0000u);
    ss += a * a + b * b;
  }
  return dpp_sum16(ss);
}
// the factor 1 / sqrt(|row|^2 + 1e-6), finite (rows never read may hold anything)
__device__ __forceinline__ float l2_factor(float ss) {
  float rf = 1.f / sqrtf(ss + 1e-6f);
  if (!(rf < 3.0e38f)) rf = 0.f;
  return rf;
}

}  // namespace flare
