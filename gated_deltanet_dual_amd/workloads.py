"""Seeded synthetic inputs for the dual-stream Gated DeltaNet layer.

This module only draws numbers.  It holds none of the layer's arithmetic and is
shared by the HIP path's tests/benchmark and by the oracle's tests, so both
sides always see bit-identical inputs.  All arrays are numpy float32 (values
that travel as bf16 are rounded to bf16 here, round-to-nearest-even, so the
float32 array holds exactly the bf16 value) or int32.

Workload shapes follow the ones the FLARE notes describe (papernotes.org,
"FLARE: Diffusion for Hybrid Language Model", Overall framework and Key designs
items 2-4): a clean prompt followed by a response cut into blocks of B (default
4), packed documents whose boundaries are multiples of B, width-4 ShortConv, and
a serving pool of per-request recurrent states.  Distributions (normal q/k/v with
L2-normalised q and k, gates alpha = exp(-0.1 softplus(z)), beta = sigmoid(z))
are synthetic stand-ins: the pages print no data.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True))
    return (x / n).astype(np.float32)


def _softplus(z):
    return np.logaddexp(0.0, z)


def _gates_smooth(rng, shape):
    """alpha = exp(-0.1*softplus(z)), beta = sigmoid(z'), z, z' ~ N(0,1)."""
    z = rng.standard_normal(shape)
    z2 = rng.standard_normal(shape)
    a = np.exp(-0.1 * _softplus(z)).astype(np.float32)
    b = (1.0 / (1.0 + np.exp(-z2))).astype(np.float32)
    return a, b


def _gates_uniform(rng, shape):
    """alpha ~ U[0.9, 1), beta ~ U(0, 1)."""
    a = rng.uniform(0.9, 1.0, shape).astype(np.float32)
    b = rng.uniform(0.0, 1.0, shape).astype(np.float32)
    b = np.where(b == 0.0, np.float32(0.5), b).astype(np.float32)
    return a, b


@dataclass
class GDNInputs:
    cu_seqlens: np.ndarray          # [N+1] int32
    prompt_lens: np.ndarray         # [N] int32
    block_size: int
    io: str                         # "f32" or "bf16"
    q: np.ndarray                   # [T,H,dk]
    k: np.ndarray
    v: np.ndarray                   # [T,H,dv]
    alpha: np.ndarray               # [T,H]
    beta: np.ndarray
    qn: np.ndarray
    kn: np.ndarray
    vn: np.ndarray
    alpha_n: np.ndarray
    beta_n: np.ndarray
    h0: np.ndarray | None = None    # [N,H,dk,dv] float32
    do: np.ndarray | None = None    # [T,H,dv]
    don: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return int(self.cu_seqlens[-1])

    @property
    def H(self):
        return self.q.shape[1]

    def clean_args(self):
        return (self.q, self.k, self.v, self.alpha, self.beta)

    def noisy_args(self):
        return (self.qn, self.kn, self.vn, self.alpha_n, self.beta_n)


def gdn_inputs(doc_lens, prompt_lens, H, dk, dv, block_size, seed, io="bf16",
               gates="smooth", normalize_qk=True, with_h0=False, with_grads=False,
               noisy_equals_clean=False, round_io=True):
    """Draw one packed batch: docs of the given lengths back to back.  With
    round_io=False the bf16 rounding is left to the caller (values are the
    unrounded float32 draws; converting them to bf16 on the device with
    round-to-nearest-even gives the same numbers as round_bf16)."""
    rng = np.random.default_rng(seed)
    doc_lens = np.asarray(doc_lens, dtype=np.int64)
    cu = np.zeros(len(doc_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(doc_lens)
    T = int(cu[-1])
    rnd = round_bf16 if (io == "bf16" and round_io) else (lambda x: np.asarray(x, np.float32))

    def qkv():
        q = rng.standard_normal((T, H, dk), dtype=np.float32)
        k = rng.standard_normal((T, H, dk), dtype=np.float32)
        v = rng.standard_normal((T, H, dv), dtype=np.float32)
        if normalize_qk:
            q, k = _l2n(q), _l2n(k)
        return rnd(q), rnd(k), rnd(v)

    gate = _gates_smooth if gates == "smooth" else _gates_uniform
    q, k, v = qkv()
    a, b = gate(rng, (T, H))
    if noisy_equals_clean:
        qn, kn, vn, an, bn = q.copy(), k.copy(), v.copy(), a.copy(), b.copy()
    else:
        qn, kn, vn = qkv()
        an, bn = gate(rng, (T, H))
    inp = GDNInputs(cu, np.asarray(prompt_lens, dtype=np.int32), int(block_size), io,
                    q, k, v, a, b, qn, kn, vn, an, bn)
    if with_h0:
        inp.h0 = (rng.standard_normal((len(doc_lens), H, dk, dv)) / np.sqrt(dk)).astype(np.float32)
    if with_grads:
        inp.do = rnd(rng.standard_normal((T, H, dv), dtype=np.float32))
        inp.don = rnd(rng.standard_normal((T, H, dv), dtype=np.float32))
    return inp


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

def tiny_fp32(seed=1):
    """1 doc of 64 tokens (16 prompt, 48 response = 12 blocks of 4), H=1,
    d=16, fp32, alpha ~ U[0.9,1), beta ~ U(0,1), zero initial state."""
    return gdn_inputs([64], [16], 1, 16, 16, 4, seed, io="f32", gates="uniform")


def dual_bf16(block_size=4, seed=2, batch=4, seqlen=4096, prompt=1024, H=16, d=128):
    """batch x seqlen, prompt tokens clean, response in blocks, bf16 q/k/v."""
    return gdn_inputs([seqlen] * batch, [prompt] * batch, H, d, d, block_size, seed)


def headline(seed=5, with_grads=True, batch=4, seqlen=8192, prompt=2048, H=16, d=128,
             block_size=4, round_io=True):
    """4 docs x 8192 tokens (prompt 2048), B=4, H=16, d=128, bf16 q/k/v,
    upstream output gradients ~ N(0,1)."""
    return gdn_inputs([seqlen] * batch, [prompt] * batch, H, d, d, block_size, seed,
                      with_grads=with_grads, round_io=round_io)


def packed_doc_lengths(total, n_docs, block, seed, min_len=64):
    """Dirichlet(1) split of `total` tokens into n_docs lengths, each a multiple
    of `block` and >= min_len, summing exactly to total; prompt lengths are
    floor(U[0.1,0.5] * n / block) * block."""
    rng = np.random.default_rng(seed)
    w = rng.dirichlet(np.ones(n_docs))
    units = total // block
    min_u = min_len // block
    spare = units - n_docs * min_u
    alloc = np.floor(w * spare).astype(np.int64)
    rem = spare - alloc.sum()
    order = np.argsort(-(w * spare - alloc))
    alloc[order[:rem]] += 1
    lens = (alloc + min_u) * block
    frac = rng.uniform(0.1, 0.5, n_docs)
    prompts = (np.floor(frac * lens / block) * block).astype(np.int64)
    return lens.astype(np.int32), prompts.astype(np.int32)


def packed_conv(seed=3, total=32768, n_docs=8, H=32, d=128, block_size=4, width=4, round_io=True):
    """One packed row of `total` tokens, n_docs Dirichlet-split documents, ShortConv
    inputs over the q/k/v channels (3*H*d) for both streams, conv weights
    ~ U(-1/2, 1/2) [C, width], then GDN gates for both streams."""
    lens, prompts = packed_doc_lengths(total, n_docs, block_size, seed)
    rng = np.random.default_rng(seed + 1000)
    C = 3 * H * d
    T = int(lens.sum())
    rnd = round_bf16 if round_io else (lambda x: x)
    x = rnd(rng.standard_normal((T, C), dtype=np.float32))
    xn = rnd(rng.standard_normal((T, C), dtype=np.float32))
    w = rng.uniform(-0.5, 0.5, (C, width)).astype(np.float32)
    a, b = _gates_smooth(rng, (T, H))
    an, bn = _gates_smooth(rng, (T, H))
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return dict(cu_seqlens=cu, prompt_lens=prompts, x=x, xn=xn, weight=w,
                alpha=a, beta=b, alpha_n=an, beta_n=bn, H=H, d=d,
                block_size=block_size, width=width)


@dataclass
class ServingInputs:
    slot_idx: np.ndarray     # [R] int32, distinct
    pool: np.ndarray         # [n_slots,H,dk,dv] float32
    evals: list              # list of (q,k,v,alpha,beta) noisy blocks
    commit: tuple            # (q,k,v,alpha,beta) clean block


def serving(seed=4, n_req=256, H=16, d=128, block_size=4, n_slots=512, n_evals=4):
    """n_req requests with distinct random slots in a pool of fp32 d x d states
    ~ N(0, 1/d); n_evals noisy bf16 blocks of block_size tokens and one clean
    block to commit, gates as the smooth recipe."""
    rng = np.random.default_rng(seed)
    slot = rng.permutation(n_slots)[:n_req].astype(np.int32)
    pool = (rng.standard_normal((n_slots, H, d, d), dtype=np.float32) / np.sqrt(d)).astype(np.float32)

    def block():
        q = round_bf16(_l2n(rng.standard_normal((n_req, block_size, H, d), dtype=np.float32)))
        k = round_bf16(_l2n(rng.standard_normal((n_req, block_size, H, d), dtype=np.float32)))
        v = round_bf16(rng.standard_normal((n_req, block_size, H, d), dtype=np.float32))
        a, b = _gates_smooth(rng, (n_req, block_size, H))
        return q, k, v, a, b

    evals = [block() for _ in range(n_evals)]
    commit = block()
    return ServingInputs(slot, pool, evals, commit)
