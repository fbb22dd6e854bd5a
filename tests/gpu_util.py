"""Shared helpers for the GPU parity tests (no method arithmetic here)."""
import numpy as np

TOL_F32 = 1e-4   # relative RMS, fp32 io
TOL_BF16 = 3e-3  # relative RMS, bf16 io


def rel_rms(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def to_dev(x, dev, bf16=False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return t.to(torch.bfloat16) if bf16 else t


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def fwd_args(inp, dev):
    bf = inp.io == "bf16"
    return [to_dev(inp.q, dev, bf), to_dev(inp.k, dev, bf), to_dev(inp.v, dev, bf),
            to_dev(inp.alpha, dev), to_dev(inp.beta, dev),
            to_dev(inp.qn, dev, bf), to_dev(inp.kn, dev, bf), to_dev(inp.vn, dev, bf),
            to_dev(inp.alpha_n, dev), to_dev(inp.beta_n, dev)]


def sub_heads(inp, heads):
    """Inputs restricted to a subset of heads (for oracle runs at full length)."""
    import copy
    out = copy.copy(inp)
    for name in ("q", "k", "v", "alpha", "beta", "qn", "kn", "vn", "alpha_n", "beta_n", "do", "don"):
        x = getattr(inp, name)
        if x is not None:
            setattr(out, name, np.ascontiguousarray(x[:, heads]))
    if inp.h0 is not None:
        out.h0 = np.ascontiguousarray(inp.h0[:, heads])
    return out
