"""gated_deltanet_dual_amd -- MI355X (gfx950) dual-stream Gated DeltaNet layer.

A thin ctypes binding over ``libflare_gdn.so`` (the C ABI declared in
``include/flare_gdn.h``).  This module only marshals arguments: every step of
the computation runs in the library's HIP kernels.  PyTorch provides device
memory and the current stream.  There is no fallback: if the library is not
built, every call raises.

Method: "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes),
Overall framework and Key designs items 2-4.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["Varlen", "GDNShape", "FlareError", "lib", "gdn_dual_fwd", "gdn_dual_fwd_pool", "gdn_dual_fwd_route1", "gdn_dual_bwd",
           "gdn_dual_fwd_conv", "block_step", "block_step_conv", "conv_cache_fill", "gdn_verify", "gdn_scatter", "gdn_verify_outputs", "gdn_commit_prefix", "shortconv_dual", "shortconv_dual_bwd", "shortconv_dual_bwd_workspace_bytes", "qkv_prologue",
           "qkv_prologue_bwd", "qkv_prologue_bwd_workspace_bytes", "chunk_size", "ckpt_slots", "EVAL", "COMMIT",
           "QK_L2NORM", "F32", "BF16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflare_gdn.so")

F32, BF16 = 0, 1
EVAL, COMMIT = 0, 1
QK_L2NORM = 1

_STATUS = {0: "OK", 1: "NULL", 2: "SHAPE", 3: "ALIGN", 4: "UNSUPPORTED", 5: "WORKSPACE", 6: "HIP"}


class FlareError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("flare status %s (%d): %s" % (_STATUS.get(status, "?"), status, msg))
        self.status = status


class _Varlen(ctypes.Structure):
    _fields_ = [("num_docs", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
                ("prompt_lens", ctypes.c_void_p), ("prompt_lens_host", ctypes.c_void_p)]


class GDNShape(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("scale", ctypes.c_float)]


_lib = None


def lib():
    """Load libflare_gdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libflare_gdn.so is not built: run `python -m gated_deltanet_dual_amd.build`")
    # torch owns the device memory and streams this library works on, so the
    # library must bind to the HIP runtime torch already loaded (same soname);
    # loading it first would bring in a second, separate runtime.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    _check_single_hip_runtime()
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    VP, SP = ctypes.POINTER(_Varlen), ctypes.POINTER(GDNShape)
    A3 = ctypes.c_void_p * 3  # host arrays of three device pointers
    L.flare_gdn_chunk_size.restype = I32
    L.flare_version.restype = I32
    L.flare_last_error.restype = ctypes.c_char_p
    L.flare_gdn_dual_workspace_size.argtypes = [VP, SP, ctypes.c_int]
    L.flare_gdn_dual_workspace_size.restype = SZ
    L.flare_gdn_dual_workspace_size_window.argtypes = [VP, SP, ctypes.c_int, I32, I32]
    L.flare_gdn_dual_workspace_size_window.restype = SZ
    L.flare_gdn_dual_ckpt_size.argtypes = [VP, SP, I32]
    L.flare_gdn_dual_ckpt_size.restype = SZ
    L.flare_gdn_ckpt_slot.argtypes = [I32, I32, I32, I32]
    L.flare_gdn_ckpt_slot.restype = ctypes.c_int64
    L.flare_gdn_dual_fwd.argtypes = [VP, SP] + [P] * 10 + [P, P, P, P, P, I32, P, SZ, P]
    L.flare_gdn_dual_fwd.restype = ctypes.c_int
    L.flare_gdn_dual_fwd_conv.argtypes = [VP, SP, I32, A3, I32, A3, A3] + [P] * 4 + [P, P, P, P, P, I32, P, SZ, P]
    L.flare_gdn_dual_fwd_conv.restype = ctypes.c_int
    L.flare_gdn_dual_bwd.argtypes = [VP, SP] + [P] * 10 + [P, P, I32, P, P, P, P] + [P] * 11 + [P, SZ, P]
    L.flare_gdn_dual_bwd.restype = ctypes.c_int
    L.flare_gdn_block_step.argtypes = [I32, P, P, P, I32, SP, P, P, P, P, P, P, I32, P]
    L.flare_gdn_block_step.restype = ctypes.c_int
    L.flare_gdn_route1_workspace_size.argtypes = [VP, SP]
    L.flare_gdn_route1_workspace_size.restype = SZ
    L.flare_gdn_dual_fwd_route1.argtypes = [VP, SP] + [P] * 10 + [P, P, P, P, P, P, SZ, P]
    L.flare_gdn_dual_fwd_route1.restype = ctypes.c_int
    L.flare_gdn_dual_fwd_pool.argtypes = [VP, SP] + [P] * 10 + [P, P, P, I32, I32, P, P, P, I32, P, SZ, P]
    L.flare_gdn_dual_fwd_pool.restype = ctypes.c_int
    L.flare_gdn_block_step_conv.argtypes = [I32, P, P, P, P, I32, SP, I32, A3, I32, I32, P, P, P, P, P, P, I32, P]
    L.flare_gdn_block_step_conv.restype = ctypes.c_int
    L.flare_conv_cache_fill.argtypes = [VP, I32, I32, I32, I32, A3, P, P, P, I32, P]
    L.flare_conv_cache_fill.restype = ctypes.c_int
    L.flare_gdn_verify.argtypes = [I32, P, P, P, I32, SP, P, P, P, P, P, P, P, P]
    L.flare_gdn_verify.restype = ctypes.c_int
    L.flare_gdn_scatter.argtypes = [I32, P, P, P, P, P, I32, SP, P]
    L.flare_gdn_scatter.restype = ctypes.c_int
    L.flare_gdn_verify_outputs.argtypes = [I32, P, P, P, I32, SP, P, P, P, P, P, P, P]
    L.flare_gdn_verify_outputs.restype = ctypes.c_int
    L.flare_gdn_commit_prefix.argtypes = [I32, P, P, P, I32, SP, P, P, P, P, P, P, P, P]
    L.flare_gdn_commit_prefix.restype = ctypes.c_int
    L.flare_shortconv_dual.argtypes = [VP, I32, I32, I32, I32, P, P, P, P, I32, P, P, P]
    L.flare_shortconv_dual.restype = ctypes.c_int
    L.flare_shortconv_dual_bwd_workspace_size.argtypes = [VP, I32, I32, I32]
    L.flare_shortconv_dual_bwd_workspace_size.restype = SZ
    L.flare_shortconv_dual_bwd.argtypes = [VP, I32, I32, I32, I32, P, P, P, P, I32, P, P, P, P, P, P, P, SZ, P]
    L.flare_shortconv_dual_bwd.restype = ctypes.c_int
    L.flare_qkv_prologue.argtypes = [VP, I32, I32, I32, I32, I32, A3, A3, A3, I32, I32, A3, A3, P]
    L.flare_qkv_prologue.restype = ctypes.c_int
    L.flare_qkv_prologue_bwd_workspace_size.argtypes = [VP, I32, I32, I32, I32]
    L.flare_qkv_prologue_bwd_workspace_size.restype = SZ
    L.flare_qkv_prologue_bwd.argtypes = [VP, I32, I32, I32, I32, I32, A3, A3, A3, I32, I32, A3, A3, A3, A3, A3,
                                         P, SZ, P]
    L.flare_qkv_prologue_bwd.restype = ctypes.c_int
    L.flare_noalloc_scratch_bytes.argtypes = []
    L.flare_noalloc_scratch_bytes.restype = SZ
    L.flare_qkv_prologue_bwd_noalloc.argtypes = [VP, I32, I32, I32, I32, I32, A3, A3, A3, I32, I32, A3, A3, A3, A3,
                                                 A3, P]
    L.flare_qkv_prologue_bwd_noalloc.restype = ctypes.c_int
    L.flare_timing_enable.argtypes = [I32]
    L.flare_timing_enable.restype = I32
    L.flare_timing_avg_ms.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64)]
    L.flare_timing_avg_ms.restype = ctypes.c_double
    L.flare_timing_reset.argtypes = []
    L.flare_timing_reset.restype = None
    _lib = L
    return L


def _check_single_hip_runtime():
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    if len(libs) > 1:
        raise ImportError("two HIP runtimes are mapped in this process: %s" % sorted(libs))


def _check(status):
    if status != 0:
        raise FlareError(status, lib().flare_last_error().decode())


def chunk_size() -> int:
    return int(lib().flare_gdn_chunk_size())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ---------------------------------------------------------------- argument checks
# The library sees bare device pointers, so every tensor is checked here
# before the call: dtype, shape (the one the shape struct implies), C
# contiguity and device.  A mismatch raises FlareError and nothing is launched.

def _fail(msg, status=2):
    raise FlareError(status, msg)


def _gpu_device(t, name):
    if t is None:
        _fail("%s is required" % name, 1)
    if not t.is_cuda:
        _fail("%s must be a GPU tensor (it is on %s)" % (name, t.device))
    return t.device


def _chk(t, name, shape, dtype, device, optional=False):
    """t has exactly this shape and dtype, is C-contiguous and on device."""
    if t is None:
        if optional:
            return
        _fail("%s is required" % name, 1)
    if t.dtype != dtype:
        _fail("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        _fail("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        _fail("%s must be contiguous" % name, 3)
    if t.device != device:
        _fail("%s is on %s, expected %s" % (name, t.device, device))


def _chk_buf(t, name, need_bytes, dtype, device, optional=False):
    """A flat buffer (workspace, checkpoints, candidates): dtype, contiguity,
    device, and at least need_bytes."""
    if t is None:
        if optional:
            return
        _fail("%s is required" % name, 1)
    if t.dtype != dtype:
        _fail("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        _fail("%s must be contiguous" % name, 3)
    if t.device != device:
        _fail("%s is on %s, expected %s" % (name, t.device, device))
    have = t.numel() * t.element_size()
    if have < need_bytes:
        _fail("%s holds %d bytes, %d needed" % (name, have, need_bytes), 5)


def _chk_varlen(varlen, T, device):
    if varlen.cu_dev.device != device:
        _fail("varlen's device arrays are on %s, the tensors on %s" % (varlen.cu_dev.device, device))
    if T != varlen.total_tokens:
        _fail("tensors hold %d tokens, cu_seqlens[-1] = %d" % (T, varlen.total_tokens))


def _io_dtype_of(t, name="q"):
    torch = _torch()
    if t is None:
        _fail("%s is required" % name, 1)
    if t.dtype not in (torch.bfloat16, torch.float32):
        _fail("%s: io tensors must be bfloat16 or float32, got %s" % (name, t.dtype), 4)
    return t.dtype


def _chk_gdn_inputs(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0=None):
    """The ten layer inputs and h0; returns (T, H, d, io dtype, device)."""
    torch = _torch()
    dev = _gpu_device(q, "q")
    io = _io_dtype_of(q)
    if q.dim() != 3:
        _fail("q must be [T, H, d], got shape %s" % (tuple(q.shape),))
    T, H, d = q.shape
    _chk_varlen(varlen, T, dev)
    for name, t in (("q", q), ("k", k), ("v", v), ("qn", qn), ("kn", kn), ("vn", vn)):
        _chk(t, name, (T, H, d), io, dev)
    for name, t in (("alpha", alpha), ("beta", beta), ("alpha_n", alpha_n), ("beta_n", beta_n)):
        _chk(t, name, (T, H), torch.float32, dev)
    _chk(h0, "h0", (varlen.num_docs, H, d, d), torch.float32, dev, optional=True)
    return T, H, d, io, dev


def _chk_rows(t, name, lead, H, d, io, dev, optional=False):
    """A serving-step tensor [lead..., H, d] of the io dtype."""
    _chk(t, name, tuple(lead) + (H, d), io, dev, optional)


def _chk_pool(pool, H, d, dev):
    torch = _torch()
    if pool is None or pool.dim() != 4:
        _fail("pool must be [n_slots, H, d, d]")
    _chk(pool, "pool", (pool.shape[0], H, d, d), torch.float32, dev)


def _chk_conv_inputs(varlen, x, xn, weight, bias):
    """ShortConv inputs x, xn [T, C] io, weight [C, W] fp32, bias [C] fp32 or
    None; returns (T, C, W, device)."""
    torch = _torch()
    dev = _gpu_device(x, "x")
    io = _io_dtype_of(x, "x")
    if x.dim() != 2 or weight is None or weight.dim() != 2:
        _fail("x must be [T, C] and weight [C, W]")
    T, C = x.shape
    W = weight.shape[1]
    _chk_varlen(varlen, T, dev)
    _chk(x, "x", (T, C), io, dev)
    _chk(xn, "xn", (T, C), io, dev)
    _chk(weight, "weight", (C, W), torch.float32, dev)
    _chk(bias, "bias", (C,), torch.float32, dev, optional=True)
    return T, C, W, dev


def _chk_three(ts, name, shape, dtype, dev):
    if ts is None or len(ts) != 3:
        _fail("%s must be a list of three tensors" % name, 1)
    for i, t in enumerate(ts):
        _chk(t, "%s[%d]" % (name, i), shape, dtype, dev)


def _chk_prologue_inputs(varlen, xs, xns, weights):
    """The prologue's three clean and three noisy projections [T, C] io and
    three weights [C, W] fp32; returns (T, C, W, device)."""
    torch = _torch()
    if xs is None or len(xs) != 3 or xs[0] is None or xs[0].dim() != 2:
        _fail("xs must be three [T, H*head_dim] io tensors")
    if weights is None or len(weights) != 3 or weights[0] is None or weights[0].dim() != 2:
        _fail("weights must be three [H*head_dim, W] fp32 tensors")
    dev = _gpu_device(xs[0], "xs[0]")
    io = _io_dtype_of(xs[0], "xs[0]")
    T, C = xs[0].shape
    W = weights[0].shape[1]
    _chk_varlen(varlen, T, dev)
    _chk_three(xs, "xs", (T, C), io, dev)
    _chk_three(xns, "xns", (T, C), io, dev)
    _chk_three(weights, "weights", (C, W), torch.float32, dev)
    return T, C, W, dev


def _chk_step_inputs(slot_idx, pool, q, k, v, alpha, beta):
    """Serving-step inputs q, k, v [R, B, H, d] io, gates [R, B, H] fp32,
    slot_idx [R] int32, pool [n_slots, H, d, d] fp32; returns (R, B, H, d, dev)."""
    torch = _torch()
    dev = _gpu_device(q, "q")
    io = _io_dtype_of(q)
    if q.dim() != 4:
        _fail("q must be [R, B, H, d], got shape %s" % (tuple(q.shape),))
    R, B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _chk_rows(t, name, (R, B), H, d, io, dev)
    for name, t in (("alpha", alpha), ("beta", beta)):
        _chk(t, name, (R, B, H), torch.float32, dev)
    _chk(slot_idx, "slot_idx", (R,), torch.int32, dev)
    _chk_pool(pool, H, d, dev)
    return R, B, H, d, dev


class Varlen:
    """Packed batch description: cu_seqlens [N+1] and prompt_lens [N], kept both on
    the host (validated before launch) and on the device (read by the kernels)."""

    def __init__(self, cu_seqlens, prompt_lens, device="cuda"):
        torch = _torch()
        self.cu_host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        self.pl_host = np.ascontiguousarray(np.asarray(prompt_lens, dtype=np.int32))
        self.cu_dev = torch.from_numpy(self.cu_host).to(device)
        self.pl_dev = torch.from_numpy(self.pl_host).to(device)
        self._s = _Varlen(len(self.pl_host), self.cu_dev.data_ptr(),
                          self.cu_host.ctypes.data, self.pl_dev.data_ptr(), self.pl_host.ctypes.data)

    @property
    def num_docs(self):
        return len(self.pl_host)

    @property
    def total_tokens(self):
        return int(self.cu_host[-1])

    def ref(self):
        return ctypes.byref(self._s)


def _shape(H, d, B, io, flags=0, scale=0.0):
    return GDNShape(H, d, d, B, io, flags, scale)


def _io_of(t):
    torch = _torch()
    return BF16 if _io_dtype_of(t) == torch.bfloat16 else F32


def ckpt_slots(varlen: Varlen, H: int, d: int, B: int, io: int, stride: int = 1) -> int:
    nbytes = lib().flare_gdn_dual_ckpt_size(varlen.ref(), ctypes.byref(_shape(H, d, B, io)), stride)
    return nbytes // (H * d * d * 4)


def gdn_dual_fwd(varlen: Varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, block_size,
                 h0=None, scale=0.0, flags=0, want_h_final=True, want_ckpt=False, out=None, ckpt=None,
                 workspace=None, ckpt_stride=1, window=0):
    """Dual-stream forward.  q,k,qn,kn [T,H,d]; v,vn [T,H,d]; gates [T,H] fp32;
    h0 [N,H,d,d] fp32 or None.  `out` = (o, on) reuses output buffers, `ckpt`
    a buffer for the chunk-start states (implies saving them) of every
    `ckpt_stride`-th chunk, `workspace` a uint8 device buffer of at least
    workspace_bytes(..., window=window) bytes (allocated here when needed and
    not given); window > 0 runs the chunked path in windows of that many
    chunks of every document.  Returns (o, on, h_final, ckpt)."""
    torch = _torch()
    T, H, d, iot, dev = _chk_gdn_inputs(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0)
    io = _io_of(q)
    shp = _shape(H, d, block_size, io, flags, scale)
    if out is None:
        o = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
        on = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    else:
        o, on = out
        _chk(o, "o", (T, H, d), iot, dev)
        _chk(on, "on", (T, H, d), iot, dev)
    hf = torch.empty((varlen.num_docs, H, d, d), dtype=torch.float32, device=q.device) if want_h_final else None
    ck = ckpt
    if ck is not None or want_ckpt:
        nbytes = lib().flare_gdn_dual_ckpt_size(varlen.ref(), ctypes.byref(shp), int(ckpt_stride))
        if nbytes == 0:
            raise FlareError(2, "invalid arguments for the checkpoint size")
        if ck is None:
            ck = torch.empty((nbytes // (H * d * d * 4), H, d, d), dtype=torch.float32, device=q.device)
        _chk_buf(ck, "ckpt", nbytes, torch.float32, dev)
    ws_bytes = _ws_bytes(varlen, shp, False, 1, window)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    _chk_buf(workspace, "workspace", ws_bytes, torch.uint8, dev, optional=ws_bytes == 0)
    # the library runs in windows when the workspace it is told of holds less
    # than one pass: hand it exactly the size asked for
    _check(lib().flare_gdn_dual_fwd(varlen.ref(), ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(alpha), _ptr(beta), _ptr(qn), _ptr(kn), _ptr(vn),
                                    _ptr(alpha_n), _ptr(beta_n), _ptr(h0), _ptr(o), _ptr(on),
                                    _ptr(hf), _ptr(ck), int(ckpt_stride), _ptr(workspace),
                                    ws_bytes if workspace is not None else 0, _stream(q.device)))
    return o, on, hf, ck


def gdn_dual_fwd_conv(varlen: Varlen, xs, xns, weights, alpha, beta, alpha_n, beta_n, block_size, activation=1,
                      h0=None, scale=0.0, flags=0, want_h_final=True, want_ckpt=False, out=None, ckpt=None,
                      workspace=None, ckpt_stride=1, window=0):
    """The dual-stream forward with the layer's ShortConv in its loads: xs,
    xns are the clean and noisy q, k, v projections (three [T, H*128] bf16
    tensors each), weights three [H*128, W] fp32 (W <= 4), SiLU when
    activation = 1; flags = QK_L2NORM normalises the q, k rows after the
    convolution.  Same results as qkv_prologue(..., qk_l2norm=False) followed
    by gdn_dual_fwd.  Returns (o, on, h_final, ckpt)."""
    torch = _torch()
    T, C, W, dev = _chk_prologue_inputs(varlen, xs, xns, weights)
    d = 128
    if C % d != 0:
        _fail("the projections must hold whole heads of 128 channels (got %d channels)" % C)
    H = C // d
    iot = _io_dtype_of(xs[0], "xs[0]")
    for name, t in (("alpha", alpha), ("beta", beta), ("alpha_n", alpha_n), ("beta_n", beta_n)):
        _chk(t, name, (T, H), torch.float32, dev)
    _chk(h0, "h0", (varlen.num_docs, H, d, d), torch.float32, dev, optional=True)
    shp = _shape(H, d, block_size, _io_of(xs[0]), flags, scale)
    if out is None:
        o = torch.empty((T, H, d), dtype=iot, device=dev)
        on = torch.empty((T, H, d), dtype=iot, device=dev)
    else:
        o, on = out
        _chk(o, "o", (T, H, d), iot, dev)
        _chk(on, "on", (T, H, d), iot, dev)
    hf = torch.empty((varlen.num_docs, H, d, d), dtype=torch.float32, device=dev) if want_h_final else None
    ck = ckpt
    if ck is not None or want_ckpt:
        nbytes = lib().flare_gdn_dual_ckpt_size(varlen.ref(), ctypes.byref(shp), int(ckpt_stride))
        if nbytes == 0:
            raise FlareError(2, "invalid arguments for the checkpoint size")
        if ck is None:
            ck = torch.empty((nbytes // (H * d * d * 4), H, d, d), dtype=torch.float32, device=dev)
        _chk_buf(ck, "ckpt", nbytes, torch.float32, dev)
    ws_bytes = _ws_bytes(varlen, shp, False, 1, window)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    _chk_buf(workspace, "workspace", ws_bytes, torch.uint8, dev, optional=ws_bytes == 0)
    _check(lib().flare_gdn_dual_fwd_conv(varlen.ref(), ctypes.byref(shp), W, _a3(weights), int(activation), _a3(xs),
                                         _a3(xns), _ptr(alpha), _ptr(beta), _ptr(alpha_n), _ptr(beta_n), _ptr(h0),
                                         _ptr(o), _ptr(on), _ptr(hf), _ptr(ck), int(ckpt_stride), _ptr(workspace),
                                         ws_bytes if workspace is not None else 0, _stream(dev)))
    return o, on, hf, ck


def _ws_bytes(varlen, shp, for_bwd, stride, window):
    if window < 0:
        _fail("window must be >= 0")
    if stride == 1 and window == 0:
        return int(lib().flare_gdn_dual_workspace_size(varlen.ref(), ctypes.byref(shp), 1 if for_bwd else 0))
    n = int(lib().flare_gdn_dual_workspace_size_window(varlen.ref(), ctypes.byref(shp), 1 if for_bwd else 0,
                                                        int(stride), int(window)))
    if n == 0:
        _fail("no %s workspace for checkpoint stride %d and window %d with this shape (windows need bf16 io at "
              "d = 128 and, for the backward, a multiple of the stride)" % ("backward" if for_bwd else "forward",
                                                                            stride, window))
    return n


def gdn_dual_fwd_route1(varlen: Varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, block_size, h0=None,
                        scale=0.0, out=None, ckpt=None, workspace=None, want_h_final=True):
    """The chunk-then-refine route for the dual forward: the clean stream with
    its chunk-start states, every block-boundary state materialised, every
    noisy block refined from it.  Returns (o, on, h_final, ckpt)."""
    torch = _torch()
    T, H, d, iot, dev = _chk_gdn_inputs(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0)
    shp = _shape(H, d, block_size, _io_of(q), 0, scale)
    if out is None:
        o = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
        on = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    else:
        o, on = out
        _chk(o, "o", (T, H, d), iot, dev)
        _chk(on, "on", (T, H, d), iot, dev)
    hf = torch.empty((varlen.num_docs, H, d, d), dtype=torch.float32, device=q.device) if want_h_final else None
    nbytes = lib().flare_gdn_dual_ckpt_size(varlen.ref(), ctypes.byref(shp), 1)
    if ckpt is None:
        ckpt = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=q.device)
    _chk_buf(ckpt, "ckpt", nbytes, torch.float32, dev)
    need = int(lib().flare_gdn_route1_workspace_size(varlen.ref(), ctypes.byref(shp)))
    call = lambda ws, nbytes: lib().flare_gdn_dual_fwd_route1(
        varlen.ref(), ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(qn), _ptr(kn),
        _ptr(vn), _ptr(alpha_n), _ptr(beta_n), _ptr(h0), _ptr(o), _ptr(on), _ptr(hf), _ptr(ckpt), ws, nbytes,
        _stream(q.device))
    if need == 0:  # the size query rejected the call: the entry point names the reason
        _check(call(None, 0))
        raise FlareError(4, "route1: unsupported shape")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    _chk_buf(workspace, "workspace", need, torch.uint8, dev)
    _check(call(_ptr(workspace), workspace.numel()))
    return o, on, hf, ckpt


def gdn_dual_fwd_pool(varlen: Varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, block_size, doc_slot,
                      pool, read_initial=False, doc_slot_host=None, scale=0.0, flags=0, out=None, workspace=None):
    """Prefill into a state pool: the dual forward with document i starting
    from pool[doc_slot[i]] (read_initial) or zero, and its final state written
    to pool[doc_slot[i]].  doc_slot: device int32 [N].  Returns (o, on)."""
    torch = _torch()
    T, H, d, iot, dev = _chk_gdn_inputs(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n)
    _chk(doc_slot, "doc_slot", (varlen.num_docs,), torch.int32, dev)
    _chk_pool(pool, H, d, dev)
    shp = _shape(H, d, block_size, _io_of(q), flags, scale)
    if out is None:
        o = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
        on = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    else:
        o, on = out
        _chk(o, "o", (T, H, d), iot, dev)
        _chk(on, "on", (T, H, d), iot, dev)
    ws_bytes = lib().flare_gdn_dual_workspace_size(varlen.ref(), ctypes.byref(shp), 0)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    _chk_buf(workspace, "workspace", ws_bytes, torch.uint8, dev, optional=ws_bytes == 0)
    host = None
    if doc_slot_host is not None:
        host = np.ascontiguousarray(np.asarray(doc_slot_host, dtype=np.int32))
    _check(lib().flare_gdn_dual_fwd_pool(varlen.ref(), ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                         _ptr(beta), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(alpha_n), _ptr(beta_n),
                                         _ptr(doc_slot), None if host is None else host.ctypes.data, _ptr(pool),
                                         pool.shape[0], 1 if read_initial else 0, _ptr(o), _ptr(on), None, 1,
                                         _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                         _stream(q.device)))
    return o, on


def gdn_dual_bwd(varlen: Varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, block_size,
                 ckpt, d_o, d_on, h0=None, dh_final=None, scale=0.0, flags=0, want_dh0=True,
                 workspace=None, out=None, fwd_workspace=None, ckpt_stride=1, window=0):
    """Reverse mode.  Returns a dict of gradients (same names as the oracle);
    `out` = such a dict reuses its buffers, `workspace` a uint8 device buffer of
    at least workspace_bytes(..., for_bwd=True, stride=ckpt_stride,
    window=window) bytes, `fwd_workspace` the workspace of the one-pass
    forward call that produced `ckpt` (its chunk matrices are then reused).
    `ckpt` holds every `ckpt_stride`-th chunk-start state; the others are
    rebuilt.  window > 0 runs in windows of that many chunks of every document
    (a multiple of ckpt_stride)."""
    torch = _torch()
    T, H, d, iot, dev = _chk_gdn_inputs(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0)
    io = _io_of(q)
    shp = _shape(H, d, block_size, io, flags, scale)
    N = varlen.num_docs
    _chk(d_o, "d_o", (T, H, d), iot, dev)
    _chk(d_on, "d_on", (T, H, d), iot, dev)
    _chk(dh_final, "dh_final", (N, H, d, d), torch.float32, dev, optional=True)
    ck_bytes = lib().flare_gdn_dual_ckpt_size(varlen.ref(), ctypes.byref(shp), int(ckpt_stride))
    if ck_bytes == 0:
        _fail("invalid checkpoint stride %r" % (ckpt_stride,))
    _chk_buf(ckpt, "ckpt", ck_bytes, torch.float32, dev)
    _chk_buf(fwd_workspace, "fwd_workspace", lib().flare_gdn_dual_workspace_size(varlen.ref(), ctypes.byref(shp), 0),
             torch.uint8, dev, optional=True)
    ws_bytes = _ws_bytes(varlen, shp, True, ckpt_stride, window)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=dev)
    _chk_buf(workspace, "workspace", ws_bytes, torch.uint8, dev)
    g = out if out is not None else {
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
        "dalpha": torch.empty_like(alpha), "dbeta": torch.empty_like(beta),
        "dqn": torch.empty_like(qn), "dkn": torch.empty_like(kn), "dvn": torch.empty_like(vn),
        "dalpha_n": torch.empty_like(alpha_n), "dbeta_n": torch.empty_like(beta_n),
        "dh0": torch.empty((N, H, d, d), dtype=torch.float32, device=dev) if want_dh0 else None,
    }
    for name in ("dq", "dk", "dv", "dqn", "dkn", "dvn"):
        _chk(g.get(name), name, (T, H, d), iot, dev)
    for name in ("dalpha", "dbeta", "dalpha_n", "dbeta_n"):
        _chk(g.get(name), name, (T, H), torch.float32, dev)
    _chk(g.get("dh0"), "dh0", (N, H, d, d), torch.float32, dev, optional=True)
    _check(lib().flare_gdn_dual_bwd(
        varlen.ref(), ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(qn), _ptr(kn), _ptr(vn), _ptr(alpha_n), _ptr(beta_n), _ptr(h0), _ptr(ckpt), int(ckpt_stride),
        _ptr(fwd_workspace), _ptr(d_o), _ptr(d_on), _ptr(dh_final), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
        _ptr(g["dalpha"]), _ptr(g["dbeta"]), _ptr(g["dqn"]), _ptr(g["dkn"]), _ptr(g["dvn"]),
        _ptr(g["dalpha_n"]), _ptr(g["dbeta_n"]), _ptr(g["dh0"]), _ptr(workspace),
        ws_bytes, _stream(dev)))
    return g


def block_step(slot_idx, pool, q, k, v, alpha, beta, mode, scale=0.0, slot_idx_host=None, o=None):
    """Serving EVAL / COMMIT.  slot_idx [R] int32 (device); pool [n_slots,H,d,d] fp32;
    q,k,v [R,B,H,d]; gates [R,B,H].  Returns o [R,B,H,d] (None for COMMIT when
    o is not wanted: pass o=False)."""
    torch = _torch()
    R, B, H, d, dev = _chk_step_inputs(slot_idx, pool, q, k, v, alpha, beta)
    shp = _shape(H, d, B, _io_of(q), 0, scale)
    if o is None:
        o = torch.empty((R, B, H, d), dtype=q.dtype, device=q.device)
    elif o is False:
        o = None
    _chk_rows(o, "o", (R, B), H, d, q.dtype, dev, optional=True)
    host = None
    if slot_idx_host is not None:
        host = np.ascontiguousarray(np.asarray(slot_idx_host, dtype=np.int32))
    _check(lib().flare_gdn_block_step(R, _ptr(slot_idx), None if host is None else host.ctypes.data,
                                      _ptr(pool), pool.shape[0], ctypes.byref(shp), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), int(mode),
                                      _stream(q.device)))
    return o


def block_step_conv(slot_idx, pool, cache, weights, xq, xk, xv, alpha, beta, mode, activation=0, qk_l2norm=True,
                    scale=0.0, slot_idx_host=None, o=None):
    """The serving step with the ShortConv in front: xq, xk, xv [R,B,H,d] raw
    projections; cache [n_slots, W-1, 3, H*d] io clean histories (None for
    W = 1); weights: three [H*d, W] fp32.  Returns o [R,B,H,d]."""
    torch = _torch()
    R, B, H, d, dev = _chk_step_inputs(slot_idx, pool, xq, xk, xv, alpha, beta)
    if weights is None or len(weights) != 3 or weights[0] is None or weights[0].dim() != 2:
        _fail("weights must be three [H*d, W] fp32 tensors")
    W = weights[0].shape[1]
    for i, w in enumerate(weights):
        _chk(w, "weights[%d]" % i, (H * d, W), torch.float32, dev)
    if W > 1:
        _chk(cache, "cache", (pool.shape[0], W - 1, 3, H * d), xq.dtype, dev)
    shp = _shape(H, d, B, _io_of(xq), 0, scale)
    if o is None:
        o = torch.empty((R, B, H, d), dtype=xq.dtype, device=xq.device)
    elif o is False:
        o = None
    _chk_rows(o, "o", (R, B), H, d, xq.dtype, dev, optional=True)
    host = None
    if slot_idx_host is not None:
        host = np.ascontiguousarray(np.asarray(slot_idx_host, dtype=np.int32))
    _check(lib().flare_gdn_block_step_conv(R, _ptr(slot_idx), None if host is None else host.ctypes.data,
                                           _ptr(pool), _ptr(cache), pool.shape[0], ctypes.byref(shp), W,
                                           _a3(weights), int(activation), 1 if qk_l2norm else 0, _ptr(xq),
                                           _ptr(xk), _ptr(xv), _ptr(alpha), _ptr(beta), _ptr(o), int(mode),
                                           _stream(xq.device)))
    return o


def conv_cache_fill(varlen: Varlen, head_dim, width, xs, doc_slot, cache, doc_slot_host=None):
    """Each document's clean history (its last W-1 projection rows, zero
    before its start) into cache[doc_slot[i]]; xs: three [T, H*d] io."""
    torch = _torch()
    if xs is None or len(xs) != 3 or xs[0] is None or xs[0].dim() != 2:
        _fail("xs must be three [T, H*d] io tensors")
    dev = _gpu_device(xs[0], "xs[0]")
    T, C = xs[0].shape
    _chk_varlen(varlen, T, dev)
    for i, x in enumerate(xs):
        _chk(x, "xs[%d]" % i, (T, C), _io_dtype_of(xs[0], "xs[0]"), dev)
    _chk(doc_slot, "doc_slot", (varlen.num_docs,), torch.int32, dev)
    if int(width) > 1:
        if cache is None or cache.dim() != 4:
            _fail("cache must be [n_slots, W-1, 3, H*d]")
        _chk(cache, "cache", (cache.shape[0], int(width) - 1, 3, C), xs[0].dtype, dev)
    host = None
    if doc_slot_host is not None:
        host = np.ascontiguousarray(np.asarray(doc_slot_host, dtype=np.int32))
    _check(lib().flare_conv_cache_fill(varlen.ref(), C // int(head_dim), int(head_dim), int(width), _io_of(xs[0]),
                                       _a3(xs), _ptr(doc_slot), None if host is None else host.ctypes.data,
                                       _ptr(cache), cache.shape[0] if cache is not None else 0,
                                       _stream(xs[0].device)))
    return cache


def gdn_verify(slot_idx, pool, q, k, v, alpha, beta, scale=0.0, slot_idx_host=None, o=None, cand=None):
    """AR-Trust verify of K drafted tokens per request (q,k,v [R,K,H,d];
    gates [R,K,H]) from the pool states (read only).  Returns (o [R,K,H,d],
    cand [R,K,H,d,d] fp32: the state after every token)."""
    torch = _torch()
    R, K, H, d, dev = _chk_step_inputs(slot_idx, pool, q, k, v, alpha, beta)
    shp = _shape(H, d, K, _io_of(q), 0, scale)
    if o is None:
        o = torch.empty((R, K, H, d), dtype=q.dtype, device=q.device)
    if cand is None:
        cand = torch.empty((R, K, H, d, d), dtype=torch.float32, device=q.device)
    _chk_rows(o, "o", (R, K), H, d, q.dtype, dev)
    _chk(cand, "cand", (R, K, H, d, d), torch.float32, dev)
    host = None
    if slot_idx_host is not None:
        host = np.ascontiguousarray(np.asarray(slot_idx_host, dtype=np.int32))
    _check(lib().flare_gdn_verify(R, _ptr(slot_idx), None if host is None else host.ctypes.data, _ptr(pool),
                                  pool.shape[0], ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                  _ptr(beta), _ptr(o), _ptr(cand), _stream(q.device)))
    return o, cand


def gdn_scatter(slot_idx, accepted, cand, pool, slot_idx_host=None):
    """AR-Trust rollback: pool[slot_idx[r]] = cand[r, accepted[r] - 1] for the
    device int32 counts accepted [R], clamped to [0, K] (0 leaves the slot)."""
    torch = _torch()
    dev = _gpu_device(cand, "cand")
    if cand.dim() != 5:
        _fail("cand must be [R, K, H, d, d]")
    R, K, H, d, _ = cand.shape
    _chk(cand, "cand", (R, K, H, d, d), torch.float32, dev)
    _chk(accepted, "accepted", (R,), torch.int32, dev)
    _chk(slot_idx, "slot_idx", (R,), torch.int32, dev)
    _chk_pool(pool, H, d, dev)
    shp = _shape(H, d, K, BF16, 0, 0.0)
    host = None
    if slot_idx_host is not None:
        host = np.ascontiguousarray(np.asarray(slot_idx_host, dtype=np.int32))
    _check(lib().flare_gdn_scatter(R, _ptr(slot_idx), None if host is None else host.ctypes.data, _ptr(accepted),
                                   _ptr(cand), _ptr(pool), pool.shape[0], ctypes.byref(shp), _stream(cand.device)))
    return pool


def gdn_verify_outputs(slot_idx, pool, q, k, v, alpha, beta, scale=0.0, slot_idx_host=None, o=None):
    """The causal outputs of gdn_verify without the candidate states (pool
    read only).  Returns o [R,K,H,d]."""
    torch = _torch()
    R, K, H, d, dev = _chk_step_inputs(slot_idx, pool, q, k, v, alpha, beta)
    shp = _shape(H, d, K, _io_of(q), 0, scale)
    if o is None:
        o = torch.empty((R, K, H, d), dtype=q.dtype, device=q.device)
    _chk_rows(o, "o", (R, K), H, d, q.dtype, dev)
    host = None
    if slot_idx_host is not None:
        host = np.ascontiguousarray(np.asarray(slot_idx_host, dtype=np.int32))
    _check(lib().flare_gdn_verify_outputs(R, _ptr(slot_idx), None if host is None else host.ctypes.data, _ptr(pool),
                                          pool.shape[0], ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                          _ptr(beta), _ptr(o), _stream(q.device)))
    return o


def gdn_commit_prefix(slot_idx, pool, q, k, v, alpha, beta, accepted, scale=0.0, slot_idx_host=None, o=None):
    """COMMIT of each request's first accepted[r] drafted tokens (device int32,
    clamped to [0, K]) into its pool slot, in place; 0 leaves the slot.
    o (optional) receives the causal outputs of the replayed tokens."""
    torch = _torch()
    R, K, H, d, dev = _chk_step_inputs(slot_idx, pool, q, k, v, alpha, beta)
    _chk(accepted, "accepted", (R,), torch.int32, dev)
    _chk_rows(o, "o", (R, K), H, d, q.dtype, dev, optional=True)
    shp = _shape(H, d, K, _io_of(q), 0, scale)
    host = None
    if slot_idx_host is not None:
        host = np.ascontiguousarray(np.asarray(slot_idx_host, dtype=np.int32))
    _check(lib().flare_gdn_commit_prefix(R, _ptr(slot_idx), None if host is None else host.ctypes.data, _ptr(pool),
                                         pool.shape[0], ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                         _ptr(beta), _ptr(accepted), _ptr(o), _stream(q.device)))
    return pool


def shortconv_dual(varlen: Varlen, block_size, x, xn, weight, bias=None, activation=0, out=None):
    """x, xn [T,C] io; weight [C,W] fp32; bias [C] fp32 or None.  Returns (y, yn)."""
    torch = _torch()
    T, C, W, dev = _chk_conv_inputs(varlen, x, xn, weight, bias)
    if out is None:
        y, yn = torch.empty_like(x), torch.empty_like(x)
    else:
        y, yn = out
        _chk(y, "y", (T, C), x.dtype, dev)
        _chk(yn, "yn", (T, C), x.dtype, dev)
    _check(lib().flare_shortconv_dual(varlen.ref(), int(block_size), C, W, _io_of(x), _ptr(x), _ptr(xn),
                                      _ptr(weight), _ptr(bias), int(activation), _ptr(y), _ptr(yn),
                                      _stream(x.device)))
    return y, yn


def shortconv_dual_bwd_workspace_bytes(varlen: Varlen, block_size, channels, width) -> int:
    """flare_shortconv_dual_bwd_workspace_size for this batch and shape."""
    return int(lib().flare_shortconv_dual_bwd_workspace_size(varlen.ref(), int(block_size), int(channels),
                                                             int(width)))


def shortconv_dual_bwd(varlen: Varlen, block_size, x, xn, weight, dy, dyn, bias=None, activation=0,
                       workspace=None, out=None, want_dbias=True):
    """Reverse mode of shortconv_dual.  Returns (dx, dxn, dweight, dbias);
    dbias is None when want_dbias is False."""
    torch = _torch()
    T, C, W, dev = _chk_conv_inputs(varlen, x, xn, weight, bias)
    _chk(dy, "dy", (T, C), x.dtype, dev)
    _chk(dyn, "dyn", (T, C), x.dtype, dev)
    if out is None:
        dx, dxn = torch.empty_like(x), torch.empty_like(x)
        dw = torch.empty((C, W), dtype=torch.float32, device=x.device)
        db = torch.empty((C,), dtype=torch.float32, device=x.device) if want_dbias else None
    else:
        dx, dxn, dw, db = out
    _chk(dx, "dx", (T, C), x.dtype, dev)
    _chk(dxn, "dxn", (T, C), x.dtype, dev)
    _chk(dw, "dweight", (C, W), torch.float32, dev)
    _chk(db, "dbias", (C,), torch.float32, dev, optional=True)
    need = shortconv_dual_bwd_workspace_bytes(varlen, block_size, C, W)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    _chk_buf(workspace, "workspace", need, torch.uint8, dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().flare_shortconv_dual_bwd(varlen.ref(), int(block_size), C, W, _io_of(x), _ptr(x), _ptr(xn),
                                          _ptr(weight), _ptr(bias), int(activation), _ptr(dy), _ptr(dyn),
                                          _ptr(dx), _ptr(dxn), _ptr(dw), _ptr(db), _ptr(workspace), nbytes,
                                          _stream(x.device)))
    return dx, dxn, dw, db


def _a3(ts):
    return (ctypes.c_void_p * 3)(*[_ptr(t) for t in ts])


def qkv_prologue(varlen: Varlen, block_size, head_dim, xs, xns, weights, activation=0, qk_l2norm=True, out=None):
    """The GDN layer's fused input prologue: ShortConv on the clean and noisy
    q, k, v projections (xs, xns: three [T, H*head_dim] io tensors each;
    weights: three [H*head_dim, W] fp32), optional SiLU, per-head L2 norm of
    q and k.  Returns (ys, yns), lists of three tensors shaped like xs."""
    torch = _torch()
    T, C, W, dev = _chk_prologue_inputs(varlen, xs, xns, weights)
    if out is None:
        ys, yns = [torch.empty_like(x) for x in xs], [torch.empty_like(x) for x in xs]
    else:
        ys, yns = out
    _chk_three(ys, "ys", (T, C), xs[0].dtype, dev)
    _chk_three(yns, "yns", (T, C), xs[0].dtype, dev)
    _check(lib().flare_qkv_prologue(varlen.ref(), int(block_size), C // int(head_dim), int(head_dim), W,
                                    _io_of(xs[0]), _a3(xs), _a3(xns), _a3(weights), int(activation),
                                    1 if qk_l2norm else 0, _a3(ys), _a3(yns), _stream(xs[0].device)))
    return ys, yns


def qkv_prologue_bwd_workspace_bytes(varlen: Varlen, block_size, heads, head_dim, width) -> int:
    """flare_qkv_prologue_bwd_workspace_size for this batch and shape."""
    return int(lib().flare_qkv_prologue_bwd_workspace_size(varlen.ref(), int(block_size), int(heads),
                                                           int(head_dim), int(width)))


def qkv_prologue_bwd(varlen: Varlen, block_size, head_dim, xs, xns, weights, dys, dyns, activation=0,
                     qk_l2norm=True, workspace=None, out=None):
    """Reverse mode of qkv_prologue.  Returns (dxs, dxns, dws), lists of three."""
    torch = _torch()
    T, C, W, dev = _chk_prologue_inputs(varlen, xs, xns, weights)
    io = xs[0].dtype
    _chk_three(dys, "dys", (T, C), io, dev)
    _chk_three(dyns, "dyns", (T, C), io, dev)
    H = C // int(head_dim)
    if out is None:
        dxs, dxns = [torch.empty_like(x) for x in xs], [torch.empty_like(x) for x in xs]
        dws = [torch.empty((C, W), dtype=torch.float32, device=xs[0].device) for _ in range(3)]
    else:
        dxs, dxns, dws = out
    _chk_three(dxs, "dxs", (T, C), io, dev)
    _chk_three(dxns, "dxns", (T, C), io, dev)
    _chk_three(dws, "dws", (C, W), torch.float32, dev)
    need = qkv_prologue_bwd_workspace_bytes(varlen, block_size, H, head_dim, W)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=xs[0].device)
    _chk_buf(workspace, "workspace", need, torch.uint8, dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().flare_qkv_prologue_bwd(varlen.ref(), int(block_size), H, int(head_dim), W, _io_of(xs[0]),
                                        _a3(xs), _a3(xns), _a3(weights), int(activation), 1 if qk_l2norm else 0,
                                        _a3(dys), _a3(dyns), _a3(dxs), _a3(dxns), _a3(dws), _ptr(workspace),
                                        nbytes, _stream(xs[0].device)))
    return dxs, dxns, dws


def qkv_prologue_bwd_noalloc(varlen: Varlen, block_size, head_dim, xs, xns, weights, dys, dyns, out,
                             activation=0, qk_l2norm=True):
    """qkv_prologue_bwd with the weight-gradient partials in the library's
    static device scratch (flare_qkv_prologue_bwd_noalloc): the library
    allocates nothing, so the caller passes every output buffer, out =
    (dxs, dxns, dws).  Returns out."""
    torch = _torch()
    T, C, W, dev = _chk_prologue_inputs(varlen, xs, xns, weights)
    io = xs[0].dtype
    _chk_three(dys, "dys", (T, C), io, dev)
    _chk_three(dyns, "dyns", (T, C), io, dev)
    if out is None or len(out) != 3:
        _fail("out must be (dxs, dxns, dws)", 1)
    dxs, dxns, dws = out
    _chk_three(dxs, "dxs", (T, C), io, dev)
    _chk_three(dxns, "dxns", (T, C), io, dev)
    _chk_three(dws, "dws", (C, W), torch.float32, dev)
    H = C // int(head_dim)
    _check(lib().flare_qkv_prologue_bwd_noalloc(varlen.ref(), int(block_size), H, int(head_dim), W, _io_of(xs[0]),
                                                _a3(xs), _a3(xns), _a3(weights), int(activation),
                                                1 if qk_l2norm else 0, _a3(dys), _a3(dyns), _a3(dxs), _a3(dxns),
                                                _a3(dws), _stream(xs[0].device)))
    return out


def noalloc_scratch_bytes() -> int:
    """Bytes of the static device scratch behind qkv_prologue_bwd_noalloc."""
    return int(lib().flare_noalloc_scratch_bytes())


def workspace_bytes(varlen: Varlen, H: int, d: int, block_size: int, io: int, flags: int = 0,
                    for_bwd: bool = False, stride: int = 1, window: int = 0) -> int:
    """flare_gdn_dual_workspace_size for this batch and shape (one pass,
    stride-1 checkpoints), or flare_gdn_dual_workspace_size_window for a
    checkpoint stride and a window of chunks."""
    return _ws_bytes(varlen, _shape(H, d, block_size, io, flags), for_bwd, stride, window)


def timing_enable(on: bool = True) -> bool:
    """Bracket every kernel launch of the library with HIP events on its
    stream (flare_timing_enable); returns the previous state."""
    return bool(lib().flare_timing_enable(1 if on else 0))


def timing_avg_ms(kernel: str):
    """(mean duration in ms, launches) of the recorded launches of `kernel`
    (flare_timing_avg_ms); waits for them to finish."""
    n = ctypes.c_int64(0)
    ms = lib().flare_timing_avg_ms(kernel.encode(), ctypes.byref(n))
    return (ms if n.value > 0 else None), n.value


def timing_reset() -> None:
    lib().flare_timing_reset()
