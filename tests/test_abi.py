"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, and its host-side validation returns the documented status
before anything is launched.  Device pointers here are dummies; every call is
built so that validation fails (or the call is a pure size query), so nothing
is ever dereferenced or launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import gated_deltanet_dual_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flare_gdn.h")
FAKE = ctypes.c_void_p(0x7F0000001000)  # never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(g.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return g.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(flare_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"flare_gdn_dual_fwd", "flare_gdn_dual_bwd", "flare_gdn_block_step",
            "flare_shortconv_dual"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_constants(L):
    assert L.flare_gdn_chunk_size() == 32
    assert L.flare_version() >= 100


def varlen(cu, pl, dev=True):
    cu = np.ascontiguousarray(np.asarray(cu, np.int32))
    pl = np.ascontiguousarray(np.asarray(pl, np.int32))
    v = g._Varlen(len(pl), FAKE.value if dev else None, cu.ctypes.data,
                  FAKE.value if dev else None, pl.ctypes.data)
    v._keep = (cu, pl)
    return v


def fwd_status(L, v, shape, ckpt=None, stride=1, null_q=False):
    P = [None if null_q else FAKE] + [FAKE] * 9
    return L.flare_gdn_dual_fwd(ctypes.byref(v), ctypes.byref(shape), *P, None, FAKE, FAKE, None,
                                ckpt, stride, None, 0, None)


def test_fwd_validation(L):
    ok_shape = g.GDNShape(16, 128, 128, 4, g.BF16, 0, 0.0)
    # cu_seqlens must start at 0
    assert fwd_status(L, varlen([1, 9], [0]), ok_shape) == 2
    # decreasing cu_seqlens
    assert fwd_status(L, varlen([0, 9, 5], [0, 0]), ok_shape) == 2
    # prompt longer than the document
    assert fwd_status(L, varlen([0, 8], [12]), ok_shape) == 2
    # prompt not a multiple of the block size
    assert fwd_status(L, varlen([0, 16], [6]), ok_shape) == 3
    # NULL input with tokens present
    assert fwd_status(L, varlen([0, 16], [8]), ok_shape, null_q=True) == 1
    # unsupported head dim / unequal dk, dv / block size / dtype / flags
    for bad in [g.GDNShape(16, 64, 64, 4, g.BF16, 0, 0.0), g.GDNShape(16, 128, 16, 4, g.BF16, 0, 0.0),
                g.GDNShape(16, 128, 128, 3, g.BF16, 0, 0.0), g.GDNShape(16, 128, 128, 64, g.BF16, 0, 0.0),
                g.GDNShape(16, 128, 128, 4, 7, 0, 0.0), g.GDNShape(16, 128, 128, 4, g.BF16, 4, 0.0),
                g.GDNShape(16, 128, 128, 4, g.F32, 0, 0.0)]:
        assert fwd_status(L, varlen([0, 16], [8]), bad) == 4
    assert fwd_status(L, varlen([0, 16], [8]), g.GDNShape(0, 128, 128, 4, g.BF16, 0, 0.0)) == 2
    # checkpoint stride below 1
    assert fwd_status(L, varlen([0, 16], [8]), ok_shape, ckpt=FAKE, stride=0) == 2
    # missing host copies
    v = g._Varlen(1, FAKE.value, None, FAKE.value, None)
    assert fwd_status(L, v, ok_shape) == 1
    assert b"cu_seqlens" in L.flare_last_error()


def test_fwd_workspace_checked_before_launch(L):
    shape = g.GDNShape(4, 128, 128, 4, g.BF16, 0, 0.0)
    v = varlen([0, 100, 164], [20, 0])
    need = L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(shape), 0)
    # per chunk slot and head (fp32 words): six 32 x 32 chunk matrices, the
    # pre-pass's hand-over to the scan (R 128 x 128 fp32, W 32 x 32 as hi and
    # lo bf16, K twice as 32 x 128 bf16, the decay padded to 64 words), and a
    # 128 x 128 chunk-start state
    pack = 128 * 128 + 2 * 32 * 32 // 2 + 2 * (32 * 128 // 2) + 64
    assert need == (164 // 32 + 2) * 4 * (6 * 32 * 32 + pack + 128 * 128) * 4 + 256
    P = [FAKE] * 10
    # a smaller workspace runs in windows of chunks; below one chunk's window it is refused
    w1 = L.flare_gdn_dual_workspace_size_window(ctypes.byref(v), ctypes.byref(shape), 0, 1, 1)
    assert 0 < w1 < need
    st = L.flare_gdn_dual_fwd(ctypes.byref(v), ctypes.byref(shape), *P, None, FAKE, FAKE, None, None, 1,
                              FAKE, w1 - 1, None)
    assert st == 5
    st = L.flare_gdn_dual_fwd(ctypes.byref(v), ctypes.byref(shape), *P, None, FAKE, FAKE, None, None, 1,
                              None, 0, None)
    assert st == 5
    # configurations served by the fused kernel need none
    other = g.GDNShape(4, 16, 16, 4, g.BF16, 0, 0.0)
    assert L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(other), 0) == 0
    # the q/k L2 flag adds the per-(token, head) factors (four fp32) after the
    # per-slot part, which starts the region on a 256-byte boundary
    l2 = g.GDNShape(4, 128, 128, 4, g.BF16, 1, 0.0)
    base = need - 256
    assert L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(l2), 0) == \
        (base + 255) // 256 * 256 + 164 * 4 * 16 + 256


def test_bwd_workspace_checked_before_launch(L):
    shape = g.GDNShape(2, 16, 16, 4, g.F32, 0, 0.0)
    v = varlen([0, 40, 64], [8, 0])
    need = L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(shape), 1)
    # per chunk slot ((T/32 + N) slots) and head, fp32: the end-state adjoint
    # (d x d) and six 32 x 32 chunk matrices
    assert need == (64 // 32 + 2) * 2 * (16 * 16 + 6 * 32 * 32) * 4 + 256
    args = [FAKE] * 10 + [None, FAKE, 1, None, FAKE, FAKE, None] + [FAKE] * 10 + [None]
    st = L.flare_gdn_dual_bwd(ctypes.byref(v), ctypes.byref(shape), *args, FAKE, need - 1, None)
    assert st == 5
    mis = ctypes.c_void_p(FAKE.value + 4)
    st = L.flare_gdn_dual_bwd(ctypes.byref(v), ctypes.byref(shape), *args, mis, need + 64, None)
    assert st == 5
    # bf16 io at d = 128 adds the pre-pass's hand-over to the reverse scan:
    # (fp32 words): R (128 x 128 fp32), W (32 x 32 as hi and lo bf16), K twice
    # (32 x 128 bf16 each), the chunk decay padded to 64 words
    big = g.GDNShape(2, 128, 128, 4, g.BF16, 0, 0.0)
    need = L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(big), 1)
    pack = 128 * 128 + 2 * 32 * 32 // 2 + 2 * (32 * 128 // 2) + 64
    assert need == (64 // 32 + 2) * 2 * (128 * 128 + 6 * 32 * 32 + pack) * 4 + 256


def test_ckpt_slots_never_overlap(L):
    rng = np.random.default_rng(0)
    C = 32
    for trial in range(20):
        lens = rng.integers(0, 300, size=rng.integers(1, 12))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        used = set()
        for i, n in enumerate(lens):
            for c in range((n + C - 1) // C):
                s = L.flare_gdn_ckpt_slot(int(cu[i]), i, c, 1)
                assert s == cu[i] // C + i + c
                assert s not in used
                used.add(s)
        v = varlen(cu, [0] * len(lens))
        shape = g.GDNShape(3, 16, 16, 4, g.F32, 0, 0.0)
        nbytes = L.flare_gdn_dual_ckpt_size(ctypes.byref(v), ctypes.byref(shape), 1)
        n_slots = nbytes // (3 * 16 * 16 * 4)
        assert n_slots == cu[-1] // C + len(lens)
        assert not used or max(used) < n_slots


def test_block_step_validation(L):
    shape = g.GDNShape(16, 128, 128, 4, g.BF16, 0, 0.0)
    host = np.array([3, 1, 3], np.int32)
    P = [FAKE] * 5
    st = L.flare_gdn_block_step(3, FAKE, host.ctypes.data, FAKE, 8, ctypes.byref(shape), *P, FAKE, 0, None)
    assert st == 2 and b"two requests" in L.flare_last_error()
    host = np.array([3, 1, 9], np.int32)
    st = L.flare_gdn_block_step(3, FAKE, host.ctypes.data, FAKE, 8, ctypes.byref(shape), *P, FAKE, 0, None)
    assert st == 2
    st = L.flare_gdn_block_step(3, FAKE, None, FAKE, 8, ctypes.byref(shape), *P, None, 0, None)
    assert st == 1  # EVAL without an output
    st = L.flare_gdn_block_step(3, FAKE, None, FAKE, 8, ctypes.byref(shape), *P, FAKE, 5, None)
    assert st == 2  # unknown mode
    st = L.flare_gdn_block_step(9, FAKE, None, FAKE, 8, ctypes.byref(shape), *P, FAKE, 0, None)
    assert st == 2  # more requests than slots
    assert L.flare_gdn_block_step(0, None, None, None, 0, ctypes.byref(shape), *([None] * 6), 0, None) == 0


def test_shortconv_validation(L):
    v = varlen([0, 16], [4])
    P = [FAKE, FAKE, FAKE, None]
    assert L.flare_shortconv_dual(ctypes.byref(v), 4, 12, 4, g.BF16, *P, 0, FAKE, FAKE, None) == 3
    assert L.flare_shortconv_dual(ctypes.byref(v), 4, 16, 9, g.BF16, *P, 0, FAKE, FAKE, None) == 4
    assert L.flare_shortconv_dual(ctypes.byref(v), 4, 16, 4, g.BF16, *P, 2, FAKE, FAKE, None) == 4
    assert L.flare_shortconv_dual(ctypes.byref(varlen([0, 16], [6])), 4, 16, 4, g.BF16, *P, 0, FAKE,
                                  FAKE, None) == 3
    assert L.flare_shortconv_dual(ctypes.byref(v), 4, 16, 4, g.BF16, None, FAKE, FAKE, None, 0, FAKE,
                                  FAKE, None) == 1


def test_shortconv_bwd_workspace_and_validation(L):
    cu, pl = [0, 37, 37, 100], [8, 0, 4]
    v = varlen(cu, pl)
    blocks = (100 + 255) // 256  # weight-gradient partials per 256-token block
    for C, W in ((16, 4), (48, 1), (64, 8)):
        assert L.flare_shortconv_dual_bwd_workspace_size(ctypes.byref(v), 4, C, W) == blocks * C * (W + 1) * 4 + 256
    v2 = varlen([0, 300, 600], [0, 0])
    assert L.flare_shortconv_dual_bwd_workspace_size(ctypes.byref(v2), 4, 16, 4) == 3 * 16 * 5 * 4 + 256
    assert L.flare_shortconv_dual_bwd_workspace_size(ctypes.byref(v), 4, 16, 9) == 0
    assert L.flare_shortconv_dual_bwd_workspace_size(ctypes.byref(v), 4, 0, 4) == 0
    need = L.flare_shortconv_dual_bwd_workspace_size(ctypes.byref(v), 4, 16, 4)
    ok = [FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None]

    def call(C=16, W=4, io=g.BF16, args=ok, ws=FAKE, nbytes=need):
        return L.flare_shortconv_dual_bwd(ctypes.byref(v), 4, C, W, io, *args, ws, nbytes, None)

    assert call(C=12) == 3                                   # bf16 needs channels % 8
    assert call(W=9) == 4
    assert call(io=7) == 4
    bad = list(ok); bad[4] = 2
    assert call(args=bad) == 4                               # unknown activation
    bad = list(ok); bad[5] = None
    assert call(args=bad) == 1                               # dy NULL
    bad = list(ok); bad[9] = None
    assert call(args=bad) == 1                               # dweight NULL
    assert call(nbytes=need - 1) == 5
    assert call(ws=None) == 5
    assert call(ws=ctypes.c_void_p(FAKE.value + 16)) == 5    # misaligned
    assert L.flare_shortconv_dual_bwd(ctypes.byref(varlen([0, 16], [6])), 4, 16, 4, g.BF16, *ok, FAKE, need,
                                      None) == 3


def test_qkv_prologue_validation(L):
    v = varlen([0, 300, 600], [0, 0])
    A3 = ctypes.c_void_p * 3
    P3 = A3(FAKE, FAKE, FAKE)
    # three sections of partials
    assert L.flare_qkv_prologue_bwd_workspace_size(ctypes.byref(v), 4, 4, 32, 4) == 3 * 3 * 128 * 5 * 4 + 256
    assert L.flare_qkv_prologue_bwd_workspace_size(ctypes.byref(v), 4, 0, 32, 4) == 0

    def fwd(H=4, d=32, W=4, io=g.BF16, l2=1, x=P3, y=P3):
        return L.flare_qkv_prologue(ctypes.byref(v), 4, H, d, W, io, x, P3, P3, 0, l2, y, P3, None)

    assert fwd(H=3, d=12) == 3            # bf16 channels (36) must be a multiple of 8
    assert fwd(d=8 * 68) == 4             # 136 lanes per head: too wide for the in-wave L2 sum
    assert fwd(d=24) == 4                 # 6 lanes per head: not a power of two
    assert fwd(l2=2) == 4
    assert fwd(x=A3(FAKE, None, FAKE)) == 1
    assert fwd(y=A3(FAKE, FAKE, None)) == 1
    # without the L2 step the head size is free
    assert fwd(d=24, l2=0, x=A3(FAKE, None, FAKE)) == 1


def test_verify_scatter_validation(L):
    shape = g._shape(2, 16, 4, g.F32)
    host = np.array([3, 1], np.int32)
    args = [FAKE] * 5
    # verify: the COMMIT checks plus required outputs and candidates
    assert L.flare_gdn_verify(2, FAKE, host.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, FAKE, None, None) == 1
    assert L.flare_gdn_verify(2, FAKE, host.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, None, FAKE, None) == 1
    dup = np.array([3, 3], np.int32)
    assert L.flare_gdn_verify(2, FAKE, dup.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, FAKE, FAKE, None) == 2
    assert L.flare_gdn_verify(0, None, None, None, 0, ctypes.byref(shape), *([None] * 7), None) == 0
    # scatter
    assert L.flare_gdn_scatter(2, FAKE, host.ctypes.data, None, FAKE, FAKE, 8, ctypes.byref(shape), None) == 1
    assert L.flare_gdn_scatter(2, FAKE, dup.ctypes.data, FAKE, FAKE, FAKE, 8, ctypes.byref(shape), None) == 2
    assert L.flare_gdn_scatter(9, FAKE, None, FAKE, FAKE, FAKE, 8, ctypes.byref(shape), None) == 2
    assert L.flare_gdn_scatter(0, None, None, None, None, None, 0, ctypes.byref(shape), None) == 0
    # the replay pair: outputs required for the read, counts for the commit
    assert L.flare_gdn_verify_outputs(2, FAKE, host.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, None,
                                      None) == 1
    assert L.flare_gdn_verify_outputs(2, FAKE, dup.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, FAKE,
                                      None) == 2
    assert L.flare_gdn_commit_prefix(2, FAKE, host.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, None, None,
                                     None) == 1
    assert L.flare_gdn_commit_prefix(2, FAKE, dup.ctypes.data, FAKE, 8, ctypes.byref(shape), *args, FAKE, None,
                                     None) == 2
    assert L.flare_gdn_commit_prefix(0, None, None, None, 0, ctypes.byref(shape), *([None] * 5), None, None,
                                     None) == 0


def test_fwd_pool_validation(L):
    v = varlen([0, 40, 80], [8, 8])
    shape = g._shape(1, 16, 4, g.F32)
    P10 = [FAKE] * 10
    host = np.array([1, 3], np.int32)
    dup = np.array([3, 3], np.int32)

    def call(slot=FAKE, slot_host=host, pool=FAKE, n_slots=4, read=1):
        return L.flare_gdn_dual_fwd_pool(ctypes.byref(v), ctypes.byref(shape), *P10, slot,
                                         None if slot_host is None else slot_host.ctypes.data, pool, n_slots, read,
                                         FAKE, FAKE, None, 1, FAKE, 1 << 20, None)

    assert call(slot=None) == 1
    assert call(pool=None) == 1
    assert call(slot_host=dup) == 2
    assert call(n_slots=1) == 2          # two documents, one slot
    assert call(read=2) == 2
    assert call(slot_host=np.array([1, 4], np.int32)) == 2  # slot out of range


def test_block_step_conv_and_cache_fill_validation(L):
    A3 = ctypes.c_void_p * 3
    W3 = A3(FAKE, FAKE, FAKE)
    host = np.array([3, 1], np.int32)

    def step(B=4, width=4, flags=0, act=0, l2=1, cache=FAKE, w=W3):
        shape = g._shape(2, 16, B, g.F32, flags)
        return L.flare_gdn_block_step_conv(2, FAKE, host.ctypes.data, FAKE, cache, 8, ctypes.byref(shape), width, w,
                                           act, l2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)

    assert step(B=16) == 4               # blocks of up to 8 tokens with the conv
    assert step(width=9) == 4
    assert step(flags=1) == 4            # the L2 step is its own argument
    assert step(act=3) == 4
    assert step(l2=2) == 4
    assert step(cache=None) == 1         # a history is needed for width > 1
    assert step(w=A3(FAKE, None, FAKE)) == 1
    v = varlen([0, 10, 30], [4, 8])
    dup = np.array([2, 2], np.int32)
    fill = lambda **k: L.flare_conv_cache_fill(ctypes.byref(v), k.get("H", 2), 16, k.get("W", 4), g.BF16, W3, FAKE,
                                               k.get("host", host).ctypes.data, FAKE, k.get("slots", 8), None)
    assert fill(host=dup) == 2
    assert fill(slots=1) == 2
    assert fill(W=0) == 4
    assert L.flare_conv_cache_fill(ctypes.byref(v), 2, 16, 1, g.BF16, W3, FAKE, None, None, 8, None) == 0  # W = 1


def test_route1_workspace_and_validation(L):
    # documents of 40 and 80 tokens with prompts 8 and 8, blocks of 4: 8 + 18
    # response blocks; the size covers the forward's workspace, one fp32 state
    # per block and the per-document / per-block tables
    v = varlen([0, 40, 120], [8, 8])
    shape = g._shape(2, 16, 4, g.F32)
    need = L.flare_gdn_route1_workspace_size(ctypes.byref(v), ctypes.byref(shape))
    fwd = L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(shape), 0)
    r = lambda x: (x + 255) // 256 * 256
    assert need == r(fwd) + r(26 * 2 * 16 * 16 * 4) + r((2 * 2 + 5 * 26) * 4) + 256
    # no response tokens: no block states
    v0 = varlen([0, 40], [40])
    need0 = L.flare_gdn_route1_workspace_size(ctypes.byref(v0), ctypes.byref(shape))
    assert need0 == r(L.flare_gdn_dual_workspace_size(ctypes.byref(v0), ctypes.byref(shape), 0)) + r(3 * 4) + 256
    # unsupported shapes report 0 and fail the call
    odd = g._shape(2, 16, 4, g.F32, g.QK_L2NORM)
    assert L.flare_gdn_route1_workspace_size(ctypes.byref(v), ctypes.byref(odd)) == 0
    P10 = [FAKE] * 10

    def call(shp=shape, ckpt=FAKE, ws=FAKE, nbytes=need):
        return L.flare_gdn_dual_fwd_route1(ctypes.byref(v), ctypes.byref(shp), *P10, None, FAKE, FAKE, None, ckpt,
                                           ws, nbytes, None)

    assert call(ckpt=None) == 1             # the chunk-start states are required
    assert call(nbytes=need - 1) == 5
    assert call(ws=None) == 5
    assert call(ws=ctypes.c_void_p(FAKE.value + 64)) == 5  # misaligned
    assert call(shp=odd) == 4


def test_parallel_runs_in_workspace_size(L):
    """Few long documents make the state scans run in parallel runs: their
    buffers (transfer maps, offsets, start values: 3 x runs x H x 64 KiB) show
    in the workspace size; many documents, or short ones, need none."""
    def need(cu, H, bwd=0):
        v = varlen(cu, [0] * (len(cu) - 1))
        return L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(g.GDNShape(H, 128, 128, 4, g.BF16, 0,
                                                                                          0.0)), bwd)
    slot_bytes = 16 * (6 * 32 * 32 + (128 * 128 + 1024 + 2048 + 2048 + 64) + 128 * 128) * 4
    # one document of 32768 tokens at 16 heads: 64 chains, 8 runs of 128 chunks, 9 run units
    base = (32768 // 32 + 1) * slot_bytes
    assert need([0, 32768], 16) == (base + 255) // 256 * 256 + 3 * 9 * 16 * 128 * 128 * 4 + 256
    # four documents of 8192 at 16 heads fill the chip: no runs
    assert need([0, 8192, 16384, 24576, 32768], 16) == (32768 // 32 + 4) * slot_bytes + 256
    # one short document: runs would be under 32 chunks
    assert need([0, 4096], 16) == (4096 // 32 + 1) * slot_bytes + 256


def test_strided_checkpoints_and_windows_sizes(L):
    """Checkpoints of stride s, the backward's rebuild region and chunk
    windows in the size queries; the entry points refuse what they do not
    serve before anything is launched."""
    H, D = 4, 128
    cu, pl = [0, 300, 364, 364, 1000], [20, 0, 0, 96]
    v = varlen(cu, pl)
    N, T = 4, 1000
    shape = g.GDNShape(H, D, D, 4, g.BF16, 0, 0.0)
    dd = D * D * 4
    wsw = lambda bwd, s, w, sh=shape: L.flare_gdn_dual_workspace_size_window(ctypes.byref(v), ctypes.byref(sh), bwd,
                                                                            s, w)
    one_f = L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(shape), 0)
    one_b = L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(shape), 1)
    assert wsw(0, 1, 0) == one_f and wsw(1, 1, 0) == one_b
    assert wsw(0, 4, 0) == one_f  # the forward's workspace does not depend on the stride
    slots = T // 32 + N
    pack = 128 * 128 + 1024 + 2048 + 2048 + 64
    # stride > 1: the backward keeps the rebuilt chunk-start states after the hand-over
    per_b = H * (dd + 6 * 32 * 32 * 4 + pack * 4)
    assert wsw(1, 2, 0) == (slots * (per_b + H * dd) + 255) // 256 * 256 + 256
    # windows of w chunks: N * w slots, then the carried chain [N][H][D][D]
    per_f = H * (6 * 32 * 32 * 4 + pack * 4 + dd)
    for w in (1, 3, 8):
        assert wsw(0, 1, w) == (N * w * per_f + 255) // 256 * 256 + N * H * dd + 256
    assert wsw(1, 4, 8) == (N * 8 * (per_b + H * dd) + 255) // 256 * 256 + N * H * dd + 256
    assert wsw(1, 4, 4) < one_b
    # the backward's window must be a multiple of the stride; no stride < 1
    assert wsw(1, 4, 6) == 0 and wsw(1, 0, 0) == 0 and wsw(0, 1, -1) == 0
    # shapes without the chunked path: one pass, stride 1 only
    small = g.GDNShape(2, 16, 16, 4, g.F32, 0, 0.0)
    assert wsw(0, 1, 4, small) == 0 and wsw(1, 2, 0, small) == 0
    assert wsw(1, 1, 0, small) == L.flare_gdn_dual_workspace_size(ctypes.byref(v), ctypes.byref(small), 1)
    # checkpoint buffers of stride s: floor(T / (32 s)) + N slots
    for s in (1, 2, 4, 7):
        assert L.flare_gdn_dual_ckpt_size(ctypes.byref(v), ctypes.byref(shape), s) == (T // (32 * s) + N) * H * dd
    assert L.flare_gdn_dual_ckpt_size(ctypes.byref(v), ctypes.byref(shape), 0) == 0
    # the backward: stride 0 is a shape error, stride > 1 needs the chunked path
    args = [FAKE] * 10 + [None, FAKE]
    tail = [None, FAKE, FAKE, None] + [FAKE] * 10 + [None]
    sv = varlen([0, 40, 64], [8, 0])
    st = L.flare_gdn_dual_bwd(ctypes.byref(sv), ctypes.byref(small), *args, 2, *tail, FAKE, 1 << 30, None)
    assert st == 4 and b"stride" in L.flare_last_error()
    st = L.flare_gdn_dual_bwd(ctypes.byref(v), ctypes.byref(shape), *args, 0, *tail, FAKE, 1 << 30, None)
    assert st == 2
    # too small for even a one-chunk window (a multiple of the stride for the backward)
    st = L.flare_gdn_dual_bwd(ctypes.byref(v), ctypes.byref(shape), *args, 4, *tail, FAKE, wsw(1, 4, 4) - 1, None)
    assert st == 5
    P = [FAKE] * 10
    st = L.flare_gdn_dual_fwd(ctypes.byref(v), ctypes.byref(shape), *P, None, FAKE, FAKE, None, None, 1,
                              FAKE, wsw(0, 1, 1) - 1, None)
    assert st == 5
    # the pool forward runs in one pass only
    host = np.arange(N, dtype=np.int32)
    st = L.flare_gdn_dual_fwd_pool(ctypes.byref(v), ctypes.byref(shape), *P, FAKE, host.ctypes.data, FAKE, N, 1,
                                   FAKE, FAKE, None, 1, FAKE, wsw(0, 1, 4), None)
    assert st == 5 and b"one pass" in L.flare_last_error()


def test_fwd_conv_validation(L):
    """flare_gdn_dual_fwd_conv refuses what it does not serve before launching:
    widths outside 1..4, unknown activations, shapes without the chunked path,
    missing projections or weights, a workspace below one chunk's window."""
    v = varlen([0, 100, 164], [20, 0])
    shape = g.GDNShape(4, 128, 128, 4, g.BF16, 0, 0.0)
    A3 = ctypes.c_void_p * 3
    full = A3(FAKE, FAKE, FAKE)
    hole = A3(FAKE, None, FAKE)

    def call(sh=shape, width=4, act=1, x=full, xn=full, w=full, ws_bytes=1 << 34):
        return L.flare_gdn_dual_fwd_conv(ctypes.byref(v), ctypes.byref(sh), width, w, act, x, xn, FAKE, FAKE, FAKE,
                                         FAKE, None, FAKE, FAKE, None, None, 1, FAKE, ws_bytes, None)

    assert call(width=0) == 4 and call(width=5) == 4
    assert call(act=2) == 4
    assert call(sh=g.GDNShape(4, 16, 16, 4, g.F32, 0, 0.0)) == 4
    assert call(x=hole) == 1 and call(xn=hole) == 1 and call(w=hole) == 1
    w1 = L.flare_gdn_dual_workspace_size_window(ctypes.byref(v), ctypes.byref(shape), 0, 1, 1)
    assert call(ws_bytes=w1 - 1) == 5
