"""The binding checks every tensor before the library sees its bare pointer.
CPU side: the checking helpers on CPU tensors, and every entry point refusing
host tensors (nothing is launched; no GPU is needed)."""
import numpy as np
import pytest
import torch

import gated_deltanet_dual_amd as g

CPU = torch.device("cpu")


def test_chk_dtype_shape_contiguity_device():
    x = torch.zeros((4, 2, 8), dtype=torch.float32)
    g._chk(x, "x", (4, 2, 8), torch.float32, CPU)
    g._chk(None, "x", (4, 2, 8), torch.float32, CPU, optional=True)
    with pytest.raises(g.FlareError, match="required"):
        g._chk(None, "x", (4, 2, 8), torch.float32, CPU)
    with pytest.raises(g.FlareError, match="dtype"):
        g._chk(x.to(torch.bfloat16), "x", (4, 2, 8), torch.float32, CPU)
    with pytest.raises(g.FlareError, match="shape"):
        g._chk(x, "x", (4, 2, 16), torch.float32, CPU)
    with pytest.raises(g.FlareError, match="contiguous"):
        g._chk(x.transpose(0, 1).contiguous().transpose(0, 1), "x", (4, 2, 8), torch.float32, CPU)
    with pytest.raises(g.FlareError, match="on"):
        g._chk(x, "x", (4, 2, 8), torch.float32, torch.device("meta"))


def test_chk_buf_size():
    ws = torch.zeros(1024, dtype=torch.uint8)
    g._chk_buf(ws, "ws", 1024, torch.uint8, CPU)
    with pytest.raises(g.FlareError, match="1025 needed") as e:
        g._chk_buf(ws, "ws", 1025, torch.uint8, CPU)
    assert e.value.status == 5
    with pytest.raises(g.FlareError, match="dtype"):
        g._chk_buf(ws.view(torch.float32), "ws", 16, torch.uint8, CPU)


def test_io_dtype():
    with pytest.raises(g.FlareError) as e:
        g._io_of(torch.zeros(2, dtype=torch.float16))
    assert e.value.status == 4
    assert g._io_of(torch.zeros(2, dtype=torch.bfloat16)) == g.BF16


def test_entry_points_refuse_host_tensors():
    T, H, d, R, B = 8, 2, 16, 2, 4
    q = torch.zeros((T, H, d))
    a = torch.ones((T, H))
    cu = np.array([0, T], np.int32)

    class HostVarlen:  # no device arrays: the device check fires first
        num_docs = 1
        total_tokens = T
        cu_dev = torch.from_numpy(cu)

    vl = HostVarlen()
    with pytest.raises(g.FlareError, match="GPU tensor"):
        g.gdn_dual_fwd(vl, q, q, q, a, a, q, q, q, a, a, B)
    with pytest.raises(g.FlareError, match="GPU tensor"):
        g.gdn_dual_bwd(vl, q, q, q, a, a, q, q, q, a, a, B, None, q, q)
    x = torch.zeros((R, B, H, d))
    ga = torch.ones((R, B, H))
    with pytest.raises(g.FlareError, match="GPU tensor"):
        g.block_step(torch.zeros(R, dtype=torch.int32), torch.zeros((4, H, d, d)), x, x, x, ga, ga, g.EVAL)
    with pytest.raises(g.FlareError, match="GPU tensor"):
        g.shortconv_dual(vl, B, torch.zeros((T, 8)), torch.zeros((T, 8)), torch.zeros((8, 4)))
