"""The integer-tag workload of the chunked-path exactness tests tells block,
document and chunk-boundary selections apart: on the CPU, the oracle's outputs
change when a block boundary, a prompt length or a document boundary moves by
one block, so a kernel that made such a slip could not match bit for bit."""
import numpy as np
import pytest

import oracle
from test_gpu_exact_chunked import tag_inputs


def fwd(inp, B=None, prompts=None, cu=None):
    B = inp.block_size if B is None else B
    return oracle.gdn_dual_fwd(inp.cu_seqlens if cu is None else cu,
                               inp.prompt_lens if prompts is None else prompts,
                               *inp.clean_args(), *inp.noisy_args(), B, h0=inp.h0, scale=1.0)


@pytest.mark.parametrize("B", [2, 4, 8])
def test_tags_discriminate_block_anchoring(B):
    inp = tag_inputs(B, seed=300 + B)
    o, on, hf = fwd(inp)
    _, on2, _ = fwd(inp, B=2 * B)
    assert not np.array_equal(on, on2), "block size"
    pl = inp.prompt_lens.copy()
    i = int(np.argmax(inp.cu_seqlens[1:] - inp.cu_seqlens[:-1] - pl))  # the doc with the longest response
    pl[i] += B
    _, on3, _ = fwd(inp, prompts=pl)
    assert not np.array_equal(on, on3), "prompt length"


def test_tags_discriminate_document_boundaries():
    inp = tag_inputs(4, seed=310)
    o, _, _ = fwd(inp)
    cu = inp.cu_seqlens.copy()
    # move the boundary between documents 0 (200 tokens, prompt 12) and 1 by one block
    cu[1] += 4
    o2, _, _ = fwd(inp, cu=cu)
    assert not np.array_equal(o, o2), "document boundary"
