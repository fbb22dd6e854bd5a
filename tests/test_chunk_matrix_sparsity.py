"""CPU check of the rule by which only parts of the chunk-matrix records are
stored and read: the six 32 x 32 chunk matrices of the chunked dual-stream
form (the clean UT inverse T, the noisy blocks' inverse T~, and the masked
weighted Gram matrices Mwo, Mwq, Mwk, Mw~ of the readout; "FLARE: Diffusion
for Hybrid Language Model", papernotes.org notes, Key designs item 2) are
built here from their definitions with random rows and gates, and every
non-zero entry must lie in a 64-byte half-row that the rule keeps.  The rule
is the one bench.py uses to count the records' bytes, the same case analysis
as the library's."""
import numpy as np
import pytest

import bench

C = 32


def chunk_matrices(B, rng, d=8):
    """T, T~, Mwo, Mwq, Mwk, Mw~ of one chunk whose rows are all response rows,
    from their definitions (dense numpy, no structure assumed)."""
    k, q, kn, qn = (rng.standard_normal((C, d)) for _ in range(4))
    g = np.cumsum(np.log(rng.uniform(0.5, 1.0, C)))       # clean log-decay prefix
    gn = np.log(rng.uniform(0.5, 1.0, C))                 # noisy log-decays
    b, bn = rng.uniform(0.1, 1.0, C), rng.uniform(0.1, 1.0, C)
    p = np.arange(C) & -B                                 # block start of each row
    gnb = np.zeros(C)                                     # noisy prefix, restarted per block
    for i in range(C):
        gnb[i] = gn[i] + (gnb[i - 1] if i > p[i] else 0.0)
    I, J = np.meshgrid(np.arange(C), np.arange(C), indexing="ij")
    A = np.where(J < I, b[J] * np.exp(g[I] - g[J]) * (k @ k.T), 0.0)
    T = np.linalg.inv(np.eye(C) + A)
    An = np.where((J < I) & (J >= p[I]), bn[J] * np.exp(gnb[I] - gnb[J]) * (kn @ kn.T), 0.0)
    Tn = np.linalg.inv(np.eye(C) + An)
    Mwo = np.where(J <= I, b[J] * np.exp(g[I] - g[J]) * (q @ k.T), 0.0)
    gp = np.where(p > 0, g[np.maximum(p - 1, 0)], 0.0)    # clean prefix at the block boundary
    Mwq = np.where(J < p[I], b[J] * np.exp(gp[I] - g[J]) * (qn @ k.T), 0.0)
    Mwk = np.where(J < p[I], b[J] * np.exp(gp[I] - g[J]) * (kn @ k.T), 0.0)
    e = np.minimum(p + B - 1, C - 1)
    Mwn = np.where((J >= p[I]) & (J <= e[I]), bn[J] * np.exp(gnb[e[I]] - gnb[J]) * (qn @ kn.T), 0.0)
    return [T, Tn, Mwo, Mwq, Mwk, Mwn]


def live_mask(mtx, B, has_noisy):
    """Entries the stored record keeps, as a C x C boolean matrix, from the
    bench's per-half-row byte count (64 bytes = one live half-row)."""
    m = np.zeros((C, C), bool)
    for row in range(C):
        for half in (0, 1):
            lo = 16 * half
            p = row & -B
            if mtx in (0, 2):
                on = lo <= row
            elif not has_noisy:
                on = False
            elif mtx == 1:
                on = lo <= row and lo + 15 >= p
            elif mtx == 5:
                on = lo <= p + B - 1 and lo + 15 >= p
            else:
                on = lo < p
            m[row, lo:lo + 16] = on
    return m


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_nonzeros_lie_in_live_half_rows(B):
    rng = np.random.default_rng(100 + B)
    mats = chunk_matrices(B, rng)
    total = 0
    for mtx, M in enumerate(mats):
        live = live_mask(mtx, B, True)
        outside = np.abs(M[~live]).max() if (~live).any() else 0.0
        assert outside < 1e-12, (B, mtx, outside)
        total += int(live.sum()) * 4
    # the byte count the bench uses is the same rule summed
    assert total == bench.chunk_matrix_live_bytes(B, True)
    assert bench.chunk_matrix_live_bytes(B, False) == 2 * (16 * 64 + 16 * 128)  # T and Mwo only


def test_rule_is_tight_where_the_masks_are():
    """The kept half-rows are not a trivial superset: at B = 4 a noisy chunk
    keeps 62.5 % of the record and a prompt-only chunk 25 %, and each kept
    half-row of the noisy matrices holds a non-zero entry for random data."""
    B = 4
    assert bench.chunk_matrix_live_bytes(B, True) == 15360
    assert bench.chunk_matrix_live_bytes(B, False) == 6144
    mats = chunk_matrices(B, np.random.default_rng(7))
    for mtx, M in enumerate(mats):
        live = live_mask(mtx, B, True)
        for row in range(C):
            for lo in (0, 16):
                if live[row, lo]:
                    assert np.abs(M[row, lo:lo + 16]).max() > 0, (mtx, row, lo)
