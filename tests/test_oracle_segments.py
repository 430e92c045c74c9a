"""Pins of the oracle's fixed-segment (block-diagonal causal) schedule.

* page-printed block counts (tests/golden/segment_counts.txt): 288 and 160 blocks
  at S 4096 for 512- and 256-token segments, 2,080 for one segment spanning S;
* special cases that reduce to other schedules: a segment of one block is the
  diagonal, a segment of at least nb blocks is the dense causal CSR;
* brute force over token pairs: a block pair is listed exactly when some query
  token of the row block may attend to some key token of the column block, i.e.
  key <= query and both in one segment of segment_blocks * 64 tokens.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden_rows


def _rows():
    out = []
    for line in read_golden_rows("segment_counts.txt"):
        S, block, seg_tokens, blocks = (int(x) for x in line.split())
        out.append((S, block, seg_tokens, blocks))
    return out


@pytest.mark.parametrize("row", _rows())
def test_segment_counts_match_pages(row):
    S, block, seg_tokens, blocks = row
    rp, ci = oracle.fixed_segment_schedule(S // block, seg_tokens // block)
    assert int(rp[-1]) == blocks == ci.shape[0]


@pytest.mark.parametrize("nb", [1, 5, 16, 64])
def test_one_block_segments_are_the_diagonal(nb):
    rp, ci = oracle.fixed_segment_schedule(nb, 1)
    assert np.array_equal(rp, np.arange(nb + 1)) and np.array_equal(ci, np.arange(nb))


@pytest.mark.parametrize("nb,seg", [(1, 1), (7, 7), (16, 40), (64, 64)])
def test_segment_spanning_all_blocks_is_dense(nb, seg):
    rp, ci = oracle.fixed_segment_schedule(nb, seg)
    rp_d, ci_d = oracle.dense_causal_schedule(nb)
    assert np.array_equal(rp, rp_d) and np.array_equal(ci, ci_d)


@pytest.mark.parametrize("nb,seg", [(6, 2), (7, 3), (9, 4), (10, 5)])
def test_brute_force_over_token_pairs(nb, seg):
    """Row i lists block j exactly when a token pair (t in block i, u in block j) has
    u <= t in one segment of seg * 64 tokens."""
    T = nb * 64
    t = np.arange(T)
    allowed = (t[None, :] <= t[:, None]) & (t[None, :] // (64 * seg) == t[:, None] // (64 * seg))
    want = [sorted({int(u) // 64 for u in np.nonzero(allowed[64 * i : 64 * i + 64].any(0))[0]})
            for i in range(nb)]
    rp, ci = oracle.fixed_segment_schedule(nb, seg)
    got = [list(ci[rp[i] : rp[i + 1]]) for i in range(nb)]
    assert got == want


def test_rejects_empty_segments():
    with pytest.raises(ValueError):
        oracle.fixed_segment_schedule(4, 0)
