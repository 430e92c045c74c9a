"""Pins of oracle.refine_schedule (a schedule over blocks of B = 64 m rows as the
CSR over 64-row blocks) and of the oracle builder at block sizes above 64:

* the refined CSR allows exactly the keys the coarse one allows, by the forward
  oracle's mask definition (allowed_key_mask at the two block sizes), on ragged S
  and rows with empty, above-diagonal and out-of-range entries, and every fine
  block it lists holds a visible key for some query of its row;
* closed forms: the dense causal CSR refines to the dense causal CSR, fixed
  segments of L coarse blocks to fixed segments of m L fine blocks, block 64 to
  itself;
* centroids at block 128 are the means of the two 64-row halves' centroids
  (weighted by their rows for a partial last block).
"""
import numpy as np
import pytest

import oracle
import workloads


@pytest.mark.parametrize("S,block,seed", [(1000, 128, 0), (1024, 256, 1), (777, 192, 2), (576, 128, 3),
                                          (100, 128, 4), (64, 128, 5), (5000, 320, 6), (129, 128, 7)])
def test_refined_mask_equals_coarse_mask(S, block, seed):
    nbc = -(-S // block)
    rp, ci = workloads.random_csr(nbc, seed=seed, density=0.4, allow_empty=True)
    frp, fci = oracle.refine_schedule(rp, ci, S, block)
    nb64 = -(-S // 64)
    assert frp.shape[0] == nb64 + 1 and frp.dtype == np.int32 and fci.dtype == np.int32
    np.testing.assert_array_equal(oracle.allowed_key_mask(rp, ci, S, block),
                                  oracle.allowed_key_mask(frp, fci, S, 64))
    for i in range(nb64):
        row = fci[frp[i]:frp[i + 1]]
        assert np.all(np.diff(row) > 0) and (row.size == 0 or (row[0] >= 0 and row[-1] <= i))
        rows = np.arange(64 * i, min(S, 64 * i + 64))
        mask = oracle.allowed_key_mask(frp, fci, S, 64, rows)
        for c in row:
            assert mask[:, 64 * c: 64 * c + 64].any(), (i, c)


def test_refinement_ignores_entries_outside_the_row():
    S, block = 640, 128  # 5 coarse rows
    rp = np.array([0, 2, 4, 4, 7, 9], np.int32)
    ci = np.array([0, 3, 0, 1, -1, 2, 3, 4, 9], np.int32)  # 3 > 0, -1 and 9 select nothing
    frp, fci = oracle.refine_schedule(rp, ci, S, block)
    np.testing.assert_array_equal(oracle.allowed_key_mask(rp, ci, S, block),
                                  oracle.allowed_key_mask(frp, fci, S, 64))
    assert fci[frp[0]:frp[1]].tolist() == [0] and fci[frp[1]:frp[2]].tolist() == [0, 1]
    assert frp[5] == frp[4] == frp[6]  # coarse row 2 is empty: fine rows 4 and 5 are empty
    # coarse row 3 keeps {2, 3}, coarse row 4 keeps {4}
    assert fci[frp[6]:frp[7]].tolist() == [4, 5, 6] and fci[frp[7]:frp[8]].tolist() == [4, 5, 6, 7]
    assert fci[frp[8]:frp[9]].tolist() == [8] and fci[frp[9]:frp[10]].tolist() == [8, 9]


@pytest.mark.parametrize("S,block", [(4096, 128), (4096, 256), (1000, 128), (300, 192)])
def test_dense_refines_to_dense(S, block):
    frp, fci = oracle.refine_schedule(*oracle.dense_causal_schedule(-(-S // block)), S, block)
    drp, dci = oracle.dense_causal_schedule(-(-S // 64))
    np.testing.assert_array_equal(frp, drp)
    np.testing.assert_array_equal(fci, dci)


@pytest.mark.parametrize("nbc,L,block", [(32, 4, 128), (16, 2, 256), (13, 5, 128)])
def test_segments_refine_to_segments(nbc, L, block):
    m = block // 64
    frp, fci = oracle.refine_schedule(*oracle.fixed_segment_schedule(nbc, L), nbc * block, block)
    srp, sci = oracle.fixed_segment_schedule(nbc * m, m * L)
    np.testing.assert_array_equal(frp, srp)
    np.testing.assert_array_equal(fci, sci)


def test_block_64_is_identity_on_valid_rows():
    rp, ci = workloads.random_csr(40, seed=9, density=0.3, allow_empty=True)
    frp, fci = oracle.refine_schedule(rp, ci, 40 * 64 - 7, 64)
    np.testing.assert_array_equal(frp, rp)
    np.testing.assert_array_equal(fci, ci)


def test_rejects_block_not_a_multiple_of_64():
    with pytest.raises(ValueError):
        oracle.refine_schedule(np.zeros(2, np.int32), np.zeros(0, np.int32), 100, 96)


@pytest.mark.parametrize("S", [1024, 1000, 960])
def test_block_128_centroids_are_means_of_halves(S):
    keys = np.random.default_rng(3).standard_normal((S, 16))
    c64 = oracle.block_centroids(keys, 64)
    c128 = oracle.block_centroids(keys, 128)
    rows64 = np.minimum(64, S - 64 * np.arange(c64.shape[0]))
    assert c128.shape[0] == -(-S // 128)
    for J in range(c128.shape[0]):
        parts = [2 * J, 2 * J + 1][: c64.shape[0] - 2 * J]
        w = rows64[parts]
        np.testing.assert_allclose(c128[J], (c64[parts] * w[:, None]).sum(0) / w.sum(), rtol=1e-13, atol=1e-15)
