"""Pins for the oracle's schedule builder, against facts fixed outside the oracle.

What pins what:
* page-printed block counts (tests/golden/block_counts.txt) -> dense CSR and the
  sink/local window widths;
* closed-form special cases (k >= nb, radius >= nb - 1, all-zero parameters);
* library routines (scipy MST, scipy single-linkage, numpy mean/cdist) -> the
  centroids, the distances and the H0 barcode;
* the elder-rule invariants the port's commit note states (one zero, multiset
  invariance under block permutation);
* hand-worked examples (tests/golden/elder_rule_line_examples.txt) -> per-block
  assignment and the size-tie direction;
* an MST-edge computation of the same salience, which the mirror page's
  ``schedule.py`` note says is bit-identical to all pairs.
"""
import itertools

import numpy as np
import pytest
from scipy.cluster.hierarchy import linkage
from scipy.sparse.csgraph import minimum_spanning_tree
from scipy.spatial.distance import cdist, pdist

import oracle
from conftest import read_golden_rows


def _golden_counts():
    out = []
    for row in read_golden_rows("block_counts.txt"):
        kind, nb, sink, local, topk, value = row.split()
        out.append((kind, nb, sink, local, topk, value))
    return out


def _keys_with_centroids(cents, block=4):
    """Keys whose blocks are constant rows, so block j's centroid is cents[j]."""
    cents = np.asarray(cents, dtype=np.float64)
    return np.repeat(cents, block, axis=0)


def _random_keys(nb, D=8, block=4, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((nb * block, D))


# ---------------------------------------------------------------- dense CSR / counts


@pytest.mark.parametrize("row", [r for r in _golden_counts() if r[0] == "dense"])
def test_dense_counts_match_page_table(row):
    _, nb, _, _, _, value = row
    rp, ci = oracle.dense_causal_schedule(int(nb))
    assert rp[-1] == int(value) == ci.shape[0]


@pytest.mark.parametrize("nb", [1, 2, 7, 16, 64])
def test_dense_is_exact_lower_triangle(nb):
    rp, ci = oracle.dense_causal_schedule(nb)
    sets = oracle.csr_to_block_sets(rp, ci)
    tri = np.tril(np.ones((nb, nb), dtype=bool))
    for i in range(nb):
        assert sets[i] == set(np.nonzero(tri[i])[0].tolist())
        assert list(ci[rp[i] : rp[i + 1]]) == sorted(sets[i])
    assert rp.dtype == np.int32 and ci.dtype == np.int32


def test_sink_local_count_45():
    (row,) = [r for r in _golden_counts() if r[0] == "sink_local"]
    _, nb, sink, local, topk, value = row
    keys = _random_keys(int(nb), block=64)
    rp, _, _ = oracle.build_schedule(keys, 64, int(sink), int(local), int(topk))
    assert rp[-1] == int(value)


@pytest.mark.parametrize("seed", range(20))
def test_topk2_count_in_page_range(seed):
    (row,) = [r for r in _golden_counts() if r[0] == "topk_range"]
    _, nb, sink, local, topk, value = row
    lo, hi = (int(x) for x in value.split(".."))
    rp, _, _ = oracle.build_schedule(_random_keys(int(nb), block=64, seed=seed), 64, int(sink), int(local), int(topk))
    assert lo <= rp[-1] <= hi


def test_every_topk2_set_stays_in_page_range():
    """All C(16, 2) global top-2 sets give a count within the page's range."""
    (row,) = [r for r in _golden_counts() if r[0] == "topk_range"]
    lo, hi = (int(x) for x in row[5].split(".."))
    for a, b in itertools.combinations(range(16), 2):
        sal = np.zeros(16)
        sal[a], sal[b] = 2.0, 1.0
        rp, _ = oracle.schedule_from_salience(sal, 1, 1, 2)
        assert lo <= rp[-1] <= hi


@pytest.mark.parametrize("nb", [1, 5, 16])
def test_topk_at_least_nb_is_dense(nb):
    keys = _random_keys(nb, seed=nb)
    rp, ci, _ = oracle.build_schedule(keys, 4, 0, 0, nb)
    drp, dci = oracle.dense_causal_schedule(nb)
    assert np.array_equal(rp, drp) and np.array_equal(ci, dci)
    rp, ci, _ = oracle.build_schedule(keys, 4, 0, 0, nb + 5)
    assert np.array_equal(ci, dci)


@pytest.mark.parametrize("nb", [1, 5, 16])
def test_wide_window_or_sink_is_dense(nb):
    keys = _random_keys(nb, seed=3)
    drp, dci = oracle.dense_causal_schedule(nb)
    for s, r in [(0, nb - 1), (nb, 0), (nb + 3, nb + 3)]:
        rp, ci, _ = oracle.build_schedule(keys, 4, s, r, 0)
        assert np.array_equal(rp, drp) and np.array_equal(ci, dci)


@pytest.mark.parametrize("nb", [1, 9])
def test_no_sink_no_window_no_topk_is_diagonal(nb):
    rp, ci, _ = oracle.build_schedule(_random_keys(nb), 4, 0, 0, 0)
    assert np.array_equal(rp, np.arange(nb + 1)) and np.array_equal(ci, np.arange(nb))


def test_schedule_rows_ascending_causal_and_contain_diagonal():
    keys = _random_keys(40, seed=11)
    rp, ci, sal = oracle.build_schedule(keys, 4, 2, 1, 5)
    top = set(np.argsort(-sal, kind="stable")[:5].tolist())
    for i in range(40):
        cols = ci[rp[i] : rp[i + 1]]
        assert np.all(np.diff(cols) > 0) and cols[-1] == i and cols[0] >= 0
        assert set(cols.tolist()) == {j for j in range(i + 1) if j < 2 or j >= i - 1 or j in top}


# ---------------------------------------------------------------- centroids / distances


def test_centroids_are_block_means_including_partial_block():
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((64 * 3 + 17, 16))
    c = oracle.block_centroids(keys, 64)
    assert c.shape == (4, 16)
    for j in range(3):
        assert np.allclose(c[j], np.mean(keys[64 * j : 64 * (j + 1)], axis=0), rtol=0, atol=1e-15)
    assert np.allclose(c[3], np.mean(keys[192:], axis=0), rtol=0, atol=1e-15)


def test_centroids_exact_for_half_precision_inputs():
    """fp16/bf16 keys sum exactly in fp64, so each centroid is the exactly rounded mean."""
    import torch

    for dt in (torch.float16, torch.bfloat16):
        keys = torch.randn(256, 32, generator=torch.Generator().manual_seed(0)).to(dt)
        k64 = keys.to(torch.float64).numpy()
        c = oracle.block_centroids(keys, 64)
        for j in range(4):
            # math.fsum gives the exactly rounded sum; /64 is exact
            import math

            exact = np.array([math.fsum(k64[64 * j : 64 * j + 64, d]) for d in range(32)]) / 64
            assert np.array_equal(c[j], exact)


def test_distances_match_cdist():
    c = np.random.default_rng(2).standard_normal((13, 7))
    d = oracle.centroid_distances(c)
    assert np.allclose(d, cdist(c, c), rtol=1e-14, atol=1e-14)
    assert np.array_equal(d, d.T) and np.all(np.diag(d) == 0)


# ---------------------------------------------------------------- salience


@pytest.mark.parametrize("seed", range(8))
def test_exactly_one_zero_salience(seed):
    sal = oracle.elder_rule_salience(oracle.block_centroids(_random_keys(25, seed=seed), 4))
    assert np.count_nonzero(sal == 0) == 1


@pytest.mark.parametrize("nb,seed", [(2, 0), (3, 1), (16, 2), (64, 3), (100, 4)])
def test_nonzero_salience_is_mst_barcode(nb, seed):
    c = oracle.block_centroids(_random_keys(nb, D=6, seed=seed), 4)
    sal = oracle.elder_rule_salience(c)
    mst = minimum_spanning_tree(cdist(c, c)).tocoo()
    assert np.allclose(np.sort(sal[sal > 0]), np.sort(mst.data), rtol=1e-14, atol=0)
    heights = linkage(pdist(c), method="single")[:, 2]
    assert np.allclose(np.sort(sal[sal > 0]), np.sort(heights), rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", range(5))
def test_barcode_multiset_invariant_under_block_permutation(seed):
    rng = np.random.default_rng(100 + seed)
    c = rng.standard_normal((30, 5))
    perm = rng.permutation(30)
    a = np.sort(oracle.elder_rule_salience(c))
    b = np.sort(oracle.elder_rule_salience(c[perm]))
    assert np.allclose(a, b, rtol=1e-14, atol=0)


def test_hand_worked_elder_examples():
    for row in read_golden_rows("elder_rule_line_examples.txt"):
        pos, expect = row.split("|")
        xs = [float(x) for x in pos.split()]
        want = np.array([float(x) for x in expect.split()])
        cents = np.zeros((len(xs), 3))
        cents[:, 0] = xs
        keys = _keys_with_centroids(cents, block=64)
        sal = oracle.elder_rule_salience(oracle.block_centroids(keys, 64))
        assert np.array_equal(sal, want), (xs, sal, want)


def _salience_from_mst_edges(c):
    """Same elder rule driven by MST edges (Prim on the distance matrix).

    The oracle's own distance matrix is used so that only the algorithm path
    (all pairs against MST edges) differs; the distances are pinned to cdist
    separately.
    """
    nb = c.shape[0]
    d = oracle.centroid_distances(c)
    in_tree = np.zeros(nb, dtype=bool)
    in_tree[0] = True
    best = d[0].copy()
    src = np.zeros(nb, dtype=np.int64)
    edges = []
    for _ in range(nb - 1):
        cand = np.where(in_tree, np.inf, best)
        u = int(np.argmin(cand))
        edges.append((best[u], min(u, src[u]), max(u, src[u])))
        in_tree[u] = True
        closer = d[u] < best
        best = np.where(closer, d[u], best)
        src = np.where(closer, u, src)
    edges.sort()
    root = list(range(nb))
    members = {i: 1 for i in range(nb)}
    sal = np.zeros(nb)

    def top(x):
        while root[x] != x:
            x = root[x]
        return x

    for w, a, b in edges:
        ra, rb = top(a), top(b)
        keep, drop = (ra, rb) if (members[ra], -ra) > (members[rb], -rb) else (rb, ra)
        root[drop] = keep
        members[keep] += members[drop]
        sal[drop] = w
    return sal


@pytest.mark.parametrize("nb,seed", [(5, 0), (16, 1), (64, 2), (130, 3)])
def test_all_pairs_equals_mst_edges_bitwise(nb, seed):
    c = np.random.default_rng(seed).standard_normal((nb, 8))
    assert np.array_equal(oracle.elder_rule_salience(c), _salience_from_mst_edges(c))


def test_topk_ranking_matches_stable_argsort():
    rng = np.random.default_rng(9)
    sal = np.round(rng.random(50) * 8) / 8  # many ties: lower index must win
    for k in [0, 1, 5, 17, 50, 80]:
        want = sorted(np.argsort(-sal, kind="stable")[: min(k, 50)].tolist())
        assert oracle.top_k_blocks(sal, k) == want


def test_single_block_schedule():
    rp, ci, sal = oracle.build_schedule(np.ones((10, 4)), 64, 1, 1, 2)
    assert list(rp) == [0, 1] and list(ci) == [0] and list(sal) == [0.0]
