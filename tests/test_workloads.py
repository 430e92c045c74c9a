"""The seeded workload inputs: determinism, shapes, and the no-tie margins that a
bit-exact CSR comparison between two implementations needs.

A CSR built by two different float64 pipelines (the oracle's all-pairs order and
an MST-based builder) can only be compared bit for bit when no decision sits
near a tie.  For each topology workload the lane-(0, 0) keys must have, relative
to the distances involved:
  (i)   distinct MST edge lengths (gap between consecutive sorted lengths),
  (ii)  every non-tree pair longer than the longest edge on its tree path,
  (iii) a gap between the k-th and (k+1)-th largest salience.
Margins are required to be at least 1e-9, far above fp64 rounding (~1e-15).
"""
import numpy as np
import pytest
from scipy.sparse.csgraph import minimum_spanning_tree

import oracle
import workloads

MARGIN = 1e-9


def _margins(keys, topk):
    c = oracle.block_centroids(keys, workloads.BLOCK)
    d = oracle.centroid_distances(c)
    nb = c.shape[0]
    mst = minimum_spanning_tree(d).tocoo()
    w = np.sort(mst.data)
    gap_edges = float(np.min(np.diff(w) / w[1:])) if w.shape[0] > 1 else np.inf
    adj = [[] for _ in range(nb)]
    for a, b, x in zip(mst.row, mst.col, mst.data):
        adj[a].append((b, x))
        adj[b].append((a, x))
    in_tree = np.zeros((nb, nb), dtype=bool)
    in_tree[mst.row, mst.col] = True
    in_tree[mst.col, mst.row] = True
    cycle = np.inf
    for s in range(nb):
        path_max = np.full(nb, -1.0)
        path_max[s] = 0.0
        stack = [s]
        while stack:
            u = stack.pop()
            for nxt, x in adj[u]:
                if path_max[nxt] < 0:
                    path_max[nxt] = max(path_max[u], x)
                    stack.append(nxt)
        off = ~in_tree[s]
        off[: s + 1] = False
        if off.any():
            cycle = min(cycle, float(np.min((d[s, off] - path_max[off]) / d[s, off])))
    sal = np.sort(oracle.elder_rule_salience(c))[::-1]
    k = min(topk, nb)
    gap_topk = float((sal[k - 1] - sal[k]) / sal[k - 1]) if 0 < k < nb else np.inf
    return gap_edges, cycle, gap_topk


TOPOLOGY = [w for w in workloads.WORKLOADS.values() if not w.dense]


@pytest.mark.parametrize("w", TOPOLOGY, ids=lambda w: w.name)
def test_workload_keys_have_no_near_ties(w):
    _, k, _ = workloads.make_qkv(w)
    keys = k.reshape(-1, w.S, w.D)[0]
    m = _margins(keys, w.topk)
    assert min(m) >= MARGIN, (w.name, m)


def test_generation_is_deterministic_and_typed():
    w = workloads.WORKLOADS["single_s1024_d64_f16"]
    a = workloads.make_qkv(w)
    b = workloads.make_qkv(w)
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and x.shape == w.shape
        assert bool((x == y).all())
    c = workloads.make_qkv(w, seed=w.seed + 1)
    assert not bool((a[0] == c[0]).all())


def test_mixture_keys_cluster_per_block():
    w = workloads.WORKLOADS["single_s4096_d64_f16_mix8"]
    _, k, _ = workloads.make_qkv(w)
    kk = k.double().numpy().reshape(w.nb, workloads.BLOCK, w.D)
    within = kk.std(axis=1).mean()
    assert 0.4 < within < 0.6  # within-block noise std 0.5
    assert kk.mean(axis=1).std() > 1.5  # means spread with std 2


def test_random_csr_rows_are_causal_ascending():
    rp, ci = workloads.random_csr(20, seed=1, density=0.3)
    for i in range(20):
        cols = ci[rp[i] : rp[i + 1]]
        assert np.all(np.diff(cols) > 0) and cols[-1] == i
