"""Pins of the oracle's per-row top-k reading (each row takes its own top-k among
its causal blocks j <= i, under the global (-salience, index) ranking).

* page configuration (16 blocks, sink 1, radius 1, top-2): constructed salience
  orders reach the closed-form counts 45, 58 and 70 of
  tests/golden/per_row_topk_counts.txt, and random saliences stay in [45, 70];
* special cases: topk >= nb gives the dense CSR, topk 0 equals the global
  reading with topk 0, and the last row's top-k set is the global top-k set;
* an independent characterisation: block j is in row i's top-k set exactly when
  j <= i < e_j, where e_j is the k-th smallest index among the blocks ranked
  above j (nb when fewer than k are).
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden_rows

ORDERS = {
    "rising": lambda nb: np.arange(nb, dtype=np.float64),
    "falling": lambda nb: np.arange(nb, dtype=np.float64)[::-1].copy(),
    "blocks_1_2_first": lambda nb: np.array([0.5, 100.0, 90.0] + [float(x) for x in range(nb - 3)]),
}


def _rows():
    out = []
    for line in read_golden_rows("per_row_topk_counts.txt"):
        nb, sink, r, k, order, count = line.split()
        out.append((int(nb), int(sink), int(r), int(k), order, int(count)))
    return out


@pytest.mark.parametrize("row", _rows())
def test_page_configuration_counts(row):
    nb, sink, r, k, order, count = row
    rp, _ = oracle.schedule_from_salience(ORDERS[order](nb), sink, r, k, per_row=True)
    assert int(rp[-1]) == count


def test_random_saliences_stay_in_range():
    rng = np.random.default_rng(5)
    counts = set()
    for _ in range(300):
        rp, _ = oracle.schedule_from_salience(rng.permutation(16).astype(float), 1, 1, 2, per_row=True)
        counts.add(int(rp[-1]))
    assert min(counts) >= 45 and max(counts) <= 70


@pytest.mark.parametrize("nb", [1, 7, 20])
def test_topk_at_least_nb_is_dense(nb):
    sal = np.random.default_rng(nb).standard_normal(nb)
    rp, ci = oracle.schedule_from_salience(sal, 0, 0, nb, per_row=True)
    rp_d, ci_d = oracle.dense_causal_schedule(nb)
    assert np.array_equal(rp, rp_d) and np.array_equal(ci, ci_d)


@pytest.mark.parametrize("nb,s,r", [(9, 1, 1), (20, 2, 0), (33, 0, 3)])
def test_topk_zero_matches_global(nb, s, r):
    sal = np.random.default_rng(nb).standard_normal(nb)
    a = oracle.schedule_from_salience(sal, s, r, 0, per_row=True)
    b = oracle.schedule_from_salience(sal, s, r, 0, per_row=False)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_last_row_takes_the_global_set():
    rng = np.random.default_rng(3)
    for _ in range(20):
        nb, k = int(rng.integers(2, 40)), int(rng.integers(1, 8))
        sal = rng.standard_normal(nb)
        rp_p, ci_p = oracle.schedule_from_salience(sal, 0, 0, k, per_row=True)
        rp_g, ci_g = oracle.schedule_from_salience(sal, 0, 0, k, per_row=False)
        assert np.array_equal(ci_p[rp_p[-2]:], ci_g[rp_g[-2]:])


@pytest.mark.parametrize("seed", range(6))
def test_interval_characterisation(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(5, 60))
    k = int(rng.integers(1, 10))
    s, r = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    sal = np.round(rng.standard_normal(nb), 1)  # ties happen: ranked by index
    better = lambda u, j: sal[u] > sal[j] or (sal[u] == sal[j] and u < j)
    e = []
    for j in range(nb):
        idx = [u for u in range(nb) if better(u, j)]
        e.append(sorted(idx)[k - 1] if len(idx) >= k else nb)
    rows = [[j for j in range(i + 1) if j < s or j >= i - r or j < i + 1 <= e[j]] for i in range(nb)]
    want_rp = np.cumsum([0] + [len(x) for x in rows])
    rp, ci = oracle.schedule_from_salience(sal, s, r, k, per_row=True)
    assert np.array_equal(rp, want_rp)
    assert np.array_equal(ci, np.array([j for x in rows for j in x], dtype=np.int32))
