"""Pins of the gradient oracle (oracle/attention_grad.py) and of the schedule
transpose (oracle.schedule.transpose_schedule) to things other than themselves:

* central finite differences of the pinned forward oracle (the definition of
  the function being differentiated), on tiny ragged inputs with small blocks;
* torch's autograd through its own causal scaled-dot-product attention, on the
  full-causal schedule (a library routine the dense schedule reduces to);
* identities the gradients must satisfy (key and value gradient sums), closed
  forms of the log-sum-exp (one allowed key, equal scores), empty rows;
* closed forms of the transpose of the dense causal and fixed-segment schedules
  and a hand-worked example (tests/golden/transpose_example.txt).
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from conftest import read_golden_rows


def _tiny(seed, S=18, D=3, lanes_shape=()):
    rng = np.random.default_rng(seed)
    shp = tuple(lanes_shape) + (S, D)
    return tuple(rng.standard_normal(shp) for _ in range(4))


def _loss(q, k, v, do, rp, ci, block):
    return float((oracle.masked_attention(q, k, v, rp, ci, block=block) * do).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_match_central_differences(seed):
    """Every element of dq, dk, dv against a central difference of
    sum(dO * attention(q, k, v)), with 5 blocks of 4 and a ragged last block of 2."""
    block, S, D = 4, 18, 3
    q, k, v, do = _tiny(seed, S, D)
    rp, ci = workloads.random_csr(-(-S // block), seed=seed, density=0.5)
    dq, dk, dv, out, lse = oracle.attention_backward(q, k, v, do, rp, ci, block=block)
    h = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(q, k, v, do, rp, ci, block)
            x[idx] = keep - h
            lm = _loss(q, k, v, do, rp, ci, block)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_directional_derivative_batched_lanes_and_scale():
    """[B, H, S, D] with an explicit scale: <grad, E> against a central difference
    along a random direction E of every input at once."""
    block, S, D = 8, 37, 5
    q, k, v, do = _tiny(7, S, D, (2, 3))
    rp, ci = workloads.random_csr(-(-S // block), seed=7, density=0.4)
    scale = 0.3
    dq, dk, dv, _, _ = oracle.attention_backward(q, k, v, do, rp, ci, block=block, scale=scale)
    rng = np.random.default_rng(8)
    eq, ek, ev = (rng.standard_normal(q.shape) for _ in range(3))

    def f(t):
        o = oracle.masked_attention(q + t * eq, k + t * ek, v + t * ev, rp, ci, block=block, scale=scale)
        return float((o * do).sum())

    h = 1e-5
    fd = (f(h) - f(-h)) / (2 * h)
    an = float((dq * eq).sum() + (dk * ek).sum() + (dv * ev).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_dense_schedule_matches_torch_causal_sdpa_autograd():
    """Full-causal schedule: the gradients equal torch's autograd of its own causal
    scaled-dot-product attention in float64 (ragged S, two lanes)."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    block, S, D = 16, 70, 8
    q, k, v, do = _tiny(11, S, D, (1, 2))
    rp, ci = oracle.dense_causal_schedule(-(-S // block))
    dq, dk, dv, out, lse = oracle.attention_backward(q, k, v, do, rp, ci, block=block)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(out, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_gradient_sum_identities(seed):
    """Row softmax: sum over keys of dS_t is 0 for every query row, so the key
    gradients sum to 0; probabilities sum to 1 on rows with an allowed key, so
    the value gradients sum to the upstream gradients of those rows."""
    block, S, D = 4, 30, 4
    q, k, v, do = _tiny(seed, S, D)
    rp, ci = workloads.random_csr(-(-S // block), seed=seed, density=0.3, allow_empty=True)
    dq, dk, dv, out, lse = oracle.attention_backward(q, k, v, do, rp, ci, block=block)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    live = np.isfinite(lse)
    np.testing.assert_allclose(dv.sum(axis=0), do[live].sum(axis=0), atol=1e-12)
    # rows with no allowed key: zero output, zero query gradient, lse -inf
    assert (~live).any(), "the seed must give at least one empty row"
    assert np.all(out[~live] == 0.0) and np.all(dq[~live] == 0.0)
    assert np.all(np.isneginf(lse[~live]))


def test_lse_closed_forms():
    """lse of a row with one allowed key is its scaled score; with n equal scores
    it is that score plus log n; the output the gradient routine returns is the
    pinned forward oracle's."""
    block, S, D = 4, 12, 3
    q, k, v, do = _tiny(5, S, D)
    rp, ci = oracle.dense_causal_schedule(3)
    scale = 0.7
    lse = oracle.masked_lse(q, k, rp, ci, block=block, scale=scale)
    assert lse[0] == pytest.approx(scale * float(q[0] @ k[0]), abs=1e-14)
    k_eq = np.tile(k[:1], (S, 1))
    lse_eq = oracle.masked_lse(q, k_eq, rp, ci, block=block, scale=scale)
    for t in range(S):
        assert lse_eq[t] == pytest.approx(scale * float(q[t] @ k[0]) + math.log(t + 1), abs=1e-12)
    _, _, _, out, lse2 = oracle.attention_backward(q, k, v, do, rp, ci, block=block, scale=scale)
    np.testing.assert_allclose(out, oracle.masked_attention(q, k, v, rp, ci, block=block, scale=scale),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_rows_routine_equals_full_routine():
    block, S, D = 8, 53, 6
    q, k, v, do = _tiny(9, S, D)
    rp, ci = workloads.random_csr(-(-S // block), seed=9, density=0.4)
    dq, dk, dv, _, lse = oracle.attention_backward(q, k, v, do, rp, ci, block=block)
    qr = np.array([0, 7, 8, 31, 52])
    kr = np.array([0, 1, 15, 40, 52])
    a, b, c, d = oracle.attention_backward_rows(q, k, v, do, rp, ci, qr, kr, block=block, chunk=16)
    np.testing.assert_allclose(a, dq[qr], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b, dk[kr], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(c, dv[kr], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(d, lse[qr], rtol=1e-13, atol=1e-13)


def test_value_gradient_of_first_row_alone():
    """Query 0 sees key 0 only (P = 1): it adds dO_0 to dV_0 and gets dQ_0 = 0."""
    block, S, D = 4, 8, 3
    q, k, v, do = _tiny(6, S, D)
    rp = np.array([0, 1, 2], np.int32)  # row 0 lists block 0; row 1 lists block 1
    ci = np.array([0, 1], np.int32)
    dq, dk, dv, out, lse = oracle.attention_backward(q, k, v, do, rp, ci, block=block)
    np.testing.assert_allclose(dq[0], 0.0, atol=1e-15)
    np.testing.assert_allclose(out[0], v[0], atol=1e-15)
    # keys of block 0 are seen by queries 0..3 only
    mask = np.tril(np.ones((4, 4), bool))
    z = (q[:4] @ k[:4].T) / math.sqrt(D)
    p = np.where(mask, np.exp(z - z.max(axis=1, keepdims=True)), 0.0)
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(dv[:4], p.T @ do[:4], atol=1e-13)


# ---------------------------------------------------------------- transpose


def test_transpose_of_dense_causal_is_closed_form():
    for nb in (1, 2, 7, 64):
        cp, ri = oracle.transpose_schedule(*oracle.dense_causal_schedule(nb))
        assert cp.dtype == np.int32 and ri.dtype == np.int32
        expect_ptr = np.concatenate([[0], np.cumsum([nb - j for j in range(nb)])])
        np.testing.assert_array_equal(cp, expect_ptr)
        for j in range(nb):
            np.testing.assert_array_equal(ri[cp[j] : cp[j + 1]], np.arange(j, nb))


@pytest.mark.parametrize("nb,L", [(64, 8), (64, 4), (13, 5), (5, 1), (6, 9)])
def test_transpose_of_segments_is_closed_form(nb, L):
    """Column j of the L-block segment schedule lists j .. min(nb, L*(j//L + 1)) - 1."""
    cp, ri = oracle.transpose_schedule(*oracle.fixed_segment_schedule(nb, L))
    for j in range(nb):
        np.testing.assert_array_equal(ri[cp[j] : cp[j + 1]], np.arange(j, min(nb, L * (j // L + 1))))


def test_transpose_golden_example():
    """Hand-worked example with out-of-range and above-diagonal entries."""
    rows = read_golden_rows("transpose_example.txt")
    sect = {}
    for line in rows:
        key, _, val = line.partition(":")
        sect[key.strip()] = [int(x) for x in val.split()]
    cp, ri = oracle.transpose_schedule(np.array(sect["row_ptr"], np.int32), np.array(sect["col_idx"], np.int32))
    np.testing.assert_array_equal(cp, sect["col_ptr"])
    np.testing.assert_array_equal(ri, sect["row_idx"])


def test_transpose_keeps_every_causal_entry():
    """For a causal ascending CSR the column view has the same number of entries,
    and entry (i, j) is in column j exactly when it is in row i."""
    for seed in range(4):
        rp, ci = workloads.random_csr(23, seed=seed, density=0.35)
        cp, ri = oracle.transpose_schedule(rp, ci)
        assert cp[-1] == rp[-1]
        pairs_r = {(i, int(j)) for i in range(23) for j in ci[rp[i] : rp[i + 1]]}
        pairs_c = {(int(i), j) for j in range(23) for i in ri[cp[j] : cp[j + 1]]}
        assert pairs_r == pairs_c
