"""Pins for the oracle at 32-row blocks, against facts fixed outside it.

The forward and the builder also take schedules over 32-row blocks; the
oracle's functions are written for any block size, and these checks pin them
at 32:

* dense 32-row CSR = causal attention (torch's scaled_dot_product_attention in
  float64 on the CPU, is_causal=True);
* arbitrary 32-row CSRs = that routine with an explicit boolean mask built here
  by a Kronecker expansion of the block matrix;
* lse = scipy's logsumexp over the same masked scores;
* a 64-row CSR and its 32-row expansion (row 2I + a lists 2J + b for every J
  of row I, b = 0, 1, kept within the row's causal range) allow the same keys,
  so the outputs agree;
* the 64-row centroids are the means of the two 32-row centroids they cover;
* the gradients over a 32-row CSR = torch's autograd through that routine under
  the explicit mask, and those of a 64-row CSR = those of its 32-row expansion.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads


def _qkv(shape, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape) for _ in range(3)]


def _kron_mask(row_ptr, col_idx, S, block):
    nb = -(-S // block)
    bm = np.zeros((nb, nb))
    for i in range(nb):
        for j in col_idx[row_ptr[i] : row_ptr[i + 1]]:
            bm[i, j] = 1.0
    return (np.kron(bm, np.ones((block, block)))[:S, :S] > 0) & np.tril(np.ones((S, S), dtype=bool))


def _sdpa(q, k, v, mask=None, causal=False):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=m,
                                                            is_causal=causal).numpy()


def _expand_to_32(rp, ci, S):
    nb64, nb32 = len(rp) - 1, -(-S // 32)
    rows = []
    for i in range(nb32):
        I = i // 2
        rows.append([2 * J + b for J in ci[rp[I] : rp[I + 1]] for b in (0, 1) if 2 * J + b <= i])
    rp32 = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci32 = np.array([c for r in rows for c in r], np.int32)
    assert nb64 == -(-S // 64)
    return rp32, ci32


@pytest.mark.parametrize("S,D", [(32, 16), (200, 32), (256, 64)])
def test_dense_32_row_csr_equals_causal_sdpa(S, D):
    q, k, v = _qkv((S, D), seed=S + 1)
    rp, ci = oracle.dense_causal_schedule(-(-S // 32))
    got = oracle.masked_attention(q, k, v, rp, ci, 32)
    assert np.max(np.abs(got - _sdpa(q, k, v, causal=True))) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_random_32_row_csr_equals_masked_sdpa(seed):
    S, D = 32 * 9 + 13, 32
    q, k, v = _qkv((2, 2, S, D), seed=40 + seed)
    nb = -(-S // 32)
    rp, ci = workloads.random_csr(nb, seed=seed, density=0.4, allow_empty=True)
    mask = _kron_mask(rp, ci, S, 32)
    got = oracle.masked_attention(q, k, v, rp, ci, 32)
    want = _sdpa(q, k, v, mask=mask)
    visible = mask.any(axis=1)  # rows with no allowed key: 0 by the schedule's rule
    assert np.max(np.abs(got[..., visible, :] - want[..., visible, :])) < 1e-12
    assert not np.any(got[..., ~visible, :])


def test_lse_at_32_row_blocks_equals_logsumexp():
    S, D = 32 * 6 + 5, 16
    q, k, _ = _qkv((S, D), seed=51)
    nb = -(-S // 32)
    rp, ci = workloads.random_csr(nb, seed=5, density=0.5, allow_empty=True)
    mask = _kron_mask(rp, ci, S, 32)
    scores = (q @ k.T) / np.sqrt(D)
    want = scipy.special.logsumexp(np.where(mask, scores, -np.inf), axis=1)
    got = oracle.masked_lse(q, k, rp, ci, 32)
    assert np.array_equal(np.isneginf(got), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.max(np.abs(got[fin] - want[fin])) < 1e-12


@pytest.mark.parametrize("S", [256, 300, 64 * 7 - 20])
def test_64_row_csr_and_its_32_row_expansion_agree(S):
    q, k, v = _qkv((S, 32), seed=S)
    nb = -(-S // 64)
    rp, ci = workloads.random_csr(nb, seed=S, density=0.5)
    rp32, ci32 = _expand_to_32(rp, ci, S)
    a = oracle.masked_attention(q, k, v, rp, ci, 64)
    b = oracle.masked_attention(q, k, v, rp32, ci32, 32)
    assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("S", [1024, 1000, 992])
def test_64_row_centroids_are_means_of_32_row_ones(S):
    keys = np.random.default_rng(9).standard_normal((S, 8))
    c32 = oracle.block_centroids(keys, 32)
    c64 = oracle.block_centroids(keys, 64)
    rows32 = np.minimum(32, S - 32 * np.arange(c32.shape[0]))
    assert c32.shape[0] == -(-S // 32)
    for J in range(c64.shape[0]):
        parts = [2 * J, 2 * J + 1][: c32.shape[0] - 2 * J]
        w = rows32[parts]
        np.testing.assert_allclose(c64[J], (c32[parts] * w[:, None]).sum(0) / w.sum(), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("seed", range(2))
def test_gradients_at_32_row_blocks_equal_masked_sdpa_autograd(seed):
    """dq, dk and dv over a 32-row CSR equal torch's autograd through its own
    scaled-dot-product attention under the explicit 32-row mask (float64 on the
    CPU; ragged S, two lanes; every row lists at least one block)."""
    S, D = 32 * 5 + 11, 16
    rng = np.random.default_rng(70 + seed)
    q, k, v, do = (rng.standard_normal((1, 2, S, D)) for _ in range(4))
    nb = -(-S // 32)
    rp, ci = workloads.random_csr(nb, seed=seed + 7, density=0.4)
    dq, dk, dv, out, _ = oracle.attention_backward(q, k, v, do, rp, ci, block=32)
    mask = torch.from_numpy(_kron_mask(rp, ci, S, 32))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(out, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("S", [256, 300])
def test_gradients_of_64_row_csr_and_its_32_row_expansion_agree(S):
    q, k, v, do = _qkv((S, 32), seed=S + 3) + [np.random.default_rng(S).standard_normal((S, 32))]
    nb = -(-S // 64)
    rp, ci = workloads.random_csr(nb, seed=S + 1, density=0.5)
    rp32, ci32 = _expand_to_32(rp, ci, S)
    a = oracle.attention_backward(q, k, v, do, rp, ci, block=64)[:3]
    b = oracle.attention_backward(q, k, v, do, rp32, ci32, block=32)[:3]
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < 1e-12
