"""Pins for the oracle's dense masked attention, against facts fixed outside it.

* torch's scaled_dot_product_attention in float64 on the CPU (a library
  routine): with is_causal=True for the dense CSR, and with an explicit boolean
  mask, built here from the CSR by a Kronecker expansion, for arbitrary CSRs;
* closed forms: query 0 sees only key 0, so its output is v_0; with q = 0 the
  softmax is uniform, so each output is the mean of the allowed values;
* a per-query brute-force loop in plain Python (math.exp) on tiny inputs;
* the block loop with running max and denominator rescaled by exp(m_prev -
  m_new), which the mirror page's Rust-port note says equals dense masked
  attention (there to 1e-12 in fp64).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _qkv(shape, seed, dtype=np.float64):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape).astype(dtype) for _ in range(3)]


def _block_mask(row_ptr, col_idx, S, block):
    """Key-allowed mask from CSR block sets expanded with np.kron, plus tril."""
    nb = -(-S // block)
    bm = np.zeros((nb, nb))
    for i in range(nb):
        for j in col_idx[row_ptr[i] : row_ptr[i + 1]]:
            bm[i, j] = 1.0
    full = np.kron(bm, np.ones((block, block)))[:S, :S] > 0
    return full & np.tril(np.ones((S, S), dtype=bool))


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], attn_mask=m, is_causal=causal, scale=scale
    ).numpy()


@pytest.mark.parametrize("S,D", [(64, 16), (200, 32), (256, 64)])
def test_dense_csr_equals_causal_sdpa(S, D):
    q, k, v = _qkv((S, D), seed=S)
    rp, ci = oracle.dense_causal_schedule(-(-S // 64))
    got = oracle.masked_attention(q, k, v, rp, ci, 64)
    want = _sdpa(q, k, v, causal=True)
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_random_csr_equals_masked_sdpa(seed):
    S, D = 64 * 5 + 23, 32
    q, k, v = _qkv((2, 3, S, D), seed=seed)
    nb = -(-S // 64)
    rp, ci = workloads.random_csr(nb, seed=seed, density=0.4)
    got = oracle.masked_attention(q, k, v, rp, ci, 64)
    mask = _block_mask(rp, ci, S, 64)
    want = _sdpa(q, k, v, mask=mask)
    assert np.max(np.abs(got - want)) < 1e-12


def test_explicit_scale_matches_sdpa():
    S, D = 128, 64
    q, k, v = _qkv((S, D), seed=7)
    rp, ci = oracle.dense_causal_schedule(2)
    got = oracle.masked_attention(q, k, v, rp, ci, 64, scale=0.37)
    want = _sdpa(q, k, v, causal=True, scale=0.37)
    assert np.max(np.abs(got - want)) < 1e-12


def test_query_zero_is_v0():
    q, k, v = _qkv((4, 256, 64), seed=1)[0:3]
    q, k, v = q[0], k[0], v[0]
    rp, ci = workloads.random_csr(4, seed=3, density=0.5)
    got = oracle.masked_attention(q, k, v, rp, ci, 64)
    assert np.array_equal(got[0], v[0])


def test_zero_query_gives_mean_of_allowed_values():
    S, D = 64 * 4, 16
    _, k, v = _qkv((S, D), seed=2)
    q = np.zeros((S, D))
    rp, ci = workloads.random_csr(4, seed=5, density=0.5)
    got = oracle.masked_attention(q, k, v, rp, ci, 64)
    mask = _block_mask(rp, ci, S, 64)
    for t in range(S):
        assert np.allclose(got[t], v[mask[t]].mean(axis=0), rtol=0, atol=1e-13)


def test_brute_force_loop_tiny():
    S, D, block = 40, 5, 8
    q, k, v = _qkv((S, D), seed=4)
    rp, ci = workloads.random_csr(5, seed=8, density=0.5, allow_empty=True)
    got = oracle.masked_attention(q, k, v, rp, ci, block)
    scale = 1 / math.sqrt(D)
    for t in range(S):
        i = t // block
        listed = set(int(x) for x in ci[rp[i] : rp[i + 1]])
        keys = [u for u in range(t + 1) if u // block in listed]
        if not keys:
            assert np.all(got[t] == 0)
            continue
        z = [scale * sum(q[t, d] * k[u, d] for d in range(D)) for u in keys]
        zm = max(z)
        w = [math.exp(x - zm) for x in z]
        tot = sum(w)
        for d in range(D):
            want = sum(wi * v[u, d] for wi, u in zip(w, keys)) / tot
            assert abs(got[t, d] - want) < 1e-12


def test_empty_rows_give_zero_output():
    S, D = 192, 8
    q, k, v = _qkv((S, D), seed=6)
    rp = np.array([0, 0, 1, 1], dtype=np.int32)  # block rows 0 and 2 empty
    ci = np.array([0], dtype=np.int32)
    got = oracle.masked_attention(q, k, v, rp, ci, 64)
    assert np.all(got[0:64] == 0) and np.all(got[128:] == 0)
    z = k[0:64] @ q[64] / math.sqrt(D)  # query 64 sees every key of block 0
    w = np.exp(z - z.max())
    assert np.allclose(got[64], (w / w.sum()) @ v[0:64], rtol=0, atol=1e-13)


def test_future_or_out_of_range_blocks_select_nothing():
    S, D = 128, 8
    q, k, v = _qkv((S, D), seed=9)
    rp_a = np.array([0, 1, 2], dtype=np.int32)
    ci_a = np.array([0, 1], dtype=np.int32)
    rp_b = np.array([0, 3, 5], dtype=np.int32)
    ci_b = np.array([0, 1, 7, 1, 9], dtype=np.int32)  # block 1 in row 0 is in the future
    a = oracle.masked_attention(q, k, v, rp_a, ci_a, 64)
    b = oracle.masked_attention(q, k, v, rp_b, ci_b, 64)
    assert np.array_equal(a, b)


def _online_block_loop(q, k, v, row_ptr, col_idx, block, scale):
    """Per query block: visit the CSR row's key blocks keeping a running max m
    and denominator l per row, rescaling the accumulator by exp(m_prev - m_new)."""
    S, D = q.shape
    out = np.zeros((S, D))
    for i in range(-(-S // block)):
        rows = np.arange(i * block, min(S, (i + 1) * block))
        m = np.full(rows.shape[0], -np.inf)
        l = np.zeros(rows.shape[0])
        acc = np.zeros((rows.shape[0], D))
        for j in col_idx[row_ptr[i] : row_ptr[i + 1]]:
            cols = np.arange(j * block, min(S, (j + 1) * block))
            z = (q[rows] @ k[cols].T) * scale
            z[cols[None, :] > rows[:, None]] = -np.inf
            m_new = np.maximum(m, z.max(axis=1))
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.where(np.isfinite(z), np.exp(z - m_new[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        nz = l > 0
        out[rows[nz]] = acc[nz] / l[nz, None]
    return out


@pytest.mark.parametrize("seed", range(3))
def test_online_block_loop_equals_dense_masked(seed):
    S, D = 64 * 6 + 10, 64
    q, k, v = _qkv((S, D), seed=20 + seed)
    keys = workloads.cast(k, "bf16")
    rp, ci, _ = oracle.build_schedule(keys, 64, 1, 1, 2)
    got = oracle.masked_attention(q, k, v, rp, ci, 64)
    want = _online_block_loop(q, k, v, rp, ci, 64, 1 / math.sqrt(D))
    assert np.max(np.abs(got - want)) < 1e-12


def test_rows_api_matches_full():
    S, D = 300, 16
    q, k, v = _qkv((S, D), seed=31)
    rp, ci = workloads.random_csr(5, seed=2, density=0.5)
    full = oracle.masked_attention(q, k, v, rp, ci, 64)
    rows = np.array([0, 5, 63, 64, 200, 299])
    part = oracle.masked_attention_rows(q, k, v, rp, ci, rows, 64)
    assert np.allclose(part, full[rows], rtol=0, atol=1e-14)
