"""GPU parity of the backward surface, through the C ABI (the ctypes binding):

* tsa_schedule_transpose: bit-exact against oracle.transpose_schedule (and the
  closed forms of the dense and segment schedules), including rows with entries
  the kernels skip;
* tsa_scheduled_attention_fwd_lse: lse against the oracle's fp64 log-sum-exp,
  and the output bit-identical to tsa_scheduled_attention_fwd;
* tsa_scheduled_attention_bwd: dq, dk, dv against the oracle's fp64 closed form
  on several tiles with ragged tails, empty rows and D 64/128; at the batched
  workload's full size on sampled rows (dq rows from their own P row, dk/dv rows
  from full P columns of two lanes); the autograd wrapper equals the direct call.

Tolerances (derived from the arithmetic).  P and dS are rounded to the input
dtype as MFMA operands (relative 2^-9 for bf16, 2^-12 for fp16 per element), the
forward's output O that enters Delta = dO . O is rounded the same way, lse
comes from the forward's denominator of rounded probabilities, and the result
is rounded once more.  Each gradient element sums many such terms with
independent rounding signs, so the error is a small multiple of the unit
roundoff times the gradient's own scale.  Bar per gradient g:
    max |g - g_ref| <= TOL * max |g_ref|   and   ||g - g_ref||_2 <= TOL_RMS * ||g_ref||_2
with TOL = 1e-2 / 2e-3 (the forward's bars, taken relative to the gradient's
scale) and TOL_RMS = 5e-3 / 1e-3 for bf16 / fp16; measured: max 4.3e-3 / 5.5e-4,
rms 2.8e-3 / 3.3e-4.  lse: |err| <= 4e-3
(bf16) / 1e-3 (fp16): the denominator sums probabilities rounded to the input type
(relative error at most 2^-9 / 2^-12 in the sum, worst case with equal signs).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp16": 2e-3}
TOL_RMS = {"bf16": 5e-3, "fp16": 1e-3}
TOL_LSE = {"bf16": 4e-3, "fp16": 1e-3}
DEV = "cuda:0"


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _dev(x):
    return torch.as_tensor(np.asarray(x)).to(DEV)


def _compare(name, got, ref, dtype):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    scale = float(np.abs(ref).max())
    rms = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    print(f"{name}: max err {err.max():.3e}  max|ref| {scale:.3e}  rel {err.max() / max(scale, 1e-30):.3e}  "
          f"rms rel {rms:.3e}")
    assert np.all(np.isfinite(g)), name
    assert err.max() <= TOL[dtype] * scale, (name, err.max(), scale)
    assert rms <= TOL_RMS[dtype], (name, rms)


# ----------------------------------------------------------------- transpose


def _accepted_rows(rp, ci):
    """Entries of each row the attention kernels accept (the rule in include/tsa.h):
    within 0..i and above every earlier entry of the row that lies in 0..i."""
    rows = []
    nnz = len(ci)
    for i in range(len(rp) - 1):
        lo = min(max(int(rp[i]), 0), nnz)
        hi = max(min(int(rp[i + 1]), nnz), lo)
        best, keep = -1, []
        for c in ci[lo:hi]:
            c = int(c)
            if 0 <= c <= i:
                if c > best:
                    keep.append(c)
                best = max(best, c)
        rows.append(keep)
    return rows


def _check_transpose(tsa, rp, ci):
    cp_g, ri_g = tsa.schedule_transpose(_dev(rp.astype(np.int32)), _dev(ci.astype(np.int32)))
    cp_o, ri_o = oracle.transpose_schedule(rp, ci)
    np.testing.assert_array_equal(cp_g.cpu().numpy(), cp_o)
    np.testing.assert_array_equal(ri_g.cpu().numpy(), ri_o)


@pytest.mark.parametrize("nb", [1, 2, 5, 31, 32, 33, 64, 100, 512])
def test_transpose_dense(tsa, nb):
    _check_transpose(tsa, *oracle.dense_causal_schedule(nb))


def test_transpose_dense_largest(tsa):
    nb = 4096
    rp, ci = tsa.dense_causal_schedule(nb, DEV)
    cp, ri = tsa.schedule_transpose(rp, ci)
    cp, ri = cp.cpu().numpy(), ri.cpu().numpy()
    expect = np.concatenate([[0], np.cumsum(nb - np.arange(nb))])
    np.testing.assert_array_equal(cp, expect)
    j = np.repeat(np.arange(nb), nb - np.arange(nb))
    np.testing.assert_array_equal(ri, j + (np.arange(len(ri)) - expect[j]))


@pytest.mark.parametrize("nb,L", [(64, 8), (64, 4), (13, 5), (512, 8), (70, 64)])
def test_transpose_segments(tsa, nb, L):
    _check_transpose(tsa, *oracle.fixed_segment_schedule(nb, L))


@pytest.mark.parametrize("seed,nb,density,empty", [(0, 64, 0.3, False), (1, 100, 0.1, True),
                                                   (2, 257, 0.05, True), (3, 7, 0.9, False)])
def test_transpose_random(tsa, seed, nb, density, empty):
    _check_transpose(tsa, *workloads.random_csr(nb, seed=seed, density=density, allow_empty=empty))


def test_transpose_of_built_schedules(tsa):
    for name in ("single_s1024_d64_f16", "single_s4096_d64_f16_mix8", "batched_b4h16_s4096_d64_bf16",
                 "long_b1h32_s32768_d64_bf16_mix32"):
        w = workloads.WORKLOADS[name]
        q, k, v = workloads.make_qkv(w, shape=(w.S, w.D))
        rp, ci = tsa.build_schedule(k.to(DEV), 64, w.sink, w.local_radius, w.topk)
        _check_transpose(tsa, rp.cpu().numpy(), ci.cpu().numpy())


def test_transpose_skips_what_the_kernels_skip(tsa):
    """Rows with descending, repeated, negative and above-diagonal entries: the
    column view holds exactly the entries the attention kernels accept."""
    rng = np.random.default_rng(5)
    nb = 90
    rows = [rng.integers(-3, nb + 3, size=int(rng.integers(0, 40))) for _ in range(nb)]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    acc = _accepted_rows(rp, ci)
    rp2 = np.concatenate([[0], np.cumsum([len(r) for r in acc])]).astype(np.int32)
    ci2 = np.array([c for r in acc for c in r], np.int32)
    cp_g, ri_g = tsa.schedule_transpose(_dev(rp), _dev(ci))
    cp_o, ri_o = oracle.transpose_schedule(rp2, ci2)
    np.testing.assert_array_equal(cp_g.cpu().numpy(), cp_o)
    np.testing.assert_array_equal(ri_g.cpu().numpy(), ri_o)


def test_transpose_empty(tsa):
    cp, ri = tsa.schedule_transpose(_dev(np.zeros(1, np.int32)), _dev(np.zeros(0, np.int32)))
    assert cp.cpu().tolist() == [0] and ri.numel() == 0
    cp, ri = tsa.schedule_transpose(_dev(np.zeros(4, np.int32)), _dev(np.zeros(0, np.int32)))
    assert cp.cpu().tolist() == [0, 0, 0, 0] and ri.numel() == 0


# ----------------------------------------------------------------- forward lse


def _inputs(shape, dtype, seed, keys="normal"):
    w = workloads.Workload("t", tuple(shape), dtype, keys, 4 if keys == "mixture" else 0, seed=seed)
    q, k, v = workloads.make_qkv(w)
    do = workloads.random_normal(shape, dtype, seed + 1000)
    return q, k, v, do


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", [(1000, 64), (2, 3, 640, 128), (37, 64)])
def test_forward_lse(tsa, dtype, shape):
    q, k, v, _ = _inputs(shape, dtype, 21)
    S = shape[-2]
    nb = -(-S // 64)
    rp, ci = workloads.random_csr(nb, seed=4, density=0.4, allow_empty=nb > 2)
    qd, kd, vd, rpd, cid = (x.to(DEV) for x in (q, k, v, torch.from_numpy(rp), torch.from_numpy(ci)))
    out1 = tsa.scheduled_attention(qd, kd, vd, rpd, cid)
    out2, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, return_lse=True)
    assert torch.equal(out1, out2)
    ref = oracle.masked_lse(q, k, rp, ci)
    got = lse.cpu().numpy().astype(np.float64)
    live = np.isfinite(ref)
    assert np.all(np.isneginf(got[~live])), "rows with no allowed key must give -inf"
    err = np.abs(got[live] - ref[live]).max()
    print(f"lse max err {err:.3e}")
    assert err <= TOL_LSE[dtype]


# ----------------------------------------------------------------- backward


def _run_backward(tsa, q, k, v, do, rp, ci, scale=None):
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    rpd, cid = _dev(rp.astype(np.int32)), _dev(ci.astype(np.int32))
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, sm_scale=scale, return_lse=True)
    cp, ri = tsa.schedule_transpose(rpd, cid)
    return tsa.scheduled_attention_backward(qd, kd, vd, out, dod, lse, rpd, cid, cp, ri, sm_scale=scale)


def _check_backward(tsa, shape, dtype, rp, ci, seed=31, keys="normal", scale=None):
    q, k, v, do = _inputs(shape, dtype, seed, keys)
    dq, dk, dv = _run_backward(tsa, q, k, v, do, rp, ci, scale)
    rdq, rdk, rdv, _, _ = oracle.attention_backward(q, k, v, do, rp, ci, scale=scale)
    _compare("dq", dq, rdq, dtype)
    _compare("dk", dk, rdk, dtype)
    _compare("dv", dv, rdv, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", [(1000, 64), (2, 3, 640, 64), (1, 2, 700, 128), (37, 64), (64, 128)])
def test_backward_random_schedule(tsa, dtype, shape):
    nb = -(-shape[-2] // 64)
    rp, ci = workloads.random_csr(nb, seed=7, density=0.4)
    _check_backward(tsa, shape, dtype, rp, ci)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_backward_dense_schedule(tsa, dtype):
    _check_backward(tsa, (1, 2, 1088, 64), dtype, *oracle.dense_causal_schedule(17))


def test_backward_dense_d128(tsa):
    _check_backward(tsa, (1, 1, 960, 128), "bf16", *oracle.dense_causal_schedule(15))


def test_backward_segment_schedule(tsa):
    _check_backward(tsa, (2, 2, 1024, 64), "bf16", *oracle.fixed_segment_schedule(16, 4))


def test_backward_empty_rows_and_scale(tsa):
    rp, ci = workloads.random_csr(20, seed=9, density=0.2, allow_empty=True)
    assert np.any(np.diff(rp) == 0)
    _check_backward(tsa, (1, 2, 1270, 64), "fp16", rp, ci, scale=0.05)


def test_backward_topology_schedule(tsa):
    w = workloads.WORKLOADS["single_s4096_d64_f16_mix8"]
    q, k, v = workloads.make_qkv(w)
    rp, ci = tsa.build_schedule(k.to(DEV), 64, w.sink, w.local_radius, w.topk)
    _check_backward(tsa, (w.S, w.D), "fp16", rp.cpu().numpy(), ci.cpu().numpy(), seed=w.seed, keys="mixture")


def test_backward_empty_problem(tsa):
    z = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device=DEV)
    rp = torch.zeros(1, dtype=torch.int32, device=DEV)
    ci = torch.zeros(0, dtype=torch.int32, device=DEV)
    lse = torch.zeros((1, 1, 0), dtype=torch.float32, device=DEV)
    dq, dk, dv = tsa.scheduled_attention_backward(z, z, z, z, z, lse, rp, ci, rp, ci)
    assert dq.numel() == 0


def test_backward_batched_full_size_sampled(tsa):
    """The batched workload at full size ([4,16,4096,64] bf16, its topology
    schedule) in the launch configuration the bench times: dq on sampled query
    rows of 4 lanes, dk and dv on sampled key rows of 2 lanes."""
    w = workloads.WORKLOADS["batched_b4h16_s4096_d64_bf16"]
    q, k, v = workloads.make_qkv(w)
    do = workloads.random_normal(w.shape, w.dtype, 4242)
    rp, ci = tsa.build_schedule(k[0, 0].contiguous().to(DEV), 64, w.sink, w.local_radius, w.topk)
    rp_h, ci_h = rp.cpu().numpy(), ci.cpu().numpy()
    dq, dk, dv = _run_backward(tsa, q, k, v, do, rp_h, ci_h)
    rng = np.random.default_rng(1)
    q_rows = np.unique(np.concatenate([[0, 63, 64, 4095], rng.integers(0, w.S, 60)]))
    k_rows = np.unique(np.concatenate([[0, 1, 4032, 4095], rng.integers(0, w.S, 60)]))
    for (b, hh) in [(0, 0), (3, 15), (1, 7), (2, 2)]:
        full = (b, hh) in [(0, 0), (3, 15)]
        rq, rk, rv, _ = oracle.attention_backward_rows(
            q[b, hh], k[b, hh], v[b, hh], do[b, hh], rp_h, ci_h, q_rows, k_rows if full else [])
        _compare(f"dq[{b},{hh}]", dq[b, hh][torch.from_numpy(q_rows).to(DEV)], rq, "bf16")
        if full:
            kr = torch.from_numpy(k_rows).to(DEV)
            _compare(f"dk[{b},{hh}]", dk[b, hh][kr], rk, "bf16")
            _compare(f"dv[{b},{hh}]", dv[b, hh][kr], rv, "bf16")


def test_autograd_wrapper_matches_direct_call(tsa):
    q, k, v, do = _inputs((2, 2, 512, 64), "bf16", 77)
    rp, ci = workloads.random_csr(8, seed=3, density=0.5)
    dq, dk, dv = _run_backward(tsa, q, k, v, do, rp, ci)
    qd, kd, vd = (x.to(DEV).requires_grad_(True) for x in (q, k, v))
    out = tsa.attention(qd, kd, vd, _dev(rp), _dev(ci))
    out.backward(do.to(DEV))
    assert torch.equal(qd.grad, dq) and torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)


def test_backward_is_deterministic(tsa):
    q, k, v, do = _inputs((1, 4, 2048, 64), "bf16", 5)
    rp, ci = workloads.random_csr(32, seed=5, density=0.5)
    a = _run_backward(tsa, q, k, v, do, rp, ci)
    b = _run_backward(tsa, q, k, v, do, rp, ci)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
