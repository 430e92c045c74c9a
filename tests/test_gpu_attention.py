"""Parity of the HIP scheduled-attention kernel with the fp64 oracle.

The kernel is called through the C ABI (via the thin binding) exactly as the
bench calls it.  Tolerances: max abs error <= 2e-3 for fp16 and <= 1e-2 for
bf16 against the fp64 dense masked attention on the same mask.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1e-2}
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as mod

    return mod


def _dev(*ts):
    return [t.to("cuda:0") for t in ts]


def _csr_dev(rp, ci):
    return (torch.from_numpy(np.asarray(rp, np.int32)).to("cuda:0"),
            torch.from_numpy(np.asarray(ci, np.int32)).to("cuda:0"))


def _max_err(got, want):
    return float(np.max(np.abs(got.detach().to("cpu", torch.float64).numpy() - want))) if want.size else 0.0


CASES = [
    # (shape, dtype, schedule kind)
    ((64, 64), "fp16", "dense"),
    ((1024, 64), "fp16", "topology"),
    ((64 * 5 + 37, 64), "fp16", "topology"),
    ((64 * 5 + 37, 64), "bf16", "random"),
    ((2, 3, 64 * 4 + 1, 64), "bf16", "topology"),
    ((2, 3, 64 * 4 + 63, 128), "fp16", "random_empty"),
    ((1, 2, 64 * 6, 128), "bf16", "dense"),
    ((3, 1, 64 * 3 + 10, 128), "bf16", "topology"),
    ((1, 1, 1, 64), "fp16", "dense"),
    ((2, 2, 63, 128), "bf16", "dense"),
]


def _schedule(kind, k, nb, seed):
    if kind == "dense":
        return oracle.dense_causal_schedule(nb)
    if kind == "topology":
        keys = k.reshape(-1, k.shape[-2], k.shape[-1])[0]
        rp, ci, _ = oracle.build_schedule(keys, 64, 1, 1, 2)
        return rp, ci
    return workloads.random_csr(nb, seed=seed, density=0.4, allow_empty=(kind == "random_empty"))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_small_shapes_elementwise(tsa, case):
    shape, dt, kind = CASES[case]
    rng_seed = 100 + case
    q = workloads.random_normal(shape, dt, rng_seed)
    k = workloads.random_normal(shape, dt, rng_seed + 1)
    v = workloads.random_normal(shape, dt, rng_seed + 2)
    S = shape[-2]
    nb = -(-S // 64)
    rp, ci = _schedule(kind, k, nb, rng_seed)
    want = oracle.masked_attention(q, k, v, rp, ci, 64)
    out = tsa.scheduled_attention(*_dev(q, k, v), *_csr_dev(rp, ci))
    torch.cuda.synchronize()
    assert out.dtype == DT[dt] and out.shape == q.shape
    err = _max_err(out, want)
    print(f"case {case} {shape} {dt} {kind}: max abs err {err:.2e}")
    assert err <= TOL[dt]


def test_explicit_scale(tsa):
    q, k, v = (workloads.random_normal((2, 2, 200, 64), "fp16", s) for s in (1, 2, 3))
    rp, ci = workloads.random_csr(4, seed=3, density=0.6)
    want = oracle.masked_attention(q, k, v, rp, ci, 64, scale=0.05)
    out = tsa.scheduled_attention(*_dev(q, k, v), *_csr_dev(rp, ci), sm_scale=0.05)
    assert _max_err(out, want) <= TOL["fp16"]


def test_large_scores_stay_finite_and_exact_pick(tsa):
    """Scale 30 makes each softmax nearly one-hot; exp must not overflow."""
    q, k, v = (workloads.random_normal((256, 64), "bf16", s) for s in (4, 5, 6))
    rp, ci = oracle.dense_causal_schedule(4)
    want = oracle.masked_attention(q, k, v, rp, ci, 64, scale=30.0)
    out = tsa.scheduled_attention(*_dev(q, k, v), *_csr_dev(rp, ci), sm_scale=30.0)
    assert torch.isfinite(out).all()
    assert _max_err(out, want) <= TOL["bf16"]


def test_two_dim_equals_four_dim_and_deterministic(tsa):
    q, k, v = (workloads.random_normal((512, 64), "bf16", s) for s in (7, 8, 9))
    rp, ci = _csr_dev(*workloads.random_csr(8, seed=1, density=0.5))
    a = tsa.scheduled_attention(*_dev(q, k, v), rp, ci)
    b = tsa.scheduled_attention(*_dev(q[None, None], k[None, None], v[None, None]), rp, ci)
    c = tsa.scheduled_attention(*_dev(q, k, v), rp, ci)
    assert torch.equal(a, b[0, 0]) and torch.equal(a, c)


def test_lanes_are_independent(tsa):
    """Each lane of a batched call equals the same lane run alone."""
    q, k, v = (workloads.random_normal((2, 2, 300, 128), "fp16", s) for s in (10, 11, 12))
    rp, ci = _csr_dev(*workloads.random_csr(5, seed=2, density=0.5))
    full = tsa.scheduled_attention(*_dev(q, k, v), rp, ci)
    one = tsa.scheduled_attention(*_dev(q[1, 0].contiguous(), k[1, 0].contiguous(), v[1, 0].contiguous()), rp, ci)
    assert torch.equal(full[1, 0], one)


def test_empty_inputs_are_noops(tsa):
    for shape in [(0, 2, 128, 64), (2, 0, 128, 64), (1, 1, 0, 64)]:
        q = torch.empty(shape, dtype=torch.float16, device="cuda:0")
        nb = -(-shape[2] // 64)
        rp = torch.zeros(nb + 1, dtype=torch.int32, device="cuda:0")
        ci = torch.zeros(0, dtype=torch.int32, device="cuda:0")
        out = tsa.scheduled_attention(q, q.clone(), q.clone(), rp, ci)
        assert out.shape == shape


def test_all_empty_rows_give_zeros(tsa):
    q = workloads.random_normal((1, 2, 192, 64), "bf16", 1)
    rp, ci = _csr_dev(np.zeros(4, np.int32), np.zeros(0, np.int32))
    out = tsa.scheduled_attention(*_dev(q, q, q), rp, ci)
    assert torch.count_nonzero(out) == 0


@pytest.mark.parametrize("shape,block", [((4, 4, 2112, 64), 64), ((8, 32, 1024, 64), 64), ((2, 4, 1000, 128), 64),
                                         ((2, 4, 640, 32), 32), ((4, 8, 700, 256), 64)])
def test_empty_rows_are_positive_zero_bits(tsa, shape, block):
    """Rows with no visible key are +0 bit for bit (no -0), on launches of both
    forward kernels that fill many workgroup slots; lse is -inf there."""
    q = workloads.random_normal(shape, "bf16", 21)
    nrows = -(-shape[2] // block)
    rp, ci = _csr_dev(np.zeros(nrows + 1, np.int32), np.zeros(0, np.int32))
    qd = q.to("cuda:0")
    out = torch.full_like(qd, 7.0)
    out, lse = tsa.scheduled_attention(qd, qd, qd, rp, ci, block=block, out=out, return_lse=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0
    assert bool(torch.isneginf(lse).all())


def test_invalid_entries_are_skipped_like_the_oracle(tsa):
    """Future blocks, duplicates-after-sort and out-of-range entries are skipped."""
    q, k, v = (workloads.random_normal((256, 64), "fp16", s) for s in (13, 14, 15))
    rp = np.array([0, 2, 5, 6, 9], np.int32)
    ci = np.array([0, 3, 0, 1, 2, 2, 0, 3, 7], np.int32)  # row0: future 3; row1: future 2; row3: 7 out of range
    want = oracle.masked_attention(q, k, v, rp, ci, 64)
    out = tsa.scheduled_attention(*_dev(q, k, v), *_csr_dev(rp, ci))
    assert _max_err(out, want) <= TOL["fp16"]


def test_validation_errors(tsa):
    q = torch.zeros(128, 64, dtype=torch.float16, device="cuda:0")
    rp, ci = _csr_dev(*oracle.dense_causal_schedule(2))
    with pytest.raises(TypeError):
        tsa.scheduled_attention(q.float(), q.float(), q.float(), rp, ci)
    with pytest.raises(TypeError):
        tsa.scheduled_attention(q, q, q, rp.long(), ci)
    with pytest.raises(ValueError):
        tsa.scheduled_attention(q, q, q, rp[:2], ci)
    with pytest.raises(ValueError):
        tsa.scheduled_attention(q, q, q, rp.cpu(), ci)
    q96 = torch.zeros(128, 96, dtype=torch.float16, device="cuda:0")
    with pytest.raises(ValueError, match="UNSUPPORTED"):
        tsa.scheduled_attention(q96, q96, q96, rp, ci)
    with pytest.raises(ValueError, match="UNSUPPORTED"):  # one 128-row block: a valid CSR length
        tsa.scheduled_attention(q, q, q, rp[:2].contiguous(), ci, block=128)
    with pytest.raises(ValueError, match="nb\\+1"):  # 32-row blocks: a 64-row CSR has too few rows
        tsa.scheduled_attention(q, q, q, rp, ci, block=32)
    q256 = torch.zeros(128, 256, dtype=torch.float16, device="cuda:0")
    rp4, ci4 = _csr_dev(*oracle.dense_causal_schedule(4))
    with pytest.raises(ValueError, match="UNSUPPORTED"):  # 32-row blocks stop at head dim 128
        tsa.scheduled_attention(q256, q256, q256, rp4, ci4, block=32)


def test_host_pointer_is_rejected_by_the_abi(tsa):
    import ctypes

    q = torch.zeros(64, 64, dtype=torch.float16, device="cuda:0")
    host = torch.zeros(64, 64, dtype=torch.float16)
    rp, ci = _csr_dev(*oracle.dense_causal_schedule(1))
    out = torch.empty_like(q)
    lib = tsa._lib
    st = lib.tsa_scheduled_attention_fwd(
        ctypes.c_void_p(host.data_ptr()), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), 0, 1, 1, 64, 64, ctypes.c_void_p(rp.data_ptr()),
        ctypes.c_void_p(ci.data_ptr()), 1, 64, 0.0, None)
    assert st == -5
    assert b"q" in lib.tsa_last_error()


# ------------------------------------------------------------------ full workloads


def _sample_rows(S, rng, n_random=64):
    rows = set(range(min(64, S))) | set(range(max(0, S - 64), S))
    rows |= set(rng.integers(0, S, n_random).tolist())
    return np.array(sorted(rows))


def _workload_schedule(w, k):
    if w.dense:
        return oracle.dense_causal_schedule(w.nb)
    keys = k.reshape(-1, w.S, w.D)[0]
    rp, ci, _ = oracle.build_schedule(keys, 64, w.sink, w.local_radius, w.topk)
    return rp, ci


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_parity(tsa, name):
    """Full-size workloads in the bench's launch configuration.  Single-lane
    workloads are compared on every output; multi-lane ones on every lane, each
    on sampled rows (block 0, the last block, 64 random rows), computed one by
    one (every output of the batched workload is compared in test_gpu_lanes.py).
    The output buffer starts as NaN, so an element no workgroup writes fails the
    finiteness check over the whole tensor."""
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_qkv(w)
    rp, ci = _workload_schedule(w, k)
    qd, kd, vd = _dev(q, k, v)
    out = torch.full(q.shape, float("nan"), dtype=DT[w.dtype], device="cuda:0")
    out = tsa.scheduled_attention(qd, kd, vd, *_csr_dev(rp, ci), out=out).cpu()
    assert out.dtype == DT[w.dtype] and out.shape == q.shape
    assert bool(torch.isfinite(out).all()), "an output element was not written"
    ql, kl, vl, ol = (t.reshape(-1, w.S, w.D) for t in (q, k, v, out))
    rng = np.random.default_rng(0)
    if w.lanes == 1 and w.S <= 4096:
        rows = np.arange(w.S)
    else:
        rows = None
    worst, worst_out = 0.0, 0.0
    for lane in range(w.lanes):
        rr = rows if rows is not None else _sample_rows(w.S, rng)
        want = oracle.masked_attention_rows(ql[lane], kl[lane], vl[lane], rp, ci, rr, 64)
        err = _max_err(ol[lane][rr], want)
        worst = max(worst, err)
        worst_out = max(worst_out, float(np.abs(want).max()))
    print(f"{name}: nnz {ci.shape[0]}, max abs err {worst:.2e} over all {w.lanes} lanes, "
          f"max|O| {worst_out:.3f}")
    assert worst <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_all_scores_strongly_negative(tsa, dtype):
    """Queries pointing against every key: every scaled score is far below zero, so
    the softmax offset, and with it the rescale threshold, is negative.  The output
    and lse still match the oracle."""
    k = workloads.random_normal((640, 64), dtype, 31, std=0.2)
    kf = k.double().numpy() + 1.0  # keys around +1 in every dim
    k = workloads.cast(kf, dtype)
    q = workloads.cast(-4.0 * np.ones((640, 64)) + workloads.random_normal((640, 64), "fp16", 32, std=0.1).double().numpy(), dtype)
    v = workloads.random_normal((640, 64), dtype, 33)
    rp, ci = workloads.random_csr(10, seed=34, density=0.6)
    want = oracle.masked_attention(q, k, v, rp, ci, 64)
    lse_want = oracle.masked_lse(q, k, rp, ci)
    assert np.nanmax(lse_want) < -20.0
    out, lse = tsa.scheduled_attention(*_dev(q, k, v), *_csr_dev(rp, ci), return_lse=True)
    assert _max_err(out, want) <= TOL[dtype]
    assert float(np.abs(lse.cpu().numpy() - lse_want).max()) <= (1e-3 if dtype == "fp16" else 4e-3)
