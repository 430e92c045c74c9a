"""Full-output parity of the forward's two-query-block workgroups.

At head dim 64, launches with many workgroups take a kernel in which one
workgroup serves two adjacent query blocks of a lane: it walks the union of
the two CSR rows, copies each union block once, and each of its waves takes
both key halves of the blocks its own row lists.  These cases are sized to
take that kernel (at least 2048 (lane, query block) pairs), with 17 query
blocks, so that the last pair has one block past the end, and they cover both
lane orders (lane counts with and without a factor of 8), both input types,
topology, dense, random and irregular CSR rows (also rows of up to 200
entries out of order), empty rows, a large softmax
scale, the lse output and the backward that consumes it, whose dq kernel takes
the same two-block form at these sizes (D 32, 64 and 128).  Every output element
is compared with the fp64 oracle; output buffers are filled with NaN first,
so an element the kernel skips fails.  One CSR is shared by every lane (PR
page "Add topology-derived sparse attention kernel", Summary, third bullet).
Bars as in the other parity tests: max abs error <= 2e-3 (fp16) / 1e-2
(bf16); lse within 1e-3 / 4e-3; gradients within 2e-3 / 1e-2 of each
gradient's largest value.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"fp16": 2e-3, "bf16": 1e-2}
TOL_LSE = {"fp16": 1e-3, "bf16": 4e-3}
S = 17 * 64  # 17 query blocks: the last pair holds one


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _csr(rp, ci):
    return (torch.from_numpy(np.asarray(rp, np.int32)).to(DEV),
            torch.from_numpy(np.asarray(ci, np.int32)).to(DEV))


def _irregular_csr(nb, seed, max_len=9, shuffle=False):
    """Ascending rows with entries the kernels must skip: negative entries,
    repeats, future blocks and blocks past the end (a row is read front to
    back, and an entry is taken only when it lies in 0..i and exceeds the last
    one taken; the oracle ignores the same entries).  With ``shuffle`` the rows
    are in random order."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(nb):
        n = int(rng.integers(0, max_len))
        r = np.sort(rng.integers(-2, nb + 3, n))
        rows.append(rng.permutation(r) if shuffle else r)
    rp = np.zeros(nb + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return rp, ci


def _accepted_csr(rp, ci):
    """The entries the kernels take from each row (the rule in include/tsa.h):
    within 0..i and above every earlier entry of the row that lies in 0..i.
    The oracle gets this CSR for rows that are not in order."""
    rows, nnz = [], len(ci)
    for i in range(len(rp) - 1):
        lo = min(max(int(rp[i]), 0), nnz)
        hi = max(min(int(rp[i + 1]), nnz), lo)
        best, keep = -1, []
        for c in ci[lo:hi]:
            if 0 <= int(c) <= i and int(c) > best:
                keep.append(int(c))
                best = int(c)
        rows.append(keep)
    out_rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    return out_rp, np.array([c for r in rows for c in r], np.int32)


def _schedule(kind, k, nb, seed):
    if kind == "topology":
        rp, ci, _ = oracle.build_schedule(k[0, 0].contiguous(), 64, 1, 2, 3)
        return rp, ci
    if kind == "dense":
        return oracle.dense_causal_schedule(nb)
    if kind == "random":
        return workloads.random_csr(nb, seed=seed, density=0.35, allow_empty=True)
    if kind == "irregular":
        return _irregular_csr(nb, seed)
    if kind == "unordered_long":  # rows of up to 200 entries in random order: several windows
        return _irregular_csr(nb, seed, max_len=200, shuffle=True)
    if kind == "empty":
        return np.zeros(nb + 1, np.int32), np.zeros(0, np.int32)
    raise ValueError(kind)


CASES = [
    # (B, H, dtype, schedule, sm_scale)
    (8, 16, "bf16", "topology", None),   # 128 lanes: per-XCD lane order
    (3, 43, "fp16", "random", None),     # 129 lanes: plain lane order
    (2, 64, "bf16", "irregular", None),
    (8, 16, "fp16", "dense", None),
    # Nearly one-hot rows: each output is close to one row of v, so v is drawn
    # with std 0.5 to keep |O| below 4, where half a bf16 ulp of the output
    # alone would exceed the absolute bar.
    (8, 17, "bf16", "topology", 30.0),
    (4, 32, "fp16", "empty", None),
    (2, 64, "fp16", "unordered_long", None),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_two_block_workgroups_every_output(tsa, case):
    B, H, dtype, kind, scale = CASES[case]
    shape = (B, H, S, 64)
    w = workloads.Workload("two_block", shape, dtype, seed=800 + case)
    q, k, v = workloads.make_qkv(w)
    if scale is not None:
        v = workloads.random_normal(shape, dtype, 950 + case, std=0.5)
    nb = S // 64
    assert B * H * nb >= 2048
    rp, ci = _schedule(kind, k, nb, 900 + case)
    rpd, cid = _csr(rp, ci)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device=DEV)
    kwargs = {} if scale is None else {"sm_scale": scale}
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, out=out, return_lse=True, **kwargs)
    torch.cuda.synchronize()
    if kind.startswith("unordered"):
        rp, ci = _accepted_csr(rp, ci)
    want = oracle.masked_attention(q, k, v, rp, ci, 64, scale=scale)
    want_lse = oracle.masked_lse(q, k, rp, ci, 64, scale=scale)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    err = float(np.abs(got - want).max())
    gl = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(want_lse)), "rows without a visible key"
    fin = np.isfinite(want_lse)
    lerr = float(np.abs(gl[fin] - want_lse[fin]).max()) if fin.any() else 0.0
    print(f"[{B},{H},{S},64] {dtype} {kind}: nnz {len(ci)}, max abs err {err:.2e}, lse {lerr:.2e}, "
          f"max|O| {np.abs(want).max():.2f}")
    assert err <= TOL[dtype]
    assert lerr <= TOL_LSE[dtype]
    if kind == "empty":
        assert torch.count_nonzero(out) == 0


EDGE_CASES = [
    # (B, H, S, dtype, schedule, v std): sizes at the edges of the two-block grid.
    # With one or two blocks per lane many rows see a handful of keys, so outputs
    # come close to single rows of v; v is drawn with std 0.5 there to keep |O|
    # below 4, where half an ulp of the output's own rounding nears the bars.
    (8, 16, 17 * 64 - 37, "bf16", "topology", 1.0),  # ragged last block (rows past S)
    (32, 64, 64, "fp16", "dense", 0.5),              # one block per lane: every pair's second block is past the end
    (16, 64, 100, "bf16", "random", 0.5),            # two blocks per lane, the second ragged
]


@pytest.mark.parametrize("case", range(len(EDGE_CASES)))
def test_two_block_edge_sizes(tsa, case):
    B, H, S_, dtype, kind, v_std = EDGE_CASES[case]
    shape = (B, H, S_, 64)
    nb = -(-S_ // 64)
    assert B * H * nb >= 2048
    w = workloads.Workload("two_block_edge", shape, dtype, seed=880 + case)
    q, k, v = workloads.make_qkv(w)
    if v_std != 1.0:
        v = workloads.random_normal(shape, dtype, 885 + case, std=v_std)
    rp, ci = _schedule(kind, k, nb, 890 + case)
    rpd, cid = _csr(rp, ci)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device=DEV)
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, out=out, return_lse=True)
    torch.cuda.synchronize()
    want = oracle.masked_attention(q, k, v, rp, ci, 64)
    want_lse = oracle.masked_lse(q, k, rp, ci, 64)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    err = float(np.abs(got - want).max())
    gl = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(want_lse))
    fin = np.isfinite(want_lse)
    lerr = float(np.abs(gl[fin] - want_lse[fin]).max()) if fin.any() else 0.0
    print(f"[{B},{H},{S_},64] {dtype} {kind}: nnz {len(ci)}, max abs err {err:.2e}, lse {lerr:.2e}")
    assert err <= TOL[dtype]
    assert lerr <= TOL_LSE[dtype]
    # the backward at the same size (its dq kernel in the two-block form too)
    do = workloads.random_normal(shape, dtype, 895 + case)
    cp, ri = tsa.schedule_transpose(rpd, cid)
    dq, dk, dv = tsa.scheduled_attention_backward(qd, kd, vd, out, do.to(DEV), lse, rpd, cid, cp, ri)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _, _ = oracle.attention_backward(q, k, v, do, rp, ci)
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        gg = g.double().cpu().numpy()
        assert np.isfinite(gg).all(), name
        scale = max(float(np.abs(r).max()), 1e-30)
        gerr = float(np.abs(gg - r).max())
        print(f"  {name}: max err {gerr:.2e} of max|ref| {scale:.2e}")
        assert gerr <= TOL[dtype] * scale, (name, gerr, scale)


BWD_CASES = [
    # (B, H, D, dtype, schedule)
    (8, 16, 64, "bf16", "topology"),
    (4, 32, 128, "fp16", "random"),
    (8, 16, 32, "bf16", "irregular"),
]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_backward_after_two_block_forward(tsa, case):
    """The backward takes its lse from the forward; at these sizes the forward
    and the dq kernel run in their two-block form."""
    B, H, D, dtype, kind = BWD_CASES[case]
    shape = (B, H, S, D)
    w = workloads.Workload("two_block_bwd", shape, dtype, seed=850 + case)
    q, k, v = workloads.make_qkv(w)
    rp, ci = _schedule(kind, k, S // 64, 860 + case)
    rpd, cid = _csr(rp, ci)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    do = workloads.random_normal(shape, dtype, 870 + case)
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, return_lse=True)
    cp, ri = tsa.schedule_transpose(rpd, cid)
    dq, dk, dv = tsa.scheduled_attention_backward(qd, kd, vd, out, do.to(DEV), lse, rpd, cid, cp, ri)
    torch.cuda.synchronize()
    rdq, rdk, rdv, rout, _ = oracle.attention_backward(q, k, v, do, rp, ci)
    assert float(np.abs(out.double().cpu().numpy() - rout).max()) <= TOL[dtype]
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        gg = g.double().cpu().numpy()
        assert np.isfinite(gg).all(), name
        scale = float(np.abs(r).max())
        gerr = float(np.abs(gg - r).max())
        print(f"{list(shape)} {dtype} {name}: max err {gerr:.2e} of max|ref| {scale:.2e}")
        assert gerr <= TOL[dtype] * scale, (name, gerr, scale)
