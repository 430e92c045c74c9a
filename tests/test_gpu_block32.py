"""GPU parity for schedules over 32-row blocks, through the C ABI.

The builder and the forward also take 32-row blocks (one CSR row per 32 query
rows, one listed entry per 32 keys).  The forward serves them with the
two-block kernel: each workgroup holds four 32-row query blocks, each wave
walks its own CSR row, and the 64-key tiles it copies are the union of the
64-key blocks those rows touch.  Checked here:

* the builder at block 32 against the oracle builder at block 32: CSR
  bit-exact, salience to a relative 1e-12 (ragged S, the LDS and the larger
  path, both top-k scopes);
* every output element and lse against the fp64 oracle at block 32: topology,
  dense, random, irregular (entries the kernel must skip, also in rows of up
  to 200 entries and in rows out of order) and empty schedules,
  lane counts with and without a factor of 8, ragged S, one- and two-row
  sequences, fp16 and bf16, head dims 32, 64 and 128, a large softmax scale;
* at the batched workload's full size ([4, 16, 4096, 64] bf16, the schedule
  built from lane (0, 0) at block 32), sampled rows of every lane;
* a 64-row CSR and its 32-row expansion allow the same keys, and on the
  two-block kernel they take the same tiles in the same order, so their
  outputs and lse are bitwise equal;
* the backward at block 32 (the two-block dq and dk/dv kernels with four
  32-row rows or 32-key columns per workgroup): every dq, dk and dv against the
  fp64 oracle at block 32 over the same kinds of schedule, the autograd
  wrapper, and bitwise equality with the 64-row backward of the expanded CSR.

Bars as in the other parity tests: max abs error <= 2e-3 (fp16) / 1e-2
(bf16); lse within 1e-3 / 4e-3.  Output buffers are filled with NaN first, so
an element the kernel skips fails.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"fp16": 2e-3, "bf16": 1e-2}
TOL_LSE = {"fp16": 1e-3, "bf16": 4e-3}


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _dev(x):
    return torch.as_tensor(np.asarray(x)).to(DEV)


def _irregular_csr(nb, seed, max_len=12, shuffle=False):
    """Ascending rows with entries the kernel must skip: negative entries,
    repeats, future blocks and blocks past the end.  With ``shuffle`` the rows
    are in random order, so that earlier larger entries hide later ones."""
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(nb):
        r = np.sort(rng.integers(-2, nb + 3, int(rng.integers(0, max_len))))
        rows.append(rng.permutation(r) if shuffle else r)
    rp = np.zeros(nb + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return rp, ci


def _accepted_csr(rp, ci):
    """The entries the kernel takes from each row (the rule in include/tsa.h):
    within 0..i and above every earlier entry of the row that lies in 0..i.
    For rows in ascending order these are the row's entries in 0..i; the oracle
    gets this CSR for rows that are not in order."""
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
        rp, ci, _ = oracle.build_schedule(k[0, 0].contiguous(), 32, 1, 2, 4)
        return rp, ci
    if kind == "dense":
        return oracle.dense_causal_schedule(nb)
    if kind == "random":
        return workloads.random_csr(nb, seed=seed, density=0.35, allow_empty=True)
    if kind == "irregular":
        return _irregular_csr(nb, seed)
    if kind == "irregular_long":  # rows of up to 200 entries: several 64-entry windows
        return _irregular_csr(nb, seed, max_len=200)
    if kind == "unordered_long":
        return _irregular_csr(nb, seed, max_len=200, shuffle=True)
    if kind == "empty":
        return np.zeros(nb + 1, np.int32), np.zeros(0, np.int32)
    raise ValueError(kind)


def _build_compare(tsa, keys, sink, radius, topk, per_row, label):
    rp_o, ci_o, sal_o = oracle.build_schedule(keys, 32, sink, radius, topk, per_row=per_row)
    rp, ci, sal = tsa.build_schedule(keys.to(DEV), 32, sink, radius, topk, return_salience=True,
                                     per_row=per_row)
    rp, ci, sal = rp.cpu().numpy(), ci.cpu().numpy(), sal.cpu().numpy()
    assert rp.shape[0] == -(-keys.shape[0] // 32) + 1, label
    assert np.array_equal(rp, rp_o), label
    assert np.array_equal(ci, ci_o), label
    assert np.allclose(sal, sal_o, rtol=1e-12, atol=0), label


@pytest.mark.parametrize("name,per_row", [("single_s1024_d64_f16", False),
                                          ("single_s4096_d64_f16_mix8", False),
                                          ("batched_b4h16_s4096_d64_bf16", True),
                                          ("long_b1h32_s32768_d64_bf16_mix32", False)])
def test_builder_at_32_row_blocks(tsa, name, per_row):
    w = workloads.WORKLOADS[name]
    _, k, _ = workloads.make_qkv(w, shape=(w.S, w.D))
    _build_compare(tsa, k, w.sink, w.local_radius, 2 * w.topk, per_row, f"{name} block 32")


@pytest.mark.parametrize("S", [1, 31, 33, 1000, 4100])
def test_builder_32_ragged(tsa, S):
    keys = workloads.random_normal((S, 64), "fp16", 7000 + S)
    _build_compare(tsa, keys, 1, 1, 3, False, f"S {S}")


CASES = [
    # (B, H, S, D, dtype, schedule, sm_scale, v std)
    (2, 4, 1000, 64, "bf16", "topology", None, 1.0),   # 8 lanes: per-XCD lane order; ragged S
    (1, 3, 1088, 32, "fp16", "random", None, 1.0),     # 3 lanes: plain lane order
    (2, 8, 777, 128, "fp16", "irregular", None, 1.0),
    (1, 5, 256, 64, "bf16", "dense", None, 0.5),
    (1, 8, 33, 64, "fp16", "dense", None, 0.5),        # two 32-row blocks, the second of one row
    (1, 2, 31, 32, "bf16", "dense", None, 0.5),        # one partial block
    (3, 3, 300, 128, "bf16", "random", None, 1.0),
    (4, 4, 640, 64, "fp16", "irregular", None, 1.0),
    (2, 8, 512, 64, "bf16", "topology", 30.0, 0.5),    # nearly one-hot rows
    (2, 4, 200, 64, "fp16", "empty", None, 1.0),
    (8, 16, 1088, 64, "fp16", "random", None, 1.0),    # 128 lanes, 34 rows per lane
    (1, 4, 2500, 64, "fp16", "dense", None, 1.0),      # rows of up to 79 entries
    (2, 2, 3000, 128, "bf16", "irregular_long", None, 1.0),
    (1, 8, 3000, 32, "fp16", "unordered_long", None, 1.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_at_32_row_blocks_every_output(tsa, case):
    B, H, S, D, dtype, kind, scale, v_std = CASES[case]
    shape = (B, H, S, D)
    q, k, v = workloads.make_qkv(workloads.Workload("block32", shape, dtype, seed=1200 + case))
    if v_std != 1.0:
        v = workloads.random_normal(shape, dtype, 1250 + case, std=v_std)
    nb = -(-S // 32)
    rp, ci = _schedule(kind, k, nb, 1300 + case)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device=DEV)
    kwargs = {} if scale is None else {"sm_scale": scale}
    out, lse = tsa.scheduled_attention(qd, kd, vd, _dev(rp), _dev(ci), block=32, out=out,
                                       return_lse=True, **kwargs)
    torch.cuda.synchronize()
    if kind.startswith("unordered"):
        rp, ci = _accepted_csr(rp, ci)
    want = oracle.masked_attention(q, k, v, rp, ci, 32, scale=scale)
    want_lse = oracle.masked_lse(q, k, rp, ci, 32, scale=scale)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    err = float(np.abs(got - want).max())
    gl = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(want_lse)), "rows without a visible key"
    fin = np.isfinite(want_lse)
    lerr = float(np.abs(gl[fin] - want_lse[fin]).max()) if fin.any() else 0.0
    print(f"[{B},{H},{S},{D}] {dtype} {kind} block 32: nnz {len(ci)}, max abs err {err:.2e}, "
          f"lse {lerr:.2e}")
    assert err <= TOL[dtype]
    assert lerr <= TOL_LSE[dtype]
    if kind == "empty":
        assert torch.count_nonzero(out) == 0


def test_forward_at_32_row_blocks_full_size_sampled(tsa):
    """The batched workload at its full size with its schedule built on the GPU
    at block 32 (checked bit-exact against the oracle builder), then sampled
    query rows of every lane against the oracle."""
    w = workloads.WORKLOADS["batched_b4h16_s4096_d64_bf16"]
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    rpd, cid = tsa.build_schedule(kd[0, 0].contiguous(), 32, w.sink, w.local_radius, 2 * w.topk)
    rp, ci = rpd.cpu().numpy(), cid.cpu().numpy()
    rp_o, ci_o, _ = oracle.build_schedule(k[0, 0].contiguous(), 32, w.sink, w.local_radius, 2 * w.topk)
    assert np.array_equal(rp, rp_o) and np.array_equal(ci, ci_o)
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, block=32, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 31, 32, 63, 64, w.S - 1], rng.integers(0, w.S, 40)]))
    got = out.double().cpu().numpy()[:, :, rows]
    gl = lse.double().cpu().numpy()[:, :, rows]
    # lse of the sampled rows: logsumexp of the scaled scores over the keys the
    # oracle's mask allows (every row sees at least its own key)
    mask = oracle.allowed_key_mask(rp, ci, w.S, 32, rows=rows)
    err = lerr = 0.0
    for b in range(w.shape[0]):
        for h in range(w.shape[1]):
            want = oracle.masked_attention_rows(q[b, h], k[b, h], v[b, h], rp, ci, rows, 32)
            err = max(err, float(np.abs(got[b, h] - want).max()))
            scores = q[b, h].double().numpy()[rows] @ k[b, h].double().numpy().T / np.sqrt(w.D)
            want_lse = scipy.special.logsumexp(np.where(mask, scores, -np.inf), axis=-1)
            lerr = max(lerr, float(np.abs(gl[b, h] - want_lse).max()))
    print(f"{list(w.shape)} bf16 block 32: nnz {len(ci)}, {len(rows)} rows x 64 lanes: err {err:.2e}, "
          f"lse {lerr:.2e}")
    assert err <= TOL["bf16"]
    assert lerr <= TOL_LSE["bf16"]


def _expand_to_32(rp, ci, S):
    rows = []
    for i in range(-(-S // 32)):
        I = i // 2
        rows.append([2 * J + b for J in ci[rp[I] : rp[I + 1]] for b in (0, 1) if 2 * J + b <= i])
    rp32 = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci32 = np.array([c for r in rows for c in r], np.int32)
    return rp32, ci32


@pytest.mark.parametrize("B,H,S,D,dtype", [(8, 16, 1088, 64, "bf16"), (2, 8, 1000, 128, "fp16")])
def test_32_row_expansion_is_bitwise_equal_on_the_two_block_kernel(tsa, B, H, S, D, dtype):
    shape = (B, H, S, D)
    q, k, v = workloads.make_qkv(workloads.Workload("block32_eq", shape, dtype, seed=1400 + D))
    nb = -(-S // 64)
    if D == 64:
        assert B * H * nb >= 2048  # the two-block kernel serves the 64-row CSR too
    rp, ci = workloads.random_csr(nb, seed=1410 + D, density=0.4)
    rp32, ci32 = _expand_to_32(rp, ci, S)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o64, l64 = tsa.scheduled_attention(qd, kd, vd, _dev(rp), _dev(ci), return_lse=True)
    o32, l32 = tsa.scheduled_attention(qd, kd, vd, _dev(rp32), _dev(ci32), block=32, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o64.view(torch.int16), o32.view(torch.int16))
    assert torch.equal(l64.view(torch.int32), l32.view(torch.int32))


# ---------------------------------------------------------------- backward

BWD_CASES = [
    # (B, H, S, D, dtype, schedule)
    (2, 4, 1000, 64, "bf16", "topology"),   # 8 lanes: per-XCD lane order; ragged S
    (1, 3, 1088, 32, "fp16", "random"),     # 3 lanes: plain order; empty rows
    (2, 8, 777, 128, "fp16", "irregular"),  # entries the kernels must skip
    (1, 5, 256, 64, "bf16", "dense"),
    (1, 2, 33, 64, "fp16", "dense"),        # two 32-row blocks, the second of one row
    (1, 2, 31, 32, "bf16", "dense"),        # one partial block
    (3, 3, 300, 128, "bf16", "random"),
    (2, 4, 200, 64, "fp16", "empty"),
    (1, 2, 3000, 64, "bf16", "irregular_long"),  # rows and columns of many windows
]


def _grad_bar_check(name, got, ref, dtype):
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all(), f"{name}: an element was not written"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(g - ref).max()) if ref.size else 0.0
    assert err <= TOL[dtype] * max(scale, 1e-30), (name, err, scale)
    return err, scale


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_backward_at_32_row_blocks_every_gradient(tsa, case):
    """dq, dk and dv of every element over a 32-row CSR against the fp64 oracle
    at block 32 (bars relative to each gradient's largest value)."""
    B, H, S, D, dtype, kind = BWD_CASES[case]
    shape = (B, H, S, D)
    q, k, v = workloads.make_qkv(workloads.Workload("block32_bwd", shape, dtype, seed=1500 + case))
    do = workloads.random_normal(shape, dtype, 1550 + case)
    nb = -(-S // 32)
    rp, ci = _schedule(kind, k, nb, 1600 + case)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    rpd, cid = _dev(rp), _dev(ci)
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, block=32, return_lse=True)
    cp, ri = tsa.schedule_transpose(rpd, cid)
    dq, dk, dv = tsa.scheduled_attention_backward(qd, kd, vd, out, do.to(DEV), lse, rpd, cid, cp, ri,
                                                  block=32)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _, _ = oracle.attention_backward(q, k, v, do, rp, ci, block=32)
    msg = []
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        err, scale = _grad_bar_check(name, g, r, dtype)
        msg.append(f"{name} {err:.2e}/{scale:.2e}")
    print(f"[{B},{H},{S},{D}] {dtype} {kind} block 32 backward: nnz {len(ci)}; " + ", ".join(msg))
    if kind == "empty":
        assert all(torch.count_nonzero(g) == 0 for g in (dq, dk, dv))


def test_backward_at_32_row_blocks_through_autograd(tsa):
    """The autograd wrapper at block 32 gives the direct call's gradients bit for bit."""
    shape = (2, 4, 520, 64)
    q, k, v = workloads.make_qkv(workloads.Workload("block32_ag", shape, "bf16", seed=1700))
    do = workloads.random_normal(shape, "bf16", 1701).to(DEV)
    rp, ci = workloads.random_csr(-(-520 // 32), seed=1702, density=0.4)
    rpd, cid = _dev(rp), _dev(ci)
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    tsa.attention(qd, kd, vd, rpd, cid, block=32).backward(do)
    out, lse = tsa.scheduled_attention(qd.detach(), kd.detach(), vd.detach(), rpd, cid, block=32,
                                       return_lse=True)
    cp, ri = tsa.schedule_transpose(rpd, cid)
    ref = tsa.scheduled_attention_backward(qd.detach(), kd.detach(), vd.detach(), out, do, lse, rpd, cid,
                                           cp, ri, block=32)
    torch.cuda.synchronize()
    for g, r in zip((qd.grad, kd.grad, vd.grad), ref):
        assert torch.equal(g.view(torch.int16), r.view(torch.int16))


@pytest.mark.parametrize("B,H,S,D,dtype", [(2, 16, 4096, 64, "bf16"), (2, 16, 4096, 128, "fp16")])
def test_backward_32_row_expansion_is_bitwise_equal_on_the_two_block_kernels(tsa, B, H, S, D, dtype):
    """A 64-row CSR and its 32-row expansion give bitwise-equal gradients where
    the 64-row backward also takes the two-block kernels (from 2048 (lane, block)
    pairs up, here 32 lanes x 64 blocks): each wave walks the same tiles in the
    same order."""
    shape = (B, H, S, D)
    q, k, v = workloads.make_qkv(workloads.Workload("block32_bwd_eq", shape, dtype, seed=1800 + D))
    do = workloads.random_normal(shape, dtype, 1801 + D).to(DEV)
    nb = -(-S // 64)
    assert B * H * nb >= 2048
    rp, ci = workloads.random_csr(nb, seed=1810 + D, density=0.4)
    rp32, ci32 = _expand_to_32(rp, ci, S)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    grads = []
    for rpn, cin, block in ((rp, ci, 64), (rp32, ci32, 32)):
        rpd, cid = _dev(rpn), _dev(cin)
        out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, block=block, return_lse=True)
        cp, ri = tsa.schedule_transpose(rpd, cid)
        grads.append(tsa.scheduled_attention_backward(qd, kd, vd, out, do, lse, rpd, cid, cp, ri, block=block))
    torch.cuda.synchronize()
    for a, b in zip(*grads):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
