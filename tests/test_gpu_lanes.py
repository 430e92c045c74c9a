"""Full-output parity of launches whose lane count is a multiple of 8.

The attention kernels map workgroups to (lane, query block) in one of two ways:
a plain lane-fastest order, and, when the lane count is a multiple of 8, an order
that gives each of the chip's 8 XCDs a contiguous range of lanes.  The bench's
workloads all take the second map, so every output element of such launches is
compared here with the fp64 oracle (a dropped or doubled lane range would leave
unwritten memory, which these tests fill with NaN first).

Cases: [2, 4, 1088, D] for D = 32, 64, 128, 256 (17 query blocks, a ragged
count), forward output and lse; 16 and 32 lanes at D = 128, where each XCD runs
its lanes two at a time (64- and 32-row blocks); the backward's dq, dk and dv at [1, 8, 1024, 64],
[2, 4, 640, D] for D = 32, 128, 256 and [1, 8, 700, 256] (two head-dim halves per
key or query block); and the batched workload (64 lanes x 4096 rows) in full.
One CSR, built from lane (0, 0)'s keys, is shared by every lane (PR page
"Add topology-derived sparse attention kernel", Summary, third bullet).
Bars as in the other parity tests: forward max abs error <= 2e-3 (fp16) /
1e-2 (bf16); lse within 1e-3 / 4e-3; gradients within 2e-3 / 1e-2 of each
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


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _csr(rp, ci):
    return (torch.from_numpy(np.asarray(rp, np.int32)).to(DEV),
            torch.from_numpy(np.asarray(ci, np.int32)).to(DEV))


def _poisoned(like):
    """An output buffer filled with NaN, so that any element the kernel skips fails."""
    return torch.full(like.shape, float("nan"), dtype=like.dtype, device=DEV)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_forward_every_lane_and_row(tsa, D, dtype):
    shape = (2, 4, 1088, D)
    w = workloads.Workload("lanes", shape, dtype, seed=600 + D)
    q, k, v = workloads.make_qkv(w)
    rp, ci, _ = oracle.build_schedule(k[0, 0].contiguous(), 64, 1, 2, 4)
    rpd, cid = _csr(rp, ci)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = _poisoned(qd)
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, out=out, return_lse=True)
    torch.cuda.synchronize()
    want_out = oracle.masked_attention(q, k, v, rp, ci)
    want_lse = oracle.masked_lse(q, k, rp, ci)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    err = float(np.abs(got - want_out).max())
    lerr = float(np.abs(lse.double().cpu().numpy() - want_lse).max())
    print(f"[2,4,1088,{D}] {dtype}: nnz {len(ci)}, max abs err {err:.2e}, lse {lerr:.2e}, "
          f"max|O| {np.abs(want_out).max():.2f}")
    assert err <= TOL[dtype]
    assert lerr <= TOL_LSE[dtype]


@pytest.mark.parametrize("shape,dtype,block", [((2, 8, 1088, 128), "bf16", 64), ((4, 8, 700, 128), "fp16", 64),
                                               ((2, 8, 1000, 128), "bf16", 32)])
def test_forward_lane_pairs_per_xcd_every_output(tsa, shape, dtype, block):
    """At head dim 128 with a lane count that is a multiple of 16, each XCD runs
    its lanes two at a time (pairs of lanes, every pair position longest first):
    every output and lse element of such launches against the oracle."""
    w = workloads.Workload("lane_pairs", shape, dtype, seed=650 + shape[0] + block)
    q, k, v = workloads.make_qkv(w)
    rp, ci, _ = oracle.build_schedule(k[0, 0].contiguous(), block, 1, 2, 4)
    rpd, cid = _csr(rp, ci)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = _poisoned(qd)
    out, lse = tsa.scheduled_attention(qd, kd, vd, rpd, cid, block=block, out=out, return_lse=True)
    torch.cuda.synchronize()
    want_out = oracle.masked_attention(q, k, v, rp, ci, block)
    want_lse = oracle.masked_lse(q, k, rp, ci, block)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    err = float(np.abs(got - want_out).max())
    lerr = float(np.abs(lse.double().cpu().numpy() - want_lse).max())
    print(f"{list(shape)} {dtype} block {block}: nnz {len(ci)}, max abs err {err:.2e}, lse {lerr:.2e}")
    assert err <= TOL[dtype]
    assert lerr <= TOL_LSE[dtype]


@pytest.mark.parametrize("shape,dtype", [((1, 8, 1024, 64), "bf16"), ((2, 4, 640, 128), "fp16"),
                                         ((2, 4, 640, 32), "bf16"), ((2, 4, 640, 256), "bf16"),
                                         ((1, 8, 700, 256), "fp16")])
def test_backward_every_lane_and_row(tsa, shape, dtype):
    w = workloads.Workload("lanes_bwd", shape, dtype, seed=700 + shape[-1])
    q, k, v = workloads.make_qkv(w)
    rp, ci, _ = oracle.build_schedule(k[0, 0].contiguous(), 64, 1, 2, 4)
    rpd, cid = _csr(rp, ci)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    do = workloads.random_normal(shape, dtype, 701)
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


def test_batched_workload_every_output(tsa):
    """The bench's batched workload (64 lanes of [4096, 64] bf16) in the launch
    configuration the bench times: the GPU-built schedule, then every one of the
    16.8 M outputs against the oracle."""
    w = workloads.WORKLOADS["batched_b4h16_s4096_d64_bf16"]
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    rpd, cid = tsa.build_schedule(kd[0, 0], 64, w.sink, w.local_radius, w.topk)
    rp, ci = rpd.cpu().numpy(), cid.cpu().numpy()
    rpo, cio, _ = oracle.build_schedule(k[0, 0].contiguous(), 64, w.sink, w.local_radius, w.topk)
    assert np.array_equal(rp, rpo) and np.array_equal(ci, cio)
    out = tsa.scheduled_attention(qd, kd, vd, rpd, cid, out=_poisoned(qd))
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    want = oracle.masked_attention(q, k, v, rp, ci)
    err = np.abs(got - want)
    lane_err = err.reshape(w.lanes, -1).max(axis=1)
    print(f"batched: nnz {len(ci)}, max abs err {err.max():.3e} (worst lane {int(lane_err.argmax())}), "
          f"max|O| {np.abs(want).max():.3f}")
    assert float(err.max()) <= TOL[w.dtype]
