"""GPU parity for schedules over blocks larger than 64 rows, through the C ABI:

* the builder at block 128 / 256 (and 192, 320) against the oracle builder at
  the same block: CSR bit-exact, salience to a relative 1e-12;
* tsa_refine_schedule against oracle.refine_schedule, bit-exact, on random,
  dense, segment and built schedules, ragged S, and rows with entries the
  kernels skip;
* attention (forward and backward) over a refined schedule against the oracle's
  masked attention at the coarse block, to the bars of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _dev(x):
    return torch.as_tensor(np.asarray(x)).to(DEV)


def _build_compare(tsa, keys, block, sink, radius, topk, label):
    rp_o, ci_o, sal_o = oracle.build_schedule(keys, block, sink, radius, topk)
    rp, ci, sal = tsa.build_schedule(keys.to(DEV), block, sink, radius, topk, return_salience=True)
    rp, ci, sal = rp.cpu().numpy(), ci.cpu().numpy(), sal.cpu().numpy()
    assert rp.shape[0] == -(-keys.shape[0] // block) + 1, label
    assert np.array_equal(rp, rp_o), label
    assert np.array_equal(ci, ci_o), label
    assert np.allclose(sal, sal_o, rtol=1e-12, atol=0), label
    return rp, ci


@pytest.mark.parametrize("block", [128, 256])
@pytest.mark.parametrize("name", ["single_s1024_d64_f16", "single_s4096_d64_f16_mix8",
                                  "batched_b4h16_s4096_d64_bf16", "long_b1h32_s32768_d64_bf16_mix32"])
def test_builder_at_coarse_blocks(tsa, name, block):
    w = workloads.WORKLOADS[name]
    _, k, _ = workloads.make_qkv(w, shape=(w.S, w.D))
    _build_compare(tsa, k, block, w.sink, w.local_radius, max(1, w.topk // (block // 64)), f"{name} block {block}")


@pytest.mark.parametrize("seed", range(8))
def test_builder_random_coarse_blocks(tsa, seed):
    rng = np.random.default_rng(100 + seed)
    block = int(rng.choice([128, 192, 256, 320]))
    nb = int(rng.integers(1, 40))
    S = block * nb - int(rng.integers(0, block)) if nb > 1 else int(rng.integers(1, block + 1))
    D = int(rng.choice([16, 64, 128]))
    dt = "bf16" if seed % 2 else "fp16"
    sink, radius, topk = (int(x) for x in rng.integers(0, 4, 3))
    keys = workloads.random_normal((S, D), dt, 5000 + seed)
    _build_compare(tsa, keys, block, sink, radius, topk, f"seed {seed} block {block} S {S}")


def _refine_compare(tsa, rp, ci, S, block):
    frp, fci = tsa.refine_schedule(_dev(rp.astype(np.int32)), _dev(ci.astype(np.int32)), S, block)
    orp, oci = oracle.refine_schedule(rp, ci, S, block)
    np.testing.assert_array_equal(frp.cpu().numpy(), orp)
    np.testing.assert_array_equal(fci.cpu().numpy(), oci)
    return frp, fci


@pytest.mark.parametrize("S,block,seed", [(1000, 128, 0), (4096, 256, 1), (777, 192, 2), (100, 128, 3),
                                          (64, 128, 4), (32768, 128, 5), (5000, 320, 6), (4096, 64, 7),
                                          (64 * 1030, 4096, 8)])
def test_refine_random(tsa, S, block, seed):
    rp, ci = workloads.random_csr(-(-S // block), seed=seed, density=0.4, allow_empty=True)
    _refine_compare(tsa, rp, ci, S, block)


@pytest.mark.parametrize("S,block", [(4096, 128), (32768, 256), (1000, 192)])
def test_refine_dense_and_segments(tsa, S, block):
    nbc = -(-S // block)
    _refine_compare(tsa, *oracle.dense_causal_schedule(nbc), S, block)
    _refine_compare(tsa, *oracle.fixed_segment_schedule(nbc, 3), S, block)


def test_refine_skips_what_the_kernels_skip(tsa):
    rng = np.random.default_rng(11)
    S, block = 3000, 128
    nbc = -(-S // block)
    rows = [rng.integers(-2, nbc + 2, size=int(rng.integers(0, 12))) for _ in range(nbc)]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    # the rule of include/tsa.h, applied on the host before the oracle's refinement
    keep = []
    for i in range(nbc):
        best, row = -1, []
        for c in ci[rp[i]:rp[i + 1]]:
            c = int(c)
            if 0 <= c <= i:
                if c > best:
                    row.append(c)
                best = max(best, c)
        keep.append(row)
    rp2 = np.concatenate([[0], np.cumsum([len(r) for r in keep])]).astype(np.int32)
    ci2 = np.array([c for r in keep for c in r], np.int32)
    frp, fci = tsa.refine_schedule(_dev(rp), _dev(ci), S, block)
    orp, oci = oracle.refine_schedule(rp2, ci2, S, block)
    np.testing.assert_array_equal(frp.cpu().numpy(), orp)
    np.testing.assert_array_equal(fci.cpu().numpy(), oci)


def test_refine_empty(tsa):
    rp, ci = tsa.refine_schedule(_dev(np.zeros(1, np.int32)), _dev(np.zeros(0, np.int32)), 0, 128)
    assert rp.cpu().tolist() == [0] and ci.numel() == 0


@pytest.mark.parametrize("dtype,shape,block", [("fp16", (1000, 64), 128), ("bf16", (1, 2, 1024, 64), 256),
                                               ("bf16", (1, 1, 900, 128), 192)])
def test_attention_over_refined_schedule(tsa, dtype, shape, block):
    """Forward and backward over the refined CSR equal the oracle's masked
    attention with the coarse CSR at the coarse block."""
    S = shape[-2]
    rp, ci = workloads.random_csr(-(-S // block), seed=21, density=0.5, allow_empty=True)
    w = workloads.Workload("t", shape, dtype, seed=33)
    q, k, v = workloads.make_qkv(w)
    do = workloads.random_normal(shape, dtype, 34)
    frp, fci = tsa.refine_schedule(_dev(rp), _dev(ci), S, block)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    out, lse = tsa.scheduled_attention(qd, kd, vd, frp, fci, return_lse=True)
    ref = oracle.masked_attention(q, k, v, rp, ci, block=block)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= (2e-3 if dtype == "fp16" else 1e-2), err
    cp, ri = tsa.schedule_transpose(frp, fci)
    dq, dk, dv = tsa.scheduled_attention_backward(qd, kd, vd, out, dod, lse, frp, fci, cp, ri)
    rdq, rdk, rdv, _, _ = oracle.attention_backward(q, k, v, do, rp, ci, block=block)
    tol = 2e-3 if dtype == "fp16" else 1e-2
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        e = np.abs(g.float().cpu().numpy() - r).max()
        print(f"{name}: rel {e / np.abs(r).max():.2e}")
        assert e <= tol * np.abs(r).max(), (name, e)
