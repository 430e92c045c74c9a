"""Parity of the fixed-segment (block-diagonal causal) CSR path with the oracle.

The GPU schedule must equal oracle.fixed_segment_schedule bit for bit; the
attention kernel over it must match the fp64 dense masked attention on the same
mask (max abs error <= 2e-3 fp16, <= 1e-2 bf16), including at the batched
benchmark shape with 512-token segments, in the bench's launch configuration.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1e-2}


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as mod

    return mod


@pytest.mark.parametrize("nb,seg", [(64, 8), (64, 4), (64, 64), (64, 1), (13, 5), (100, 7),
                                    (512, 8), (1, 1), (0, 3), (70, 200)])
def test_segment_schedule_bit_exact(tsa, nb, seg):
    rp, ci = tsa.segment_schedule(nb, seg, "cuda:0")
    rp_o, ci_o = oracle.fixed_segment_schedule(nb, seg)
    assert np.array_equal(rp.cpu().numpy(), rp_o) and np.array_equal(ci.cpu().numpy(), ci_o)


@pytest.mark.parametrize("shape,dt,seg", [((64 * 6 + 17, 64), "fp16", 2),
                                          ((2, 3, 64 * 5, 128), "bf16", 3),
                                          ((1, 2, 64 * 9 - 1, 64), "bf16", 4)])
def test_attention_on_segments_elementwise(tsa, shape, dt, seg):
    q = workloads.random_normal(shape, dt, 7100)
    k = workloads.random_normal(shape, dt, 7101)
    v = workloads.random_normal(shape, dt, 7102)
    S = shape[-2]
    nb = -(-S // 64)
    rp, ci = tsa.segment_schedule(nb, seg, "cuda:0")
    out = tsa.scheduled_attention(q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0"), rp, ci).cpu()
    rp_o, ci_o = oracle.fixed_segment_schedule(nb, seg)
    ql, kl, vl, ol = (t.reshape(-1, S, shape[-1]) for t in (q, k, v, out))
    worst = 0.0
    for lane in range(ql.shape[0]):
        want = oracle.masked_attention(ql[lane], kl[lane], vl[lane], rp_o, ci_o, 64)
        worst = max(worst, float(np.max(np.abs(ol[lane].to(torch.float64).numpy() - want))))
    print(f"{shape} {dt} seg {seg}: max abs err {worst:.2e}")
    assert worst <= TOL[dt]


def test_attention_on_512_token_segments_at_bench_shape(tsa):
    """[4, 16, 4096, 64] bf16 with 8-block segments (288 of 2,080 causal blocks):
    sampled lanes and rows, each compared with the oracle row by row."""
    w = workloads.WORKLOADS["batched_b4h16_s4096_d64_bf16"]
    q, k, v = workloads.make_qkv(w)
    rp, ci = tsa.segment_schedule(w.nb, 8, "cuda:0")
    assert int(rp[-1]) == 288
    out = tsa.scheduled_attention(q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0"), rp, ci).cpu()
    rp_o, ci_o = oracle.fixed_segment_schedule(w.nb, 8)
    ql, kl, vl, ol = (t.reshape(-1, w.S, w.D) for t in (q, k, v, out))
    rng = np.random.default_rng(1)
    worst = 0.0
    for lane in sorted({0, w.lanes - 1, int(rng.integers(0, w.lanes))}):
        rows = np.array(sorted(set(range(64)) | set(range(w.S - 64, w.S)) | set(range(448, 576))
                               | set(rng.integers(0, w.S, 128).tolist())))
        want = oracle.masked_attention_rows(ql[lane], kl[lane], vl[lane], rp_o, ci_o, rows, 64)
        worst = max(worst, float(np.max(np.abs(ol[lane][rows].to(torch.float64).numpy() - want))))
    print(f"512-token segments: max abs err {worst:.2e}")
    assert worst <= TOL["bf16"]
