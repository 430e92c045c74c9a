"""Parity of the HIP builder's per-row top-k scope (TSA_TOPK_PER_ROW) with the
fp64 oracle (oracle.build_schedule(..., per_row=True)), through the C ABI.

CSR row_ptr/col_idx must be bit-identical and salience equal to a relative
1e-12, on the one-wavefront path (nb <= 128) and the large path (nb > 128);
attention over a per-row schedule must match the fp64 masked attention.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as mod

    return mod


def _compare(tsa, keys_cpu, sink, radius, topk, label=""):
    rp_o, ci_o, sal_o = oracle.build_schedule(keys_cpu, 64, sink, radius, topk, per_row=True)
    rp, ci, sal = tsa.build_schedule(keys_cpu.to("cuda:0"), 64, sink, radius, topk,
                                     return_salience=True, per_row=True)
    rp, ci, sal = rp.cpu().numpy(), ci.cpu().numpy(), sal.cpu().numpy()
    assert np.array_equal(rp, rp_o), label
    assert np.array_equal(ci, ci_o), label
    assert np.allclose(sal, sal_o, rtol=1e-12, atol=0), label
    return rp, ci


@pytest.mark.parametrize("name", [n for n, w in workloads.WORKLOADS.items() if not w.dense])
def test_workload_schedules_per_row(tsa, name):
    w = workloads.WORKLOADS[name]
    _, k, _ = workloads.make_qkv(w)
    rp, ci = _compare(tsa, k.reshape(-1, w.S, w.D)[0].contiguous(), w.sink, w.local_radius, w.topk, name)
    print(f"{name} per-row: nnz {ci.shape[0]}")


@pytest.mark.parametrize("seed", range(16))
def test_random_small_configurations_per_row(tsa, seed):
    rng = np.random.default_rng(seed + 500)
    nb = int(rng.integers(1, 21))
    S = 64 * nb - int(rng.integers(0, 64)) if nb > 1 else int(rng.integers(1, 65))
    D = int(rng.choice([8, 64, 128]))
    sink, radius, topk = (int(x) for x in rng.integers(0, 5, 3))
    keys = workloads.random_normal((S, D), "bf16" if seed % 2 else "fp16", 5000 + seed)
    _compare(tsa, keys, sink, radius, topk, f"seed {seed} nb {nb}")


@pytest.mark.parametrize("nb,topk", [(64, 16), (100, 7), (128, 40), (130, 17), (300, 5), (700, 33)])
def test_sizes_across_both_paths(tsa, nb, topk):
    keys = workloads.random_normal((64 * nb - 3, 32), "bf16", 6000 + nb)
    _compare(tsa, keys, 2, 3, topk, f"nb {nb}")


@pytest.mark.parametrize("nb", [5, 64, 200])
def test_topk_extremes(tsa, nb):
    keys = workloads.random_normal((64 * nb, 16), "fp16", 6100 + nb)
    rp, ci = _compare(tsa, keys, 0, 0, nb + 3, f"nb {nb} dense")
    rp_d, ci_d = oracle.dense_causal_schedule(nb)
    assert np.array_equal(rp, rp_d) and np.array_equal(ci, ci_d)
    rp0, ci0 = _compare(tsa, keys, 1, 2, 0, f"nb {nb} topk 0")
    rp_g, ci_g, _ = oracle.build_schedule(keys, 64, 1, 2, 0)
    assert np.array_equal(rp0, rp_g) and np.array_equal(ci0, ci_g)


def test_per_row_buffers_reused_with_global_builds(tsa):
    """One workspace alternates between the two scopes; each build matches."""
    w = workloads.WORKLOADS["batched_b4h16_s4096_d64_bf16"]
    _, k, _ = workloads.make_qkv(w)
    keys = k.reshape(-1, w.S, w.D)[0].contiguous()
    bp = tsa.ScheduleBuffers(w.S, w.D, w.sink, w.local_radius, w.topk, "cuda:0", per_row=True)
    bg = tsa.ScheduleBuffers(w.S, w.D, w.sink, w.local_radius, w.topk, "cuda:0")
    bg._ws = bp._ws
    bg.ws_ptr = bp.ws_ptr
    for per_row, bufs in [(True, bp), (False, bg), (True, bp)]:
        tsa.build_schedule_into(keys.to("cuda:0"), bufs)
        rp_o, ci_o, _ = oracle.build_schedule(keys, 64, w.sink, w.local_radius, w.topk, per_row=per_row)
        rp = bufs.row_ptr.cpu().numpy()
        assert np.array_equal(rp, rp_o)
        assert np.array_equal(bufs.col_idx[: int(rp[-1])].cpu().numpy(), ci_o)


def test_attention_on_per_row_schedule(tsa):
    w = workloads.WORKLOADS["batched_b4h16_s4096_d64_bf16"]
    q, k, v = workloads.make_qkv(w)
    rp, ci = tsa.build_schedule(k.to("cuda:0"), 64, w.sink, w.local_radius, w.topk, per_row=True)
    out = tsa.scheduled_attention(q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0"), rp, ci).cpu()
    rp_o, ci_o = rp.cpu().numpy(), ci.cpu().numpy()
    ql, kl, vl, ol = (t.reshape(-1, w.S, w.D) for t in (q, k, v, out))
    rng = np.random.default_rng(2)
    worst = 0.0
    for lane in sorted({0, w.lanes - 1, int(rng.integers(0, w.lanes))}):
        rows = np.array(sorted(set(range(64)) | set(range(w.S - 64, w.S)) | set(rng.integers(0, w.S, 128).tolist())))
        want = oracle.masked_attention_rows(ql[lane], kl[lane], vl[lane], rp_o, ci_o, rows, 64)
        worst = max(worst, float(np.max(np.abs(ol[lane][rows].to(torch.float64).numpy() - want))))
    print(f"per-row schedule nnz {ci_o.shape[0]}: max abs err {worst:.2e}")
    assert worst <= 1e-2
