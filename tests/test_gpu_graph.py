"""Schedule build + attention captured in a HIP graph and replayed, through the
C ABI: every replay, with new keys copied into the captured buffers between
replays (eager work and synchronisations in between), must give the oracle's
schedule (bit-exact) and attention (fp16: max abs error <= 2e-3).  The
one-launch builder's election token changes per replay through the epoch word
in its workspace, so a replay never reuses the previous call's token.
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


@pytest.mark.parametrize("S", [4096, 64 * 200])  # one-launch builder (64 blocks), multi-launch (200)
def test_replayed_graph_rebuilds_the_schedule(tsa, S):
    D = 64
    bufs = tsa.ScheduleBuffers(S, D, 1, 1, 4, DEV)
    q_s = torch.zeros((S, D), dtype=torch.float16, device=DEV)
    k_s = torch.zeros_like(q_s)
    v_s = torch.zeros_like(q_s)
    out = torch.empty_like(q_s)
    # one eager call before capture (the library allocates nothing; this warms the buffers)
    tsa.build_schedule_into(k_s, bufs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tsa.build_schedule_into(k_s, bufs)
        tsa.scheduled_attention(q_s, k_s, v_s, bufs.row_ptr, bufs.col_idx, out=out)
    for rep, seed in enumerate([11, 12, 13, 12]):
        q, k, v = workloads.make_qkv(workloads.Workload("t", (S, D), "fp16", seed=seed))
        q_s.copy_(q.to(DEV))
        k_s.copy_(k.to(DEV))
        v_s.copy_(v.to(DEV))
        _ = (q_s.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rp_o, ci_o, _ = oracle.build_schedule(k, 64, 1, 1, 4)
        nnz = int(bufs.row_ptr[-1].item())
        np.testing.assert_array_equal(bufs.row_ptr.cpu().numpy(), rp_o)
        np.testing.assert_array_equal(bufs.col_idx[:nnz].cpu().numpy(), ci_o)
        rows = np.arange(0, S, 37)
        ref = oracle.masked_attention_rows(q, k, v, rp_o, ci_o, rows)
        err = float(np.abs(out[torch.from_numpy(rows).to(DEV)].double().cpu().numpy() - ref).max())
        print(f"S {S} replay {rep} seed {seed}: nnz {nnz}, max err {err:.2e}")
        assert err <= 2e-3
