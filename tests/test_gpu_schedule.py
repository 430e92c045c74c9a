"""Parity of the HIP schedule builder with the fp64 all-pairs oracle.

CSR row_ptr/col_idx must be bit-identical on inputs without near-ties (the
workload seeds are checked for that in test_workloads.py); salience must match
to a relative 1e-12 (fp64 distances summed in a different order).
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
    rp_o, ci_o, sal_o = oracle.build_schedule(keys_cpu, 64, sink, radius, topk)
    rp, ci, sal = tsa.build_schedule(keys_cpu.to("cuda:0"), 64, sink, radius, topk, return_salience=True)
    assert rp.device.type == "cuda" and rp.dtype == torch.int32 and ci.dtype == torch.int32
    rp, ci, sal = rp.cpu().numpy(), ci.cpu().numpy(), sal.cpu().numpy()
    assert np.array_equal(rp, rp_o), label
    assert np.array_equal(ci, ci_o), label
    assert np.allclose(sal, sal_o, rtol=1e-12, atol=0), (label, np.max(np.abs(sal - sal_o)))
    assert np.count_nonzero(sal == 0) == (1 if sal.shape[0] > 0 else 0)
    return rp, ci


@pytest.mark.parametrize("name", [n for n, w in workloads.WORKLOADS.items() if not w.dense])
def test_workload_schedules_bit_exact(tsa, name):
    w = workloads.WORKLOADS[name]
    _, k, _ = workloads.make_qkv(w)
    keys = k.reshape(-1, w.S, w.D)[0].contiguous()
    rp, ci = _compare(tsa, keys, w.sink, w.local_radius, w.topk, name)
    print(f"{name}: nnz {ci.shape[0]} of {w.nb * (w.nb + 1) // 2} causal blocks")


def test_page_configuration_count_range(tsa):
    """16 blocks, sink 1, radius 1, top-2: 45 + a term in [0, 27] (pages' port: 56 of 136)."""
    counts = []
    for seed in range(10):
        keys = workloads.random_normal((1024, 64), "fp16", 1000 + seed)
        rp, _ = _compare(tsa, keys, 1, 1, 2, f"seed {seed}")
        counts.append(int(rp[-1]))
    assert all(45 <= c <= 72 for c in counts), counts


@pytest.mark.parametrize("seed", range(24))
def test_random_small_configurations(tsa, seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 21))
    S = 64 * nb - int(rng.integers(0, 64)) if nb > 1 else int(rng.integers(1, 65))
    D = int(rng.choice([8, 64, 128]))
    dt = "bf16" if seed % 2 else "fp16"
    sink, radius, topk = (int(x) for x in rng.integers(0, 5, 3))
    keys = workloads.random_normal((S, D), dt, 2000 + seed, std=float(rng.choice([0.5, 1.0, 3.0])))
    _compare(tsa, keys, sink, radius, topk, f"seed {seed} nb {nb} S {S}")


@pytest.mark.parametrize("nb", [65, 130, 300, 700])
def test_multi_slot_sizes(tsa, nb):
    keys = workloads.random_normal((64 * nb - 5, 32), "bf16", 3000 + nb)
    _compare(tsa, keys, 2, 3, 17, f"nb {nb}")


def test_topk_at_least_nb_gives_dense(tsa):
    keys = workloads.random_normal((64 * 9, 64), "fp16", 7)
    rp, ci = tsa.build_schedule(keys.to("cuda:0"), 64, 0, 0, 9)
    drp, dci = oracle.dense_causal_schedule(9)
    assert np.array_equal(rp.cpu().numpy(), drp) and np.array_equal(ci.cpu().numpy(), dci)


def test_four_dim_keys_use_lane_zero(tsa):
    k = workloads.random_normal((2, 3, 64 * 10, 64), "bf16", 8)
    a = tsa.build_schedule(k.to("cuda:0"), 64, 1, 1, 3)
    b = tsa.build_schedule(k[0, 0].contiguous().to("cuda:0"), 64, 1, 1, 3)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_keys_give_empty_schedule(tsa):
    keys = torch.empty(0, 64, dtype=torch.float16, device="cuda:0")
    rp, ci = tsa.build_schedule(keys, 64, 1, 1, 2)
    assert rp.cpu().tolist() == [0] and ci.numel() == 0


def test_hand_worked_elder_examples_on_gpu(tsa):
    from conftest import read_golden_rows

    for row in read_golden_rows("elder_rule_line_examples.txt"):
        pos, expect = row.split("|")
        xs = [float(x) for x in pos.split()]
        keys = torch.zeros(64 * len(xs), 64, dtype=torch.float16)
        for j, x in enumerate(xs):
            keys[64 * j : 64 * (j + 1), 0] = x
        _, _, sal = tsa.build_schedule(keys.to("cuda:0"), 64, 0, 0, 0, return_salience=True)
        assert sal.cpu().tolist() == [float(x) for x in expect.split()]


@pytest.mark.parametrize("nb", [0, 1, 16, 64, 128, 517])
def test_dense_schedule(tsa, nb):
    rp, ci = tsa.dense_causal_schedule(nb, "cuda:0")
    drp, dci = oracle.dense_causal_schedule(nb)
    assert np.array_equal(rp.cpu().numpy(), drp) and np.array_equal(ci.cpu().numpy(), dci)


def test_builder_validation(tsa):
    keys = torch.zeros(128, 64, dtype=torch.float16, device="cuda:0")
    for bad_block in (16, 48, 96):  # 32 and multiples of 64 are the accepted sizes
        with pytest.raises(ValueError, match="UNSUPPORTED"):
            tsa.build_schedule(keys, bad_block, 1, 1, 2)
    with pytest.raises(ValueError, match="INVALID_ARG"):
        tsa.build_schedule(keys, 64, -1, 1, 2)
    with pytest.raises(TypeError):
        tsa.build_schedule(keys.float(), 64, 1, 1, 2)
    big = torch.zeros(64 * 4097, 8, dtype=torch.float16, device="cuda:0")
    with pytest.raises(ValueError, match="UNSUPPORTED"):
        tsa.build_schedule(big, 64, 1, 1, 2)


def test_builder_then_attention_end_to_end(tsa):
    w = workloads.WORKLOADS["single_s1024_d64_f16"]
    q, k, v = workloads.make_qkv(w)
    rp, ci = tsa.build_schedule(k.to("cuda:0"), 64, w.sink, w.local_radius, w.topk)
    out = tsa.scheduled_attention(q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0"), rp, ci)
    rp_o, ci_o, _ = oracle.build_schedule(k, 64, w.sink, w.local_radius, w.topk)
    want = oracle.masked_attention(q, k, v, rp_o, ci_o, 64)
    assert float(np.max(np.abs(out.cpu().double().numpy() - want))) <= 2e-3


def _compare_tied(tsa, keys_cpu, sink, radius, topk, label):
    """Inputs with exactly tied distances: the edge order (length, lower, higher)
    decides, on both sides, which pair is taken first."""
    rp_o, ci_o, sal_o = oracle.build_schedule(keys_cpu, 64, sink, radius, topk)
    rp, ci, sal = tsa.build_schedule(keys_cpu.to("cuda:0"), 64, sink, radius, topk, return_salience=True)
    assert np.array_equal(rp.cpu().numpy(), rp_o), label
    assert np.array_equal(ci.cpu().numpy(), ci_o), label
    # squared distances are small integers here, so only the square root rounds
    assert np.allclose(sal.cpu().numpy(), sal_o, rtol=1e-15, atol=0), label


def _keys_at(points, D=64):
    """Keys whose block j has every row equal to points[j] (zero-padded to D)."""
    nb, p = points.shape
    keys = torch.zeros(64 * nb, D, dtype=torch.float16)
    keys[:, :p] = torch.from_numpy(np.repeat(points, 64, axis=0)).to(torch.float16)
    return keys


@pytest.mark.parametrize("nb", [1, 2, 20, 64, 100, 128, 200])
def test_exact_ties_identical_blocks(tsa, nb):
    # every distance is 0: the MST is the star of block 0 and every merge is a size tie
    _compare_tied(tsa, torch.zeros(64 * nb, 64, dtype=torch.float16), 1, 1, 3, f"zeros nb {nb}")


@pytest.mark.parametrize("nb", [20, 64, 128, 300])
def test_exact_ties_shuffled_lattice(tsa, nb):
    rng = np.random.default_rng(nb)
    side = int(np.ceil(np.sqrt(nb)))
    pts = np.array([(x, y) for x in range(side) for y in range(side)][:nb], dtype=np.float64)
    pts = pts[rng.permutation(nb)]
    _compare_tied(tsa, _keys_at(pts), 1, 2, 5, f"lattice nb {nb}")


@pytest.mark.parametrize("nb", [40, 128, 260])
def test_exact_ties_repeated_points(tsa, nb):
    rng = np.random.default_rng(10 + nb)
    pts = rng.integers(-2, 3, size=(nb, 3)).astype(np.float64)  # many exact duplicates
    _compare_tied(tsa, _keys_at(pts, D=8), 2, 1, 7, f"repeats nb {nb}")


@pytest.mark.parametrize("nb,D", [(3, 20), (17, 200), (64, 64), (100, 72), (128, 128)])
def test_reused_and_prefilled_workspace(tsa, nb, D):
    """One set of buffers serves several builds with different keys, and the
    workspace is filled with zeros, ones or a byte pattern before some builds:
    every schedule still matches the oracle, so the builder needs no cleared
    workspace and leaves nothing behind that misleads the next call."""
    S = 64 * nb - 7
    bufs = tsa.ScheduleBuffers(S, D, 1, 2, 5, "cuda:0", salience=True)
    for it, fill in enumerate([None, 0x00, 0xFF, None, 0x5A, None]):
        keys = workloads.random_normal((S, D), "bf16", 4000 + 10 * nb + it)
        if fill is not None:
            bufs._ws.fill_(fill)
        tsa.build_schedule_into(keys.to("cuda:0"), bufs)
        rp_o, ci_o, sal_o = oracle.build_schedule(keys, 64, 1, 2, 5)
        rp = bufs.row_ptr.cpu().numpy()
        nnz = int(rp[-1])
        label = f"nb {nb} D {D} build {it} fill {fill}"
        assert np.array_equal(rp, rp_o), label
        assert np.array_equal(bufs.col_idx[:nnz].cpu().numpy(), ci_o), label
        assert np.allclose(bufs.salience.cpu().numpy(), sal_o, rtol=1e-12, atol=0), label


def test_workspace_shared_across_block_counts(tsa):
    """One workspace serves builds of several block counts in turn, on both
    builder paths, with repeats and changes of size: the words one size uses to
    elect its last workgroup then sit where another size keeps its flags.  Every
    schedule still matches the oracle."""
    D = 64
    seq = [64, 16, 64, 64, 300, 300, 64, 16, 16, 300, 100]
    need = [int(tsa._lib.tsa_build_schedule_workspace_bytes(64 * nb, D, 64)) for nb in seq]
    shared = torch.empty(max(need) + 256, dtype=torch.uint8, device="cuda:0")
    shared.fill_(0x3C)
    for it, nb in enumerate(seq):
        S = 64 * nb
        bufs = tsa.ScheduleBuffers(S, D, 1, 2, 5, "cuda:0", salience=True)
        bufs.ws_ptr = (shared.data_ptr() + 255) // 256 * 256
        bufs.ws_bytes = max(need)
        keys = workloads.random_normal((S, D), "fp16", 4500 + it)
        tsa.build_schedule_into(keys.to("cuda:0"), bufs)
        rp_o, ci_o, sal_o = oracle.build_schedule(keys, 64, 1, 2, 5)
        rp = bufs.row_ptr.cpu().numpy()
        nnz = int(rp[-1])
        label = f"build {it} nb {nb}"
        assert np.array_equal(rp, rp_o), label
        assert np.array_equal(bufs.col_idx[:nnz].cpu().numpy(), ci_o), label
        assert np.allclose(bufs.salience.cpu().numpy(), sal_o, rtol=1e-12, atol=0), label


@pytest.mark.parametrize("nb", [256, 512])
def test_more_boruvka_rounds_than_launched(tsa, nb):
    """Block v's rows sit at the point whose coordinate l is 2^l times bit l of v.
    Every Boruvka round then pairs each component with the one that differs in
    its lowest free bit (all such edges tie in length), so the tree needs exactly
    log2(nb) rounds, more than the large path launches: the last launch's
    elected workgroup runs the remaining rounds itself.  Every merge is between
    equal sizes, so the elder rule's index tie-break decides each one."""
    bits = int(np.log2(nb))
    pts = np.array([[((v >> b) & 1) * 2.0 ** b for b in range(bits)] for v in range(nb)])
    _compare_tied(tsa, _keys_at(pts, D=16), 1, 2, 5, f"binary nb {nb}")


def test_largest_schedule(tsa):
    """The builder's limit, 4096 blocks (S = 262,144; the multi-launch path with the
    LDS edge sort), bit-exact against the oracle's all-pairs scan."""
    keys = workloads.random_normal((64 * 4096, 8), "fp16", 4096)
    rp, ci = _compare(tsa, keys, 2, 2, 24, "nb 4096")
    assert rp.shape[0] == 4097
