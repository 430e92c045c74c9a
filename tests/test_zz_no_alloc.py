"""tsa_build_schedule_noalloc (the builder with the library's fixed device
workspace, for callers that cannot allocate) against tsa_build_schedule_ex (the
same build with a caller-owned workspace): row_ptr and col_idx bit for bit and
salience bit for bit, on consecutive calls that each use a smaller input than
the one before, so that every call runs over what the previous one left in the
shared array.  Also: a build too large for the array is rejected before any
GPU work and writes nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _keys(S, D, dtype, seed, mixture):
    shape = (S, D)
    w = workloads.Workload("noalloc", shape, dtype, "mixture" if mixture else "normal", 8 if mixture else 0,
                           seed=seed)
    return workloads.make_qkv(w)[1].to(DEV)


def _reference(tsa, keys, block, sink, r, k, per_row):
    bufs = tsa.ScheduleBuffers(keys.shape[0], keys.shape[1], sink, r, k, DEV, salience=True, per_row=per_row,
                               block=block)
    tsa.build_schedule_into(keys, bufs)
    torch.cuda.synchronize()
    nnz = int(bufs.row_ptr[-1].item())
    return bufs.row_ptr.cpu().numpy(), bufs.col_idx[:nnz].cpu().numpy(), bufs.salience[:bufs.nb].cpu().numpy()


def _noalloc(tsa, keys, block, sink, r, k, per_row):
    S, D = keys.shape
    nb = -(-S // block)
    cap = int(tsa._lib.tsa_schedule_max_nnz(nb, sink, r, k))
    row_ptr = torch.full((nb + 1,), -3, dtype=torch.int32, device=DEV)
    col_idx = torch.full((max(cap, 1),), -3, dtype=torch.int32, device=DEV)
    sal = torch.full((max(nb, 1),), float("nan"), dtype=torch.float64, device=DEV)
    code = 1 if keys.dtype == torch.bfloat16 else 0
    vp = ctypes.c_void_p
    st = tsa._lib.tsa_build_schedule_noalloc(
        vp(keys.data_ptr()), code, S, D, block, sink, r, k, 1 if per_row else 0, vp(row_ptr.data_ptr()),
        vp(col_idx.data_ptr()), cap, vp(sal.data_ptr()), vp(torch.cuda.current_stream().cuda_stream))
    assert st == 0, tsa._lib.tsa_last_error()
    torch.cuda.synchronize()
    nnz = int(row_ptr[-1].item())
    return row_ptr.cpu().numpy(), col_idx[:nnz].cpu().numpy(), sal[:nb].cpu().numpy()


# largest first: each call runs over the previous call's contents of the array
CALLS = [
    # (S, D, dtype, block, sink, r, k, per_row, mixture, seed)
    (32768, 64, "bf16", 64, 2, 4, 32, False, True, 11),  # 512 blocks: multi-launch path, 2 MB of distances
    (16384, 128, "fp16", 64, 1, 2, 16, True, True, 12),  # 256 blocks, per-row top-k
    (4096, 64, "bf16", 64, 1, 2, 16, False, False, 13),  # 64 blocks: one-launch path
    (3000, 64, "fp16", 128, 1, 1, 4, False, True, 14),   # 24 blocks of 128 rows, ragged tail
    (1024, 32, "bf16", 64, 1, 1, 2, True, False, 15),    # 16 blocks
]


def test_noalloc_matches_workspace_build_on_shrinking_calls(tsa):
    for S, D, dtype, block, sink, r, k, per_row, mixture, seed in CALLS:
        print(f"noalloc build S={S} D={D} {dtype} block {block} ({sink},{r},{k}) per_row={per_row}", flush=True)
        keys = _keys(S, D, dtype, seed, mixture)
        want = _reference(tsa, keys, block, sink, r, k, per_row)
        got = _noalloc(tsa, keys, block, sink, r, k, per_row)
        assert np.array_equal(got[0], want[0]), "row_ptr"
        assert np.array_equal(got[1], want[1]), "col_idx"
        assert np.array_equal(got[2], want[2]), "salience"
    # the first (largest) build again, over the smallest one's leftovers
    S, D, dtype, block, sink, r, k, per_row, mixture, seed = CALLS[0]
    keys = _keys(S, D, dtype, seed, mixture)
    want = _reference(tsa, keys, block, sink, r, k, per_row)
    got = _noalloc(tsa, keys, block, sink, r, k, per_row)
    assert all(np.array_equal(a, b) for a, b in zip(got, want))


def test_noalloc_rejects_builds_beyond_the_array(tsa):
    S, D, block = 65536, 64, 64  # 1024 blocks: 8 MB of distances > TSA_NOALLOC_SCRATCH_BYTES
    need = int(tsa._lib.tsa_build_schedule_workspace_bytes(S, D, block))
    assert need > 4 << 20
    keys = torch.zeros((S, D), dtype=torch.bfloat16, device=DEV)
    nb = S // block
    cap = int(tsa._lib.tsa_schedule_max_nnz(nb, 1, 1, 2))
    row_ptr = torch.full((nb + 1,), -3, dtype=torch.int32, device=DEV)
    col_idx = torch.full((cap,), -3, dtype=torch.int32, device=DEV)
    vp = ctypes.c_void_p
    st = tsa._lib.tsa_build_schedule_noalloc(vp(keys.data_ptr()), 1, S, D, block, 1, 1, 2, 0,
                                             vp(row_ptr.data_ptr()), vp(col_idx.data_ptr()), cap, vp(None),
                                             vp(None))
    torch.cuda.synchronize()
    assert st == -2
    assert b"workspace" in tsa._lib.tsa_last_error()
    assert bool((row_ptr == -3).all()) and bool((col_idx == -3).all())


def test_binding_wrapper(tsa):
    keys = _keys(2048, 64, "bf16", 16, True)
    want = _reference(tsa, keys, 64, 1, 1, 4, False)
    nb = 32
    row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=DEV)
    col_idx = torch.empty(int(tsa.schedule_max_nnz(nb, 1, 1, 4)), dtype=torch.int32, device=DEV)
    tsa.build_schedule_noalloc(keys, row_ptr, col_idx, 64, 1, 1, 4)
    torch.cuda.synchronize()
    nnz = int(row_ptr[-1].item())
    assert np.array_equal(row_ptr.cpu().numpy(), want[0])
    assert np.array_equal(col_idx[:nnz].cpu().numpy(), want[1])
