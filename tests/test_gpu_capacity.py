"""Output capacity of the column view and the refinement for CSRs whose rows
share entries (a row_ptr that is not non-decreasing).

Both entry points size their output by a host bound that holds for a
non-decreasing row_ptr.  When rows re-read the same entries the output can need
more; the kernels then write nothing at or past the given capacity, and a call
that reads the count back returns TSA_ERR_SCHEDULE.  Each test passes a buffer
longer than the capacity it declares, filled with a sentinel, so that a write
past the capacity would land inside the allocation and show up as a changed
sentinel.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = -7
TSA_ERR_SCHEDULE = -4


@pytest.fixture(scope="module")
def tsa():
    import block_sparse_causal_amd as m

    return m


def _i32(x):
    return torch.as_tensor(np.asarray(x, np.int32)).to(DEV)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_transpose_overlapping_rows_stop_at_capacity(tsa):
    nb = 8
    row_ptr = _i32([0, 8, 0, 8, 0, 8, 0, 8, 0])  # rows 0, 2, 4, 6 each read all 8 entries
    col_idx = _i32(np.arange(8))
    cap = min(8, nb * (nb + 1) // 2)  # the host bound: 8; the rows accept 1 + 3 + 5 + 7 = 16
    col_ptr = torch.empty(nb + 1, dtype=torch.int32, device=DEV)
    row_idx = torch.full((cap + 64,), SENTINEL, dtype=torch.int32, device=DEV)
    ws_bytes = int(tsa._lib.tsa_schedule_transpose_workspace_bytes(nb))
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=DEV)
    aligned = ctypes.c_void_p((ws.data_ptr() + 255) // 256 * 256)
    total = ctypes.c_int64(0)
    st = tsa._lib.tsa_schedule_transpose(nb, _p(row_ptr), _p(col_idx), 8, _p(col_ptr), _p(row_idx), cap,
                                         aligned, ws_bytes, ctypes.byref(total), None)
    torch.cuda.synchronize()
    assert st == TSA_ERR_SCHEDULE, st
    assert b"row_capacity" in tsa._lib.tsa_last_error()
    assert total.value == 16
    tail = row_idx[cap:].cpu().numpy()
    assert (tail == SENTINEL).all(), tail
    head = row_idx[:cap].cpu().numpy()
    assert ((head >= 0) & (head < nb)).all(), head
    # the binding raises instead of returning a truncated view
    with pytest.raises(ValueError, match="row_capacity"):
        tsa.schedule_transpose(row_ptr, col_idx)


def test_refine_overlapping_rows_stop_at_capacity(tsa):
    S, block = 1024, 128  # 8 coarse rows, 16 fine rows
    row_ptr = _i32([0, 8, 0, 8, 0, 8, 0, 8, 0])
    col_idx = _i32(np.arange(8))
    cap = int(tsa._lib.tsa_refine_schedule_max_nnz(S, block, 8))  # min(4 * 8, 136) = 32
    assert cap == 32
    rp64 = torch.empty(S // 64 + 1, dtype=torch.int32, device=DEV)
    ci64 = torch.full((cap + 64,), SENTINEL, dtype=torch.int32, device=DEV)
    total = ctypes.c_int64(0)
    st = tsa._lib.tsa_refine_schedule(S, block, _p(row_ptr), _p(col_idx), 8, _p(rp64), _p(ci64), cap,
                                      ctypes.byref(total), None)
    torch.cuda.synchronize()
    assert st == TSA_ERR_SCHEDULE, st
    # fine rows 0,1 | 4,5 | 8,9 | 12,13 hold 1+2 | 5+6 | 9+10 | 13+14 entries
    assert total.value == 60
    tail = ci64[cap:].cpu().numpy()
    assert (tail == SENTINEL).all(), tail
    with pytest.raises(ValueError, match="capacity"):
        tsa.refine_schedule(row_ptr, col_idx, S, block)
