"""The C ABI library on any host: it loads, exports every declared entry point,
and its host-side logic (capacity bound, workspace size, argument checks that
precede any GPU call) behaves as include/tsa.h states.  No compute call is made.
"""
import ctypes
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsa.h")


@pytest.fixture(scope="module")
def lib():
    path = os.environ.get("TSA_ABI_LIBRARY")
    if path:
        # another build of the library (test_abi_sanitized.py's host-sanitizer
        # build), with the package's signatures, without importing the package
        spec = importlib.util.spec_from_file_location(
            "_tsa_abi", os.path.join(ROOT, "block_sparse_causal_amd", "_abi.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        other = ctypes.CDLL(path)
        mod.declare_signatures(other)
        return other
    import block_sparse_causal_amd as tsa

    return tsa._lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for required in ("tsa_build_schedule", "tsa_scheduled_attention_fwd", "tsa_dense_causal_schedule",
                     "tsa_segment_schedule", "tsa_segment_schedule_nnz", "tsa_schedule_max_nnz",
                     "tsa_build_schedule_ex",
                     "tsa_build_schedule_workspace_bytes", "tsa_last_error", "tsa_version",
                     "tsa_scheduled_attention_fwd_lse", "tsa_schedule_transpose",
                     "tsa_schedule_transpose_workspace_bytes", "tsa_scheduled_attention_bwd",
                     "tsa_scheduled_attention_bwd_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


@pytest.mark.skipif(bool(os.environ.get("TSA_ABI_LIBRARY")), reason="checks the package's own library")
def test_library_file_is_in_tree():
    import block_sparse_causal_amd as tsa

    assert os.path.dirname(tsa.library_path()) == os.path.join(ROOT, "block_sparse_causal_amd")


@pytest.mark.parametrize("nb,s,r,k", [(16, 1, 1, 2), (64, 1, 1, 8), (64, 1, 2, 16), (512, 2, 4, 32),
                                      (0, 1, 1, 1), (5, 0, 0, 0), (3, 10, 10, 10)])
def test_max_nnz_bound(lib, nb, s, r, k):
    brute = sum(min(i + 1, s + r + 1 + k) for i in range(nb))
    assert lib.tsa_schedule_max_nnz(nb, s, r, k) == brute


def test_max_nnz_bound_holds_for_oracle_schedules(lib):
    import oracle

    rng = np.random.default_rng(0)
    for _ in range(20):
        nb = int(rng.integers(1, 40))
        s, r, k = (int(x) for x in rng.integers(0, 6, 3))
        rp, _, _ = oracle.build_schedule(rng.standard_normal((64 * nb, 4)), 64, s, r, k)
        assert rp[-1] <= lib.tsa_schedule_max_nnz(nb, s, r, k)


@pytest.mark.parametrize("nb,seg", [(64, 8), (64, 4), (64, 64), (64, 100), (0, 3), (1, 1), (13, 5),
                                    (100, 7)])
def test_segment_nnz_matches_oracle(lib, nb, seg):
    import oracle

    rp, _ = oracle.fixed_segment_schedule(nb, seg)
    assert lib.tsa_segment_schedule_nnz(nb, seg) == int(rp[-1])


def test_segment_schedule_checks_before_gpu(lib):
    vp = ctypes.c_void_p
    assert lib.tsa_segment_schedule_nnz(4, 0) == -1 and lib.tsa_segment_schedule_nnz(-1, 2) == -1
    assert lib.tsa_segment_schedule(4, 0, vp(None), vp(None), 10, vp(None)) == -1
    assert b"segment_blocks" in lib.tsa_last_error()
    assert lib.tsa_segment_schedule(64, 8, vp(None), vp(None), 287, vp(None)) == -4  # short col_idx
    assert lib.tsa_segment_schedule(64, 8, vp(None), vp(None), 288, vp(None)) == -1  # NULL outputs


def test_build_schedule_ex_rejects_unknown_scope(lib):
    vp = ctypes.c_void_p
    f = lib.tsa_build_schedule_ex
    f.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, ctypes.c_int64, vp, vp,
                  ctypes.c_size_t, ctypes.POINTER(ctypes.c_int64), vp]
    assert f(None, 1, 128, 64, 64, 1, 1, 2, 2, None, None, 10, None, None, 0, None, None) == -1
    assert b"topk_scope" in lib.tsa_last_error()


def test_max_nnz_bound_holds_for_per_row_oracle_schedules(lib):
    import oracle

    rng = np.random.default_rng(1)
    for _ in range(20):
        nb = int(rng.integers(1, 40))
        s, r, k = (int(x) for x in rng.integers(0, 6, 3))
        rp, _, _ = oracle.build_schedule(rng.standard_normal((64 * nb, 4)), 64, s, r, k, per_row=True)
        assert rp[-1] <= lib.tsa_schedule_max_nnz(nb, s, r, k)


def test_max_nnz_rejects_negative(lib):
    assert lib.tsa_schedule_max_nnz(4, -1, 0, 0) == -1
    assert b"must be" in lib.tsa_last_error()


def test_workspace_bytes(lib):
    # centroids always; the distance matrix only when it does not stay in LDS (nb > 128)
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 64) >= 64 * 64 * 8
    assert lib.tsa_build_schedule_workspace_bytes(64 * 200, 64, 64) >= 200 * 64 * 8 + 200 * 200 * 8
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 32) >= 128 * 64 * 8  # 32-row blocks
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 16) == 0
    assert lib.tsa_build_schedule_workspace_bytes(64 * 5000, 64, 64) == 0


def _fwd(lib, **kw):
    args = dict(q=None, k=None, v=None, out=None, dtype=0, B=1, H=1, S=128, D=64, row_ptr=None,
                col_idx=None, nnz=3, block=64, scale=0.0, stream=None)
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.tsa_scheduled_attention_fwd(
        vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["out"]), args["dtype"], args["B"], args["H"],
        args["S"], args["D"], vp(args["row_ptr"]), vp(args["col_idx"]), args["nnz"], args["block"],
        args["scale"], vp(args["stream"]))


def test_attention_argument_checks_before_gpu(lib):
    assert _fwd(lib, dtype=5) == -1
    assert _fwd(lib, B=-1) == -1
    assert _fwd(lib, block=32) == -1  # 32-row blocks at D 64: the NULL pointers are what fail
    for d in (32, 128):
        assert _fwd(lib, block=32, D=d) == -1
    assert _fwd(lib, block=32, D=256) == -2  # 32-row blocks stop at head dim 128
    assert b"32-row blocks" in lib.tsa_last_error()
    assert _fwd(lib, block=32, S=65535 * 128 + 1) == -2  # past the grid's pair count
    assert _fwd(lib, block=16) == -2
    assert _fwd(lib, block=128) == -2
    assert _fwd(lib, D=96) == -2
    assert b"32, 64, 128 or 256" in lib.tsa_last_error()
    assert _fwd(lib, D=512) == -2
    for d in (32, 256):
        assert _fwd(lib, D=d) == -1  # a supported head dim: the NULL pointers are what fail
    assert _fwd(lib, scale=float("nan")) == -1
    assert _fwd(lib) == -1  # NULL pointers for a non-empty problem
    assert _fwd(lib, S=0) == 0  # empty problem is a no-op
    assert _fwd(lib, B=0) == 0
    assert lib.tsa_last_error() == b""


def test_attention_rejects_overlapping_output(lib):
    base = 1 << 40  # never dereferenced: the overlap check precedes any GPU call
    st = _fwd(lib, q=base, k=base + (1 << 20), v=base + (2 << 20), out=base + 64, row_ptr=base, col_idx=base)
    assert st == -1 and b"overlap" in lib.tsa_last_error()


def test_builder_argument_checks_before_gpu(lib):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64

    def call(dtype=0, S=1024, D=64, block=64, s=1, r=1, k=2, cap=1000, ws=1 << 20):
        return lib.tsa_build_schedule(vp(None), dtype, S, D, block, s, r, k, vp(None), vp(None), cap,
                                      vp(None), vp(None), ws, None, vp(None))

    assert call(dtype=3) == -1
    assert call(S=-1) == -1
    assert call(s=-2) == -1
    assert call(block=96) == -2  # not a multiple of 64
    assert call(block=128) == -1  # a valid block; the NULL row_ptr is what fails
    assert call(S=64 * 4097) == -2
    assert call() == -1  # NULL row_ptr
    assert b"row_ptr" in lib.tsa_last_error()


def test_dense_schedule_argument_checks_before_gpu(lib):
    vp = ctypes.c_void_p
    assert lib.tsa_dense_causal_schedule(-1, vp(None), vp(None), 0, vp(None)) == -1
    assert lib.tsa_dense_causal_schedule(10, vp(None), vp(None), 54, vp(None)) == -4
    assert lib.tsa_dense_causal_schedule(10, vp(None), vp(None), 55, vp(None)) == -1
    assert lib.tsa_dense_causal_schedule(70000, vp(None), vp(None), 1 << 40, vp(None)) == -3


def test_fwd_lse_requires_lse(lib):
    vp = ctypes.c_void_p
    base = 1 << 40  # never dereferenced: the NULL check precedes any GPU call
    st = lib.tsa_scheduled_attention_fwd_lse(vp(base), vp(base + (1 << 24)), vp(base + (2 << 24)),
                                             vp(base + (3 << 24)), vp(None), 1, 1, 1, 128, 64,
                                             vp(base), vp(base), 3, 64, 0.0, vp(None))
    assert st == -1 and b"NULL" in lib.tsa_last_error()
    # lse overlapping out
    st = lib.tsa_scheduled_attention_fwd_lse(vp(base), vp(base + (1 << 24)), vp(base + (2 << 24)),
                                             vp(base + (3 << 24)), vp(base + (3 << 24) + 64), 1, 1, 1, 128,
                                             64, vp(base), vp(base), 3, 64, 0.0, vp(None))
    assert st == -1 and b"overlap" in lib.tsa_last_error()
    assert lib.tsa_scheduled_attention_fwd_lse(vp(None), vp(None), vp(None), vp(None), vp(None), 1, 0, 1,
                                               128, 64, vp(None), vp(None), 0, 64, 0.0, vp(None)) == 0


def test_transpose_workspace_and_checks_before_gpu(lib):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    assert lib.tsa_schedule_transpose_workspace_bytes(0) == 0
    assert lib.tsa_schedule_transpose_workspace_bytes(-3) == 0
    assert lib.tsa_schedule_transpose_workspace_bytes(4097) == 0
    for nb in (1, 31, 32, 33, 64, 512, 4096):
        nw = -(-nb // 32)
        assert lib.tsa_schedule_transpose_workspace_bytes(nb) == 4 * (nw * nb + nb)

    def call(nb=10, nnz=55, cap=55, ws=1 << 20, rp=None, ci=None, cp=None, ri=None, wsp=None):
        return lib.tsa_schedule_transpose(nb, vp(rp), vp(ci), nnz, vp(cp), vp(ri), cap, vp(wsp), ws, None,
                                          vp(None))

    assert call(nb=-1) == -1
    assert call(nnz=-1) == -1
    assert call(nb=4097, nnz=0, cap=0) == -2
    assert call(cap=54) == -4  # min(nnz, nb(nb+1)/2) = 55
    assert call(nnz=100, cap=54) == -4
    assert b"row_capacity" in lib.tsa_last_error()
    assert call() == -1  # NULL pointers
    base = 1 << 40
    assert call(rp=base, ci=base, cp=base, ri=base, wsp=base, ws=10) == -1
    assert b"workspace" in lib.tsa_last_error()
    assert call(rp=base, ci=base, cp=base, ri=base, wsp=base + 16) == -1
    assert b"aligned" in lib.tsa_last_error()


def _bwd(lib, **kw):
    vp = ctypes.c_void_p
    a = dict(q=None, k=None, v=None, out=None, dout=None, lse=None, dtype=1, B=1, H=1, S=128, D=64,
             row_ptr=None, col_idx=None, nnz=3, col_ptr=None, row_idx=None, nnz_t=3, block=64, scale=0.0,
             dq=None, dk=None, dv=None, ws=None, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.tsa_scheduled_attention_bwd(
        vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["out"]), vp(a["dout"]), vp(a["lse"]), a["dtype"], a["B"],
        a["H"], a["S"], a["D"], vp(a["row_ptr"]), vp(a["col_idx"]), a["nnz"], vp(a["col_ptr"]),
        vp(a["row_idx"]), a["nnz_t"], a["block"], a["scale"], vp(a["dq"]), vp(a["dk"]), vp(a["dv"]),
        vp(a["ws"]), a["ws_bytes"], vp(a["stream"]))


def test_backward_workspace_and_checks_before_gpu(lib):
    assert lib.tsa_scheduled_attention_bwd_workspace_bytes(4, 16, 4096) == 4 * 16 * 4096 * 8 + 64 * 4
    assert lib.tsa_scheduled_attention_bwd_workspace_bytes(1, 1, 100) == 800 + 2 * 4
    assert lib.tsa_scheduled_attention_bwd_workspace_bytes(1, 1, 3) == 32 + 4
    assert lib.tsa_scheduled_attention_bwd_workspace_bytes(-1, 1, 1) == 0
    assert lib.tsa_scheduled_attention_bwd_workspace_bytes(1, 1, 1 << 62) == 0
    assert _bwd(lib, dtype=7) == -1
    assert _bwd(lib, D=96) == -2
    assert _bwd(lib, D=256) == -1  # head dim 256 passes the checks; the NULL pointers fail
    assert _bwd(lib, D=256, block=32) == -2  # 32-row blocks stop at head dim 128
    assert _bwd(lib, D=32) == -1
    assert _bwd(lib, block=128) == -2
    assert _bwd(lib, block=48) == -2
    assert _bwd(lib, block=32) == -1  # 32-row blocks pass the block check; the NULL pointers fail
    assert _bwd(lib, nnz_t=-1) == -1
    assert _bwd(lib, scale=float("inf")) == -1
    assert _bwd(lib) == -1 and b"NULL" in lib.tsa_last_error()
    assert _bwd(lib, S=0) == 0 and _bwd(lib, H=0) == 0
    base = 1 << 40  # never dereferenced: these checks precede any GPU call
    mb = 1 << 24
    good = dict(q=base, k=base + mb, v=base + 2 * mb, out=base + 3 * mb, dout=base + 4 * mb, lse=base + 5 * mb,
                row_ptr=base, col_idx=base, col_ptr=base, row_idx=base, dq=base + 6 * mb, dk=base + 7 * mb,
                dv=base + 8 * mb, ws=base + 9 * mb)
    assert _bwd(lib, **{**good, "ws_bytes": 128 * 8 - 1}) == -1
    assert b"workspace" in lib.tsa_last_error()
    assert _bwd(lib, **{**good, "dq": base + 2 * mb + 256}) == -1  # dq overlaps v
    assert b"overlap" in lib.tsa_last_error()
    assert _bwd(lib, **{**good, "dv": base + 6 * mb + 512}) == -1  # dv overlaps dq
    assert b"overlap" in lib.tsa_last_error()
    assert _bwd(lib, **{**good, "ws": base + 5 * mb + 16}) == -1  # workspace overlaps lse
    assert _bwd(lib, **{**good, "dk": base + 7 * mb + 8}) == -1  # misaligned
    assert b"aligned" in lib.tsa_last_error()


def test_block_sizes_accepted_by_builder_and_refinement(lib):
    vp = ctypes.c_void_p
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 128) > 0
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 4096) > 0
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 96) == 0
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 8192) == 0
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 32) > 0
    assert lib.tsa_build_schedule_workspace_bytes(4096, 64, 48) == 0
    # block 32 is valid: the NULL row_ptr is what fails
    assert lib.tsa_build_schedule(vp(None), 0, 4096, 64, 32, 1, 1, 2, vp(None), vp(None), 1000, vp(None),
                                  vp(None), 1 << 20, None, vp(None)) == -1
    # the refinement keeps to multiples of 64
    assert lib.tsa_refine_schedule_max_nnz(4096, 32, 10) == -1
    # block 96 is not a multiple of 64: unsupported before any GPU call
    assert lib.tsa_build_schedule(vp(None), 0, 4096, 64, 96, 1, 1, 2, vp(None), vp(None), 1000, vp(None),
                                  vp(None), 1 << 20, None, vp(None)) == -2
    # block 128 at S = 128 * 4097 blocks exceeds the builder's limit
    assert lib.tsa_build_schedule(vp(None), 0, 128 * 4097, 64, 128, 1, 1, 2, vp(None), vp(None), 1 << 30,
                                  vp(None), vp(None), 1 << 20, None, vp(None)) == -2


@pytest.mark.parametrize("S,block,nnz", [(4096, 128, 100), (4096, 256, 10), (1000, 128, 0), (4096, 128, 10**6),
                                         (0, 128, 5), (64 * 100, 64, 50)])
def test_refine_max_nnz(lib, S, block, nnz):
    m, nb64 = block // 64, -(-S // 64)
    assert lib.tsa_refine_schedule_max_nnz(S, block, nnz) == min(m * m * nnz, nb64 * (nb64 + 1) // 2)


def test_refine_checks_before_gpu(lib):
    vp = ctypes.c_void_p
    assert lib.tsa_refine_schedule_max_nnz(100, 96, 5) == -1
    assert lib.tsa_refine_schedule_max_nnz(-1, 128, 5) == -1

    def call(S=1024, block=128, nnz=10, cap=40, rp=None, ci=None, rp64=None, ci64=None):
        return lib.tsa_refine_schedule(S, block, vp(rp), vp(ci), nnz, vp(rp64), vp(ci64), cap, None, vp(None))

    assert call(S=-1) == -1
    assert call(block=96) == -2
    assert call(S=64 * ((1 << 22) + 1), nnz=0, cap=0) == -2
    assert call(cap=39) == -4 and b"capacity" in lib.tsa_last_error()
    assert call() == -1 and b"NULL" in lib.tsa_last_error()


def test_noalloc_build_checks_before_gpu(lib):
    """tsa_build_schedule_noalloc: the argument checks of tsa_build_schedule_ex, then
    the fixed array's size limit, both before any GPU call."""
    vp = ctypes.c_void_p
    base = 1 << 40  # never dereferenced: every check below precedes any GPU call

    def call(S=1024, D=64, block=64, scope=0, cap=1000, row_ptr=base):
        return lib.tsa_build_schedule_noalloc(vp(base), 1, S, D, block, 1, 1, 2, scope, vp(row_ptr),
                                              vp(base + (1 << 24)), cap, vp(None), vp(None))

    assert call(scope=5) == -1
    assert call(block=96) == -2
    assert call(row_ptr=None) == -1
    assert call(cap=3) == -4
    big_S = 65536  # 1024 blocks: an 8 MB distance matrix does not fit the fixed array
    assert lib.tsa_build_schedule_workspace_bytes(big_S, 64, 64) > (4 << 20)
    assert call(S=big_S, cap=1 << 20) == -2
    assert b"workspace" in lib.tsa_last_error()
