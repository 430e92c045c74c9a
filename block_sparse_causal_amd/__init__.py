"""Topology-scheduled block-sparse causal attention for AMD Instinct MI355X.

Thin Python binding over ``libtsa.so`` (C ABI in ``include/tsa.h``).  This module
only marshals arguments: it turns torch tensors into device pointers, sizes and
the current HIP stream, allocates outputs and workspaces with torch, and maps
status codes to exceptions.  Every step of the computation runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

Operations (pages "Add topology-derived sparse attention kernel",
triton-lang/kernels PR 22, Summary):

* ``build_schedule``       sink + local window + top-k salient key blocks -> CSR
* ``dense_causal_schedule`` the lower-triangular CSR
* ``segment_schedule``      the fixed-segment (block-diagonal causal) CSR
* ``refine_schedule``       a schedule over blocks of 128, 256, ... rows as the
  equivalent 64-row-block CSR the attention entry points take
* ``scheduled_attention``  forward causal attention over a CSR block schedule
  (optionally with each row's log-sum-exp)

and, beyond the pages (whose kernel is forward-only), the backward pass:

* ``schedule_transpose``            column view (CSC) of a CSR schedule
* ``scheduled_attention_backward``  dq, dk, dv over the same schedule
* ``attention``                     forward with torch autograd support
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._abi import declare_signatures

__all__ = [
    "BLOCK",
    "SUB_BLOCK",
    "TsaError",
    "library_path",
    "schedule_max_nnz",
    "build_schedule",
    "ScheduleBuffers",
    "build_schedule_into",
    "dense_causal_schedule",
    "segment_schedule",
    "refine_schedule",
    "scheduled_attention",
    "schedule_transpose",
    "scheduled_attention_backward",
    "attention",
]

BLOCK = 64
SUB_BLOCK = 32  # the smaller block the builder and the forward also take
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtsa.so")

TSA_OK = 0
_STATUS_NAMES = {
    -1: "TSA_ERR_INVALID_ARG",
    -2: "TSA_ERR_UNSUPPORTED",
    -3: "TSA_ERR_SHAPE",
    -4: "TSA_ERR_SCHEDULE",
    -5: "TSA_ERR_DEVICE",
    -6: "TSA_ERR_HIP",
}
_DTYPES = {torch.float16: 0, torch.bfloat16: 1}


class TsaError(RuntimeError):
    """A libtsa call failed inside the HIP runtime."""


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m block_sparse_causal_amd.build` "
            "(this package has no non-HIP code path)"
        )
    lib = ctypes.CDLL(_LIB_PATH)
    declare_signatures(lib)
    return lib


_lib = _load()


def library_path() -> str:
    """Path of the loaded native library."""
    return _LIB_PATH


def _check(status: int, what: str) -> None:
    if status == TSA_OK:
        return
    msg = _lib.tsa_last_error().decode(errors="replace")
    name = _STATUS_NAMES.get(status, str(status))
    if status == -6:
        raise TsaError(f"{what}: {name}: {msg}")
    raise ValueError(f"{what}: {name}: {msg}")


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else None)


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
    return _DTYPES[t.dtype]


def schedule_max_nnz(nb: int, sink: int, local_radius: int, topk: int) -> int:
    """Upper bound on the entries a built schedule can hold (host arithmetic in libtsa)."""
    n = _lib.tsa_schedule_max_nnz(nb, sink, local_radius, topk)
    if n < 0:
        _check(-1, "schedule_max_nnz")
    return int(n)


def build_schedule(keys: torch.Tensor, block: int = BLOCK, sink: int = 1, local_radius: int = 1,
                   topk: int = 2, return_salience: bool = False, per_row: bool = False):
    """Topology-derived CSR schedule from the keys of lane (0, 0).

    keys: [S, D] or [B, H, S, D] float16/bfloat16 on a GPU.  Returns int32
    (row_ptr [nb+1], col_idx [nnz]) on the keys' device, nb = ceil(S / block),
    plus the fp64 salience [nb] when ``return_salience``.  Waits for the stream
    to read back nnz.  block: 32 or a multiple of 64; schedules over blocks larger
    than 64 reach the attention entry points through ``refine_schedule``, those
    over 32-row blocks go to ``scheduled_attention(..., block=32)`` as they are.
    per_row: each row takes its own top-k among its blocks j <= i instead of
    one global top-k set (TSA_TOPK_PER_ROW).
    """
    if not isinstance(keys, torch.Tensor):
        raise TypeError("keys must be a torch.Tensor")
    if keys.dim() == 4:
        keys = keys[0, 0]
    if keys.dim() != 2:
        raise ValueError(f"keys must be [S, D] or [B, H, S, D], got {tuple(keys.shape)}")
    if not keys.is_cuda:
        raise ValueError("keys must be on a GPU device")
    if not keys.is_contiguous():
        raise ValueError("keys (lane 0, 0) must be contiguous")
    code = _dtype_code(keys, "keys")
    S, D = keys.shape
    dev = keys.device
    nb = -(-S // block) if block > 0 else 0  # the library rejects unsupported blocks
    cap = schedule_max_nnz(nb, sink, local_radius, topk) if min(sink, local_radius, topk) >= 0 else 0
    ws_bytes = _lib.tsa_build_schedule_workspace_bytes(S, D, block)
    with torch.cuda.device(dev):
        row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        sal = torch.empty(max(nb, 1), dtype=torch.float64, device=dev) if return_salience else None
        ws = torch.empty(max(int(ws_bytes), 1) + 256, dtype=torch.uint8, device=dev)
        base = ws.data_ptr()
        aligned = (base + 255) // 256 * 256
        nnz = ctypes.c_int64(0)
        status = _lib.tsa_build_schedule_ex(
            _ptr(keys), code, S, D, block, sink, local_radius, topk, 1 if per_row else 0,
            _ptr(row_ptr), _ptr(col_idx), cap, _ptr(sal), ctypes.c_void_p(aligned), int(ws_bytes),
            ctypes.byref(nnz), _stream(dev),
        )
    _check(status, "build_schedule")
    out = (row_ptr, col_idx[: nnz.value])
    if return_salience:
        out = out + (sal[:nb],)
    return out


class ScheduleBuffers:
    """Preallocated device buffers for repeated schedule builds of one shape.

    Holds row_ptr [nb+1], col_idx at its capacity bound, an optional salience
    [nb] and the builder workspace, so ``build_schedule_into`` allocates
    nothing and never waits for the stream.
    """

    def __init__(self, S: int, D: int, sink: int, local_radius: int, topk: int, device,
                 salience: bool = False, per_row: bool = False, block: int = BLOCK):
        dev = torch.device(device)
        self.S, self.D, self.sink, self.local_radius, self.topk = S, D, sink, local_radius, topk
        self.per_row = per_row
        self.block = block
        self.nb = -(-S // block)
        self.capacity = schedule_max_nnz(self.nb, sink, local_radius, topk)
        self.ws_bytes = int(_lib.tsa_build_schedule_workspace_bytes(S, D, block))
        if self.ws_bytes == 0 and self.nb > 0:
            _check(-2, "ScheduleBuffers: unsupported size")
        self.row_ptr = torch.empty(self.nb + 1, dtype=torch.int32, device=dev)
        self.col_idx = torch.empty(max(self.capacity, 1), dtype=torch.int32, device=dev)
        self.salience = torch.empty(max(self.nb, 1), dtype=torch.float64, device=dev) if salience else None
        self._ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=dev)
        self.ws_ptr = (self._ws.data_ptr() + 255) // 256 * 256


def build_schedule_into(keys: torch.Tensor, bufs: ScheduleBuffers) -> None:
    """Queue a schedule build into ``bufs`` on the current stream (no host wait).

    keys: [S, D] (lane 0, 0) float16/bfloat16, contiguous, matching ``bufs``.
    Entries past row_ptr[nb] in ``bufs.col_idx`` are unspecified.
    """
    if keys.dim() == 4:
        keys = keys[0, 0]
    if tuple(keys.shape) != (bufs.S, bufs.D) or not keys.is_contiguous() or not keys.is_cuda:
        raise ValueError("keys must be a contiguous GPU tensor of the buffers' [S, D]")
    code = _dtype_code(keys, "keys")
    with torch.cuda.device(keys.device):
        status = _lib.tsa_build_schedule_ex(
            _ptr(keys), code, bufs.S, bufs.D, bufs.block, bufs.sink, bufs.local_radius, bufs.topk,
            1 if bufs.per_row else 0, _ptr(bufs.row_ptr), _ptr(bufs.col_idx), bufs.capacity,
            _ptr(bufs.salience), ctypes.c_void_p(bufs.ws_ptr), bufs.ws_bytes, None,
            _stream(keys.device),
        )
    _check(status, "build_schedule_into")


def build_schedule_noalloc(keys: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor, block: int,
                           sink: int, local_radius: int, topk: int, per_row: bool = False,
                           salience: torch.Tensor | None = None) -> None:
    """Queue a schedule build into caller-provided int32 ``row_ptr`` [nb+1] and
    ``col_idx`` (capacity = its length) on the current stream, with the library's
    fixed device workspace (tsa_build_schedule_noalloc): no allocation, no host
    wait.  The entry count is row_ptr[nb]."""
    if keys.dim() == 4:
        keys = keys[0, 0]
    if keys.dim() != 2 or not keys.is_contiguous() or not keys.is_cuda:
        raise ValueError("keys must be a contiguous [S, D] GPU tensor")
    code = _dtype_code(keys, "keys")
    _check_index("row_ptr", row_ptr, keys.device)
    _check_index("col_idx", col_idx, keys.device)
    S, D = keys.shape
    if row_ptr.numel() != -(-S // block) + 1:
        raise ValueError(f"row_ptr must have ceil(S/block)+1 = {-(-S // block) + 1} entries")
    with torch.cuda.device(keys.device):
        status = _lib.tsa_build_schedule_noalloc(
            _ptr(keys), code, S, D, block, sink, local_radius, topk, 1 if per_row else 0, _ptr(row_ptr),
            _ptr(col_idx), col_idx.numel(), _ptr(salience), _stream(keys.device),
        )
    _check(status, "build_schedule_noalloc")


def refine_schedule(row_ptr: torch.Tensor, col_idx: torch.Tensor, S: int, block: int):
    """The CSR over 64-row blocks that allows exactly the keys the CSR over blocks
    of ``block`` rows allows (tsa_refine_schedule), for the attention entry
    points.  Returns int32 (row_ptr [ceil(S/64)+1], col_idx); waits for the
    stream to read back the entry count."""
    dev = row_ptr.device
    _check_index("row_ptr", row_ptr, dev)
    _check_index("col_idx", col_idx, dev)
    nnz = col_idx.numel()
    cap = int(_lib.tsa_refine_schedule_max_nnz(S, block, nnz))
    if cap < 0:
        _check(-1, "refine_schedule")
    nb64 = -(-S // BLOCK)
    with torch.cuda.device(dev):
        rp = torch.empty(nb64 + 1, dtype=torch.int32, device=dev)
        ci = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        total = ctypes.c_int64(0)
        status = _lib.tsa_refine_schedule(S, block, _ptr(row_ptr), _ptr(col_idx), nnz, _ptr(rp), _ptr(ci),
                                          cap, ctypes.byref(total), _stream(dev))
    _check(status, "refine_schedule")
    return rp, ci[: total.value]


def dense_causal_schedule(nb: int, device, out: tuple[torch.Tensor, torch.Tensor] | None = None
                          ) -> tuple[torch.Tensor, torch.Tensor]:
    """Lower-triangular CSR for nb blocks on ``device`` (int32 row_ptr, col_idx).
    ``out``: preallocated (row_ptr [nb+1], col_idx [>= nb(nb+1)/2]) to write into,
    so that the call allocates nothing."""
    dev = torch.device(device)
    nnz = nb * (nb + 1) // 2
    with torch.cuda.device(dev):
        if out is None:
            row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
            col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        else:
            row_ptr, col_idx = out
            _check_index("row_ptr", row_ptr, dev)
            _check_index("col_idx", col_idx, dev)
            if row_ptr.numel() != nb + 1 or col_idx.numel() < nnz:
                raise ValueError("out must hold row_ptr [nb+1] and col_idx [>= nb(nb+1)/2]")
        status = _lib.tsa_dense_causal_schedule(nb, _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _stream(dev))
    _check(status, "dense_causal_schedule")
    return row_ptr, col_idx[:nnz]


def segment_schedule(nb: int, segment_blocks: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Fixed-segment (block-diagonal causal) CSR for nb blocks on ``device``: row i
    lists blocks L*(i//L) .. i for L = segment_blocks (int32 row_ptr, col_idx)."""
    dev = torch.device(device)
    nnz = int(_lib.tsa_segment_schedule_nnz(nb, segment_blocks))
    if nnz < 0:
        raise ValueError(f"segment_schedule: invalid nb={nb} or segment_blocks={segment_blocks}")
    with torch.cuda.device(dev):
        row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        status = _lib.tsa_segment_schedule(nb, segment_blocks, _ptr(row_ptr), _ptr(col_idx), nnz,
                                           _stream(dev))
    _check(status, "segment_schedule")
    return row_ptr, col_idx[:nnz]


def _attention_shape(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share a shape, got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share a dtype")
    code = _dtype_code(q, "q")
    if q.dim() == 2:
        B, H, (S, D) = 1, 1, q.shape
    elif q.dim() == 4:
        B, H, S, D = q.shape
    else:
        raise ValueError(f"q must be [S, D] or [B, H, S, D], got {tuple(q.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    return code, B, H, S, D


def _check_index(name, t, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_block(block):
    # the row_ptr length check needs a positive block; the library decides the rest
    if not isinstance(block, int) or block <= 0:
        raise ValueError(f"block must be a positive int, got {block!r}")


def _scale_arg(sm_scale):
    scale = 0.0 if sm_scale is None else float(sm_scale)
    if sm_scale is not None and scale <= 0:
        raise ValueError("sm_scale must be positive")
    return scale


def scheduled_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                        col_idx: torch.Tensor, block: int = BLOCK, sm_scale: float | None = None,
                        out: torch.Tensor | None = None, return_lse: bool = False):
    """Forward scheduled attention; returns a tensor of q's shape and dtype, or
    (out, lse) with ``return_lse`` (lse float32 [..., S], natural log of each
    row's softmax denominator, -inf for rows with no allowed key).

    q, k, v: [S, D] or [B, H, S, D], one float16/bfloat16 dtype, contiguous, on
    one GPU.  row_ptr/col_idx: int32 CSR on the same device, shared by every
    (b, h) lane, over blocks of ``block`` rows: 64, or SUB_BLOCK (32) at head
    dims 32, 64 and 128.  sm_scale defaults to 1/sqrt(D).
    """
    code, B, H, S, D = _attention_shape(q, k, v)
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        _check_index(name, t, q.device)
    _check_block(block)
    nb = -(-S // block)
    if row_ptr.numel() != nb + 1:
        raise ValueError(f"row_ptr must have nb+1 = {nb + 1} entries for S={S}, got {row_ptr.numel()}")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")
    scale = _scale_arg(sm_scale)
    with torch.cuda.device(q.device):
        if return_lse:
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
            status = _lib.tsa_scheduled_attention_fwd_lse(
                _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), code, B, H, S, D, _ptr(row_ptr),
                _ptr(col_idx), col_idx.numel(), block, scale, _stream(q.device),
            )
        else:
            status = _lib.tsa_scheduled_attention_fwd(
                _ptr(q), _ptr(k), _ptr(v), _ptr(out), code, B, H, S, D, _ptr(row_ptr), _ptr(col_idx),
                col_idx.numel(), block, scale, _stream(q.device),
            )
    _check(status, "scheduled_attention")
    return (out, lse) if return_lse else out


def prepare_scheduled_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                                col_idx: torch.Tensor, out: torch.Tensor, sm_scale: float | None = None,
                                block: int = BLOCK):
    """``scheduled_attention(q, k, v, row_ptr, col_idx, out=out, block=block)``
    with the arguments checked and marshalled once: returns a callable that
    queues the forward on the current stream of q's device with one C ABI call
    (which still validates its arguments).  For loops that launch the same call
    many times, where the per-call Python work would otherwise set the pace."""
    code, B, H, S, D = _attention_shape(q, k, v)
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        _check_index(name, t, q.device)
    _check_block(block)
    if row_ptr.numel() != -(-S // block) + 1:
        raise ValueError("row_ptr must have nb+1 entries")
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")
    keep = (q, k, v, row_ptr, col_idx, out)  # the callable holds the tensors alive
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), code, B, H, S, D, _ptr(row_ptr), _ptr(col_idx),
            col_idx.numel(), block, _scale_arg(sm_scale))
    fn, dev = _lib.tsa_scheduled_attention_fwd, q.device

    def call():
        status = fn(*args, _stream(dev))
        if status != TSA_OK:
            _check(status, "scheduled_attention")

    call.tensors = keep
    return call


def schedule_transpose(row_ptr: torch.Tensor, col_idx: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Column view (CSC) of a causal CSR schedule, built on the GPU: column j
    lists, ascending, the query blocks whose rows list key block j.  Returns
    int32 (col_ptr [nb+1], row_idx [nnz']); waits for the stream to read nnz'."""
    dev = row_ptr.device
    _check_index("row_ptr", row_ptr, dev)
    _check_index("col_idx", col_idx, dev)
    if not row_ptr.is_cuda:
        raise ValueError("row_ptr must be on a GPU device")
    nb = row_ptr.numel() - 1
    if nb < 0:
        raise ValueError("row_ptr must have at least one entry")
    nnz = col_idx.numel()
    cap = min(nnz, nb * (nb + 1) // 2)
    ws_bytes = int(_lib.tsa_schedule_transpose_workspace_bytes(nb))
    with torch.cuda.device(dev):
        col_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
        row_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
        aligned = (ws.data_ptr() + 255) // 256 * 256
        total = ctypes.c_int64(0)
        status = _lib.tsa_schedule_transpose(
            nb, _ptr(row_ptr), _ptr(col_idx), nnz, _ptr(col_ptr), _ptr(row_idx), cap,
            ctypes.c_void_p(aligned if ws_bytes else None), ws_bytes, ctypes.byref(total), _stream(dev),
        )
    _check(status, "schedule_transpose")
    return col_ptr, row_idx[: total.value]


def scheduled_attention_backward(q, k, v, out, dout, lse, row_ptr, col_idx, col_ptr, row_idx,
                                 block: int = BLOCK, sm_scale: float | None = None):
    """Gradients (dq, dk, dv) of ``scheduled_attention`` for the upstream gradient
    ``dout``; ``out`` and ``lse`` are the forward's (``return_lse=True``) and
    (col_ptr, row_idx) is ``schedule_transpose(row_ptr, col_idx)``.  The schedule
    is over blocks of ``block`` rows: 64 (head dims 32, 64, 128 and 256), or
    SUB_BLOCK (32) at head dims up to 128.  Returns tensors of q's shape and
    dtype."""
    code, B, H, S, D = _attention_shape(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a tensor of q's shape and dtype")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on q's device")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or lse.shape != q.shape[:-1]:
        raise ValueError("lse must be a float32 tensor of q's shape without the head dim")
    if lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be contiguous on q's device")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx), ("col_ptr", col_ptr), ("row_idx", row_idx)):
        _check_index(name, t, q.device)
    _check_block(block)
    nb = -(-S // block)
    if row_ptr.numel() != nb + 1 or col_ptr.numel() != nb + 1:
        raise ValueError(f"row_ptr and col_ptr must have nb+1 = {nb + 1} entries for S={S}")
    scale = _scale_arg(sm_scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_bytes = int(_lib.tsa_scheduled_attention_bwd_workspace_bytes(B, H, S))
    with torch.cuda.device(q.device):
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        status = _lib.tsa_scheduled_attention_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), code, B, H, S, D,
            _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(col_ptr), _ptr(row_idx),
            row_idx.numel(), block, scale, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes,
            _stream(q.device),
        )
    _check(status, "scheduled_attention_backward")
    return dq, dk, dv


class _ScheduledAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, row_ptr, col_idx, col_ptr, row_idx, sm_scale, block):
        out, lse = scheduled_attention(q, k, v, row_ptr, col_idx, block=block, sm_scale=sm_scale,
                                       return_lse=True)
        ctx.save_for_backward(q, k, v, out, lse, row_ptr, col_idx, col_ptr, row_idx)
        ctx.sm_scale = sm_scale
        ctx.block = block
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, row_ptr, col_idx, col_ptr, row_idx = ctx.saved_tensors
        dq, dk, dv = scheduled_attention_backward(q, k, v, out, dout.contiguous(), lse, row_ptr, col_idx,
                                                  col_ptr, row_idx, block=ctx.block, sm_scale=ctx.sm_scale)
        return dq, dk, dv, None, None, None, None, None, None


def attention(q, k, v, row_ptr, col_idx, col_ptr=None, row_idx=None, sm_scale: float | None = None,
              block: int = BLOCK):
    """Scheduled attention that torch autograd can differentiate: the forward
    keeps lse, the backward runs ``scheduled_attention_backward``.  Pass the
    schedule's column view (``schedule_transpose``) to reuse it across calls;
    otherwise it is built here.  ``block``: the schedule's block rows (64, or 32)."""
    if col_ptr is None or row_idx is None:
        col_ptr, row_idx = schedule_transpose(row_ptr, col_idx)
    return _ScheduledAttention.apply(q, k, v, row_ptr, col_idx, col_ptr, row_idx, sm_scale, block)
