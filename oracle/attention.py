"""Dense masked attention in fp64 (oracle).  TEST INFRASTRUCTURE ONLY.

Sources (pages "Add topology-derived sparse attention kernel", triton-lang/kernels
pull request 22, and its mirror page):

* PR page, Summary, first bullet: forward causal attention that consumes a
  causal CSR block schedule; third bullet: [seq, dim] and [batch, heads, seq,
  dim] inputs with one CSR shared by every batch/head lane.
* PR page, Local benchmark: the kernel is checked against a dense masked
  computation on the same mask ("max abs error" column).
* Mirror page, Rust-port commit note: the scheduled result equals dense masked
  attention.

Definition used here.  Query row t lies in query block i = t // block.  Its
allowed keys are A(t) = {u <= t : u // block is listed in CSR row i}.  With
z_u = scale * (q_t . k_u), o_t = sum_{u in A(t)} softmax(z)_u v_u, evaluated
as a full-width softmax over all S keys with the disallowed ones at -inf.
Readings: scale defaults to 1/sqrt(D); an empty A(t) gives o_t = 0.  Rows are
processed in chunks only to bound memory; every row is a plain full-width
masked softmax.
"""
from __future__ import annotations

import math

import numpy as np


def _to_f64(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def allowed_key_mask(row_ptr, col_idx, S: int, block: int = 64, rows=None) -> np.ndarray:
    """Boolean [len(rows), S] mask: True where key u is allowed for query t.

    u is allowed for t when u <= t and u's key block is listed in the CSR row
    of t's query block (PR page, Summary, first bullet).  Listed blocks outside
    0 .. nb-1 select no keys.
    """
    rp = np.asarray(row_ptr).astype(np.int64)
    ci = np.asarray(col_idx).astype(np.int64)
    nb = -(-S // block)
    if rp.shape[0] != nb + 1:
        raise ValueError(f"row_ptr must have nb+1 = {nb + 1} entries, got {rp.shape[0]}")
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    key_block = np.arange(S) // block
    mask = np.zeros((rows.shape[0], S), dtype=bool)
    for r, t in enumerate(rows):
        i = int(t) // block
        listed = np.zeros(nb, dtype=bool)
        for j in ci[rp[i] : rp[i + 1]]:
            if 0 <= j < nb:
                listed[j] = True
        mask[r] = listed[key_block] & (np.arange(S) <= t)
    return mask


def _attend(qf_rows, kf, vf, mask, scale):
    """Full-width masked softmax attention for a slab of query rows (fp64)."""
    z = (qf_rows @ kf.T) * scale
    z = np.where(mask, z, -np.inf)
    out = np.zeros((qf_rows.shape[0], kf.shape[1]), dtype=np.float64)
    has_key = mask.any(axis=1)
    if has_key.any():
        zz = z[has_key]
        zmax = zz.max(axis=1, keepdims=True)
        p = np.exp(zz - zmax)
        out[has_key] = (p @ vf) / p.sum(axis=1, keepdims=True)
    return out


def masked_attention_rows(q, k, v, row_ptr, col_idx, rows, block: int = 64, scale=None):
    """Oracle output for selected query rows of ONE lane.

    q, k, v: [S, D] (any float type; converted to fp64).  rows: query indices.
    Returns fp64 [len(rows), D].
    """
    qf, kf, vf = _to_f64(q), _to_f64(k), _to_f64(v)
    S, D = qf.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    mask = allowed_key_mask(row_ptr, col_idx, S, block, rows)
    return _attend(qf[rows], kf, vf, mask, scale)


def masked_attention(q, k, v, row_ptr, col_idx, block: int = 64, scale=None, chunk: int = 256):
    """Oracle output for every query row of every lane.

    q, k, v: [S, D] or [B, H, S, D]; one CSR is shared by every lane (PR page,
    Summary, third bullet).  Returns fp64 of the same shape.
    """
    qf, kf, vf = _to_f64(q), _to_f64(k), _to_f64(v)
    if qf.shape != kf.shape or qf.shape != vf.shape:
        raise ValueError("q, k, v must share one shape")
    if qf.ndim not in (2, 4):
        raise ValueError("q must be [S, D] or [B, H, S, D]")
    S, D = qf.shape[-2], qf.shape[-1]
    lanes_q = qf.reshape(-1, S, D)
    lanes_k = kf.reshape(-1, S, D)
    lanes_v = vf.reshape(-1, S, D)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros_like(lanes_q)
    for t0 in range(0, S, chunk):
        rows = np.arange(t0, min(S, t0 + chunk))
        mask = allowed_key_mask(row_ptr, col_idx, S, block, rows)  # shared by every lane
        for lane in range(lanes_q.shape[0]):
            out[lane, rows] = _attend(lanes_q[lane, rows], lanes_k[lane], lanes_v[lane], mask, scale)
    return out.reshape(qf.shape)
