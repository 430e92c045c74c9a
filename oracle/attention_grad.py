"""Gradients of scheduled attention in fp64 (oracle).  TEST INFRASTRUCTURE ONLY.

Sources: the pages "Add topology-derived sparse attention kernel"
(triton-lang/kernels pull request 22) and its mirror page.  The PR page's
kernel is forward-only (Summary, first bullet), and the mirror page's note on
learned segment boundaries says that, lacking a backward, training would have to
run dense.  The backward pass here is therefore a new surface; what it computes
is fixed by the forward it differentiates:

    o_t = sum_{u in A(t)} P_tu v_u,   P_tu = exp(z_tu - lse_t),
    z_tu = scale * (q_t . k_u),       lse_t = log sum_{u in A(t)} exp(z_tu),

with A(t) the allowed keys of query row t (defined in the forward oracle,
``attention.allowed_key_mask``).  For an upstream gradient dO of the output,
the chain rule through the row softmax gives the plain closed form

    dV = P^T dO,  dP = dO V^T,  Delta_t = sum_d dO_td o_td,
    dS = P * (dP - Delta),  dQ = scale * dS K,  dK = scale * dS^T Q,

where P is zero outside the mask.  A row with no allowed key has o_t = 0 and
lse_t = -inf and contributes nothing.  Everything is full width: P is
materialised for a slab of rows at a time, with no blocking beyond that slab.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _to_f64, allowed_key_mask


def _scale_of(D: int, scale):
    return 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)


def _row_stats(qf_rows, kf, mask, scale):
    """Masked scores z, probabilities P and lse for a slab of rows of one lane."""
    z = (qf_rows @ kf.T) * scale
    z = np.where(mask, z, -np.inf)
    lse = np.full(qf_rows.shape[0], -np.inf)
    p = np.zeros_like(z)
    has_key = mask.any(axis=1)
    if has_key.any():
        zz = z[has_key]
        zmax = zz.max(axis=1, keepdims=True)
        e = np.exp(zz - zmax)
        ssum = e.sum(axis=1, keepdims=True)
        lse[has_key] = (zmax + np.log(ssum))[:, 0]
        p[has_key] = e / ssum
    return p, lse


def masked_lse(q, k, row_ptr, col_idx, block: int = 64, scale=None, chunk: int = 256):
    """Log-sum-exp of each row's allowed scaled scores, fp64 [..., S].

    q, k: [S, D] or [B, H, S, D] (one CSR shared by every lane).  Rows with no
    allowed key get -inf.
    """
    qf, kf = _to_f64(q), _to_f64(k)
    S, D = qf.shape[-2], qf.shape[-1]
    scale = _scale_of(D, scale)
    lq, lk = qf.reshape(-1, S, D), kf.reshape(-1, S, D)
    out = np.zeros((lq.shape[0], S))
    for t0 in range(0, S, chunk):
        rows = np.arange(t0, min(S, t0 + chunk))
        mask = allowed_key_mask(row_ptr, col_idx, S, block, rows)
        for lane in range(lq.shape[0]):
            out[lane, rows] = _row_stats(lq[lane, rows], lk[lane], mask, scale)[1]
    return out.reshape(qf.shape[:-1])


def attention_backward(q, k, v, do, row_ptr, col_idx, block: int = 64, scale=None,
                       chunk: int = 256):
    """(dq, dk, dv, out, lse) of scheduled attention, all fp64.

    q, k, v, do: [S, D] or [B, H, S, D]; one CSR shared by every lane.  Follows
    the closed form in the module docstring, a slab of query rows at a time: each
    slab adds its P^T dO to dV and its scale * dS^T Q to dK.
    """
    qf, kf, vf, dof = _to_f64(q), _to_f64(k), _to_f64(v), _to_f64(do)
    if not (qf.shape == kf.shape == vf.shape == dof.shape):
        raise ValueError("q, k, v, do must share one shape")
    if qf.ndim not in (2, 4):
        raise ValueError("q must be [S, D] or [B, H, S, D]")
    S, D = qf.shape[-2], qf.shape[-1]
    scale = _scale_of(D, scale)
    lq, lk, lv, ldo = (x.reshape(-1, S, D) for x in (qf, kf, vf, dof))
    dq, dk, dv, out = (np.zeros_like(lq) for _ in range(4))
    lse = np.zeros((lq.shape[0], S))
    for t0 in range(0, S, chunk):
        rows = np.arange(t0, min(S, t0 + chunk))
        mask = allowed_key_mask(row_ptr, col_idx, S, block, rows)
        for lane in range(lq.shape[0]):
            p, lse[lane, rows] = _row_stats(lq[lane, rows], lk[lane], mask, scale)
            o = p @ lv[lane]
            out[lane, rows] = o
            g = ldo[lane, rows]
            dv[lane] += p.T @ g
            dp = g @ lv[lane].T
            delta = (g * o).sum(axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[lane, rows] = scale * (ds @ lk[lane])
            dk[lane] += scale * (ds.T @ lq[lane, rows])
    shp = qf.shape
    return dq.reshape(shp), dk.reshape(shp), dv.reshape(shp), out.reshape(shp), lse.reshape(shp[:-1])


def attention_backward_rows(q, k, v, do, row_ptr, col_idx, q_rows, k_rows, block: int = 64,
                            scale=None, chunk: int = 512):
    """Selected rows of the gradients of ONE lane, for sizes where the full
    gradients are too costly to hold as fp64 reference.

    q, k, v, do: [S, D].  Returns (dq[q_rows], dk[k_rows], dv[k_rows], lse[q_rows]).
    dq rows need only their own P row; dk and dv rows need the P columns of all
    query rows, which this walks in slabs (the same closed form).
    """
    qf, kf, vf, dof = _to_f64(q), _to_f64(k), _to_f64(v), _to_f64(do)
    S, D = qf.shape
    scale = _scale_of(D, scale)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    mask = allowed_key_mask(row_ptr, col_idx, S, block, q_rows)
    p, lse_sel = _row_stats(qf[q_rows], kf, mask, scale)
    o = p @ vf
    g = dof[q_rows]
    ds = p * (g @ vf.T - (g * o).sum(axis=1, keepdims=True))
    dq_sel = scale * (ds @ kf)
    dk_sel = np.zeros((k_rows.shape[0], D))
    dv_sel = np.zeros((k_rows.shape[0], D))
    for t0 in range(0, S if k_rows.size else 0, chunk):
        rows = np.arange(t0, min(S, t0 + chunk))
        m = allowed_key_mask(row_ptr, col_idx, S, block, rows)
        pr, _ = _row_stats(qf[rows], kf, m, scale)
        orow = pr @ vf
        gr = dof[rows]
        dsr = pr * (gr @ vf.T - (gr * orow).sum(axis=1, keepdims=True))
        dv_sel += pr[:, k_rows].T @ gr
        dk_sel += scale * (dsr[:, k_rows].T @ qf[rows])
    return dq_sel, dk_sel, dv_sel, lse_sel
