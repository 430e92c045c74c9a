"""Brute-force fp64 schedule builder (oracle).  TEST INFRASTRUCTURE ONLY.

Sources (pages "Add topology-derived sparse attention kernel", triton-lang/kernels
pull request 22, and the mirror of that page):

* PR page, Summary, second bullet: the schedule is built from sink blocks,
  local-window blocks and a 0D-persistence-style salience score over key-block
  centroids; first bullet: the kernel consumes causal CSR block schedules.
* Mirror page, commit note of the Rust port: salience follows the elder rule,
  exactly one block scores zero, the non-zero scores form the H0 barcode, and
  when two components tie on size the absorbed one depends on index order; the
  dense schedule is the lower-triangular CSR.
* Mirror page, commit note on ``schedule.py``: computing the same salience from
  MST edges instead of all pairs gives bit-identical results.  This oracle
  deliberately keeps the all-pairs form; the MST form lives in the GPU path.

Readings where the pages are silent (each is also listed in the design notes):

* size tie in the elder rule: the root with the LARGER index is absorbed, so
  the lower index is the elder;
* salience = Euclidean distance between MEAN centroids at which the block's
  component is absorbed; the last surviving root scores 0;
* pairs are processed in ascending (distance, i, j) order with i < j;
* top-k is ONE global set: the first min(k, nb) blocks under the order
  (-salience, index); a row i takes the members t <= i;
* local window of row i is blocks max(0, i - r) .. i; sink blocks are the first
  ``sink`` blocks, clipped causally;
* a partial last block (S not a multiple of ``block``) has as centroid the mean
  of its valid rows.
"""
from __future__ import annotations

import numpy as np


def _as_f64_2d(keys) -> np.ndarray:
    """Convert one lane of keys, shape [S, D], to float64 (exact for fp16/bf16)."""
    try:  # torch tensors: go through float64 on the CPU, which is exact
        import torch

        if isinstance(keys, torch.Tensor):
            keys = keys.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    arr = np.asarray(keys, dtype=np.float64)
    if arr.ndim != 2:
        raise ValueError(f"keys must be [S, D], got shape {arr.shape}")
    return arr


def block_centroids(keys, block: int = 64) -> np.ndarray:
    """Centroid of each key block: the mean of its key rows (fp64).

    PR page, Summary, second bullet ("salience score over key-block centroids").
    Block j covers key rows j*block .. min(S, (j+1)*block) - 1.
    """
    k = _as_f64_2d(keys)
    S = k.shape[0]
    nb = -(-S // block)
    cents = np.zeros((nb, k.shape[1]), dtype=np.float64)
    for j in range(nb):
        rows = k[j * block : min(S, (j + 1) * block)]
        cents[j] = rows.sum(axis=0) / rows.shape[0]
    return cents


def centroid_distances(cents: np.ndarray) -> np.ndarray:
    """Full symmetric matrix of Euclidean distances between centroids (fp64).

    d_ij = sqrt(sum_d (c_i[d] - c_j[d])^2), formed from the differences (no
    Gram-matrix expansion).
    """
    c = np.asarray(cents, dtype=np.float64)
    diff = c[:, None, :] - c[None, :, :]
    return np.sqrt(np.sum(diff * diff, axis=-1))


def elder_rule_salience(cents: np.ndarray) -> np.ndarray:
    """Per-block elder-rule H0 salience by single linkage over ALL pairs.

    Mirror page, Rust-port commit note: salience is the elder rule; exactly one
    block scores zero; the non-zero scores are the H0 barcode; on a size tie the
    absorbed component depends on index order.

    Every block starts as its own component.  Pairs (i < j) are visited in
    ascending (d_ij, i, j).  When a pair joins two different components, the
    smaller component is absorbed (on equal size: the one whose root has the
    larger index), and that root's salience is d_ij.  The root that is never
    absorbed keeps salience 0.
    """
    c = np.asarray(cents, dtype=np.float64)
    nb = c.shape[0]
    sal = np.zeros(nb, dtype=np.float64)
    if nb <= 1:
        return sal
    dist = centroid_distances(c)
    iu, ju = np.triu_indices(nb, k=1)
    dij = dist[iu, ju]
    order = np.lexsort((ju, iu, dij))  # primary key d, then i, then j

    parent = list(range(nb))
    size = [1] * nb

    def find(x: int) -> int:
        while parent[x] != x:
            x = parent[x]
        return x

    merges = 0
    for p in order:
        i, j, d = int(iu[p]), int(ju[p]), float(dij[p])
        ri, rj = find(i), find(j)
        if ri == rj:
            continue
        if size[ri] > size[rj] or (size[ri] == size[rj] and ri < rj):
            survivor, absorbed = ri, rj
        else:
            survivor, absorbed = rj, ri
        parent[absorbed] = survivor
        size[survivor] += size[absorbed]
        sal[absorbed] = d
        merges += 1
        if merges == nb - 1:
            break
    return sal


def top_k_blocks(salience: np.ndarray, topk: int) -> list[int]:
    """The global top-k salient blocks, returned in ascending index order.

    PR page, Summary, second bullet (blocks ranked by the salience score).
    Ranking key is (-salience, index): higher salience first, ties to the lower
    index.  topk >= nb selects every block.
    """
    sal = np.asarray(salience, dtype=np.float64)
    ranked = sorted(range(sal.shape[0]), key=lambda j: (-sal[j], j))
    return sorted(ranked[: max(0, min(int(topk), sal.shape[0]))])


def _csr_from_rows(rows: list[list[int]]) -> tuple[np.ndarray, np.ndarray]:
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int32)
    for i, cols in enumerate(rows):
        row_ptr[i + 1] = row_ptr[i] + len(cols)
    col_idx = np.array([j for cols in rows for j in cols], dtype=np.int32)
    return row_ptr, col_idx


def schedule_from_salience(
    salience: np.ndarray, sink: int, local_radius: int, topk: int, per_row: bool = False
) -> tuple[np.ndarray, np.ndarray]:
    """CSR rows: sink blocks, local window and top-k blocks, each clipped causally.

    PR page, Summary, first and second bullets.  Row i lists, in ascending order,
    every key block j <= i with j < sink, or i - local_radius <= j, or j in the
    top-k set.  With per_row=False the top-k set is global: the first topk
    blocks of the whole ranking.  With per_row=True each row takes its own
    top-k among its causal blocks j <= i under the same ranking, and may
    overlap the sink and local blocks.  The pages do not settle which of the
    two readings the kernel used.
    """
    nb = len(salience)
    top = set(top_k_blocks(salience, topk))
    rows = []
    for i in range(nb):
        if per_row:
            top = set(j for j in top_k_blocks(np.asarray(salience)[: i + 1], topk))
        rows.append(
            [j for j in range(i + 1) if j < sink or j >= i - local_radius or j in top]
        )
    return _csr_from_rows(rows)


def build_schedule(
    keys, block: int = 64, sink: int = 1, local_radius: int = 1, topk: int = 2,
    per_row: bool = False,
) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Topology-derived CSR schedule from one lane of keys [S, D].

    Returns (row_ptr int32 [nb+1], col_idx int32 [nnz], salience fp64 [nb]).
    PR page, Summary, second bullet; salience as in ``elder_rule_salience``;
    per_row as in ``schedule_from_salience``.
    """
    if block <= 0:
        raise ValueError("block must be positive")
    if min(sink, local_radius, topk) < 0:
        raise ValueError("sink, local_radius and topk must be >= 0")
    sal = elder_rule_salience(block_centroids(keys, block))
    row_ptr, col_idx = schedule_from_salience(sal, sink, local_radius, topk, per_row)
    return row_ptr, col_idx, sal


def dense_causal_schedule(nb: int) -> tuple[np.ndarray, np.ndarray]:
    """Lower-triangular CSR: row i lists blocks 0..i.

    PR page, Summary (its tests cover the dense causal CSR) and Local
    benchmark table (dense block counts 136 / 528 / 2080).
    """
    return _csr_from_rows([list(range(i + 1)) for i in range(nb)])


def fixed_segment_schedule(nb: int, segment_blocks: int) -> tuple[np.ndarray, np.ndarray]:
    """Block-diagonal causal CSR: row i lists the blocks j <= i of its own segment.

    Mirror page, commit note on learned segment boundaries: attention does not
    cross a segment boundary, and with fixed segments of 512 or 256 tokens
    (8 or 4 blocks of 64) a causal CSR kernel visits 288 or 160 of the 2,080
    causal blocks at S 4096.  Segments are the runs [m*L, (m+1)*L) of
    L = segment_blocks blocks; the last run may be shorter.
    """
    if segment_blocks < 1:
        raise ValueError("segment_blocks must be >= 1")
    rows = []
    for i in range(nb):
        rows.append([j for j in range(i + 1) if j // segment_blocks == i // segment_blocks])
    return _csr_from_rows(rows)


def csr_to_block_sets(row_ptr, col_idx) -> list[set[int]]:
    """The set of key blocks listed in each CSR row."""
    rp = np.asarray(row_ptr).astype(np.int64)
    ci = np.asarray(col_idx).astype(np.int64)
    return [set(int(x) for x in ci[rp[i] : rp[i + 1]]) for i in range(len(rp) - 1)]


def transpose_schedule(row_ptr, col_idx) -> tuple[np.ndarray, np.ndarray]:
    """Column view (CSC) of a causal CSR schedule: column j lists, ascending,
    the query blocks i whose row lists key block j, j <= i.

    The gradients of keys and values (dK, dV) of key block j gather over exactly
    these query blocks (the backward of the forward on the PR page, Summary,
    first bullet).  Listed blocks outside 0..i select no keys and do not appear.
    Returns int32 (col_ptr [nb+1], row_idx [nnz']).
    """
    sets = csr_to_block_sets(row_ptr, col_idx)
    nb = len(sets)
    cols = [[i for i in range(nb) if j in sets[i] and j <= i] for j in range(nb)]
    return _csr_from_rows(cols)


def refine_schedule(row_ptr, col_idx, S: int, block: int) -> tuple[np.ndarray, np.ndarray]:
    """The CSR over 64-row blocks that allows exactly the keys a CSR over blocks
    of ``block`` rows allows.

    The pages validate a schedule's block size (PR page, Summary, fifth bullet)
    and benchmark at 64.  With m = block / 64, fine row i lists block c exactly
    when coarse row i // m lists c // m and c <= i; listed coarse blocks outside
    0..i // m select no keys.  Returns int32 (row_ptr [ceil(S/64)+1], col_idx).
    """
    if block < 64 or block % 64:
        raise ValueError("block must be a positive multiple of 64")
    m = block // 64
    sets = csr_to_block_sets(row_ptr, col_idx)
    nb64 = -(-S // 64)
    rows = []
    for i in range(nb64):
        I = i // m
        rows.append([c for c in range(i + 1) if (c // m) in sets[I] and c // m <= I])
    return _csr_from_rows(rows)
