"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic (no centroids, distances, salience, masks or softmax), so
both the oracle side and the HIP side can take their inputs from it.

Recipe (numpy ``default_rng(seed)`` in float64, then one round-to-nearest cast
to fp16/bf16 through torch on the CPU).  Tensors are drawn in the order q, k, v.

* "normal" keys: i.i.d. N(0, 1), like q and v.
* "mixture" keys (clustered key blocks): per lane, ``ncomp`` means ~ N(0, 4 I)
  (std 2), then one component id per 64-key block, uniform, then per-key noise
  ~ N(0, 0.25 I) (std 0.5); key t = mean[id[t // 64]] + noise[t].

The workloads below follow the head dimension (64), block size (64) and
sequence lengths the pages benchmark at, widened to batched, long-context and
full-causal-density cases.  The pages name no dataset; everything is synthetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    shape: tuple  # (S, D) or (B, H, S, D)
    dtype: str  # "fp16" | "bf16"
    keys: str = "normal"  # "normal" | "mixture"
    ncomp: int = 0
    sink: int = 1
    local_radius: int = 1
    topk: int = 2
    dense: bool = False  # True: the full lower-triangular CSR, no topology schedule
    seed: int = 1
    note: str = field(default="", compare=False)

    @property
    def S(self) -> int:
        return self.shape[-2]

    @property
    def D(self) -> int:
        return self.shape[-1]

    @property
    def lanes(self) -> int:
        return int(np.prod(self.shape[:-2])) if len(self.shape) == 4 else 1

    @property
    def nb(self) -> int:
        return -(-self.S // BLOCK)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            "single_s1024_d64_f16", (1024, 64), "fp16", "normal", 0, 1, 1, 2, seed=1,
            note="single head, 16 blocks, sink 1, radius 1, top-2",
        ),
        Workload(
            "single_s4096_d64_f16_mix8", (4096, 64), "fp16", "mixture", 8, 1, 1, 8, seed=2,
            note="single head, 64 blocks, keys clustered in 8 components, top-8",
        ),
        Workload(
            "batched_b4h16_s4096_d64_bf16", (4, 16, 4096, 64), "bf16", "normal", 0, 1, 2, 16, seed=3,
            note="64 lanes share one schedule built from lane (0, 0); radius 2, top-16",
        ),
        Workload(
            "long_b1h32_s32768_d64_bf16_mix32", (1, 32, 32768, 64), "bf16", "mixture", 32, 2, 4, 32,
            seed=4, note="long context, 512 blocks, 32-component clustered keys per head",
        ),
        Workload(
            "dense_b2h32_s8192_d128_bf16", (2, 32, 8192, 128), "bf16", "normal", dense=True, seed=5,
            note="full causal density (8256 blocks), head dim 128",
        ),
    ]
}

# the workload bench.py times by default: the batched one, where every lane shares
# one schedule and the chip is filled (4096 workgroups)
BENCH_WORKLOAD = "batched_b4h16_s4096_d64_bf16"


def _torch_dtype(dtype: str):
    import torch

    return {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32, "fp64": torch.float64}[dtype]


def cast(arr: np.ndarray, dtype: str):
    """Round a float64 array to ``dtype`` (round to nearest even) as a CPU torch tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).to(_torch_dtype(dtype))


def draw_keys(rng: np.random.Generator, shape, kind: str = "normal", ncomp: int = 0) -> np.ndarray:
    """Keys in float64 following the recipe in the module docstring."""
    if kind == "normal":
        return rng.standard_normal(shape)
    if kind != "mixture":
        raise ValueError(f"unknown key distribution {kind!r}")
    S, D = shape[-2], shape[-1]
    lanes = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    out = np.empty((lanes, S, D), dtype=np.float64)
    nb = -(-S // BLOCK)
    for lane in range(lanes):
        means = rng.normal(0.0, 2.0, size=(ncomp, D))
        comp = rng.integers(0, ncomp, size=nb)
        noise = rng.normal(0.0, 0.5, size=(S, D))
        out[lane] = means[comp[np.arange(S) // BLOCK]] + noise
    return out.reshape(shape)


def make_qkv(workload, seed=None, shape=None):
    """(q, k, v) CPU torch tensors of the workload's dtype, drawn q then k then v.

    ``shape`` overrides the workload's shape (used for reduced-size variants of a
    workload with the same distributions).
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp = tuple(shape) if shape is not None else w.shape
    q = rng.standard_normal(shp)
    k = draw_keys(rng, shp, w.keys, w.ncomp)
    v = rng.standard_normal(shp)
    return cast(q, w.dtype), cast(k, w.dtype), cast(v, w.dtype)


def random_normal(shape, dtype: str, seed: int, std: float = 1.0):
    """One N(0, std^2) tensor of ``dtype``."""
    rng = np.random.default_rng(seed)
    return cast(rng.normal(0.0, std, size=shape), dtype)


def random_csr(nb: int, seed: int, density: float = 0.3, allow_empty: bool = False, causal: bool = True):
    """A random CSR block schedule (int32 row_ptr [nb+1], col_idx [nnz]).

    Row i lists a random subset of blocks 0..i in ascending order (or of 0..nb-1
    when ``causal`` is False).  Unless ``allow_empty``, the diagonal block is
    always listed.
    """
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(nb):
        hi = i + 1 if causal else nb
        pick = rng.random(hi) < density
        if not allow_empty and i < hi:
            pick[i] = True
        rows.append(np.nonzero(pick)[0])
    row_ptr = np.zeros(nb + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return row_ptr, col_idx
