"""Seeded synthetic inputs for the fused chunked KL loss.

This module only draws random numbers and casts them; it holds none of the
loss arithmetic. Both the CPU oracle tests and the GPU path are fed from it,
so they see byte-identical inputs.

The workloads stand in for the teacher top-K caches of the pages (one cached
list of the teacher's 100 most likely tokens per position, with its logits:
P1 "Making knowledge distillation cheap enough to run at scale",
section "Two system changes", offline distillation paragraph). The real caches,
corpora and models are not available; synthetic values of the same shapes are
used instead.

Recipe (all draws from numpy's PCG64 ``default_rng(seed)``, in this order):

1. ``H`` ~ N(0, 1), shape [N, d], drawn in fp32, rounded to the storage dtype
   with round-to-nearest-even (torch's ``.to(bfloat16)``).
2. ``W`` ~ N(0, 1/d) (variance 1/d), shape [V, d], same rounding.
3. teacher ids, shape [N, K], int32, distinct within a row, kept in draw order:
   - ``uniform``: each draw uniform on [0, V);
   - ``zipf``: P(id = r - 1) proportional to r ** -a for r = 1..V (identity
     rank-to-id map: low ids are frequent), drawn by inverse CDF.
   Repeats inside a row are rejected and the row continues drawing until it
   holds K distinct ids.
4. teacher logits, shape [N, K], fp32: K iid draws of N(0, var) (the second
   parameter is a variance), sorted in descending order per row.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["Workload", "CONFIGS", "get_config", "other_reading", "generate", "seed_for"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int          # tokens (sequence positions)
    d: int          # hidden size
    V: int          # vocabulary size
    K: int          # teacher top-K entries per position
    chunk: int      # positions per chunk
    T: float        # temperature
    dtype: str      # "fp32" or "bf16": storage type of H and W
    id_dist: str    # "uniform" or "zipf"
    logit_var: float
    zipf_a: float = 1.1
    index: int = 0  # 1-based position in the list of workloads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Cross-references between them ("teacher top-K as the
# first one", "same generators as the third one") are read with 1-based
# numbering: the third and fifth use uniform distinct ids with logits
# N(0, 2), like the first.
CONFIGS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 128, 256, 4096, 16, 32, 1.0, "fp32",
                          "uniform", 2.0, index=1),
    "small_bf16": Workload("small_bf16", 2048, 1024, 32000, 100, 256, 1.0,
                           "bf16", "zipf", 3.0, index=2),
    "llama3b_8k": Workload("llama3b_8k", 8192, 3072, 128256, 100, 1024, 1.0,
                           "bf16", "uniform", 2.0, index=3),
    "gptoss20b_32k": Workload("gptoss20b_32k", 32768, 2880, 201088, 100, 2048,
                              1.0, "bf16", "zipf", 4.0, index=4),
    "longctx_256k": Workload("longctx_256k", 262144, 2880, 201088, 100, 4096,
                             2.0, "bf16", "uniform", 2.0, index=5),
}


def other_reading(w: Workload) -> Workload:
    """The same workload under the 0-based reading of the cross-references
    (the third workload takes the second one's teacher generator, Zipf ids
    with logits N(0, 3); the fifth takes the fourth one's, Zipf with N(0, 4)).
    Shapes and flops are unchanged; only the value distributions differ."""
    if w.index == 3:
        return w.with_(id_dist="zipf", logit_var=3.0)
    if w.index == 5:
        return w.with_(id_dist="zipf", logit_var=4.0)
    return w


def get_config(name: str) -> Workload:
    if name in CONFIGS:
        return CONFIGS[name]
    for w in CONFIGS.values():  # also accept "C1".."C5"
        if name.upper() == f"C{w.index}":
            return w
    raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")


def seed_for(w: Workload) -> int:
    return 1000 + w.index


def _first_k_distinct(cand: np.ndarray, K: int):
    """For each row of ``cand`` keep the first K distinct values in draw order.

    Returns (out [rows, K] int64, ok [rows] bool); rows with fewer than K
    distinct values have ok False.
    """
    rows, M = cand.shape
    order = np.argsort(cand, axis=1, kind="stable")
    sv = np.take_along_axis(cand, order, axis=1)
    first = np.ones_like(sv, dtype=bool)
    first[:, 1:] = sv[:, 1:] != sv[:, :-1]
    # position (in draw order) of every first occurrence; others pushed last
    pos = np.where(first, order, M + np.arange(M)[None, :])
    pos.sort(axis=1)
    ok = pos[:, K - 1] < M
    keep = np.minimum(pos[:, :K], M - 1)
    return np.take_along_axis(cand, keep, axis=1), ok


def _draw_ids(rng: np.random.Generator, N: int, K: int, V: int, dist: str,
              a: float) -> np.ndarray:
    if K > V:
        raise ValueError("K must not exceed V")
    if dist == "zipf":
        w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]

        def draw(shape):
            return np.minimum(np.searchsorted(cdf, rng.random(shape), side="right"), V - 1)
        M = max(2 * K, 256)
    elif dist == "uniform":
        def draw(shape):
            return rng.integers(0, V, size=shape)
        M = 2 * K + 8
    else:
        raise ValueError(dist)
    out = np.empty((N, K), dtype=np.int64)
    block = 8192
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        cand = draw((r1 - r0, M))
        ids, ok = _first_k_distinct(cand, K)
        while not ok.all():
            # rows that did not reach K distinct ids keep drawing
            bad = np.nonzero(~ok)[0]
            more = draw((bad.size, 4 * M))
            ids_b, ok_b = _first_k_distinct(np.concatenate([cand[bad], more], 1), K)
            ids[bad] = ids_b
            cand_new = np.zeros((r1 - r0, cand.shape[1] + 4 * M), dtype=cand.dtype)
            cand_new[:, :cand.shape[1]] = cand
            cand_new[bad, cand.shape[1]:] = more
            cand = cand_new
            ok[bad] = ok_b
        out[r0:r1] = ids
    return out


def generate(w: Workload, seed: Optional[int] = None, *, N: Optional[int] = None):
    """Return dict(H, W, ids, logits) as CPU torch tensors for workload ``w``.

    ``N`` overrides the number of positions (the other sizes are kept).
    """
    if seed is None:
        seed = seed_for(w)
    n = w.N if N is None else N
    rng = np.random.default_rng(seed)
    dt = w.torch_dtype
    H = torch.from_numpy(rng.standard_normal((n, w.d), dtype=np.float32)).to(dt)
    Wf = rng.standard_normal((w.V, w.d), dtype=np.float32)
    Wf *= np.float32(1.0 / np.sqrt(w.d))
    W = torch.from_numpy(Wf).to(dt)
    del Wf
    ids = _draw_ids(rng, n, w.K, w.V, w.id_dist, w.zipf_a).astype(np.int32)
    lg = rng.standard_normal((n, w.K)) * np.sqrt(w.logit_var)
    lg = -np.sort(-lg, axis=1)
    return {
        "H": H.contiguous(),
        "W": W.contiguous(),
        "ids": torch.from_numpy(np.ascontiguousarray(ids)),
        "logits": torch.from_numpy(lg.astype(np.float32)),
    }
