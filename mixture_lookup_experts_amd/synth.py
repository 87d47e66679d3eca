"""Seeded synthetic inputs for the MoLE hot path.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so the HIP path and the CPU oracle can both take their
inputs from it.  Every array is produced on the host with NumPy's PCG64
generator from a documented seed, so the same bytes reach the GPU and the
oracle.

Workloads (sizes from the MoLE model family: 160M / 410M / 1B-class layers,
a 50304-token vocabulary, experts D -> F -> D with GELU and no bias):

  ===== ====== ===== ==== ===== ======= ===========================
  name    V      D    N     F    dtype   token batches
  ===== ====== ===== ==== ===== ======= ===========================
  tiny    512    64    4   256   fp32    64 ids, uniform
  160m  50304   768    4  3072   bf16    1, 8, 64, 256 (Zipf 1.1)
  410m  50304  1024   16  4096   bf16    1024, 4096, 256 (Zipf 1.1)
  1b    50304  2048   16  8192   bf16    1, 16, 128, 1024 (Zipf 1.1), 16 layers
  ===== ====== ===== ==== ===== ======= ===========================

Weights, embedding and router ~ N(0, 0.02) (standard deviation 0.02),
hidden states h ~ N(0, 1); bf16 tensors are fp32 draws rounded to nearest
even.  Token ids follow a finite Zipf law: rank k in 1..V with probability
proportional to k^-1.1, drawn by inverse CDF in fp64, and mapped to ids by a
seeded permutation so that hot rows are scattered over the table.

Seeds: 20250000 + 100*config + k with k = 0 Emb, 1 W_up, 2 W_down, 3 W_r,
4 rank->id permutation, 10+step h, 50+step ids; layer l of the 16-layer
workload adds 1000*l to every per-layer seed (Emb is shared by all layers).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20250000


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # 1-based position in the workload list (seed offset)
    V: int
    D: int
    N: int
    F: int
    dtype: str            # "f32" or "bf16"
    tokens: tuple
    layers: int = 1
    zipf: bool = True
    nf3: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 512, 64, 4, 256, "f32", (64,), zipf=False,
                     notes="tiny fp32 layer, uniform ids"),
    "160m": Workload("160m", 2, 50304, 768, 4, 3072, "bf16", (1, 8, 64, 256),
                     notes="160M-class layer, decode batches"),
    "410m": Workload("410m", 3, 50304, 1024, 16, 4096, "bf16", (1024, 4096, 256),
                     notes="410M-class layer, prefill + decode"),
    "1b": Workload("1b", 4, 50304, 2048, 16, 8192, "bf16", (1, 16, 128, 1024), layers=16,
                   notes="1B-class stack of 16 layers"),
    "410m-nf3": Workload("410m-nf3", 5, 50304, 1024, 16, 4096, "bf16", (1024, 4096, 256),
                         nf3=True, notes="410M-class layer with a 3-bit NF3 table"),
}


def seed(w: Workload, k: int, layer: int = 0) -> int:
    return SEED_BASE + 100 * w.index + k + 1000 * layer


# ---- element formats -------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs are finite draws, so NaN handling is not needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# ---- token ids -------------------------------------------------------------

def zipf_cdf(V: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def zipf_probs(V: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def rank_permutation(w: Workload) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed(w, 4))).permutation(w.V).astype(np.int64)


def zipf_ids(rng: np.random.Generator, V: int, T: int, perm: np.ndarray, s: float = 1.1) -> np.ndarray:
    """T ids from a finite Zipf(s) law over V ranks, ranks mapped through perm."""
    u = rng.random(T)
    ranks = np.searchsorted(zipf_cdf(V, s), u, side="right")
    ranks = np.minimum(ranks, V - 1)
    return perm[ranks].astype(np.int64)


def uniform_ids(rng: np.random.Generator, V: int, T: int) -> np.ndarray:
    return rng.integers(0, V, size=T, dtype=np.int64)


def distinct_ids(rng: np.random.Generator, V: int, T: int) -> np.ndarray:
    """T distinct ids (sampling without replacement): gathered bytes == unique bytes."""
    return rng.choice(V, size=T, replace=False).astype(np.int64)


# ---- layer weights and batches --------------------------------------------

@dataclass
class Layer:
    emb: np.ndarray     # [V, D]
    w_up: np.ndarray    # [N, F, D]
    w_down: np.ndarray  # [N, D, F]
    w_r: np.ndarray     # [N, D]


def make_embedding(w: Workload, std: float = 0.02) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed(w, 0)))
    return _normal(rng, (w.V, w.D), std, w.dtype)


def make_expert_weights(w: Workload, layer: int = 0, std: float = 0.02):
    r1 = np.random.Generator(np.random.PCG64(seed(w, 1, layer)))
    r2 = np.random.Generator(np.random.PCG64(seed(w, 2, layer)))
    return (_normal(r1, (w.N, w.F, w.D), std, w.dtype),
            _normal(r2, (w.N, w.D, w.F), std, w.dtype))


def make_router(w: Workload, layer: int = 0, std: float = 0.02) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed(w, 3, layer)))
    return _normal(rng, (w.N, w.D), std, w.dtype)


def make_layer(w: Workload, layer: int = 0, emb: np.ndarray | None = None) -> Layer:
    emb = make_embedding(w) if emb is None else emb
    w_up, w_down = make_expert_weights(w, layer)
    return Layer(emb, w_up, w_down, make_router(w, layer))


def make_hidden(w: Workload, T: int, step: int = 0, layer: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed(w, 10 + step, layer)))
    return _normal(rng, (T, w.D), 1.0, w.dtype)


def make_ids(w: Workload, T: int, step: int = 0, kind: str | None = None,
             perm: np.ndarray | None = None) -> np.ndarray:
    """kind: 'zipf', 'uniform' or 'distinct' (default: the workload's own)."""
    rng = np.random.Generator(np.random.PCG64(seed(w, 50 + step)))
    kind = kind or ("zipf" if w.zipf else "uniform")
    if kind == "zipf":
        return zipf_ids(rng, w.V, T, rank_permutation(w) if perm is None else perm)
    if kind == "uniform":
        return uniform_ids(rng, w.V, T)
    if kind == "distinct":
        return distinct_ids(rng, w.V, T)
    raise ValueError(kind)


def expected_unique(V: int, T: int, s: float = 1.1) -> float:
    """E[#distinct ids] among T Zipf(s) draws: sum_k 1 - (1 - p_k)^T."""
    p = zipf_probs(V, s)
    return float(np.sum(1.0 - (1.0 - p) ** T))
