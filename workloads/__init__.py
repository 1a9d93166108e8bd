"""Seeded synthetic workloads for the sparse top-k MoE FFN forward.

This module only draws random numbers and stores them; it contains none of
the layer's arithmetic.  Both the HIP path and the CPU oracle consume exactly
the arrays produced here, so a test compares the two on identical bits.

Conventions
-----------
* Every tensor is drawn from ``numpy.random.default_rng([seed, tensor_id])``;
  per-expert tensors (W1, b1, W2, b2) use ``[seed, tensor_id, e]`` so experts can
  be generated in parallel and in any order.
* Floating-point draws are fp32 in C order.  For bf16 workloads they are then
  rounded to bf16 with round-to-nearest-even and stored as ``uint16`` bit
  patterns; those bits are the input to both sides.
* Weight layout is ``[in][out]`` per expert: ``W1[E,H,F]``, ``W2[E,F,H]`` and
  the gate ``Wg[H,E]`` (the transpose of how ``nn.Linear`` stores its weight,
  "moe-training" SKILL page, Quick Start, Basic MoE Architecture).

The five workloads mirror the pages' settings: a tiny fp32 layer, the
DeepSpeed-script shape (hidden 1024, seq 2048, micro-batch 4), a Switch-style
top-1 layer with 128 experts, a Zipf-skewed dropless layer, and a
Mixtral-8x7B-shaped layer (hidden 4096, FFN 14336, 8 experts, top-2,
eval capacity factor 2.0).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

# tensor ids for the seeded streams
TID_X, TID_WG, TID_BG, TID_W1, TID_B1, TID_W2, TID_B2, TID_Y = range(8)


@dataclasses.dataclass(frozen=True)
class Dist:
    """A value distribution: 'normal' (mean 0, std=scale), 'uniform'
    (U(-scale, scale)), 'zero', or 'zipf_log' (gate bias = log of a normalised
    Zipf(s=scale) popularity vector, expert 0 most popular)."""
    kind: str
    scale: float = 0.0


NONE = None  # a tensor that is absent (NULL bias)


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    T: int
    H: int
    E: int
    k: int
    F: int
    dtype: str              # "f32" or "bf16": storage type of x, weights, outputs
    cf: float               # capacity factor; <= 0 means dropless
    seed: int
    x: Dist = Dist("normal", 1.0)
    wg: Dist = Dist("normal", 0.02)
    bg: Optional[Dist] = None
    w1: Dist = Dist("normal", 0.02)
    b1: Optional[Dist] = None
    w2: Dist = Dist("normal", 0.02)
    b2: Optional[Dist] = None
    identical_experts: bool = False   # every expert gets expert 0's weights
    act: str = "gelu"                 # expert activation: "gelu" (exact erf) or "silu"
    ec_group: int = 0                 # > 0: expert-choice routing over groups of this size

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _c1() -> Spec:
    H, F = 64, 256
    u_h = Dist("uniform", 1.0 / math.sqrt(H))
    u_f = Dist("uniform", 1.0 / math.sqrt(F))
    return Spec("tiny_fp32_T256_H64_E8_k2", T=256, H=H, E=8, k=2, F=F, dtype="f32",
                cf=0.0, seed=1, x=Dist("normal", 1.0), wg=u_h, bg=u_h,
                w1=u_h, b1=u_h, w2=u_f, b2=u_f)


CONFIGS: Dict[str, Spec] = {
    "c1": _c1(),
    "c2": Spec("ds_shaped_T8192_H1024_E8_k2_cf1.25", T=8192, H=1024, E=8, k=2, F=4096,
               dtype="bf16", cf=1.25, seed=2),
    "c3": Spec("switch_T8192_H1024_E128_k1_cf1.25", T=8192, H=1024, E=128, k=1, F=4096,
               dtype="bf16", cf=1.25, seed=3, wg=Dist("normal", 0.1)),
    "c4": Spec("zipf_T16384_H2048_E64_k2_dropless", T=16384, H=2048, E=64, k=2, F=8192,
               dtype="bf16", cf=0.0, seed=4, bg=Dist("zipf_log", 1.2)),
    "c5": Spec("mixtral_T16384_H4096_E8_k2_F14336_cf2.0", T=16384, H=4096, E=8, k=2,
               F=14336, dtype="bf16", cf=2.0, seed=5),
    # the Mixtral block of the pages: bias-free, SiLU experts, no capacity
    "c5s": Spec("mixtral_silu_T16384_H4096_E8_k2_F14336_dropless", T=16384, H=4096, E=8,
                k=2, F=14336, dtype="bf16", cf=0.0, seed=6, act="silu"),
}
# Decode-shaped forwards of the Mixtral-shaped layer (the pages' inference
# setting: a few tokens, only their top-k experts active, no capacity limit).
# Every T shares the seed, so the weights are identical and x of a smaller T is
# the leading rows of x of a larger one (draws are in C order).
for _t in (1, 8, 64, 256):
    CONFIGS[f"d{_t}"] = Spec(f"mixtral_decode_T{_t}_H4096_E8_k2_F14336_dropless", T=_t, H=4096,
                             E=8, k=2, F=14336, dtype="bf16", cf=0.0, seed=8)
del _t
# Expert-choice routing on the Mixtral-shaped layer: each expert takes its
# C = ceil(2048 * 2 / 8) = 512 top tokens of every 2048-token sequence.
CONFIGS["c5e"] = Spec("mixtral_expert_choice_T16384_H4096_E8_k2_F14336_seq2048", T=16384,
                      H=4096, E=8, k=2, F=14336, dtype="bf16", cf=0.0, seed=9, ec_group=2048)


# ----------------------------------------------------------------------------
# storage conversion (bit-level; not part of the layer's arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------
def _draw(rng: np.random.Generator, dist: Dist, shape, E: int = 0) -> np.ndarray:
    if dist.kind == "normal":
        out = rng.standard_normal(size=shape, dtype=np.float32)
        if dist.scale != 1.0:
            out *= np.float32(dist.scale)
        return out
    if dist.kind == "uniform":
        out = rng.random(size=shape, dtype=np.float32)
        out *= np.float32(2.0 * dist.scale)
        out -= np.float32(dist.scale)
        return out
    if dist.kind == "zero":
        return np.zeros(shape, dtype=np.float32)
    if dist.kind == "const":
        return np.full(shape, dist.scale, dtype=np.float32)
    if dist.kind == "zipf_log":
        ranks = np.arange(1, E + 1, dtype=np.float64)
        p = ranks ** (-dist.scale)
        p /= p.sum()
        return np.log(p).astype(np.float32).reshape(shape)
    raise ValueError(f"unknown distribution {dist.kind}")


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def _expert_tensor(spec: Spec, tid: int, dist: Dist, shape_e, workers: int) -> np.ndarray:
    E = spec.E
    st_dtype = np.uint16 if spec.dtype == "bf16" else np.float32
    out = np.empty((E,) + tuple(shape_e), dtype=st_dtype)

    def one(e):
        src = 0 if spec.identical_experts else e
        rng = np.random.default_rng([spec.seed, tid, src])
        out[e] = _store(_draw(rng, dist, shape_e), spec.dtype)

    if workers > 1 and E > 1:
        with ThreadPoolExecutor(max_workers=min(workers, E)) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    return out


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def generate(spec: Spec, workers: Optional[int] = None, with_weights: bool = True
             ) -> Dict[str, Optional[np.ndarray]]:
    """Draw every input tensor of `spec`.

    Returns a dict with keys x [T,H], Wg [H,E], bg [E] or None, W1 [E,H,F],
    b1 [E,F] or None, W2 [E,F,H], b2 [E,H] or None.  Arrays are float32 for
    "f32" workloads and uint16 bf16 bit patterns for "bf16" workloads.
    """
    workers = default_workers() if workers is None else workers
    T, H, E, F = spec.T, spec.H, spec.E, spec.F
    d = spec.dtype
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = _store(_draw(np.random.default_rng([spec.seed, TID_X]), spec.x, (T, H)), d)
    out["Wg"] = _store(_draw(np.random.default_rng([spec.seed, TID_WG]), spec.wg, (H, E)), d)
    out["bg"] = (None if spec.bg is None else
                 _store(_draw(np.random.default_rng([spec.seed, TID_BG]), spec.bg, (E,), E), d))
    if with_weights:
        out["W1"] = _expert_tensor(spec, TID_W1, spec.w1, (H, F), workers)
        out["b1"] = None if spec.b1 is None else _expert_tensor(spec, TID_B1, spec.b1, (F,), 1)
        out["W2"] = _expert_tensor(spec, TID_W2, spec.w2, (F, H), workers)
        out["b2"] = None if spec.b2 is None else _expert_tensor(spec, TID_B2, spec.b2, (H,), 1)
    return out


def synthetic_rows(spec: Spec, rows: int, tid: int = TID_Y) -> np.ndarray:
    """Independent seeded rows [rows, H] in the workload's storage type, used as
    expert outputs when a combine stage is tested on its own."""
    rng = np.random.default_rng([spec.seed, tid])
    return _store(_draw(rng, Dist("normal", 1.0), (rows, spec.H)), spec.dtype)


def zero_gate(spec: Spec) -> Spec:
    """All gate weights and biases exactly zero: every logit is 0 (exact ties)."""
    return spec.replace(wg=Dist("zero"), bg=Dist("zero"))
