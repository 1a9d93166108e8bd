"""CPU oracle for the sparse top-k MoE FFN forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never imports, links or calls it, and the two share no code.

``liboracle.so`` (plain C, fp64, OpenMP) implements the per-token loop of the
"moe-training" SKILL page's reference layer (Quick Start, Basic MoE
Architecture), the losses of Core Concepts 3 (Load Balancing) and capacity
dropping in token order.  This module is argument marshalling around it, plus
``forward()``, which strings the steps together in the page's order.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB may point at another build of moe_oracle.c (used by the test
# that plants mistakes in the oracle source to show the pins catch them).
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")


class _Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32), ("cf", ctypes.c_double),
                ("dtype", ctypes.c_int32), ("act", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        L.orc_logits.argtypes = [P, vp, vp, vp, vp]
        L.orc_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_capacity.argtypes = [P]
        L.orc_capacity.restype = ctypes.c_int64
        L.orc_dispatch.argtypes = [P, vp, vp, vp, vp]
        L.orc_expert_rows.argtypes = [P, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp]
        L.orc_forward_tokens.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_int64, vp]
        L.orc_combine.argtypes = [P, vp, vp, vp, vp]
        L.orc_expert_choice.argtypes = [P, ctypes.c_int64, vp, vp, vp, vp]
        L.orc_ec_capacity.argtypes = [P, ctypes.c_int64]
        L.orc_ec_capacity.restype = ctypes.c_int64
        L.orc_backward.argtypes = [P] + [vp] * 8 + [vp, ctypes.c_double, ctypes.c_double] + [vp] * 7
        L.orc_backward_tokens.argtypes = [P] + [vp] * 8 + [vp, ctypes.c_double, ctypes.c_double,
                                                          vp, ctypes.c_int64, vp]
        L.orc_backward_weight_entries.argtypes = [P] + [vp] * 8 + [vp, vp, ctypes.c_int64, vp]
        L.orc_backward_gate.argtypes = [P] + [vp] * 8 + [vp, ctypes.c_double, ctypes.c_double,
                                                          vp, vp]
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def problem(spec, **over) -> _Problem:
    """Build the oracle's problem struct from an inputs.Spec (fields T, H, E, k,
    F, cf, dtype, act), with optional overrides."""
    g = lambda n: over.get(n, getattr(spec, n))
    act = g("act")
    if act not in ("gelu", "silu"):
        raise ValueError(f"activation {act!r}")
    return _Problem(T=int(g("T")), H=int(g("H")), E=int(g("E")), k=int(g("k")),
                    F=int(g("F")), cf=float(g("cf")),
                    dtype={"f32": 0, "bf16": 1, "f64": 2}[g("dtype")],
                    act=1 if act == "silu" else 0)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    if a is None:
        return None
    want = {"bf16": np.uint16, "f32": np.float32, "f64": np.float64}[dtype]
    if a.dtype != want:
        raise TypeError(f"oracle expects {want} storage for {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(lib().orc_num_threads())


def capacity(spec) -> int:
    return int(lib().orc_capacity(ctypes.byref(problem(spec))))


def logits(spec, x, Wg, bg=None) -> np.ndarray:
    d = spec.dtype
    x, Wg, bg = _storage(x, d), _storage(Wg, d), _storage(bg, d)
    out = np.empty((spec.T, spec.E), np.float64)
    _check(lib().orc_logits(ctypes.byref(problem(spec)), _ptr(x), _ptr(Wg), _ptr(bg),
                            _ptr(out)), "logits")
    return out


def route(spec, lg: np.ndarray) -> Dict[str, np.ndarray]:
    lg = np.ascontiguousarray(lg, np.float64)
    T, E, k = spec.T, spec.E, spec.k
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    probs = np.empty((T, E), np.float64)
    lse = np.empty((T,), np.float64)
    counts = np.empty((E,), np.int32)
    aux = ctypes.c_double()
    z = ctypes.c_double()
    _check(lib().orc_route(ctypes.byref(problem(spec)), _ptr(lg), _ptr(idx), _ptr(w),
                           _ptr(probs), _ptr(lse), _ptr(counts), ctypes.byref(aux),
                           ctypes.byref(z)), "route")
    return dict(topk_idx=idx, topk_w=w, probs=probs, lse=lse, counts=counts,
                aux=aux.value, z=z.value)


def dispatch(spec, topk_idx: np.ndarray) -> Dict[str, np.ndarray]:
    T, E, k = spec.T, spec.E, spec.k
    idx = np.ascontiguousarray(topk_idx, np.int32)
    offsets = np.empty((E + 1,), np.int32)
    pos = np.empty((T, k), np.int32)
    row_token = np.empty((T * k,), np.int32)
    _check(lib().orc_dispatch(ctypes.byref(problem(spec)), _ptr(idx), _ptr(offsets),
                              _ptr(pos), _ptr(row_token)), "dispatch")
    return dict(offsets=offsets, pos=pos, row_token=row_token)


def expert_rows(spec, rows, experts, W1, b1, W2, b2, want_h: bool = True):
    d = spec.dtype
    rows = _storage(rows, d)
    n = rows.shape[0]
    ex = np.ascontiguousarray(experts, np.int32)
    h = np.empty((n, spec.F), np.float64) if want_h else None
    y = np.empty((n, spec.H), np.float64)
    _check(lib().orc_expert_rows(ctypes.byref(problem(spec)), _ptr(rows), n, _ptr(ex),
                                 _ptr(_storage(W1, d)), _ptr(_storage(b1, d)),
                                 _ptr(_storage(W2, d)), _ptr(_storage(b2, d)),
                                 _ptr(h), _ptr(y)), "expert_rows")
    return h, y


def forward_tokens(spec, x, topk_idx, topk_w, pos, W1, b1, W2, b2,
                   tokens: Sequence[int]) -> np.ndarray:
    d = spec.dtype
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    out = np.empty((tok.shape[0], spec.H), np.float64)
    _check(lib().orc_forward_tokens(
        ctypes.byref(problem(spec)), _ptr(_storage(x, d)),
        _ptr(np.ascontiguousarray(topk_idx, np.int32)),
        _ptr(np.ascontiguousarray(topk_w, np.float64)),
        _ptr(np.ascontiguousarray(pos, np.int32)), _ptr(_storage(W1, d)),
        _ptr(_storage(b1, d)), _ptr(_storage(W2, d)), _ptr(_storage(b2, d)),
        _ptr(tok), tok.shape[0], _ptr(out)), "forward_tokens")
    return out


def combine(spec, y, pos, topk_w) -> np.ndarray:
    out = np.empty((spec.T, spec.H), np.float64)
    _check(lib().orc_combine(ctypes.byref(problem(spec)), _ptr(_storage(y, spec.dtype)),
                             _ptr(np.ascontiguousarray(pos, np.int32)),
                             _ptr(np.ascontiguousarray(topk_w, np.float64)), _ptr(out)),
           "combine")
    return out


def forward(spec, inp: Dict[str, Optional[np.ndarray]], tokens: Optional[Sequence[int]] = None,
            given_logits: Optional[np.ndarray] = None) -> Dict[str, object]:
    """The whole layer: logits -> routing and losses -> capacity dispatch ->
    expert FFN and combine.  `tokens` restricts the (expensive) FFN/combine to
    a subset of token rows (out then has one row per listed token); routing
    and dispatch always cover all T tokens because capacity dropping depends
    on every earlier token.  `given_logits` replaces the gate linear (e.g. by
    logits the GPU produced, so both sides take top-k decisions on the same
    values)."""
    lg = logits(spec, inp["x"], inp["Wg"], inp.get("bg")) if given_logits is None \
        else np.ascontiguousarray(given_logits, np.float64)
    r = route(spec, lg)
    dsp = dispatch(spec, r["topk_idx"])
    toks = np.arange(spec.T) if tokens is None else np.asarray(tokens, np.int64)
    out = forward_tokens(spec, inp["x"], r["topk_idx"], r["topk_w"], dsp["pos"],
                         inp["W1"], inp.get("b1"), inp["W2"], inp.get("b2"), toks)
    res: Dict[str, object] = dict(logits=lg, cap=capacity(spec), out=out, tokens=toks)
    res.update(r)
    res.update(dsp)
    return res


# ---------------------------------------------------------------- expert choice
def ec_capacity(spec, group: int) -> int:
    return int(lib().orc_ec_capacity(ctypes.byref(problem(spec)), int(group)))


def expert_choice(spec, lg: np.ndarray, group: int) -> Dict[str, np.ndarray]:
    """Expert-choice routing on logits [T][E]: per group of `group` tokens each
    expert takes its C tokens with the largest logits.  Returns sel
    [E][T/group][C] (ascending tokens), rowof [T][E] (expert-major row of each
    taken (token, expert), -1 when not taken), probs [T][E] (softmax weights),
    offsets [E+1] (every expert holds (T/group) * C rows) and C."""
    T, E = spec.T, spec.E
    C = ec_capacity(spec, group)
    ng = T // group
    sel = np.empty((E, ng, C), np.int32)
    rowof = np.empty((T, E), np.int32)
    probs = np.empty((T, E), np.float64)
    _check(lib().orc_expert_choice(ctypes.byref(problem(spec)), int(group),
                                   _ptr(np.ascontiguousarray(lg, np.float64)), _ptr(sel),
                                   _ptr(rowof), _ptr(probs)), "expert_choice")
    offsets = (np.arange(E + 1, dtype=np.int64) * ng * C).astype(np.int32)
    return dict(sel=sel, rowof=rowof, probs=probs, offsets=offsets, C=C)


def ec_forward_tokens(spec, x, rowof, probs, W1, b1, W2, b2,
                      tokens: Sequence[int]) -> np.ndarray:
    """Expert-choice layer output of the listed tokens: the sum, over the
    experts that took the token in expert order, of its softmax weight times
    the expert's output.  The same per-token loop as forward_tokens, with one
    slot per expert (slot e is expert e, kept when rowof[t][e] >= 0)."""
    T, E = spec.T, spec.E
    slots = np.broadcast_to(np.arange(E, dtype=np.int32), (T, E))
    return forward_tokens(spec.replace(k=E), x, slots, probs, rowof, W1, b1, W2, b2, tokens)


def ec_forward(spec, inp: Dict[str, Optional[np.ndarray]], group: int,
               tokens: Optional[Sequence[int]] = None,
               given_logits: Optional[np.ndarray] = None) -> Dict[str, object]:
    """The expert-choice layer: logits -> expert choice -> expert FFN and
    combine, for all tokens or the listed ones."""
    lg = logits(spec, inp["x"], inp["Wg"], inp.get("bg")) if given_logits is None \
        else np.ascontiguousarray(given_logits, np.float64)
    r = expert_choice(spec, lg, group)
    toks = np.arange(spec.T) if tokens is None else np.asarray(tokens, np.int64)
    out = ec_forward_tokens(spec, inp["x"], r["rowof"], r["probs"], inp["W1"], inp.get("b1"),
                            inp["W2"], inp.get("b2"), toks)
    res: Dict[str, object] = dict(logits=lg, out=out, tokens=toks)
    res.update(r)
    return res


# ---------------------------------------------------------------- backward
def _bwd_common(spec, inp, dout, given_logits):
    d = spec.dtype
    lg = None if given_logits is None else np.ascontiguousarray(given_logits, np.float64)
    return (ctypes.byref(problem(spec)), _ptr(_storage(inp["x"], d)), _ptr(_storage(inp["Wg"], d)),
            _ptr(_storage(inp.get("bg"), d)), _ptr(_storage(inp["W1"], d)),
            _ptr(_storage(inp.get("b1"), d)), _ptr(_storage(inp["W2"], d)),
            _ptr(_storage(inp.get("b2"), d)), _ptr(lg), _ptr(_storage(dout, d)))


def backward(spec, inp: Dict[str, Optional[np.ndarray]], dout: np.ndarray, g_aux: float = 0.0,
             g_z: float = 0.0, given_logits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(dout * out) + g_aux * aux + g_z * z with respect to
    x, the gate and the expert weights (fp64; biases only when present)."""
    T, H, E, F = spec.T, spec.H, spec.E, spec.F
    g = dict(dx=np.empty((T, H)), dWg=np.empty((H, E)), dbg=np.empty(E),
             dW1=np.empty((E, H, F)), db1=np.empty((E, F)), dW2=np.empty((E, F, H)),
             db2=np.empty((E, H)))
    _check(lib().orc_backward(*_bwd_common(spec, inp, dout, given_logits), float(g_aux),
                              float(g_z), *[_ptr(g[n]) for n in ("dx", "dWg", "dbg", "dW1", "db1",
                                                                  "dW2", "db2")]), "backward")
    return g


def backward_tokens(spec, inp, dout, tokens: Sequence[int], g_aux: float = 0.0, g_z: float = 0.0,
                    given_logits: Optional[np.ndarray] = None) -> np.ndarray:
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    dx = np.empty((tok.shape[0], spec.H))
    _check(lib().orc_backward_tokens(*_bwd_common(spec, inp, dout, given_logits), float(g_aux),
                                     float(g_z), _ptr(tok), tok.shape[0], _ptr(dx)),
           "backward_tokens")
    return dx


def backward_gate(spec, inp, dout, g_aux: float = 0.0, g_z: float = 0.0,
                  given_logits: Optional[np.ndarray] = None):
    """(dWg [H][E], dbg [E]) of the same objective as backward(), computed
    without the expert-weight and dx terms (one forward's work)."""
    dWg = np.empty((spec.H, spec.E))
    dbg = np.empty(spec.E)
    _check(lib().orc_backward_gate(*_bwd_common(spec, inp, dout, given_logits), float(g_aux),
                                   float(g_z), _ptr(dWg), _ptr(dbg)), "backward_gate")
    return dWg, dbg


def backward_weight_entries(spec, inp, dout, entries, given_logits=None) -> np.ndarray:
    """entries: rows (kind, e, i, j) with kind 1 dW1[e][i][j], 2 dW2[e][i][j],
    3 db1[e][j], 4 db2[e][j]."""
    ent = np.ascontiguousarray(np.asarray(entries, dtype=np.int32).reshape(-1, 4))
    out = np.empty(ent.shape[0])
    _check(lib().orc_backward_weight_entries(*_bwd_common(spec, inp, dout, given_logits),
                                             _ptr(ent), ent.shape[0], _ptr(out)),
           "backward_weight_entries")
    return out


def topk_margin(spec, lg: np.ndarray) -> float:
    """Smallest gap between the k-th and (k+1)-th largest logit of any token
    (infinite when k == E).  Used to decide whether top-k decisions taken on
    differently rounded logits are guaranteed to agree."""
    if spec.k >= spec.E:
        return float("inf")
    s = -np.sort(-np.asarray(lg, np.float64), axis=1)
    return float(np.min(s[:, spec.k - 1] - s[:, spec.k]))
