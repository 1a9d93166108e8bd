"""Independent formulations of the MoE layer used to pin the C oracle —
TEST INFRASTRUCTURE ONLY (imported by tests, never by the product path).

Each function computes the same layer as ``liboracle.so`` by a different
route, from library primitives, so that a slip in the per-token C loop (a
dropped term, a wrong sign or index, a transposed operand) shows up as a
mismatch:

* ``dense_then_mask`` — evaluate EVERY expert on EVERY token with dense
  matrix products, then gather the selected outputs by index and weight them.
  This is the "evaluate all experts, then index by the top-k" reading of the
  "moe-training" SKILL page's Top-2 routing snippet (Core Concepts,
  2. Routing Mechanisms).  Top-k here is a stable descending sort of the
  softmax probabilities; capacity ranks come from a cumulative sum of one-hot
  rows in token order.
* ``torch_masked_layer`` — the reference layer of the page (Quick Start, Basic
  MoE Architecture) built from ``torch.nn.Linear`` / ``torch.nn.GELU`` /
  ``torch.softmax`` / ``torch.topk`` in float64 on the CPU, dispatching with
  one boolean row mask per expert (no capacity limit).
* ``torch_expert_major`` — the expert-major formulation of the page's Mixtral
  block (Advanced Patterns, Mixtral 8x7B Architecture): per-expert gather of
  the (token, slot) pairs and ``index_add_`` back into token rows (no
  capacity limit).

* ``expert_choice_dense`` / ``torch_expert_choice_sets`` — expert-choice
  routing (Core Concepts, 2. Routing Mechanisms) by a stable lexicographic sort
  per (expert, group) with every expert evaluated densely, and by the page's
  own ``torch.topk`` over the sequence axis.

All of them follow ``spec.act``: ``nn.GELU`` (exact erf) as in the reference
layer, or ``nn.SiLU`` as in the Mixtral block; the numpy route evaluates SiLU
as ``a * expit(a)`` and GELU with ``scipy.special.erf``.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
from scipy import special

from workloads import to_f32


def _f64(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    return None if a is None else to_f32(a, dtype).astype(np.float64)


def _capacity(spec) -> int:
    if not spec.cf > 0:
        return spec.T
    return int(np.ceil(spec.cf * spec.T * spec.k / spec.E))


def _all_experts(spec, x, W1, b1, W2, b2) -> np.ndarray:
    """Every expert on every token, [E][T][H], with dense matrix products."""
    Y = np.empty((spec.E, x.shape[0], spec.H))
    for e in range(spec.E):
        a = x @ W1[e] + (0.0 if b1 is None else b1[e][None, :])
        if spec.act == "silu":
            g = a * special.expit(a)
        else:
            g = 0.5 * a * (1.0 + special.erf(a / np.sqrt(2.0)))
        Y[e] = g @ W2[e] + (0.0 if b2 is None else b2[e][None, :])
    return Y


def dense_then_mask(spec, inp: Dict[str, Optional[np.ndarray]]) -> Dict[str, object]:
    d = spec.dtype
    T, H, E, k, F = spec.T, spec.H, spec.E, spec.k, spec.F
    x = _f64(inp["x"], d)
    Wg = _f64(inp["Wg"], d)
    bg = _f64(inp.get("bg"), d)
    W1 = _f64(inp["W1"], d)
    W2 = _f64(inp["W2"], d)
    b1 = _f64(inp.get("b1"), d)
    b2 = _f64(inp.get("b2"), d)

    lg = x @ Wg + (0.0 if bg is None else bg[None, :])
    p = special.softmax(lg, axis=1)
    lse = special.logsumexp(lg, axis=1)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :k].astype(np.int32)
    psel = np.take_along_axis(p, idx, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)

    f = np.bincount(idx.ravel(), minlength=E) / float(T * k)
    aux = E * float(np.sum(f * p.mean(axis=0)))
    z = float(np.mean(lse ** 2))

    cap = _capacity(spec)
    onehot = np.zeros((T * k, E), np.int64)
    onehot[np.arange(T * k), idx.ravel()] = 1
    rank = (np.cumsum(onehot, axis=0) - 1)[np.arange(T * k), idx.ravel()]
    kept = rank < cap
    kept_per_e = np.bincount(idx.ravel()[kept], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(kept_per_e)]).astype(np.int32)
    pos = np.where(kept, offsets[idx.ravel()] + rank, -1).reshape(T, k).astype(np.int32)

    Y = _all_experts(spec, x, W1, b1, W2, b2)
    sel = Y[idx, np.arange(T)[:, None], :]           # [T, k, H]
    coef = w * kept.reshape(T, k)
    out = np.einsum("tk,tkh->th", coef, sel)
    return dict(logits=lg, probs=p, lse=lse, topk_idx=idx, topk_w=w, counts=np.bincount(
        idx.ravel(), minlength=E).astype(np.int32), aux=aux, z=z, cap=cap, offsets=offsets,
        pos=pos, out=out, Y=Y)


def _torch_modules(spec, inp):
    import torch
    d = spec.dtype
    E = spec.E
    t64 = lambda a: None if a is None else torch.from_numpy(_f64(a, d))
    W1, W2, b1, b2 = t64(inp["W1"]), t64(inp["W2"]), t64(inp.get("b1")), t64(inp.get("b2"))
    Wg, bg = t64(inp["Wg"]), t64(inp.get("bg"))
    experts = []
    for e in range(E):
        l1 = torch.nn.Linear(spec.H, spec.F, bias=b1 is not None, dtype=torch.float64)
        l2 = torch.nn.Linear(spec.F, spec.H, bias=b2 is not None, dtype=torch.float64)
        with torch.no_grad():
            l1.weight.copy_(W1[e].T)          # nn.Linear stores [out, in]
            l2.weight.copy_(W2[e].T)
            if b1 is not None:
                l1.bias.copy_(b1[e])
            if b2 is not None:
                l2.bias.copy_(b2[e])
        act = torch.nn.SiLU() if spec.act == "silu" else torch.nn.GELU()
        experts.append(torch.nn.Sequential(l1, act, l2))
    gate = torch.nn.Linear(spec.H, E, bias=bg is not None, dtype=torch.float64)
    with torch.no_grad():
        gate.weight.copy_(Wg.T)
        if bg is not None:
            gate.bias.copy_(bg)
    return gate, experts


def torch_masked_layer(spec, inp) -> Dict[str, object]:
    """Token-choice routing with library top-k, then one boolean row mask per
    expert: rows that picked expert e get that expert's output scaled by the
    weight they gave it (an expert appears at most once in a token's top-k, so
    the slots of a token can be merged).  No capacity limit."""
    import torch
    gate, experts = _torch_modules(spec, inp)
    xt = torch.from_numpy(_f64(inp["x"], spec.dtype))
    with torch.no_grad():
        lg = gate(xt)
        prob = torch.softmax(lg, dim=-1)
        val, sel = torch.topk(prob, spec.k, dim=-1)
        wts = val / val.sum(dim=-1, keepdim=True)
        acc = torch.zeros_like(xt)
        for e, net in enumerate(experts):
            hit = sel == e
            rows = hit.any(dim=1)
            if not bool(rows.any()):
                continue
            coef = (wts * hit).sum(dim=1)[rows]
            acc[rows] += coef[:, None] * net(xt[rows])
        hist = torch.nn.functional.one_hot(sel.reshape(-1).long(), spec.E).sum(dim=0)
        aux = spec.E * torch.dot(hist.double() / sel.numel(), prob.mean(dim=0))
        z = torch.logsumexp(lg, dim=-1).square().mean()
    return dict(logits=lg.numpy(), topk_idx=sel.numpy().astype(np.int32),
                topk_w=wts.numpy(), out=acc.numpy(), aux=float(aux), z=float(z))


def torch_expert_major(spec, inp) -> np.ndarray:
    """Expert-major accumulation: for each expert, the flat (token, slot) pairs
    that chose it are gathered, run through the expert, scaled by their weight
    and added into their token rows with index_add_.  No capacity limit."""
    import torch
    gate, experts = _torch_modules(spec, inp)
    xt = torch.from_numpy(_f64(inp["x"], spec.dtype))
    with torch.no_grad():
        prob = torch.softmax(gate(xt), dim=1)
        val, sel = torch.topk(prob, spec.k, dim=-1)
        wflat = (val / val.sum(dim=-1, keepdim=True)).reshape(-1)
        eflat = sel.reshape(-1)
        tflat = torch.arange(spec.T).repeat_interleave(spec.k)
        acc = torch.zeros_like(xt)
        for e, net in enumerate(experts):
            j = torch.nonzero(eflat == e).squeeze(1)
            if j.numel() == 0:
                continue
            toks = tflat[j]
            acc.index_add_(0, toks, net(xt[toks]) * wflat[j, None])
    return acc.numpy()


def dense_ffn(spec, inp, e: int = 0) -> np.ndarray:
    """One expert applied densely to every token with torch.nn modules (float64)."""
    import torch
    _, experts = _torch_modules(spec, inp)
    x = torch.from_numpy(_f64(inp["x"], spec.dtype))
    with torch.no_grad():
        return experts[e](x).numpy()


# ---------------------------------------------------------------- expert choice
def expert_choice_dense(spec, inp: Dict[str, Optional[np.ndarray]], group: int,
                        C: int) -> Dict[str, object]:
    """Expert-choice routing by sorting: in every group each expert's tokens are
    ordered by (descending logit, ascending token) with a stable lexicographic
    sort and the first C are taken; then every expert runs on every token and
    the taken outputs are summed with the tokens' softmax weights (a 0/1 mask
    per (token, expert))."""
    d = spec.dtype
    T, E = spec.T, spec.E
    x = _f64(inp["x"], d)
    Wg, bg = _f64(inp["Wg"], d), _f64(inp.get("bg"), d)
    lg = x @ Wg + (0.0 if bg is None else bg[None, :])
    p = special.softmax(lg, axis=1)
    ng = T // group
    mask = np.zeros((T, E), bool)
    sets = np.empty((E, ng, C), np.int64)
    for e in range(E):
        for g in range(ng):
            toks = np.arange(g * group, (g + 1) * group)
            order = np.lexsort((toks, -lg[toks, e]))    # last key is primary
            take = np.sort(toks[order[:C]])
            sets[e, g] = take
            mask[take, e] = True
    Y = _all_experts(spec, x, _f64(inp["W1"], d), _f64(inp.get("b1"), d), _f64(inp["W2"], d),
                     _f64(inp.get("b2"), d))
    out = np.einsum("te,eth->th", p * mask, Y)
    return dict(logits=lg, probs=p, mask=mask, sets=sets, out=out, Y=Y)


def torch_expert_choice_sets(lg: np.ndarray, group: int, C: int) -> np.ndarray:
    """The page's expert-choice snippet (Core Concepts, 2. Routing Mechanisms):
    scores laid out (batch, experts, seq_len), torch.topk over the sequence.
    Returns the taken tokens [E][groups][C], ascending (torch.topk leaves the
    order of equal scores open, so callers use inputs without ties)."""
    import torch
    T, E = lg.shape
    ng = T // group
    scores = torch.from_numpy(lg).reshape(ng, group, E).transpose(-1, -2)   # (ng, E, group)
    idx = torch.topk(scores, k=C, dim=-1).indices                         # (ng, E, C)
    glob = idx + (torch.arange(ng) * group)[:, None, None]
    return np.sort(glob.permute(1, 0, 2).numpy(), axis=-1)


# ---------------------------------------------------------------- backward
def torch_layer_grads(spec, inp: Dict[str, Optional[np.ndarray]], dout: np.ndarray,
                      g_aux: float, g_z: float) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(dout * out) + g_aux * aux + g_z * z by torch
    autograd in float64, for the page's layer with no capacity limit: gate
    linear, softmax, torch.topk, renormalisation, every expert evaluated
    densely and gathered by index, the aux loss with the routed fractions f
    held constant, and the z-loss.  Returned in the [in][out] weight layout."""
    import torch
    d = spec.dtype
    T, E, k = spec.T, spec.E, spec.k
    t64 = lambda a: None if a is None else torch.from_numpy(_f64(a, d)).requires_grad_(True)
    x, Wg, bg = t64(inp["x"]), t64(inp["Wg"]), t64(inp.get("bg"))
    W1, b1, W2, b2 = t64(inp["W1"]), t64(inp.get("b1")), t64(inp["W2"]), t64(inp.get("b2"))
    lg = x @ Wg + (bg if bg is not None else 0.0)
    p = torch.softmax(lg, dim=1)
    val, idx = torch.topk(p, k, dim=1)
    w = val / val.sum(dim=1, keepdim=True)
    act = torch.nn.functional.silu if spec.act == "silu" else torch.nn.functional.gelu
    Y = torch.stack([act(x @ W1[e] + (b1[e] if b1 is not None else 0.0)) @ W2[e]
                     + (b2[e] if b2 is not None else 0.0) for e in range(E)])     # [E, T, H]
    sel = Y[idx, torch.arange(T)[:, None], :]                                      # [T, k, H]
    out = (w[:, :, None] * sel).sum(dim=1)
    f = torch.bincount(idx.reshape(-1), minlength=E).double() / float(T * k)
    aux = E * (f * p.mean(dim=0)).sum()
    z = (torch.logsumexp(lg, dim=1) ** 2).mean()
    L = (torch.from_numpy(_f64(dout, d)) * out).sum() + g_aux * aux + g_z * z
    L.backward()
    g = lambda t: None if t is None else t.grad.numpy()
    return dict(dx=g(x), dWg=g(Wg), dbg=g(bg), dW1=g(W1), db1=g(b1), dW2=g(W2), db2=g(b2))
