"""MI355X (gfx950) sparse top-k Mixture-of-Experts FFN forward.

A thin ctypes binding over ``libmoe.so`` (include/moe.h).  Every function has
the name of the C entry point it calls and only marshals arguments: torch
tensors are passed as raw device pointers together with the current HIP
stream of their device; every step of the layer runs in the HIP kernels.  If
the library has not been built the calls raise; there is no fallback path.

    import sparse_mixture_experts_21_amd as moe
    prob = moe.Problem(T=..., H=..., E=..., k=..., F=..., capacity_factor=..., dtype="bf16")
    ws = torch.empty(moe.moe_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    moe.moe_forward(prob, x, Wg, bg, W1, b1, W2, b2, out, losses, ws=ws)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB may name another build of the same sources (the host-sanitizer build
# that the CPU tests load); the default is the in-tree libmoe.so.
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_SILU = 0, 1
MOE_ROUTE_LOGITS_IN = 1
(MOE_EV_ROUTE, MOE_EV_PERMUTE, MOE_EV_FFN_UP, MOE_EV_FFN_UP_FIXUP, MOE_EV_FFN_DOWN,
 MOE_EV_FFN_DOWN_FIXUP, MOE_EV_COMBINE, MOE_EV_END, MOE_FORWARD_EVENTS) = range(9)
STAGE_NAMES = ("route", "permute", "ffn_up", "ffn_up_fixup", "ffn_down", "ffn_down_fixup",
               "combine")
MOE_BACKWARD_EVENTS = 10
BACKWARD_STAGE_NAMES = ("token", "dgrad_da", "dgrad_dxe", "dx", "gather", "wgrad_w2",
                        "wgrad_w1", "bias", "gate")

EXPORTS = ("moe_capacity", "moe_workspace_bytes", "moe_route", "moe_permute",
           "moe_expert_ffn", "moe_combine", "moe_forward", "moe_status_string",
           "moe_ec_capacity", "moe_ec_workspace_bytes", "moe_route_expert_choice",
           "moe_forward_expert_choice", "moe_train_workspace_bytes", "moe_forward_train",
           "moe_backward", "moe_forward_noalloc")
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Problem(ctypes.Structure):
    """moe_problem_t.  dtype may be given as "bf16"/"f32" and activation as
    "gelu"/"silu", or either as the enum value."""
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double), ("dtype", ctypes.c_int32),
                ("activation", ctypes.c_int32)]

    def __init__(self, T, H, E, k, F, capacity_factor=0.0, dtype="bf16", activation="gelu"):
        if isinstance(dtype, str):
            dtype = {"bf16": MOE_DTYPE_BF16, "f32": MOE_DTYPE_F32}[dtype]
        if isinstance(activation, str):
            activation = {"gelu": MOE_ACT_GELU, "silu": MOE_ACT_SILU}[activation]
        super().__init__(int(T), int(H), int(E), int(k), int(F), float(capacity_factor),
                         int(dtype), int(activation))

    @classmethod
    def from_spec(cls, spec, **over) -> "Problem":
        g = lambda n: over.get(n, getattr(spec, n))
        return cls(g("T"), g("H"), g("E"), g("k"), g("F"), over.get("cf", spec.cf),
                   g("dtype"), g("act"))

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == MOE_DTYPE_BF16 else 4

    def __repr__(self):
        return (f"Problem(T={self.T}, H={self.H}, E={self.E}, k={self.k}, F={self.F}, "
                f"cf={self.capacity_factor}, dtype={'bf16' if self.dtype else 'f32'}, "
                f"activation={'silu' if self.activation == MOE_ACT_SILU else 'gelu'})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_mixture_experts_21_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, st = ctypes.c_void_p, ctypes.c_int
        L.moe_capacity.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.moe_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp,
                                ctypes.c_size_t, vp]
        L.moe_permute.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_expert_ffn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_combine.argtypes = [P, vp, vp, vp, vp, vp]
        L.moe_forward.argtypes = [P] + [vp] * 16 + [ctypes.c_size_t, vp, vp]
        L.moe_forward_noalloc.argtypes = [P] + [vp] * 17
        i64 = ctypes.c_int64
        L.moe_ec_capacity.argtypes = [P, i64, ctypes.POINTER(i64)]
        L.moe_ec_workspace_bytes.argtypes = [P, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route_expert_choice.argtypes = [P, i64, vp, vp, vp, vp, ctypes.c_uint32, vp, vp,
                                              vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_forward_expert_choice.argtypes = [P, i64] + [vp] * 13 + [ctypes.c_size_t, vp, vp]
        L.moe_train_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_forward_train.argtypes = [P] + [vp] * 10 + [ctypes.c_size_t, vp]
        fl = ctypes.c_float
        L.moe_backward.argtypes = [P] + [vp] * 5 + [fl, fl] + [vp] * 8 + [ctypes.c_size_t, vp, vp]
        for f in ("moe_capacity", "moe_workspace_bytes", "moe_route", "moe_permute",
                  "moe_expert_ffn", "moe_combine", "moe_forward", "moe_ec_capacity",
                  "moe_ec_workspace_bytes", "moe_route_expert_choice",
                  "moe_forward_expert_choice", "moe_train_workspace_bytes",
                  "moe_forward_train", "moe_backward", "moe_forward_noalloc"):
            getattr(L, f).restype = st
        L.moe_status_string.argtypes = [st]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


moe_status_string = status_string


# ---------------------------------------------------------------- marshalling
def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL).  Raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


# ---------------------------------------------------------------- entry points
def moe_capacity(p: Problem) -> int:
    cap = ctypes.c_int64()
    _check(lib().moe_capacity(ctypes.byref(p), ctypes.byref(cap)), "moe_capacity")
    return cap.value


def moe_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def moe_route(p: Problem, x, Wg, bg, logits, topk_idx, topk_w, counts, losses, ws,
              flags: int = 0, stream=None) -> None:
    _check(lib().moe_route(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(logits),
                           _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(losses),
                           flags, _ptr(ws), _nbytes(ws), _stream(stream, topk_idx)),
           "moe_route")


def moe_permute(p: Problem, x, topk_idx, offsets, pos, row_token, xp, ws, stream=None) -> None:
    _check(lib().moe_permute(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(offsets),
                             _ptr(pos), _ptr(row_token), _ptr(xp), _ptr(ws), _nbytes(ws),
                             _stream(stream, topk_idx)), "moe_permute")


def moe_expert_ffn(p: Problem, xp, offsets, W1, b1, W2, b2, h, y, ws=None,
                   stream=None) -> None:
    _check(lib().moe_expert_ffn(ctypes.byref(p), _ptr(xp), _ptr(offsets), _ptr(W1), _ptr(b1),
                                _ptr(W2), _ptr(b2), _ptr(h), _ptr(y), _ptr(ws), _nbytes(ws),
                                _stream(stream, xp)), "moe_expert_ffn")


def moe_combine(p: Problem, y, pos, topk_w, out, stream=None) -> None:
    _check(lib().moe_combine(ctypes.byref(p), _ptr(y), _ptr(pos), _ptr(topk_w), _ptr(out),
                             _stream(stream, out)), "moe_combine")


def moe_forward(p: Problem, x, Wg, bg, W1, b1, W2, b2, out, losses, ws, logits=None,
                topk_idx=None, topk_w=None, counts=None, offsets=None, pos=None,
                stream=None, events: Optional["StageEvents"] = None) -> None:
    ev = events.array() if events is not None else None
    _check(lib().moe_forward(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(b1),
                             _ptr(W2), _ptr(b2), _ptr(out), _ptr(losses), _ptr(logits),
                             _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                             _ptr(pos), _ptr(ws), _nbytes(ws), _stream(stream, out),
                             ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None),
           "moe_forward")


def moe_forward_noalloc(p: Problem, x, Wg, bg, W1, b1, W2, b2, out, losses, logits=None,
                        topk_idx=None, topk_w=None, counts=None, offsets=None, pos=None,
                        stream=None, events: Optional["StageEvents"] = None) -> None:
    ev = events.array() if events is not None else None
    _check(lib().moe_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1),
                                     _ptr(b1), _ptr(W2), _ptr(b2), _ptr(out), _ptr(losses),
                                     _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                                     _ptr(offsets), _ptr(pos), _stream(stream, out),
                                     ctypes.cast(ev, ctypes.c_void_p) if ev is not None
                                     else None), "moe_forward_noalloc")


def moe_ec_capacity(p: Problem, group: int) -> int:
    c = ctypes.c_int64()
    _check(lib().moe_ec_capacity(ctypes.byref(p), int(group), ctypes.byref(c)),
           "moe_ec_capacity")
    return c.value


def moe_ec_workspace_bytes(p: Problem, group: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_ec_workspace_bytes(ctypes.byref(p), int(group), ctypes.byref(n)),
           "moe_ec_workspace_bytes")
    return n.value


def moe_route_expert_choice(p: Problem, group: int, x, Wg, bg, logits, probs, sel, rowof,
                            offsets, ws, flags: int = 0, stream=None) -> None:
    _check(lib().moe_route_expert_choice(ctypes.byref(p), int(group), _ptr(x), _ptr(Wg),
                                         _ptr(bg), _ptr(logits), flags, _ptr(probs), _ptr(sel),
                                         _ptr(rowof), _ptr(offsets), _ptr(ws), _nbytes(ws),
                                         _stream(stream, probs)), "moe_route_expert_choice")


def moe_forward_expert_choice(p: Problem, group: int, x, Wg, bg, W1, b1, W2, b2, out, ws,
                              logits=None, probs=None, sel=None, rowof=None, stream=None,
                              events: Optional["StageEvents"] = None) -> None:
    ev = events.array() if events is not None else None
    _check(lib().moe_forward_expert_choice(
        ctypes.byref(p), int(group), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(b1), _ptr(W2),
        _ptr(b2), _ptr(out), _ptr(logits), _ptr(probs), _ptr(sel), _ptr(rowof), _ptr(ws),
        _nbytes(ws), _stream(stream, out),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None),
        "moe_forward_expert_choice")


def moe_train_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_train_workspace_bytes(ctypes.byref(p), ctypes.byref(n)),
           "moe_train_workspace_bytes")
    return n.value


def moe_forward_train(p: Problem, x, Wg, bg, W1, b1, W2, b2, out, losses, ws, stream=None) -> None:
    _check(lib().moe_forward_train(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1),
                                   _ptr(b1), _ptr(W2), _ptr(b2), _ptr(out), _ptr(losses),
                                   _ptr(ws), _nbytes(ws), _stream(stream, out)),
           "moe_forward_train")


def moe_backward(p: Problem, x, Wg, W1, W2, dout, g_aux, g_z, dx, dWg, dW1, dW2, ws,
                 dbg=None, db1=None, db2=None, stream=None,
                 events: Optional["StageEvents"] = None) -> None:
    ev = events.array() if events is not None else None
    _check(lib().moe_backward(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(W1), _ptr(W2), _ptr(dout),
                              float(g_aux), float(g_z), _ptr(dx), _ptr(dWg), _ptr(dbg), _ptr(dW1),
                              _ptr(db1), _ptr(dW2), _ptr(db2), _ptr(ws), _nbytes(ws),
                              _stream(stream, dx),
                              ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None),
           "moe_backward")


# ---------------------------------------------------------------- stage events
_hip = None


def _hiprt() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


class StageEvents:
    """HIP events for moe_forward / moe_forward_expert_choice (n =
    MOE_FORWARD_EVENTS, the default) or moe_backward (n = MOE_BACKWARD_EVENTS)
    via events=...: the library records them on its stream around each stage,
    so stage times come from the stream the kernels actually run on."""

    def __init__(self, n: int = MOE_FORWARD_EVENTS, points: Optional[Sequence[int]] = None):
        """points: the event indices to record (default all); the others are
        NULL, which the library skips."""
        h = _hiprt()
        self.n = n
        self._ev = (ctypes.c_void_p * n)()
        for i in (range(n) if points is None else points):
            e = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._ev[i] = e.value

    def array(self):
        return self._ev

    def elapsed_ms(self, i: int, j: int) -> float:
        """Milliseconds from event i to event j of the last recorded call."""
        h = _hiprt()
        h.hipEventSynchronize(self._ev[j])
        ms = ctypes.c_float()
        if h.hipEventElapsedTime(ctypes.byref(ms), self._ev[i], self._ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def stage_ms(self) -> Sequence[float]:
        """Milliseconds of each stage of the last recorded call (waits for it;
        every event must have been recorded)."""
        return [self.elapsed_ms(i, i + 1) for i in range(self.n - 1)]

    def __del__(self):
        try:
            h = _hiprt()
            for i in range(self.n):
                if self._ev[i]:
                    h.hipEventDestroy(self._ev[i])
        except Exception:
            pass
