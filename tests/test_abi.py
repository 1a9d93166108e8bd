"""The C ABI without a GPU: libmoe.so loads, exports every entry point that
include/moe.h declares, and rejects bad arguments on the host before anything
is enqueued (every call here fails validation, so no kernel is launched and
the fake device pointers are never dereferenced)."""
import ctypes
import math
import os
import re

import pytest

import sparse_mixture_experts_21_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
A = 0x100000          # a 16-byte-aligned fake device address (never dereferenced)
MIS = A + 4           # misaligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(moe.EXPORTS), names
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), f"libmoe.so does not export {n}"


def test_status_strings():
    for s in range(5):
        assert moe.status_string(s)
    assert moe.status_string(99) == "unknown status"


def P(**kw):
    base = dict(T=64, H=32, E=8, k=2, F=64, capacity_factor=1.25, dtype="bf16")
    base.update(kw)
    return moe.Problem(**base)


def route(p, x=A, Wg=A, bg=None, logits=None, idx=A, w=A, counts=A, losses=A, flags=0, ws=A,
          ws_bytes=1 << 30):
    return moe.lib().moe_route(ctypes.byref(p), x, Wg, bg, logits, idx, w, counts, losses,
                               flags, ws, ws_bytes, None)


def permute(p, x=A, idx=A, off=A, pos=A, rt=A, xp=A, ws=A, ws_bytes=1 << 30):
    return moe.lib().moe_permute(ctypes.byref(p), x, idx, off, pos, rt, xp, ws, ws_bytes, None)


def ffn(p, xp=A, off=A, W1=A, b1=None, W2=A, b2=None, h=A, y=A):
    return moe.lib().moe_expert_ffn(ctypes.byref(p), xp, off, W1, b1, W2, b2, h, y, None, 0, None)


def combine(p, y=A, pos=A, w=A, out=A):
    return moe.lib().moe_combine(ctypes.byref(p), y, pos, w, out, None)


def forward(p, ws_bytes=1 << 40, **kw):
    a = dict(x=A, Wg=A, bg=None, W1=A, b1=None, W2=A, b2=None, out=A, losses=A, logits=None,
             idx=None, w=None, counts=None, off=None, pos=None, ws=A, ev=None)
    a.update(kw)
    return moe.lib().moe_forward(ctypes.byref(p), a["x"], a["Wg"], a["bg"], a["W1"], a["b1"],
                                 a["W2"], a["b2"], a["out"], a["losses"], a["logits"], a["idx"],
                                 a["w"], a["counts"], a["off"], a["pos"], a["ws"], ws_bytes,
                                 None, a["ev"])


BAD_PROBLEMS = [
    (dict(T=0), moe.MOE_ERR_INVALID_ARG),
    (dict(H=0), moe.MOE_ERR_INVALID_ARG),
    (dict(F=0), moe.MOE_ERR_INVALID_ARG),
    (dict(E=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=9, E=8), moe.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(activation=2), moe.MOE_ERR_INVALID_ARG),
    (dict(activation=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=math.nan), moe.MOE_ERR_INVALID_ARG),
    (dict(E=257, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=16, k=9), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=36), moe.MOE_ERR_UNSUPPORTED),
    (dict(F=68), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=34, dtype="f32"), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 30, k=2), moe.MOE_ERR_UNSUPPORTED),
    # bf16: 32-bit buffer-resource ranges (gathered token rows, one expert's
    # weights, the gate) must stay below 2^31 bytes
    (dict(T=2 ** 18, H=4096), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=32768, F=32768), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=256, k=2, H=2 ** 22, F=8), moe.MOE_ERR_UNSUPPORTED),
]


def test_problem_struct_layout_matches_header():
    # moe_problem_t: int64 T, int32 H E k F, double capacity_factor, int32 dtype activation
    assert ctypes.sizeof(moe.Problem) == 40
    assert moe.Problem.capacity_factor.offset == 24
    assert moe.Problem.dtype.offset == 32 and moe.Problem.activation.offset == 36


@pytest.mark.parametrize("act", ["gelu", "silu", moe.MOE_ACT_SILU])
def test_both_activations_accepted(act):
    p = P(activation=act)
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == moe.MOE_OK
    assert n.value > 0


@pytest.mark.parametrize("kw", [dict(T=2 ** 18 - 1, H=4096), dict(H=32768, F=32760),
                                dict(T=2 ** 18, H=4096, dtype="f32")])
def test_range_envelope_edges_accepted(kw):
    """Just inside the bf16 32-bit ranges, and fp32 (no such range): accepted
    by the host-only queries."""
    p = P(**kw)
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == moe.MOE_OK
    cap = ctypes.c_int64()
    assert moe.lib().moe_capacity(ctypes.byref(p), ctypes.byref(cap)) == moe.MOE_OK


@pytest.mark.parametrize("kw,status", BAD_PROBLEMS, ids=[str(b[0]) for b in BAD_PROBLEMS])
def test_bad_problem_rejected_by_every_entry_point(kw, status):
    p = P(**kw)
    assert route(p) == status
    assert permute(p) == status
    assert ffn(p) == status
    assert combine(p) == status
    assert forward(p) == status
    cap = ctypes.c_int64()
    assert moe.lib().moe_capacity(ctypes.byref(p), ctypes.byref(cap)) == status
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == status


def test_null_problem():
    L = moe.lib()
    assert L.moe_route(None, A, A, None, None, A, A, A, A, 0, A, 1, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(None, A, A, A, A, None) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["x", "Wg", "idx", "w", "counts", "losses", "ws"])
def test_route_null_required(arg):
    assert route(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG


def test_route_flags_and_logits_in():
    assert route(P(), flags=2) == moe.MOE_ERR_INVALID_ARG
    # logits required as input with MOE_ROUTE_LOGITS_IN; x and Wg are then optional
    assert route(P(), flags=moe.MOE_ROUTE_LOGITS_IN, logits=None) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["x", "Wg", "bg", "logits", "idx", "w", "counts", "losses", "ws"])
def test_route_misaligned(arg):
    assert route(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_route_workspace_too_small():
    assert route(P(), ws_bytes=16) == moe.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("arg", ["x", "idx", "off", "pos", "rt", "xp", "ws"])
def test_permute_null_and_misaligned(arg):
    assert permute(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG
    assert permute(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_permute_workspace_too_small():
    assert permute(P(), ws_bytes=0) == moe.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("arg", ["xp", "off", "W1", "W2", "h", "y"])
def test_ffn_null_and_misaligned(arg):
    assert ffn(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG
    assert ffn(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_ffn_misaligned_bias():
    assert ffn(P(), b1=MIS) == moe.MOE_ERR_UNSUPPORTED
    assert ffn(P(), b2=MIS) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("arg", ["y", "pos", "w", "out"])
def test_combine_null_and_misaligned(arg):
    assert combine(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG
    assert combine(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("arg", ["x", "Wg", "W1", "W2", "out", "losses", "ws"])
def test_forward_null_and_misaligned(arg):
    assert forward(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG
    assert forward(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("arg", ["bg", "b1", "b2", "logits", "idx", "w", "counts", "off", "pos"])
def test_forward_misaligned_optional(arg):
    assert forward(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_forward_workspace_exact_size():
    p = P()
    need = moe.moe_workspace_bytes(p)
    assert forward(p, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE


def test_forward_null_event_entries_are_skipped_not_rejected():
    """A NULL entry of stage_events skips that point: validation accepts an
    array of NULLs and goes on to the next check (here the workspace size),
    so nothing is launched."""
    arr = (ctypes.c_void_p * moe.MOE_FORWARD_EVENTS)()
    p = P()
    need = moe.moe_workspace_bytes(p)
    assert forward(p, ev=ctypes.cast(arr, ctypes.c_void_p), ws_bytes=need - 1) == \
        moe.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("T,k,E,cf,cap", [
    (8192, 2, 8, 1.25, 2560), (8192, 1, 128, 1.25, 80), (16384, 2, 8, 2.0, 8192),
    (16384, 2, 64, 0.0, 16384), (256, 2, 8, 0.5, 32), (10, 1, 3, 1.0, 4), (7, 2, 4, -1.0, 7)])
def test_capacity(T, k, E, cf, cap):
    assert moe.moe_capacity(P(T=T, k=k, E=E, capacity_factor=cf)) == cap


def test_workspace_grows_with_problem():
    small = moe.moe_workspace_bytes(P(T=64))
    big = moe.moe_workspace_bytes(P(T=4096))
    assert 0 < small < big
    assert moe.moe_workspace_bytes(P(T=64)) % 256 == 0


def test_binding_raises_on_error():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_bytes(P(k=0))
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


# ---------------------------------------------------------------- expert choice
def ec_route(p, group, x=A, Wg=A, bg=None, logits=None, flags=0, probs=A, sel=A, rowof=A,
             off=A, ws=A, ws_bytes=1 << 40):
    return moe.lib().moe_route_expert_choice(ctypes.byref(p), group, x, Wg, bg, logits, flags,
                                             probs, sel, rowof, off, ws, ws_bytes, None)


def ec_forward(p, group, ws_bytes=1 << 40, **kw):
    a = dict(x=A, Wg=A, bg=None, W1=A, b1=None, W2=A, b2=None, out=A, logits=None, probs=None,
             sel=None, rowof=None, ws=A, ev=None)
    a.update(kw)
    return moe.lib().moe_forward_expert_choice(
        ctypes.byref(p), group, a["x"], a["Wg"], a["bg"], a["W1"], a["b1"], a["W2"], a["b2"],
        a["out"], a["logits"], a["probs"], a["sel"], a["rowof"], a["ws"], ws_bytes, None, a["ev"])


EC_BAD = [
    (dict(), 0, moe.MOE_ERR_INVALID_ARG),
    (dict(), -64, moe.MOE_ERR_INVALID_ARG),
    (dict(T=64), 48, moe.MOE_ERR_INVALID_ARG),             # T % group != 0
    (dict(k=0), 64, moe.MOE_ERR_INVALID_ARG),              # the problem itself
    (dict(T=65536), 65536, moe.MOE_ERR_UNSUPPORTED),       # group keys exceed LDS
    (dict(H=36), 64, moe.MOE_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,group,status", EC_BAD, ids=[f"{b[0]}-{b[1]}" for b in EC_BAD])
def test_ec_bad_group_rejected_by_every_entry_point(kw, group, status):
    p = P(**kw)
    c = ctypes.c_int64()
    assert moe.lib().moe_ec_capacity(ctypes.byref(p), group, ctypes.byref(c)) == status
    n = ctypes.c_size_t()
    assert moe.lib().moe_ec_workspace_bytes(ctypes.byref(p), group, ctypes.byref(n)) == status
    assert ec_route(p, group) == status
    assert ec_forward(p, group) == status


@pytest.mark.parametrize("T,group,k,E,cf", [(16384, 2048, 2, 8, 0.0), (16384, 2048, 2, 8, 1.25),
                                            (64, 64, 1, 8, 0.0), (70, 7, 1, 8, 0.0),
                                            (40, 10, 8, 8, 2.0), (300, 100, 3, 7, 1.0)])
def test_ec_capacity_matches_oracle(oracle_mod, T, group, k, E, cf):
    import workloads as W
    spec = W.Spec("ec", T=T, H=32, E=E, k=k, F=64, dtype="bf16", cf=cf, seed=1)
    assert moe.moe_ec_capacity(P(T=T, k=k, E=E, capacity_factor=cf), group) == \
        oracle_mod.ec_capacity(spec, group)


@pytest.mark.parametrize("arg", ["probs", "sel", "rowof", "off", "ws"])
def test_ec_route_null_required(arg):
    assert ec_route(P(), 64, **{arg: None}) == moe.MOE_ERR_INVALID_ARG


def test_ec_route_flags_and_logits_in():
    assert ec_route(P(), 64, flags=2) == moe.MOE_ERR_INVALID_ARG
    assert ec_route(P(), 64, flags=moe.MOE_ROUTE_LOGITS_IN, logits=None) == \
        moe.MOE_ERR_INVALID_ARG
    assert ec_route(P(), 64, x=None) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["probs", "sel", "rowof", "off", "ws", "x"])
def test_ec_route_misaligned(arg):
    assert ec_route(P(), 64, **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("arg", ["x", "Wg", "W1", "W2", "out", "ws"])
def test_ec_forward_null_required(arg):
    assert ec_forward(P(), 64, **{arg: None}) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["x", "out", "logits", "probs", "sel", "rowof", "b1"])
def test_ec_forward_misaligned(arg):
    assert ec_forward(P(), 64, **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_ec_workspace_exact_size_and_null_events():
    p = P()
    need = moe.moe_ec_workspace_bytes(p, 64)
    assert need % 256 == 0 and need > 0
    assert ec_forward(p, 64, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert ec_route(p, 64, ws_bytes=0) == moe.MOE_ERR_WORKSPACE
    # NULL event entries are skipped, not rejected: validation reaches the workspace check
    arr = (ctypes.c_void_p * moe.MOE_FORWARD_EVENTS)()
    assert ec_forward(p, 64, ev=ctypes.cast(arr, ctypes.c_void_p), ws_bytes=need - 1) == \
        moe.MOE_ERR_WORKSPACE


# ---------------------------------------------------------------- training
def fwd_train(p, ws_bytes=1 << 40, **kw):
    a = dict(x=A, Wg=A, bg=None, W1=A, b1=None, W2=A, b2=None, out=A, losses=A, ws=A)
    a.update(kw)
    return moe.lib().moe_forward_train(ctypes.byref(p), a["x"], a["Wg"], a["bg"], a["W1"],
                                       a["b1"], a["W2"], a["b2"], a["out"], a["losses"], a["ws"],
                                       ws_bytes, None)


def bwd(p, ws_bytes=1 << 40, g_aux=0.01, g_z=0.001, **kw):
    a = dict(x=A, Wg=A, W1=A, W2=A, dout=A, dx=A, dWg=A, dbg=None, dW1=A, db1=None, dW2=A,
             db2=None, ws=A)
    a.update(kw)
    return moe.lib().moe_backward(ctypes.byref(p), a["x"], a["Wg"], a["W1"], a["W2"], a["dout"],
                                  g_aux, g_z, a["dx"], a["dWg"], a["dbg"], a["dW1"], a["db1"],
                                  a["dW2"], a["db2"], a["ws"], ws_bytes, None, a.get("ev"))


@pytest.mark.parametrize("kw,status", BAD_PROBLEMS[:10] + [
    (dict(dtype="f32"), moe.MOE_ERR_UNSUPPORTED),                 # bf16 only
    (dict(T=2 ** 17, k=2, H=4096, F=4096), moe.MOE_ERR_UNSUPPORTED),  # 32-bit row ranges
], ids=lambda v: str(v))
def test_train_bad_problem_rejected(kw, status):
    p = P(**kw)
    n = ctypes.c_size_t()
    assert moe.lib().moe_train_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == status
    assert fwd_train(p) == status
    assert bwd(p) == status


@pytest.mark.parametrize("arg", ["x", "Wg", "W1", "W2", "out", "losses", "ws"])
def test_forward_train_null_required(arg):
    assert fwd_train(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["x", "Wg", "W1", "W2", "dout", "dx", "dWg", "dW1", "dW2", "ws"])
def test_backward_null_required(arg):
    assert bwd(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["x", "dout", "dx", "dWg", "dbg", "dW1", "db1", "dW2", "db2"])
def test_backward_misaligned(arg):
    assert bwd(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_train_workspace_sizes_and_nan_weights():
    p = P()
    need = moe.moe_train_workspace_bytes(p)
    assert need > moe.moe_workspace_bytes(p) and need % 256 == 0
    assert fwd_train(p, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert bwd(p, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert bwd(p, g_aux=math.nan) == moe.MOE_ERR_INVALID_ARG
    # NULL event entries are skipped, not rejected: validation reaches the workspace check
    arr = (ctypes.c_void_p * moe.MOE_BACKWARD_EVENTS)()
    assert bwd(p, ev=ctypes.cast(arr, ctypes.c_void_p), ws_bytes=need - 1) == \
        moe.MOE_ERR_WORKSPACE


# ---------------------------------------------------------------- fixed scratch
def fwd_noalloc(p, **kw):
    a = dict(x=A, Wg=A, bg=None, W1=A, b1=None, W2=A, b2=None, out=A, losses=A, logits=None,
             idx=None, w=None, counts=None, off=None, pos=None, ev=None)
    a.update(kw)
    return moe.lib().moe_forward_noalloc(ctypes.byref(p), a["x"], a["Wg"], a["bg"], a["W1"],
                                         a["b1"], a["W2"], a["b2"], a["out"], a["losses"],
                                         a["logits"], a["idx"], a["w"], a["counts"], a["off"],
                                         a["pos"], None, a["ev"])


@pytest.mark.parametrize("kw,status", BAD_PROBLEMS, ids=[str(b[0]) for b in BAD_PROBLEMS])
def test_noalloc_bad_problem_rejected(kw, status):
    assert fwd_noalloc(P(**kw)) == status


@pytest.mark.parametrize("arg", ["x", "Wg", "W1", "W2", "out", "losses"])
def test_noalloc_null_and_misaligned(arg):
    assert fwd_noalloc(P(), **{arg: None}) == moe.MOE_ERR_INVALID_ARG
    assert fwd_noalloc(P(), **{arg: MIS}) == moe.MOE_ERR_UNSUPPORTED


def test_noalloc_scratch_limit_and_null_events():
    """A problem whose workspace exceeds the fixed scratch is refused with
    MOE_ERR_WORKSPACE before any HIP call (this runs without a GPU), also
    with an event array of NULL entries (skipped, not rejected)."""
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == moe.MOE_NOALLOC_SCRATCH_BYTES
    big = P(T=8192, H=1024, E=8, k=2, F=4096)
    assert moe.moe_workspace_bytes(big) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert fwd_noalloc(big) == moe.MOE_ERR_WORKSPACE
    arr = (ctypes.c_void_p * moe.MOE_FORWARD_EVENTS)()
    assert fwd_noalloc(big, ev=ctypes.cast(arr, ctypes.c_void_p)) == moe.MOE_ERR_WORKSPACE
