"""Pins for the CPU oracle (runs without a GPU).

The oracle (oracle/liboracle.so, a per-token fp64 C loop) is checked against
things other than itself: the worked weights the routing diagram prints,
closed forms (all-zero gate, constant and one-hot biases, identical experts,
one expert, k = E), a dense evaluate-every-expert-then-mask brute force, two
torch float64 formulations of the page's layer, and dispatch invariants.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RT, AT = 1e-10, 1e-12


def tiny(T=24, H=16, E=4, k=2, F=40, dtype="f32", cf=0.0, seed=7, biases=True, **kw):
    s = W.Spec(f"tiny_T{T}_H{H}_E{E}_k{k}_F{F}_{dtype}_cf{cf}", T=T, H=H, E=E, k=k, F=F,
               dtype=dtype, cf=cf, seed=seed, x=W.Dist("normal", 1.0),
               wg=W.Dist("normal", 0.5), w1=W.Dist("uniform", 1 / math.sqrt(H)),
               w2=W.Dist("uniform", 1 / math.sqrt(F)))
    if biases:
        s = s.replace(bg=W.Dist("uniform", 0.3), b1=W.Dist("uniform", 0.2),
                      b2=W.Dist("uniform", 0.1))
    return s.replace(**kw) if kw else s


def run_oracle(om, spec, inp, **kw):
    return om.forward(spec, inp, **kw)


# ---------------------------------------------------------------- worked example
def test_golden_diagram_weights(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "top2_diagram_weights.json")))
    spec = tiny(T=1, E=g["E"], k=g["k"])
    r = oracle_mod.route(spec, np.array([g["logits"]], np.float64))
    assert r["topk_idx"][0].tolist() == g["expected_topk_idx"]
    np.testing.assert_allclose(r["topk_w"][0], g["expected_topk_w"], rtol=0, atol=1e-15)
    assert abs(r["topk_w"][0].sum() - 1.0) < 1e-15


# ---------------------------------------------------------------- brute force
BRUTE_CASES = [
    dict(),
    dict(dtype="bf16"),
    dict(k=1),
    dict(k=3, E=5),
    dict(k=4, E=4),
    dict(E=8, k=2, T=64, H=32, F=48),
    dict(cf=0.5),
    dict(cf=1.0, k=1, E=3, T=31),
    dict(cf=1.25, dtype="bf16", T=50, E=6, k=2),
    dict(biases=False),
    dict(E=1, k=1),
    dict(T=1),
    dict(act="silu"),
    dict(act="silu", dtype="bf16", biases=False, E=8, k=2, T=40),
]


@pytest.mark.parametrize("case", BRUTE_CASES, ids=[str(c) for c in BRUTE_CASES])
def test_oracle_matches_dense_brute_force(oracle_mod, case):
    spec = tiny(**case)
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    b = bf.dense_then_mask(spec, inp)
    np.testing.assert_allclose(o["logits"], b["logits"], rtol=RT, atol=AT)
    assert np.array_equal(o["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(o["topk_w"], b["topk_w"], rtol=RT, atol=AT)
    np.testing.assert_allclose(o["probs"], b["probs"], rtol=RT, atol=AT)
    np.testing.assert_allclose(o["lse"], b["lse"], rtol=RT, atol=AT)
    assert np.array_equal(o["counts"], b["counts"])
    assert o["cap"] == b["cap"]
    assert math.isclose(o["aux"], b["aux"], rel_tol=RT)
    assert math.isclose(o["z"], b["z"], rel_tol=RT, abs_tol=AT)
    assert np.array_equal(o["offsets"], b["offsets"])
    assert np.array_equal(o["pos"], b["pos"])
    np.testing.assert_allclose(o["out"], b["out"], rtol=RT, atol=1e-11)


def test_oracle_expert_rows_match_dense_experts(oracle_mod):
    spec = tiny(E=3, T=20)
    inp = W.generate(spec, workers=1)
    b = bf.dense_then_mask(spec, inp)
    for e in range(spec.E):
        _, y = oracle_mod.expert_rows(spec, inp["x"], np.full(spec.T, e), inp["W1"],
                                      inp["b1"], inp["W2"], inp["b2"])
        np.testing.assert_allclose(y, b["Y"][e], rtol=RT, atol=1e-11)


def test_oracle_combine_matches_indexing(oracle_mod):
    spec = tiny(T=30, E=4, k=2, cf=0.75, dtype="bf16")
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    A = int(o["offsets"][-1])
    y = W.synthetic_rows(spec, A)
    out = oracle_mod.combine(spec, y, o["pos"], o["topk_w"])
    yf = W.to_f32(y, "bf16").astype(np.float64)
    ref = np.zeros((spec.T, spec.H))
    for t in range(spec.T):
        for s in range(spec.k):
            if o["pos"][t, s] >= 0:
                ref[t] += o["topk_w"][t, s] * yf[o["pos"][t, s]]
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- torch formulations
@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_oracle_matches_torch_layers_on_tiny_fp32_config(oracle_mod, act):
    spec = W.CONFIGS["c1"].replace(act=act)
    inp = W.generate(spec)
    o = run_oracle(oracle_mod, spec, inp)
    assert oracle_mod.topk_margin(spec, o["logits"]) > 1e-9      # no ties: torch.topk is safe
    t = bf.torch_masked_layer(spec, inp)
    np.testing.assert_allclose(o["logits"], t["logits"], rtol=RT, atol=AT)
    assert np.array_equal(o["topk_idx"], t["topk_idx"])
    np.testing.assert_allclose(o["topk_w"], t["topk_w"], rtol=RT, atol=AT)
    np.testing.assert_allclose(o["out"], t["out"], rtol=RT, atol=1e-11)
    assert math.isclose(o["aux"], t["aux"], rel_tol=1e-12)
    assert math.isclose(o["z"], t["z"], rel_tol=1e-12)
    em = bf.torch_expert_major(spec, inp)
    np.testing.assert_allclose(o["out"], em, rtol=RT, atol=1e-11)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("E,k", [(8, 2), (8, 1), (5, 3), (4, 4)])
def test_zero_gate_ties_and_losses(oracle_mod, E, k):
    spec = W.zero_gate(tiny(T=40, E=E, k=k))
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    assert np.all(o["logits"] == 0.0)
    assert np.array_equal(o["topk_idx"], np.tile(np.arange(k, dtype=np.int32), (spec.T, 1)))
    np.testing.assert_allclose(o["topk_w"], 1.0 / k, rtol=0, atol=1e-15)
    expect_counts = np.zeros(E, np.int32)
    expect_counts[:k] = spec.T
    assert np.array_equal(o["counts"], expect_counts)
    assert math.isclose(o["aux"], 1.0, rel_tol=1e-14)
    assert math.isclose(o["z"], math.log(E) ** 2, rel_tol=1e-14, abs_tol=1e-15)


def test_zero_gate_capacity_closed_form(oracle_mod):
    spec = W.zero_gate(tiny(T=64, E=8, k=2, cf=0.5))
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    cap = o["cap"]
    assert cap == 8                                    # ceil(0.5 * 64 * 2 / 8)
    assert o["offsets"].tolist() == [0, 8, 16] + [16] * 6
    for t in range(spec.T):
        for s in range(2):
            assert o["pos"][t, s] == (s * cap + t if t < cap else -1)
    ffn = [bf.dense_ffn(spec, inp, e) for e in (0, 1)]
    for t in range(spec.T):
        ref = 0.5 * ffn[0][t] + 0.5 * ffn[1][t] if t < cap else np.zeros(spec.H)
        np.testing.assert_allclose(o["out"][t], ref, rtol=RT, atol=1e-11)


def test_constant_bias_z_loss(oracle_mod):
    c, E = 1.5, 6
    spec = W.zero_gate(tiny(T=16, E=E, k=2)).replace(bg=W.Dist("const", c))
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    assert math.isclose(o["z"], (c + math.log(E)) ** 2, rel_tol=1e-14)
    assert math.isclose(o["aux"], 1.0, rel_tol=1e-14)


def test_one_hot_bias_losses(oracle_mod):
    c, E = 2.0, 8
    spec = W.zero_gate(tiny(T=10, E=E, k=1))
    inp = W.generate(spec, workers=1)
    bg = np.zeros(E, np.float32)
    bg[0] = c
    inp["bg"] = bg
    o = run_oracle(oracle_mod, spec, inp)
    assert np.all(o["topk_idx"] == 0) and np.all(o["topk_w"] == 1.0)
    p0 = math.exp(c) / (math.exp(c) + E - 1)
    assert math.isclose(o["aux"], E * p0, rel_tol=1e-14)
    assert math.isclose(o["z"], math.log(math.exp(c) + E - 1) ** 2, rel_tol=1e-14)


@pytest.mark.parametrize("cf", [0.0, 0.5])
def test_identical_experts_reduce_to_dense_ffn(oracle_mod, cf):
    spec = tiny(T=48, E=4, k=2, cf=cf, identical_experts=True)
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    dense = bf.dense_ffn(spec, inp, 0)
    kept_w = np.where(o["pos"] >= 0, o["topk_w"], 0.0).sum(axis=1)
    np.testing.assert_allclose(o["out"], kept_w[:, None] * dense, rtol=RT, atol=1e-11)
    if cf == 0.0:
        np.testing.assert_allclose(o["out"], dense, rtol=RT, atol=1e-11)
    else:
        assert (o["pos"] < 0).any()


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_single_expert_is_dense_ffn(oracle_mod, act):
    spec = tiny(T=33, E=1, k=1, act=act)
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    assert np.all(o["topk_w"] == 1.0)
    np.testing.assert_allclose(o["out"], bf.dense_ffn(spec, inp, 0), rtol=RT, atol=1e-11)
    assert math.isclose(o["aux"], 1.0, rel_tol=1e-14)
    np.testing.assert_allclose(o["lse"], o["logits"][:, 0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_scalar_expert_activation_values(oracle_mod, act):
    """H = F = 1, one expert with unit weights and zero biases: the output is the
    activation itself.  GELU(a) = a * Phi(a) and SiLU(a) = a / (1 + e^-a) at
    points where both are known in closed form or from the normal table."""
    a = np.array([0.0, 1.0, -2.0, 3.0], np.float32)
    spec = tiny(T=4, H=1, E=1, k=1, F=1, biases=False, act=act)
    one = np.ones((1, 1, 1), np.float32)
    inp = dict(x=a[:, None].copy(), Wg=np.ones((1, 1), np.float32), bg=None,
               W1=one, b1=None, W2=one.copy(), b2=None)
    o = run_oracle(oracle_mod, spec, inp)
    if act == "silu":
        want = [0.0, 1.0 / (1.0 + math.exp(-1.0)), -2.0 / (1.0 + math.exp(2.0)),
                3.0 / (1.0 + math.exp(-3.0))]
    else:   # Phi(1) = 0.841344746..., Phi(-2) = 0.022750131..., Phi(3) = 0.998650101...
        want = [0.0, 0.8413447460685429, -2.0 * 0.022750131948179195,
                3.0 * 0.9986501019683699]
    np.testing.assert_allclose(o["out"][:, 0], want, rtol=1e-14, atol=1e-15)


def test_k_equals_E_is_soft_mixture(oracle_mod):
    spec = tiny(T=20, E=4, k=4)
    inp = W.generate(spec, workers=1)
    o = run_oracle(oracle_mod, spec, inp)
    mix = sum(o["probs"][:, e:e + 1] * bf.dense_ffn(spec, inp, e) for e in range(4))
    np.testing.assert_allclose(o["out"], mix, rtol=RT, atol=1e-11)
    assert math.isclose(o["aux"], 1.0, rel_tol=1e-13)


def test_top_k_tie_rule(oracle_mod):
    spec = tiny(T=3, E=4, k=2)
    lg = np.array([[1.0, 2.0, 2.0, 0.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 3.0, 3.0]])
    r = oracle_mod.route(spec, lg)
    assert r["topk_idx"].tolist() == [[1, 2], [0, 1], [2, 3]]
    np.testing.assert_allclose(r["topk_w"], 0.5, atol=1e-15)


@pytest.mark.parametrize("T,k,E,cf,cap", [
    (8192, 2, 8, 1.25, 2560), (8192, 1, 128, 1.25, 80), (16384, 2, 8, 2.0, 8192),
    (16384, 2, 64, 0.0, 16384), (256, 2, 8, 0.5, 32), (10, 1, 3, 1.0, 4), (8192, 2, 8, 1.0, 2048)])
def test_capacity_values(oracle_mod, T, k, E, cf, cap):
    spec = tiny(T=T, k=k, E=E, cf=cf)
    assert oracle_mod.capacity(spec) == cap


# ---------------------------------------------------------------- invariants
def check_dispatch_invariants(spec, o):
    T, E, k = spec.T, spec.E, spec.k
    idx, pos, off, rt = o["topk_idx"], o["pos"], o["offsets"], o["row_token"]
    cap = o["cap"]
    np.testing.assert_allclose(o["topk_w"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert o["counts"].sum() == T * k
    for t in range(T):
        assert len(set(idx[t].tolist())) == k
    kept = np.diff(off)
    assert np.all(kept >= 0) and np.all(kept <= cap)
    assert np.all(kept == np.minimum(o["counts"], cap))
    A = int(off[-1])
    kp = pos[pos >= 0]
    assert kp.size == A and np.array_equal(np.sort(kp), np.arange(A))
    for t in range(T):
        for s in range(k):
            r = pos[t, s]
            if r >= 0:
                assert rt[r] == t
                assert off[idx[t, s]] <= r < off[idx[t, s] + 1]
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.all(rt[A:] == -1)


def test_dispatch_invariants_tiny(oracle_mod):
    spec = W.CONFIGS["c1"].replace(cf=0.5)
    inp = W.generate(spec)
    o = run_oracle(oracle_mod, spec, inp)
    assert o["cap"] == 32 and (o["pos"] < 0).any()
    check_dispatch_invariants(spec, o)


@pytest.mark.slow
def test_dispatch_invariants_ds_shaped_routing(oracle_mod):
    """Routing and dispatch of the T=8192, H=1024, E=8 layer at capacity
    factor 1.0 (forcing drops); the FFN is not evaluated here."""
    spec = W.CONFIGS["c2"].replace(cf=1.0)
    inp = W.generate(spec, with_weights=False)
    lg = oracle_mod.logits(spec, inp["x"], inp["Wg"], inp["bg"])
    o = oracle_mod.route(spec, lg)
    o.update(oracle_mod.dispatch(spec, o["topk_idx"]))
    o["cap"] = oracle_mod.capacity(spec)
    assert o["cap"] == 2048
    check_dispatch_invariants(spec, o)


# ---------------------------------------------------------------- expert choice
EC_CASES = [
    dict(T=24, E=4, k=1, group=24),
    dict(T=24, E=4, k=2, group=8),
    dict(T=30, E=3, k=1, cf=1.5, group=10),
    dict(T=16, E=8, k=2, cf=0.25, group=16, dtype="bf16"),
    dict(T=20, E=5, k=3, group=5, act="silu"),
    dict(T=12, E=2, k=1, cf=4.0, group=6, biases=False),   # C = group: every token
]


def _ec(case):
    case = dict(case)
    group = case.pop("group")
    return tiny(**case), group


@pytest.mark.parametrize("case", EC_CASES, ids=[str(c) for c in EC_CASES])
def test_expert_choice_matches_sorting_and_dense_experts(oracle_mod, case):
    spec, group = _ec(case)
    inp = W.generate(spec, workers=1)
    o = oracle_mod.ec_forward(spec, inp, group)
    C = o["C"]
    b = bf.expert_choice_dense(spec, inp, group, C)
    np.testing.assert_allclose(o["logits"], b["logits"], rtol=RT, atol=AT)
    assert np.array_equal(o["sel"], b["sets"])
    assert np.array_equal(o["rowof"] >= 0, b["mask"])
    np.testing.assert_allclose(o["probs"], b["probs"], rtol=RT, atol=AT)
    np.testing.assert_allclose(o["out"], b["out"], rtol=RT, atol=1e-11)


@pytest.mark.parametrize("case", EC_CASES[:5], ids=[str(c) for c in EC_CASES[:5]])
def test_expert_choice_matches_torch_topk_snippet(oracle_mod, case):
    spec, group = _ec(case)
    inp = W.generate(spec, workers=1)
    lg = oracle_mod.logits(spec, inp["x"], inp["Wg"], inp["bg"])
    r = oracle_mod.expert_choice(spec, lg, group)
    assert np.array_equal(r["sel"], bf.torch_expert_choice_sets(lg, group, r["C"]))


def test_expert_choice_structure(oracle_mod):
    spec, group = _ec(dict(T=48, E=6, k=2, cf=1.25, group=12))
    inp = W.generate(spec, workers=1)
    lg = oracle_mod.logits(spec, inp["x"], inp["Wg"], inp["bg"])
    r = oracle_mod.expert_choice(spec, lg, group)
    E, T, C, ng = spec.E, spec.T, r["C"], spec.T // group
    assert C == math.ceil(1.25 * group * 2 / E) == 5
    # perfect balance: every expert holds exactly ng * C rows
    assert np.array_equal(np.diff(r["offsets"]), np.full(E, ng * C))
    rows = r["rowof"][r["rowof"] >= 0]
    assert np.array_equal(np.sort(rows), np.arange(E * ng * C))     # a bijection onto the rows
    for e in range(E):
        for g in range(ng):
            take = r["sel"][e, g]
            assert np.all(np.diff(take) > 0) and np.all(take // group == g)
            for j, t in enumerate(take):
                assert r["rowof"][t, e] == (e * ng + g) * C + j
            rest = np.setdiff1d(np.arange(g * group, (g + 1) * group), take)
            assert lg[take, e].min() > lg[rest, e].max()              # no ties in this draw
    np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_expert_choice_ties_take_lower_tokens(oracle_mod):
    """All-zero gate: every logit ties, so each expert takes the first C
    tokens of every group; with identical experts the output is the dense FFN
    on those tokens (weight E * 1/E) and zero elsewhere."""
    spec = W.zero_gate(tiny(T=20, E=4, k=1, identical_experts=True))
    group = 10
    inp = W.generate(spec, workers=1)
    o = oracle_mod.ec_forward(spec, inp, group)
    C = o["C"]
    assert C == math.ceil(10 * 1 / 4) == 3
    for e in range(spec.E):
        for g in range(2):
            assert o["sel"][e, g].tolist() == list(range(g * group, g * group + C))
    dense = bf.dense_ffn(spec, inp, 0)
    first = np.array([t % group < C for t in range(spec.T)])
    np.testing.assert_allclose(o["out"][first], dense[first], rtol=RT, atol=1e-11)
    assert np.all(o["out"][~first] == 0.0)


def test_expert_choice_full_capacity_is_soft_mixture(oracle_mod):
    """C = group: every expert takes every token, so the layer is the soft
    mixture sum_e p_e FFN_e(x), with no renormalisation."""
    spec = tiny(T=18, E=3, k=1, cf=3.0)
    o = oracle_mod.ec_forward(spec, W.generate(spec, workers=1), 6)
    assert o["C"] == 6
    inp = W.generate(spec, workers=1)
    mix = sum(o["probs"][:, e:e + 1] * bf.dense_ffn(spec, inp, e) for e in range(3))
    np.testing.assert_allclose(o["out"], mix, rtol=RT, atol=1e-11)


@pytest.mark.parametrize("group,k,E,cf,C", [(2048, 2, 8, 0.0, 512), (2048, 2, 8, 1.25, 640),
                                            (16384, 1, 128, 1.0, 128), (7, 1, 8, 0.0, 1),
                                            (10, 8, 8, 2.0, 10), (100, 3, 7, 1.0, 43)])
def test_expert_choice_capacity_values(oracle_mod, group, k, E, cf, C):
    spec = tiny(T=group, E=E, k=k, cf=cf)
    assert oracle_mod.ec_capacity(spec, group) == C


# ---------------------------------------------------------------- backward
BWD_CASES = [
    dict(g_aux=0.3, g_z=0.1),
    dict(g_aux=0.0, g_z=0.0, act="silu"),
    dict(k=1, g_aux=1.0, g_z=0.5),
    dict(k=3, E=5, T=20, g_aux=0.01, g_z=0.001, biases=False),
    dict(dtype="bf16", E=8, T=40, g_aux=0.2, g_z=0.2),
    dict(E=1, k=1, T=10, g_aux=0.5, g_z=0.5),
]


def _bwd(case):
    case = dict(case)
    ga, gz = case.pop("g_aux"), case.pop("g_z")
    spec = tiny(**case)
    inp = W.generate(spec, workers=1)
    dout = W.synthetic_rows(spec, spec.T, tid=91)
    return spec, inp, dout, ga, gz


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_backward_matches_torch_autograd(oracle_mod, case):
    """No capacity limit: the oracle's chain rule against torch autograd through
    the page's layer (topk, renormalisation, dense experts, aux and z losses)."""
    spec, inp, dout, ga, gz = _bwd(case)
    g = oracle_mod.backward(spec, inp, dout, ga, gz)
    t = bf.torch_layer_grads(spec, inp, dout, ga, gz)
    for name, ref in t.items():
        if ref is None:
            continue
        np.testing.assert_allclose(g[name], ref, rtol=1e-10, atol=1e-12, err_msg=name)


def _f64_inputs(spec, inp):
    return {k: None if v is None else W.to_f32(v, spec.dtype).astype(np.float64)
            for k, v in inp.items()}


def _objective(om, spec, inp, dout, ga, gz):
    o = om.forward(spec, inp)
    return float(np.sum(dout * o["out"])) + ga * o["aux"] + gz * o["z"]


@pytest.mark.parametrize("cf,act", [(0.5, "gelu"), (0.75, "silu"), (0.0, "gelu")])
def test_backward_directional_finite_differences(oracle_mod, cf, act):
    """fp64 storage, capacity drops included: for a random direction v of each
    input, (L(u + e v) - L(u - e v)) / 2e equals <dL/du, v> (routing and drops
    do not change within +-e for these inputs)."""
    spec32 = tiny(T=32, E=4, k=2, cf=cf, act=act)
    inp = _f64_inputs(spec32, W.generate(spec32, workers=1))
    spec = spec32.replace(dtype="f64")
    dout = W.to_f32(W.synthetic_rows(spec32, spec32.T, tid=92), "f32").astype(np.float64)
    ga, gz = 0.3, 0.2
    if cf > 0:
        o = oracle_mod.forward(spec, inp)
        assert (o["pos"] < 0).any(), "no slot dropped: the case does not exercise drops"
    g = oracle_mod.backward(spec, inp, dout, ga, gz)
    rng = np.random.default_rng(5)
    eps = 1e-6
    for name, grad in (("x", "dx"), ("Wg", "dWg"), ("bg", "dbg"), ("W1", "dW1"), ("b1", "db1"),
                       ("W2", "dW2"), ("b2", "db2")):
        v = rng.standard_normal(inp[name].shape)
        hi, lo = dict(inp), dict(inp)
        hi[name] = inp[name] + eps * v
        lo[name] = inp[name] - eps * v
        fd = (_objective(oracle_mod, spec, hi, dout, ga, gz) -
              _objective(oracle_mod, spec, lo, dout, ga, gz)) / (2 * eps)
        an = float(np.sum(g[grad] * v))
        assert math.isclose(fd, an, rel_tol=1e-6, abs_tol=1e-8), (name, fd, an)


def test_backward_dropped_slots_pass_no_expert_gradient(oracle_mod):
    """Heavy drops (cf = 0.25): an expert's weight gradients only see its kept
    rows, so a dout that is zero on every token keeping a slot of expert e
    leaves dW1[e], dW2[e] and the biases of e exactly zero."""
    spec = tiny(T=40, E=4, k=2, cf=0.25)
    inp = W.generate(spec, workers=1)
    o = oracle_mod.forward(spec, inp)
    e = 2
    keep_e = np.any((o["topk_idx"] == e) & (o["pos"] >= 0), axis=1)
    dout = W.synthetic_rows(spec, spec.T, tid=93)
    dout[keep_e] = 0
    g = oracle_mod.backward(spec, inp, dout, 0.0, 0.0)
    for n in ("dW1", "db1", "dW2", "db2"):
        assert np.all(g[n][e] == 0.0), n
    assert np.any(g["dW1"][(e + 1) % 4] != 0.0)


def test_backward_tokens_and_weight_entries_match_full(oracle_mod):
    spec = tiny(T=30, E=5, k=2, cf=0.75, dtype="bf16")
    inp = W.generate(spec, workers=1)
    dout = W.synthetic_rows(spec, spec.T, tid=94)
    g = oracle_mod.backward(spec, inp, dout, 0.2, 0.05)
    toks = [0, 7, 13, 29]
    dx = oracle_mod.backward_tokens(spec, inp, dout, toks, 0.2, 0.05)
    np.testing.assert_allclose(dx, g["dx"][toks], rtol=1e-12, atol=1e-14)
    ent = [(1, 0, 3, 7), (1, 4, 15, 39), (2, 2, 11, 5), (2, 3, 0, 15), (3, 1, 0, 20),
           (4, 4, 0, 9)]
    v = oracle_mod.backward_weight_entries(spec, inp, dout, ent)
    ref = [g["dW1"][0, 3, 7], g["dW1"][4, 15, 39], g["dW2"][2, 11, 5], g["dW2"][3, 0, 15],
           g["db1"][1, 20], g["db2"][4, 9]]
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("case", [dict(T=30, E=5, k=2, cf=0.75, dtype="bf16"),
                                  dict(T=24, E=4, k=1, cf=0.0, act="silu"),
                                  dict(T=40, E=8, k=3, cf=0.5, dtype="bf16", biases=False)],
                         ids=["bf16_drops", "silu_k1", "k3_heavy_drops"])
def test_backward_gate_matches_full(oracle_mod, case):
    """The gate-only gradients (used where the full backward is too large)
    equal the full backward's dWg and dbg bit for bit: the same terms in the
    same order, on the oracle's own and on given logits."""
    spec = tiny(**case)
    inp = W.generate(spec, workers=1)
    dout = W.synthetic_rows(spec, spec.T, tid=99)
    g = oracle_mod.backward(spec, inp, dout, 0.2, 0.05)
    dWg, dbg = oracle_mod.backward_gate(spec, inp, dout, 0.2, 0.05)
    assert np.array_equal(dWg, g["dWg"]) and np.array_equal(dbg, g["dbg"])
    lg = oracle_mod.logits(spec, inp["x"], inp["Wg"], inp["bg"]) * 1.5
    g = oracle_mod.backward(spec, inp, dout, 0.1, 0.3, given_logits=lg)
    dWg, dbg = oracle_mod.backward_gate(spec, inp, dout, 0.1, 0.3, given_logits=lg)
    assert np.array_equal(dWg, g["dWg"]) and np.array_equal(dbg, g["dbg"])
