"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* Stage isolation: each stage is fed the oracle's inputs for that stage.
* End to end: moe_forward on small configurations and on the five full-size
  workloads in the launch configuration the benchmark uses; routing, dispatch
  and the layer output of every token are compared.
* Routing decisions are taken in fp32 on the GPU; the exact check applies the
  oracle's discrete steps to the GPU's own fp32 logits (both sides decide on
  the same values).  Against the oracle's independent fp64 logits the indices
  must also agree whenever the smallest k-th/(k+1)-th logit gap is >= 1e-5.
"""
import math
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as om
import sparse_mixture_experts_21_amd as moe
import workloads as W
from gpu_util import (DEV, alloc_forward, as_f64, assert_close_storage, assert_losses,
                      check_discrete_from_gpu_logits, dev, host_storage, logits_tol,
                      run_forward, run_stages, say, storage_dtype, upload, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    om.lib()


def S(name, T, H, E, k, F, dtype="bf16", cf=0.0, seed=11, biases=False, **kw):
    s = W.Spec(name, T=T, H=H, E=E, k=k, F=F, dtype=dtype, cf=cf, seed=seed)
    if dtype == "f32":
        s = s.replace(wg=W.Dist("uniform", 1 / math.sqrt(H)), w1=W.Dist("uniform", 1 / math.sqrt(H)),
                      w2=W.Dist("uniform", 1 / math.sqrt(F)))
    if biases:
        s = s.replace(bg=W.Dist("uniform", 0.05), b1=W.Dist("uniform", 0.05),
                      b2=W.Dist("uniform", 0.05))
    return s.replace(**kw) if kw else s


SMALL = [
    W.CONFIGS["c1"],
    W.CONFIGS["c1"].replace(name="c1_cf0.5_heavy_drops", cf=0.5),
    W.CONFIGS["c1"].replace(name="c1_T257", T=257),
    S("bf16_T2048_H512_E8_k2_F2048_cf1.25", 2048, 512, 8, 2, 2048, cf=1.25),
    S("bf16_T512_H256_E8_k2_F768_bm128", 512, 256, 8, 2, 768, cf=1.0, biases=True),
    S("bf16_ragged_T777_H264_E6_k2_F776_cf1.0", 777, 264, 6, 2, 776, cf=1.0, biases=True),
    S("bf16_T1024_H256_E128_k1_F512_cf1.25", 1024, 256, 128, 1, 512, cf=1.25,
      wg=W.Dist("normal", 0.1)),
    S("bf16_zipf_T2048_H256_E64_k2_F1024", 2048, 256, 64, 2, 1024, bg=W.Dist("zipf_log", 1.2)),
    W.zero_gate(S("bf16_zero_gate_T300_H128_E8_k2_F256_cf0.5", 300, 128, 8, 2, 256, cf=0.5)),
    S("bf16_k8_E8_dropless_T200_H128_F256", 200, 128, 8, 8, 256),
    S("bf16_E1_k1_T100_H64_F128", 100, 64, 1, 1, 128, biases=True),
    S("bf16_T1_H64_E4_k2_F128", 1, 64, 4, 2, 128, biases=True),
    S("bf16_T257_H64_E8_k2_F256", 257, 64, 8, 2, 256, cf=1.25),
    S("bf16_tiny_cf_T256_H64_E8_k2_F128_cf0.1", 256, 64, 8, 2, 128, cf=0.1),
    S("f32_k3_E5_T100_H32_F64", 100, 32, 5, 3, 64, dtype="f32", cf=0.75, biases=True),
    # SiLU experts (the Mixtral 8x7B block: no biases, no capacity), then with
    # biases, drops and a ragged width, and in fp32
    S("silu_bf16_T2048_H512_E8_k2_F2048_dropless", 2048, 512, 8, 2, 2048, act="silu"),
    S("silu_bf16_ragged_T777_H264_E6_k2_F776_cf1.0", 777, 264, 6, 2, 776, cf=1.0,
      biases=True, act="silu"),
    S("silu_f32_k2_E4_T100_H32_F64", 100, 32, 4, 2, 64, dtype="f32", biases=True, act="silu"),
]
SILU = [s for s in SMALL if s.act == "silu"]
# Tiny batches (T * E <= 64, bf16): moe_forward routes and dispatches them in
# one workgroup.  Several LDS blocks of H, a ragged H, a tail block, k = E,
# E = 1, k = 8 with heavy drops, tied logits, biases, SiLU.
TINY = [
    S("tiny_T1_H4096_E8_k2_F512", 1, 4096, 8, 2, 512),
    S("tiny_T8_H264_E8_k2_F256_cf0.5", 8, 264, 8, 2, 256, cf=0.5, biases=True),
    S("tiny_T5_H1032_E4_k4_F128", 5, 1032, 4, 4, 128, biases=True),
    S("tiny_T64_H128_E1_k1_F64", 64, 128, 1, 1, 64),
    S("tiny_T4_H256_E16_k8_F128_cf0.25", 4, 256, 16, 8, 128, cf=0.25, wg=W.Dist("normal", 0.1)),
    W.zero_gate(S("tiny_zero_gate_T3_H128_E8_k2_F64_cf0.5", 3, 128, 8, 2, 64, cf=0.5)),
    S("tiny_silu_T2_H512_E8_k2_F256", 2, 512, 8, 2, 256, act="silu"),
]
# Decode-sized batches (T <= 8): every GEMM tile holds a few real rows and is
# cut along K.  A ragged K and N (partial k-tile and column tile), more than
# 64 experts with a few active, every expert holding every token, one expert,
# and a long K (down GEMM with F = 8200).
FEW = [
    S("few_T1_H512_E8_k2_F2048", 1, 512, 8, 2, 2048, biases=True),
    S("few_T3_H264_E6_k2_F776", 3, 264, 6, 2, 776, biases=True),
    S("few_T8_H256_E128_k8_F512_cf0.5", 8, 256, 128, 8, 512, cf=0.5, wg=W.Dist("normal", 0.1)),
    S("few_silu_T7_H1032_E4_k4_F136", 7, 1032, 4, 4, 136, act="silu"),
    S("few_T2_H128_E1_k1_F64", 2, 128, 1, 1, 64, biases=True),
    S("few_T8_H128_E2_k1_F8200", 8, 128, 2, 1, 8200, biases=True),
]


# Thousands of tokens through the narrow-gate router: a ragged H (the second
# 256-wide stage half empty) and T (a last block of 8 tokens) with 16-bit gate
# reads (E % 4 != 0), and E = 16 with k = 4.
RES = [
    S("router_T8200_H264_E6_k2_F128", 8200, 264, 6, 2, 128, biases=True),
    S("router_T8192_H1024_E16_k4_F128_cf1.0", 8192, 1024, 16, 4, 128, cf=1.0,
      wg=W.Dist("normal", 0.05)),
]


# Every router shape by gate width: E in 17..32 with 16-bit gate reads
# (E % 4 != 0) and with transposing reads, E not a multiple of 16 above 128,
# and the widest gate (E = 256, k = 8) with drops.
WIDE = [
    S("wide_E17_T500_H136_k2_F64", 500, 136, 17, 2, 64, biases=True),
    S("wide_E24_T700_H264_k3_F136_cf1.0", 700, 264, 24, 3, 136, cf=1.0),
    S("wide_E200_T129_H512_k2_F64", 129, 512, 200, 2, 64, wg=W.Dist("normal", 0.1)),
    S("wide_E256_T300_H128_k8_F128_cf1.0", 300, 128, 256, 8, 128, cf=1.0, biases=True),
]


def _small_ids():
    return [s.name for s in SMALL + TINY + FEW + RES + WIDE]


# ---------------------------------------------------------------- end to end (small)
@pytest.mark.parametrize("spec", SMALL + TINY + FEW + RES + WIDE, ids=_small_ids())
def test_forward_small_all_outputs(spec):
    say(f"[forward small] {spec.name}")
    inp = W.generate(spec)
    d = upload(spec, inp)
    o = run_forward(spec, d)
    lg = as_f64(o["logits"])
    ref_lg = om.logits(spec, inp["x"], inp["Wg"], inp["bg"])
    assert np.max(np.abs(lg - ref_lg)) <= logits_tol(spec)
    r = check_discrete_from_gpu_logits(om, spec, o)
    margin = om.topk_margin(spec, ref_lg)
    if margin >= 1e-5:
        ind = om.route(spec, ref_lg)
        assert np.array_equal(o["topk_idx"].cpu().numpy(), ind["topk_idx"])
        assert_losses(o["losses"].cpu().numpy(), ind["aux"], ind["z"], "losses vs oracle")
    say(f"    top-k margin {margin:.3e}, kept rows {int(r['offsets'][-1])} of {spec.T * spec.k}")
    out_ref = om.forward_tokens(spec, inp["x"], r["topk_idx"], r["topk_w"], r["pos"], inp["W1"],
                                inp.get("b1"), inp["W2"], inp.get("b2"), np.arange(spec.T))
    assert_close_storage(as_f64(o["out"]), out_ref, spec.dtype, "out")
    dropped = np.all(r["pos"] < 0, axis=1)
    if dropped.any():
        assert np.all(as_f64(o["out"])[dropped] == 0.0)


# The second GEMM's last round cut along K with whole tiles before it (more
# than one round of 256 tiles), biases and ragged experts: moe_forward finishes
# the cut tiles inside the combine, the stages through the GEMM's own fixup.
# On 256 CUs the first cuts 16 of 272 tiles into 8 slices (4 column tiles, the
# narrow super-blocks), the second 40 of 296 into 4 (8 column tiles, the
# remaining row tiles after one super-block row).
CUT = [
    S("cut_T8192_H1024_E8_k2_F1024_cf1.25", 8192, 1024, 8, 2, 1024, cf=1.25, biases=True),
    S("cut_T4096_H2048_E8_k2_F512", 4096, 2048, 8, 2, 512, biases=True,
      bg=W.Dist("zipf_log", 1.2)),
    # 16-wide super-blocks (80 of 336 tiles cut into 3); a column count no
    # super-block width divides (5: the plain order, 120 tiles in 2); the
    # 128-row layout (128 of 384 in 2) and the 64-row layout (128 of 384 in 2)
    S("cut_T2048_H4096_E8_k2_F512", 2048, 4096, 8, 2, 512, biases=True),
    S("cut_T2500_H1280_E8_k2_F512", 2500, 1280, 8, 2, 512, biases=True),
    S("cut_T1500_H3072_E32_k2_F256", 1500, 3072, 32, 2, 256, wg=W.Dist("normal", 0.1)),
    S("cut_T800_H1536_E64_k2_F512", 800, 1536, 64, 2, 512, biases=True,
      wg=W.Dist("normal", 0.1)),
]


@pytest.mark.parametrize("spec", CUT, ids=lambda s: s.name)
def test_forward_cut_all_outputs(spec):
    """The shapes above end to end against the oracle at every token."""
    test_forward_small_all_outputs(spec)


@pytest.mark.parametrize("spec", SMALL[:8] + SILU[:2] + TINY[:3] + FEW[:3] + RES[:1] + WIDE[1:2]
                         + [SMALL[9]] + CUT, ids=lambda s: s.name)
def test_stages_equal_forward_bitwise(spec):
    say(f"[stages == forward] {spec.name}")
    inp = W.generate(spec)
    d = upload(spec, inp)
    f = run_forward(spec, d)
    s = run_stages(spec, d)
    for key in ("out", "losses", "logits", "topk_idx", "topk_w", "counts", "offsets", "pos"):
        assert torch.equal(f[key].view(torch.uint8) if f[key].dtype == torch.bfloat16 else f[key],
                           s[key].view(torch.uint8) if s[key].dtype == torch.bfloat16 else s[key]), key
    A = int(s["offsets"][-1])
    rt = s["row_token"][:A].long()
    xp, ref = s["xp"][:A], d["x"][rt]
    if spec.dtype == "bf16":
        xp, ref = xp.view(torch.int16), ref.view(torch.int16)
    assert torch.equal(xp, ref)


@pytest.mark.parametrize("spec", [SMALL[3], SMALL[5], SMALL[7], TINY[1]], ids=lambda s: s.name)
def test_forward_deterministic(spec):
    say(f"[determinism] {spec.name}")
    inp = W.generate(spec)
    d = upload(spec, inp)
    a = run_forward(spec, d)
    b = run_forward(spec, d)
    for key in a:
        x, y = a[key], b[key]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), key


def test_forward_without_optional_outputs():
    spec = SMALL[3]
    say(f"[optional outputs NULL] {spec.name}")
    inp = W.generate(spec)
    d = upload(spec, inp)
    a = run_forward(spec, d)
    b = run_forward(spec, d, with_optional=False)
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    assert torch.equal(a["losses"], b["losses"])


# ---------------------------------------------------------------- stage isolation
@pytest.mark.parametrize("spec", [SMALL[0], SMALL[3], SMALL[6], SMALL[8]], ids=lambda s: s.name)
def test_route_stage_logits_in(spec):
    """moe_route fed the oracle's logits (rounded to fp32) reproduces the oracle's
    discrete routing on those values exactly."""
    say(f"[route LOGITS_IN] {spec.name}")
    inp = W.generate(spec, with_weights=False)
    lg32 = om.logits(spec, inp["x"], inp["Wg"], inp["bg"]).astype(np.float32)
    ref = om.route(spec, lg32.astype(np.float64))
    prob = moe.Problem.from_spec(spec)
    ws = workspace(prob)
    o = alloc_forward(spec)
    lgd = dev(lg32, "f32")
    moe.moe_route(prob, None, None, None, lgd, o["topk_idx"], o["topk_w"], o["counts"],
                  o["losses"], ws, flags=moe.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    assert np.array_equal(o["topk_idx"].cpu().numpy(), ref["topk_idx"])
    assert np.array_equal(o["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_allclose(o["topk_w"].cpu().numpy(), ref["topk_w"], rtol=0, atol=1e-5)
    assert_losses(o["losses"].cpu().numpy(), ref["aux"], ref["z"], "losses")
    np.testing.assert_allclose(o["topk_w"].cpu().numpy().sum(axis=1), 1.0, atol=1e-6)


@pytest.mark.parametrize("spec", [SMALL[1], SMALL[3], SMALL[5], SMALL[6], SMALL[7], SMALL[8]],
                         ids=lambda s: s.name)
def test_permute_stage(spec):
    say(f"[permute] {spec.name}")
    inp = W.generate(spec, with_weights=False)
    ref = om.route(spec, om.logits(spec, inp["x"], inp["Wg"], inp["bg"]))
    dsp = om.dispatch(spec, ref["topk_idx"])
    prob = moe.Problem.from_spec(spec)
    ws = workspace(prob)
    T, k, H = spec.T, spec.k, spec.H
    x = dev(inp["x"], spec.dtype)
    idx = dev(ref["topk_idx"], "i32")
    off = torch.empty(spec.E + 1, dtype=torch.int32, device=DEV)
    pos = torch.empty(T, k, dtype=torch.int32, device=DEV)
    rt = torch.empty(T * k, dtype=torch.int32, device=DEV)
    xp = torch.empty(T * k, H, dtype=storage_dtype(spec), device=DEV)
    moe.moe_permute(prob, x, idx, off, pos, rt, xp, ws)
    torch.cuda.synchronize()
    A = int(dsp["offsets"][-1])
    assert np.array_equal(off.cpu().numpy(), dsp["offsets"])
    assert np.array_equal(pos.cpu().numpy(), dsp["pos"])
    assert np.array_equal(rt.cpu().numpy()[:A], dsp["row_token"][:A])
    xs = host_storage(xp[:A], spec.dtype)
    assert np.array_equal(xs, inp["x"][dsp["row_token"][:A]])


@pytest.mark.parametrize("spec", [SMALL[0], SMALL[3], SMALL[4], SMALL[5], SMALL[6], SMALL[7]]
                         + SILU + FEW, ids=lambda s: s.name)
def test_expert_ffn_stage(spec):
    say(f"[expert_ffn] {spec.name}")
    inp = W.generate(spec)
    ref = om.route(spec, om.logits(spec, inp["x"], inp["Wg"], inp["bg"]))
    dsp = om.dispatch(spec, ref["topk_idx"])
    A = int(dsp["offsets"][-1])
    rows = inp["x"][dsp["row_token"][:A]]
    experts = np.repeat(np.arange(spec.E), np.diff(dsp["offsets"]))
    h_ref, y_ref = om.expert_rows(spec, rows, experts, inp["W1"], inp.get("b1"), inp["W2"],
                                  inp.get("b2"))
    prob = moe.Problem.from_spec(spec)
    d = upload(spec, inp)
    T, k = spec.T, spec.k
    xp = torch.zeros(T * k, spec.H, dtype=storage_dtype(spec), device=DEV)
    xp[:A] = dev(rows, spec.dtype)
    off = dev(dsp["offsets"], "i32")
    h = torch.empty(T * k, spec.F, dtype=storage_dtype(spec), device=DEV)
    y = torch.empty(T * k, spec.H, dtype=storage_dtype(spec), device=DEV)
    moe.moe_expert_ffn(prob, xp, off, d["W1"], d.get("b1"), d["W2"], d.get("b2"), h, y)
    torch.cuda.synchronize()
    assert_close_storage(as_f64(h[:A]), h_ref, spec.dtype, "h")
    assert_close_storage(as_f64(y[:A]), y_ref, spec.dtype, "y")


def _tail_plan_host(offsets, bm, nt, ncu, nk, ns=4, max_units=256):
    """Host copy of the rule the GEMM applies on the device: the real tiles'
    ragged last round (R mod ncu tiles) is cut into S K-slices when S >= 2."""
    mt = sum((int(offsets[e + 1]) - int(offsets[e]) + bm - 1) // bm for e in range(len(offsets) - 1))
    tail = (mt * nt) % ncu
    S = min(ncu, max_units) // tail if tail else 1
    S = min(S, nk // ns)
    return (tail, S) if S >= 2 else (0, 1)


SPLIT = S("split_T4096_H512_E8_k2_F2048", 4096, 512, 8, 2, 2048)


# few rows per expert (64-row tiles): every tile of both GEMMs is cut along K
SPLIT_SMALL = S("split_small_T4_H512_E8_k2_F2048", 4, 512, 8, 2, 2048, biases=True)


@pytest.mark.parametrize("spec", [SPLIT, SPLIT.replace(act="silu", name=SPLIT.name + "_silu"),
                                  SPLIT_SMALL], ids=lambda s: s.name)
def test_expert_ffn_tail_split(spec):
    """With a workspace, the last round of tiles is cut along K (fp32 partials
    summed in slice order); the result must match the oracle like whole tiles
    do.  At the T=4096 shape the up GEMM cuts 40 of ~296 tiles and the down
    GEMM cuts all of its ~74 tiles (no whole tile at all); at T=4 every tile of
    both GEMMs is cut, with one or two real rows per tile."""
    say(f"[expert_ffn tail split] {spec.name}")
    inp = W.generate(spec)
    ref = om.route(spec, om.logits(spec, inp["x"], inp["Wg"], inp["bg"]))
    dsp = om.dispatch(spec, ref["topk_idx"])
    off_h = dsp["offsets"]
    A = int(off_h[-1])
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    avg = -(-spec.T * spec.k // spec.E)
    bm = 64 if avg <= 32 else 128 if avg <= 128 else 256
    up = _tail_plan_host(off_h, bm, (spec.F + 255) // 256, ncu, spec.H // 32)
    down = _tail_plan_host(off_h, bm, (spec.H + 255) // 256, ncu, spec.F // 32)
    say(f"    tail plan on {ncu} CUs: up {up}, down {down}")
    assert up[1] >= 2 and down[1] >= 2, "shape no longer exercises the K split"
    rows = inp["x"][dsp["row_token"][:A]]
    experts = np.repeat(np.arange(spec.E), np.diff(off_h))
    h_ref, y_ref = om.expert_rows(spec, rows, experts, inp["W1"], inp.get("b1"), inp["W2"],
                                  inp.get("b2"))
    prob = moe.Problem.from_spec(spec)
    d = upload(spec, inp)
    T, k = spec.T, spec.k
    xp = torch.zeros(T * k, spec.H, dtype=storage_dtype(spec), device=DEV)
    xp[:A] = dev(rows, spec.dtype)
    off = dev(off_h, "i32")
    outs = {}
    for tag, ws in (("split", workspace(prob)), ("whole", None)):
        h = torch.empty(T * k, spec.F, dtype=storage_dtype(spec), device=DEV)
        y = torch.empty(T * k, spec.H, dtype=storage_dtype(spec), device=DEV)
        moe.moe_expert_ffn(prob, xp, off, d["W1"], d.get("b1"), d["W2"], d.get("b2"), h, y, ws)
        torch.cuda.synchronize()
        assert_close_storage(as_f64(h[:A]), h_ref, spec.dtype, f"h ({tag})")
        assert_close_storage(as_f64(y[:A]), y_ref, spec.dtype, f"y ({tag})")
        outs[tag] = (h[:A].clone(), y[:A].clone())
    # the two differ only in fp32 summation order inside the cut tiles
    for a, b, nm in ((outs["split"][0], outs["whole"][0], "h"), (outs["split"][1], outs["whole"][1], "y")):
        diff = (a.float() - b.float()).abs()
        scale = b.float().abs().clamp_min(float(b.float().pow(2).mean().sqrt()))
        assert float((diff / scale).max()) <= 2.0 ** -6, f"{nm}: split and whole tiles disagree"


@pytest.mark.parametrize("spec", [SMALL[0], SMALL[1], SMALL[3], SMALL[8]], ids=lambda s: s.name)
def test_combine_stage(spec):
    say(f"[combine] {spec.name}")
    inp = W.generate(spec, with_weights=False)
    ref = om.route(spec, om.logits(spec, inp["x"], inp["Wg"], inp["bg"]))
    dsp = om.dispatch(spec, ref["topk_idx"])
    A = max(int(dsp["offsets"][-1]), 1)
    y = W.synthetic_rows(spec, A)
    w32 = ref["topk_w"].astype(np.float32)
    out_ref = om.combine(spec, y, dsp["pos"], w32.astype(np.float64))
    prob = moe.Problem.from_spec(spec)
    out = torch.empty(spec.T, spec.H, dtype=storage_dtype(spec), device=DEV)
    moe.moe_combine(prob, dev(y, spec.dtype), dev(dsp["pos"], "i32"), dev(w32, "f32"), out)
    torch.cuda.synchronize()
    assert_close_storage(as_f64(out), out_ref, spec.dtype, "out")


# ---------------------------------------------------------------- full size
FULL = ["c2", "c3", "c4", "c5", "c5s", "d1", "d8", "d64", "d256"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL + ["c2_cf1.0"])
def test_forward_full_size(name):
    """The full-size workloads in the benchmark's launch configuration: routing
    and dispatch exactly, and the layer output of EVERY token against the
    oracle's per-token loop (about 45 s of oracle time on 16 host threads for
    the 16384-token Mixtral-shaped layers)."""
    base = name.split("_")[0]
    spec = W.CONFIGS[base]
    if name.endswith("cf1.0"):
        spec = spec.replace(cf=1.0, name=spec.name.replace("cf1.25", "cf1.0"))
    say(f"[forward full size] {name}: {spec.name}")
    inp = W.generate(spec)
    d = upload(spec, inp)
    o = run_forward(spec, d)
    r = check_discrete_from_gpu_logits(om, spec, o)
    A = int(r["offsets"][-1])
    kept = np.diff(r["offsets"])
    cap = om.capacity(spec)
    assert np.all(kept <= cap)
    say(f"    cap {cap}, kept {A} of {spec.T * spec.k}, experts empty {int(np.sum(kept == 0))}, "
        f"max/min rows {kept.max()}/{kept.min()}")
    ref_lg = om.logits(spec, inp["x"], inp["Wg"], inp["bg"])
    lg_err = float(np.max(np.abs(as_f64(o["logits"]) - ref_lg)))
    assert lg_err <= logits_tol(spec), lg_err
    margin = om.topk_margin(spec, ref_lg)
    say(f"    logits max err {lg_err:.2e}, top-k margin {margin:.2e}")
    if margin >= 1e-5:
        ind = om.route(spec, ref_lg)
        assert np.array_equal(o["topk_idx"].cpu().numpy(), ind["topk_idx"])
        assert_losses(o["losses"].cpu().numpy(), ind["aux"], ind["z"], "losses vs oracle")
    got = as_f64(o["out"])
    del o, d
    t0 = time.perf_counter()
    out_ref = om.forward_tokens(spec, inp["x"], r["topk_idx"], r["topk_w"], r["pos"], inp["W1"],
                                inp.get("b1"), inp["W2"], inp.get("b2"), np.arange(spec.T))
    say(f"    oracle over all {spec.T} tokens: {time.perf_counter() - t0:.1f} s "
        f"on {om.num_threads()} threads")
    assert_close_storage(got, out_ref, spec.dtype, f"out[all {spec.T} tokens]")
    dropped = np.all(r["pos"] < 0, axis=1)
    if dropped.any():
        assert np.all(got[dropped] == 0.0)


@pytest.mark.timeout(600)
def test_expert_ffn_stage_ds_shape_every_row():
    """moe_expert_ffn at the DeepSpeed-script shape (T=8192, H=1024, E=8, top-2,
    F=4096, no capacity limit): 16384 rows in 64 row tiles of 256, so the up
    GEMM runs 4 chip-wide super-blocks of 256 tiles (every rotation of the
    XCD sub-blocks) and the down GEMM 256 tiles.  h and y of every row are
    compared with the oracle element by element."""
    spec = W.CONFIGS["c2"].replace(cf=0.0, name="ds_shaped_T8192_H1024_E8_k2_dropless")
    say(f"[expert_ffn every row] {spec.name}")
    inp = W.generate(spec)
    ref = om.route(spec, om.logits(spec, inp["x"], inp["Wg"], inp["bg"]))
    dsp = om.dispatch(spec, ref["topk_idx"])
    A = int(dsp["offsets"][-1])
    assert A == spec.T * spec.k
    rows = inp["x"][dsp["row_token"][:A]]
    experts = np.repeat(np.arange(spec.E), np.diff(dsp["offsets"]))
    prob = moe.Problem.from_spec(spec)
    d = upload(spec, inp)
    xp = dev(rows, spec.dtype)
    off = dev(dsp["offsets"], "i32")
    h = torch.empty(A, spec.F, dtype=storage_dtype(spec), device=DEV)
    y = torch.empty(A, spec.H, dtype=storage_dtype(spec), device=DEV)
    moe.moe_expert_ffn(prob, xp, off, d["W1"], d.get("b1"), d["W2"], d.get("b2"), h, y,
                       workspace(prob))
    torch.cuda.synchronize()
    gh, gy = as_f64(h), as_f64(y)
    del h, y, xp, d
    t0 = time.perf_counter()
    h_ref, y_ref = om.expert_rows(spec, rows, experts, inp["W1"], inp.get("b1"), inp["W2"],
                                  inp.get("b2"))
    say(f"    oracle over {A} rows: {time.perf_counter() - t0:.1f} s")
    assert_close_storage(gh, h_ref, spec.dtype, "h (every row)")
    assert_close_storage(gy, y_ref, spec.dtype, "y (every row)")
