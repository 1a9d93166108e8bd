"""moe_forward captured into a HIP graph (torch.cuda.CUDAGraph on the capture
stream) and replayed: the library issues only kernel launches on the caller's
stream (no memset, copy, allocation or host synchronisation), so a decode
loop can replay one forward without per-launch host overhead.

Each case captures one forward, then three times: new inputs are written
eagerly into the captured input buffers, an eager forward runs into separate
outputs, the graph is replayed, and every output of the replay must equal the
eager one bit for bit (same kernels, same inputs).  The eager result is also
checked against the oracle once, so a replay that matched a wrong eager run
would still fail.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as om
import sparse_mixture_experts_21_amd as moe
import workloads as W
from gpu_util import (DEV, alloc_forward, as_f64, assert_close_storage,
                      check_discrete_from_gpu_logits, say, upload, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    om.lib()


CASES = [
    # one-launch routing of a tiny batch, narrow GEMM layouts cut along K
    W.Spec("graph_T2_H512_E8_k2_F1024", T=2, H=512, E=8, k=2, F=1024, dtype="bf16", cf=0.0,
           seed=41),
    # router + dispatch kernels, 256-row tiles, a ragged last round, drops, biases
    W.Spec("graph_T1000_H256_E8_k2_F768_cf1.0", T=1000, H=256, E=8, k=2, F=768, dtype="bf16",
           cf=1.0, seed=42, bg=W.Dist("uniform", 0.05), b1=W.Dist("uniform", 0.05),
           b2=W.Dist("uniform", 0.05)),
]

KEYS = ("out", "losses", "logits", "topk_idx", "topk_w", "counts", "offsets", "pos")


def _forward(prob, d, o, ws):
    moe.moe_forward(prob, d["x"], d["Wg"], d.get("bg"), d["W1"], d.get("b1"), d["W2"],
                    d.get("b2"), o["out"], o["losses"], ws,
                    **{k: o[k] for k in KEYS if k not in ("out", "losses")})


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_forward_graph_replay_equals_eager(spec):
    say(f"[graph replay] {spec.name}")
    inp = W.generate(spec)
    d = upload(spec, inp)
    prob = moe.Problem.from_spec(spec)
    ws = workspace(prob)
    og, oe = alloc_forward(spec), alloc_forward(spec)
    # warm up on a side stream, then capture one forward
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _forward(prob, d, og, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _forward(prob, d, og, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for rnd in range(3):
        # new tokens, written eagerly into the captured input buffer
        xs = (rng.standard_normal((spec.T, spec.H)) * 0.5).astype(np.float32)
        d["x"].copy_(torch.from_numpy(xs).to(DEV).to(d["x"].dtype))
        torch.cuda.synchronize()
        _forward(prob, d, oe, ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(_bits(og[key]), _bits(oe[key])), f"replay {rnd}: {key}"
        if rnd == 0:
            # the eager run itself against the oracle (on the GPU's logits)
            xin = d["x"].view(torch.int16).cpu().numpy().view(np.uint16)
            r = check_discrete_from_gpu_logits(om, spec, oe)
            ref = om.forward_tokens(spec, xin, r["topk_idx"], r["topk_w"], r["pos"], inp["W1"],
                                    inp.get("b1"), inp["W2"], inp.get("b2"), np.arange(spec.T))
            assert_close_storage(as_f64(oe["out"]), ref, spec.dtype, "eager out")
