"""moe_forward_noalloc (the forward on the library's fixed device scratch,
for callers that cannot allocate) against moe_forward with a caller-owned
workspace: two calls in a row, the second on a smaller problem, must give
bit-identical outputs (the same kernels on the same inputs), and a problem
whose workspace exceeds the fixed scratch is refused before any launch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sparse_mixture_experts_21_amd as moe
import workloads as W
from gpu_util import DEV, alloc_forward, run_forward, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _noalloc(spec, d):
    o = alloc_forward(spec)
    prob = moe.Problem.from_spec(spec)
    moe.moe_forward_noalloc(prob, d["x"], d["Wg"], d.get("bg"), d["W1"], d.get("b1"), d["W2"],
                            d.get("b2"), o["out"], o["losses"], logits=o["logits"],
                            topk_idx=o["topk_idx"], topk_w=o["topk_w"], counts=o["counts"],
                            offsets=o["offsets"], pos=o["pos"])
    torch.cuda.synchronize()
    return o


def test_noalloc_equals_forward_two_calls_shrinking():
    # the 256-token Mixtral-shaped decode batch (router, dispatch kernels,
    # K-sliced GEMM tails), then 8 tokens of it (one-launch tiny routing)
    specs = [W.CONFIGS["d256"], W.CONFIGS["d8"]]
    for spec in specs:
        prob = moe.Problem.from_spec(spec)
        need = moe.moe_workspace_bytes(prob)
        say(f"[noalloc] {spec.name}: workspace {need / 2**20:.1f} MiB of "
            f"{moe.MOE_NOALLOC_SCRATCH_BYTES / 2**20:.0f} MiB")
        assert need <= moe.MOE_NOALLOC_SCRATCH_BYTES
        inp = W.generate(spec)
        d = upload(spec, inp)
        ref = run_forward(spec, d)
        got = _noalloc(spec, d)
        for key in ref:
            assert torch.equal(_bits(got[key]), _bits(ref[key])), f"{spec.name}: {key}"


def test_noalloc_bf16_small_and_fp32():
    # a capacity-dropping bf16 layer with biases and ragged widths (128-row
    # tiles), then an fp32 one (smaller)
    specs = [W.Spec("noalloc_bf16_T300_H264_E6_k2_F776_cf1.0", T=300, H=264, E=6, k=2, F=776,
                    dtype="bf16", cf=1.0, seed=41, bg=W.Dist("uniform", 0.05),
                    b1=W.Dist("uniform", 0.05), b2=W.Dist("uniform", 0.05)),
             W.CONFIGS["c1"]]
    for spec in specs:
        say(f"[noalloc] {spec.name}")
        assert moe.moe_workspace_bytes(moe.Problem.from_spec(spec)) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        inp = W.generate(spec)
        d = upload(spec, inp)
        ref = run_forward(spec, d)
        got = _noalloc(spec, d)
        for key in ref:
            assert torch.equal(_bits(got[key]), _bits(ref[key])), f"{spec.name}: {key}"


def test_noalloc_refuses_problems_beyond_the_scratch():
    spec = W.CONFIGS["c2"]                 # 224 MiB of workspace
    prob = moe.Problem.from_spec(spec)
    assert moe.moe_workspace_bytes(prob) > moe.MOE_NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(prob, t, t, None, t, None, t, None, t,
                                torch.empty(2, dtype=torch.float32, device=DEV))
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
