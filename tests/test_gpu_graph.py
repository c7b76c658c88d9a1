"""A layer step recorded into a HIP graph (``MoELayer.capture_step``) against the same steps run eagerly.

Two layers start from the same inputs and bias. One runs four eager steps; the other runs one eager
step, is recorded, and replays the recording three times, with unrelated eager device work and a
synchronisation between the replays. Every step's output, picks, loads and updated bias must equal the
eager layer's bit for bit: the kernels are deterministic, and a replay launches exactly what the eager
step launches. Replays that went wrong after the first (stale clears, recorded host values) would show
here as a mismatch at step 3 or 4.
"""
import pytest
import torch

from moe_inputs import generate, get_config
from mixture_experts_layer_gate_amd import MoELayer

pytestmark = pytest.mark.gpu

CASES = [("c1", {}), ("c2", {}), ("c2", {"gemm": "fp8"}), ("c2", {"gemm": "mxfp4"})]


@pytest.mark.parametrize("name,over", CASES, ids=["c1_f32", "c2_bf16", "c2_fp8", "c2_mxfp4"])
def test_step_graph_replays_equal_eager_steps(name, over):
    cfg = get_config(name, **over)
    print(f"[graph] {name} {over}", flush=True)
    inp = generate(cfg, "cuda")
    u = inp["u"]
    eager = MoELayer(cfg, inp, "cuda", keep_scores=False)
    graphed = MoELayer(cfg, inp, "cuda", keep_scores=False)

    def state(layer):
        return (layer.out.clone(), layer.topk_idx.clone(), layer.expert_load.clone(), layer.bias.clone())

    want = []
    for _ in range(4):
        eager.step(u)
        want.append(state(eager))
    torch.cuda.synchronize()

    graphed.step(u)                                  # the eager step before the recording
    got = [state(graphed)]
    g = graphed.capture_step(u)
    torch.cuda.synchronize()
    assert torch.equal(graphed.bias, got[0][3]), "recording must not run the step"
    for i in range(3):
        junk = torch.randn(1 << 20, device="cuda")    # unrelated eager work between replays
        _ = (junk * 2).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append(state(graphed))
    assert graphed.step_count == 4
    labels = ("out", "topk_idx", "expert_load", "bias")
    for step, (w, h) in enumerate(zip(want, got)):
        for lab, a, b in zip(labels, w, h):
            assert torch.equal(a, b), f"step {step + 1}: {lab} differs between the replay and the eager step"
    # the bias moved every step, so each replay saw the bias the previous one left
    assert not torch.equal(want[0][3], want[3][3])
