"""The library's launches can be captured in a HIP graph (torch.cuda.CUDAGraph on ROCm):
run() allocates nothing, never synchronises and takes the caller's stream. Each replay,
with eager work and synchronisations in between, must equal the eager result bit for bit."""
import math

import pytest
import torch

import datagen
import swin3d_window_attention_amd as sw
from _gpu import device_inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,plan_dtype", [("stage3_pad", "bf16"), ("stage3_pad_f32_split", "f32_split")])
def test_graph_replays_match_eager(name, plan_dtype):
    wl = datagen.WORKLOADS[name]
    x = device_inputs(wl)
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=plan_dtype, scale=wl.scale,
                   cross_region_bias=-math.inf)
    eager = torch.empty_like(x["q"])
    plan.run(x["q"], x["k"], x["v"], eager)
    torch.cuda.synchronize()
    ibits = torch.int16 if x["q"].dtype == torch.bfloat16 else torch.int32

    out = torch.zeros_like(x["q"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # capture must not run on the default stream
        plan.run(x["q"], x["k"], x["v"], out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        plan.run(x["q"], x["k"], x["v"], out)
    for rep in range(4):
        out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(ibits), eager.view(ibits)), f"replay {rep}"
    say(f"[gpu] graph {name}: 4 replays bit-identical to eager")
