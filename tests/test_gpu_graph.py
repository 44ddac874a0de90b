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


EXTRA = {w.name: w for w in (
    datagen.small_workload("graph_w2x12x12", 1, 4, 36, 48, 4, 64, (2, 12, 12), (1, 6, 6), "bf16", seed=61),  # whole window
    datagen.small_workload("graph_w2x6x6", 1, 4, 36, 48, 4, 64, (2, 6, 6), (1, 3, 3), "bf16", seed=63),      # streaming
    # streaming on a padded grid: the instance whose padding-only query blocks end early
    datagen.small_workload("graph_w3x12x12_pad", 1, 4, 24, 24, 2, 128, (3, 12, 12), (1, 6, 6), "bf16", seed=64),
)}


@pytest.mark.parametrize("name,plan_dtype", [("stage3_pad", "bf16"), ("stage3_pad_f32_split", "f32_split"),
                                             ("stage3_pad_f32", "f32"), ("graph_w2x12x12", "bf16"),
                                             ("graph_w2x6x6", "bf16"), ("graph_w3x12x12_pad", "bf16")])
def test_graph_replays_match_eager(name, plan_dtype):
    wl = EXTRA[name] if name in EXTRA else datagen.WORKLOADS[name]
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


def test_graph_replays_adaln():
    wl = datagen.AdalnWorkload("graph_adaln", 2, 700, 512, "bf16", "f32", "f32", seed=62)
    a = datagen.adaln_inputs(wl)
    x = datagen.to_torch(a["x"], "bf16").cuda()
    res = datagen.to_torch(a["res"], "f32").cuda()
    g, b = (torch.from_numpy(a[k]).cuda() for k in ("gamma", "beta"))
    eager = sw.adaln_residual(x, res, g, b, wl.eps)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sw.adaln_residual(x, res, g, b, wl.eps, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        sw.adaln_residual(x, res, g, b, wl.eps, out=out)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
    say("[gpu] graph adaln: 4 replays bit-identical to eager")


@pytest.mark.parametrize("name", ["stage3_pad", "graph_w3x12x12_pad"])
def test_one_plan_on_two_streams(name):
    """A plan holds no device state: the same plan launched on two streams at once, on different
    inputs, gives each stream its own eager result bit for bit."""
    wl = EXTRA[name] if name in EXTRA else datagen.WORKLOADS[name]
    xa = device_inputs(wl)
    xb = {t: (xa[t].float() * -0.5).to(xa[t].dtype) for t in "qkv"}  # other values, same shapes
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    ref = []
    for x in (xa, xb):
        o = torch.empty_like(x["q"])
        plan.run(x["q"], x["k"], x["v"], o)
        torch.cuda.synchronize()
        ref.append(o)
    outs = [torch.full_like(xa["q"], float("nan")) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for x, o, s_ in zip((xa, xb), outs, streams):
            with torch.cuda.stream(s_):
                plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o.view(torch.int16), r.view(torch.int16))
    say(f"[gpu] {name}: one plan on two streams, both bit-identical to eager")
