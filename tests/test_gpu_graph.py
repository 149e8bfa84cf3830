"""The library's multi-layer step graph (moe_step_graph_*): layers chained
through their outputs (layer l + 1 reads layer l's y), captured once by the
library and replayed, against the same calls made eagerly (bitwise, on every
replay) and against the oracle layer by layer (each layer fed the input the
GPU gave it)."""
import dataclasses

import pytest
import torch

import quantized_moe_expert_02_amd as moe
from quantized_moe_expert_02_amd import synth
from helpers import assert_close, oracle_y

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _log(*a):
    print(*a, flush=True)


def chain_layers(dims, n, name):
    """n layers sharing one set of experts, each with its own router.  The
    down projections are scaled up by a power of two (exactly: the row
    scales, or the tensor scale) so that outputs fed back as inputs keep a
    magnitude well inside binary16's normal range over a few layers."""
    base = synth.make_layer(dims, ("stepgraph", name))
    if dims.wfmt in synth.ROW_SCALED:
        base.s_down = base.s_down * 16
    else:
        base.g3[:, 2] *= 8
    canon = [base] + [dataclasses.replace(base, router_w=synth.make_router(dims, ("stepgraph", name, l))[0])
                      for l in range(1, n)]
    pl0 = moe.PackedLayer.from_layer(base)
    packed = [pl0] + [moe.PackedLayer(dims, pl0.packed, c.router_w.to(DEV), None) for c in canon[1:]]
    return canon, packed


CASES = [
    ("int4_t1", synth.Dims(1024, 256, 32, 4, 1, synth.INT4_ROW), 1, 3),
    ("e2m1_t4", synth.Dims(1024, 512, 32, 4, 1, synth.E2M1_B16), 4, 3),
    ("int4_prefill_t40", synth.Dims(512, 256, 16, 2, 1, synth.INT4_ROW), 40, 3),
]


@pytest.mark.parametrize("name,dims,T,n", CASES)
def test_step_graph_chain(name, dims, T, n):
    _log("step graph", name, dims, T, n)
    canon, layers = chain_layers(dims, n, name)
    ws = moe.workspace(dims, T, DEV)
    bufs = [synth.make_tokens(dims, T, ("stepgraph", name, "x")).to(DEV)] + \
        [torch.zeros((T, dims.hidden), dtype=torch.float16, device=DEV) for _ in range(n)]
    xs, ys = bufs[:-1], bufs[1:]

    def eager(x0):
        out, x = [], x0
        for pl in layers:
            x = moe.moe_w4a16_forward(pl, x, ws=ws).clone()
            out.append(x)
        return out

    sg = moe.StepGraph(layers, xs, ys, ws)
    try:
        x_alt = synth.make_tokens(dims, T, ("stepgraph", name, "x2")).to(DEV)
        x_first = bufs[0].clone()
        for rep, x0 in enumerate((x_first, x_first, x_alt, x_first)):
            bufs[0].copy_(x0)
            for y in ys:
                y.fill_(0)
            sg.launch()
            ref = eager(x0)  # eager work on the same stream after the replay
            torch.cuda.synchronize()
            for l in range(n):
                assert torch.equal(ys[l], ref[l]), (name, rep, l)
        for l in range(n):  # the last replay, layer by layer against the oracle
            a = float(ys[l].float().abs().mean())
            assert 1e-2 < a < 1e3, (name, l, a)  # the chain stays in binary16's normal range
            assert_close(ys[l], oracle_y(canon[l], xs[l].cpu()), f"{name} layer {l}")
    finally:
        sg.close()


@pytest.mark.parametrize("name", ["decode_b1", "e2m1_b1"])
def test_step_graph_full_size_chain(name):
    """Two layers of a full-size decode workload (all 256 + 1 experts
    resident, one token) chained through the step graph: each replay equals
    the eager calls bitwise, and each layer matches the oracle fed the input
    the GPU gave it (at this width the chained activations keep their scale
    without any rescaling)."""
    _log("step graph, full size", name)
    base, x0 = synth.workload(name, device=DEV)
    dims = base.dims
    canon = [base, dataclasses.replace(base, router_w=synth.make_router(dims, ("stepgraph", name, 1),
                                                                        device=DEV)[0])]
    pl0 = moe.PackedLayer.from_layer(base)
    layers = [pl0, moe.PackedLayer(dims, pl0.packed, canon[1].router_w, None)]
    T = x0.shape[0]
    ws = moe.workspace(dims, T, DEV)
    bufs = [x0.clone()] + [torch.zeros((T, dims.hidden), dtype=torch.float16, device=DEV) for _ in range(2)]
    sg = moe.StepGraph(layers, bufs[:-1], bufs[1:], ws)
    try:
        for rep in range(3):
            for y in bufs[1:]:
                y.fill_(0)
            sg.launch()
            e0 = moe.moe_w4a16_forward(layers[0], bufs[0], ws=ws).clone()
            e1 = moe.moe_w4a16_forward(layers[1], e0, ws=ws).clone()
            torch.cuda.synchronize()
            assert torch.equal(bufs[1], e0) and torch.equal(bufs[2], e1), (name, rep)
        for l in range(2):
            assert_close(bufs[l + 1], oracle_y(canon[l], bufs[l]), f"{name} layer {l}")
    finally:
        sg.close()
