"""Stream semantics and HIP graph replay of the library's entry points.

tp.h promises that every call is enqueued on the stream it is given and that
the library allocates nothing (no memory calls, no memsets), so a sequence of
calls can run on a side stream or be captured in a graph and replayed. Checked
here on the step's path at reduced sizes, including the small-M split-K plan
(its partial sums in the workspace, then the reduce launch): the same bytes on
a side stream as on the default stream, and every replay of a captured graph
equal to the eager result for the inputs the graph reads at that moment (the
inputs are rewritten by eager work between replays).
"""

import pytest
import torch

import int4_quantized_gemm_amd as tp
import workloads as W
from tests.gpu_util import announce, dev

pytestmark = pytest.mark.gpu


def _buffers(d):
    """Inputs, weights and preallocated outputs and workspaces of four calls:
    rotate + quantize, W8A8 at 300 rows (multi-stage kernel), W8A8 at 40 rows
    (small-M split-K plan) and W4 with the rotation (through the workspace)."""
    wl = W.PROJ256.with_(name="streams", m=300, n=640, k=2048, seed=91, path="w8a8")
    x, w = W.generate(wl)
    w4l = W.PROJ256.with_(name="streams_w4", m=200, n=384, k=3072, seed=92, path="w4")
    x4, w4 = W.generate(w4l)
    b = {"x": x.to(d), "x4": x4.to(d)}
    b["q8"], b["s8"] = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    b["q4"], b["s4"] = tp.tp_rotate_quantize_weights(w4.to(d), bits=4)
    m, k, n = wl.m, wl.k, wl.n
    b["qa"] = torch.empty((m, k), dtype=torch.int8, device=d)
    b["sa"] = torch.empty((m,), dtype=torch.float32, device=d)
    b["y"] = torch.empty((m, n), dtype=torch.float32, device=d)
    b["y40"] = torch.empty((40, n), dtype=torch.float32, device=d)
    b["y4"] = torch.empty((w4l.m, w4l.n), dtype=torch.bfloat16, device=d)
    need40 = tp.tp_workspace_size(tp._lib.TP_OP_QGEMM_W8A8_PREQUANTIZED, 40, n, k, 0)
    assert need40 > 0, "the 40-row case is meant to take the split-K plan"
    b["ws"] = torch.empty((max(1, tp.tp_workspace_size(tp._lib.TP_OP_QGEMM_W8A8_PREQUANTIZED, m, n, k, 0)),),
                          dtype=torch.uint8, device=d)
    b["ws40"] = torch.empty((need40,), dtype=torch.uint8, device=d)
    b["ws4"] = torch.empty((max(1, tp.tp_workspace_size(tp._lib.TP_OP_QGEMM_W4, w4l.m, w4l.n, w4l.k, 1)),),
                           dtype=torch.uint8, device=d)
    return b


def _run(b, stream=None):
    tp.tp_quantize_rows_int8(b["x"], qa=b["qa"], sa=b["sa"], stream=stream)
    tp.tp_qgemm_w8a8_prequantized(b["qa"], b["sa"], b["q8"], b["s8"], out=b["y"], workspace=b["ws"], stream=stream)
    tp.tp_qgemm_w8a8_prequantized(b["qa"][:40], b["sa"][:40], b["q8"], b["s8"], out=b["y40"], workspace=b["ws40"],
                                  stream=stream)
    tp.tp_qgemm_w4(b["x4"], b["q4"], b["s4"], rotate=True, out=b["y4"], workspace=b["ws4"], stream=stream)


def _outputs(b):
    return [b[k].clone() for k in ("qa", "sa", "y", "y40", "y4")]


def _same(got, want, what):
    for g, w, name in zip(got, want, ("qa", "sa", "y", "y40", "y4")):
        assert torch.equal(g.view(torch.uint8) if g.dtype != torch.int8 else g,
                           w.view(torch.uint8) if w.dtype != torch.int8 else w), f"{what}: {name} differs"


def test_side_stream_gives_the_same_bytes():
    d = dev()
    announce("side stream")
    b = _buffers(d)
    _run(b)
    torch.cuda.synchronize()
    want = _outputs(b)
    for k in ("qa", "y", "y40", "y4"):
        b[k].zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(b)  # the binding passes torch's current stream, here the side stream
    side.synchronize()
    _same(_outputs(b), want, "side stream (current)")
    for k in ("qa", "y", "y40", "y4"):
        b[k].zero_()
    torch.cuda.synchronize()
    _run(b, stream=side)  # the stream passed explicitly
    side.synchronize()
    _same(_outputs(b), want, "side stream (explicit)")


def test_graph_replays_match_eager():
    d = dev()
    announce("graph capture and replay")
    b = _buffers(d)
    _run(b)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(b)
    gen = torch.Generator(device=d)
    for rep in range(4):
        # eager work between replays: new inputs for the graph to read
        gen.manual_seed(100 + rep)
        b["x"].copy_(torch.randn(b["x"].shape, device=d, generator=gen).to(b["x"].dtype))
        b["x4"].copy_(torch.randn(b["x4"].shape, device=d, generator=gen).to(b["x4"].dtype))
        torch.cuda.synchronize()
        _run(b)
        torch.cuda.synchronize()
        want = _outputs(b)
        for k in ("qa", "y", "y40", "y4"):
            b[k].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_outputs(b), want, f"replay {rep}")
    del graph


def test_two_streams_at_once():
    """Calls on two streams that share no output or workspace may overlap:
    the W8A8 calls on one stream and the W4 call on another, issued together,
    give the bytes of the calls run one after the other."""
    d = dev()
    announce("two streams at once")
    b = _buffers(d)
    _run(b)
    torch.cuda.synchronize()
    want = _outputs(b)
    for k in ("qa", "y", "y40", "y4"):
        b[k].zero_()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        tp.tp_quantize_rows_int8(b["x"], qa=b["qa"], sa=b["sa"], stream=s1)
        tp.tp_qgemm_w8a8_prequantized(b["qa"], b["sa"], b["q8"], b["s8"], out=b["y"], workspace=b["ws"], stream=s1)
        tp.tp_qgemm_w8a8_prequantized(b["qa"][:40], b["sa"][:40], b["q8"], b["s8"], out=b["y40"],
                                      workspace=b["ws40"], stream=s1)
        tp.tp_qgemm_w4(b["x4"], b["q4"], b["s4"], rotate=True, out=b["y4"], workspace=b["ws4"], stream=s2)
    s1.synchronize()
    s2.synchronize()
    _same(_outputs(b), want, "two streams")
