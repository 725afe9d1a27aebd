"""The layer captured in a HIP graph: every replay gives the eager result bit
for bit (the bench times captured steps).  Replays alternate with eager
forwards and host synchronisation, so state that persists on the device
between calls -- the epoch of the one-launch decode step's workspace, the
arrival counter of the fused route+permute -- is exercised in both orders."""
import numpy as np
import pytest
import torch

from gpu_common import Case, bf16_to_np_bits, say

pytestmark = pytest.mark.gpu


def _state(case):
    b = case.buf
    return (bf16_to_np_bits(b.out).copy(), b.topk_idx.cpu().numpy().copy(),
            b.topk_w.cpu().numpy().view(np.uint32).copy())


@pytest.mark.parametrize("name,kw,fmt", [
    ("decode1", dict(), "int4"),                                         # one-launch step
    ("decode1", dict(), "fp4"),
    ("shape", dict(T=3, H=1024, E=32, k=4, I=256, n_shared=1), "int4"),  # fused route+permute, down+combine
    ("decode64", dict(), "int4"),                                        # weight-stream GEMMs
    ("decode64", dict(), "fp4"),
    ("shape", dict(T=420, H=512, E=256, k=6, I=128, n_shared=1), "int4"),  # row sums + tiled GEMMs, two streams
    ("shape", dict(T=420, H=512, E=256, k=6, I=128, n_shared=1), "fp4"),   # tiled FP4 GEMMs, two streams
])
def test_graph_replays_match_eager(name, kw, fmt):
    case = Case(name, seed=4, fmt=fmt, **kw)
    case.run()
    ref = _state(case)
    lay, buf, x = case.layer_obj, case.buf, case.xd
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            lay.forward(x, buf)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(4):
        buf.out.zero_()
        buf.topk_idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _state(case)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), "replay %d differs from the eager result" % i
        case.run()  # an eager forward between replays
        for a, b in zip(_state(case), ref):
            assert np.array_equal(a, b), "eager call after replay %d differs" % i
    if buf.decode_ws.numel() > 3:  # the one-launch step's error word
        assert int(buf.decode_ws[3].item()) == 0, "a decode-step wait timed out"
    say("  %s %s: 4 replays and 4 eager calls identical" % (name, fmt))
