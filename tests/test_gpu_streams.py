"""The entry points run on the caller's stream and under HIP graph capture.

Every C-ABI call enqueues its kernel on the stream it is given and allocates
nothing, so a caller can put it on any stream or capture it into a graph
(releases page v0.3.0: the C-ABI bridge exchanges caller-owned buffers).
Results are compared bit for bit with the same call on the default stream:
the kernels are deterministic (no atomics, fixed summation order).
"""
import numpy as np
import pytest

import synth
import quantized_prefill_gemm_codec_amd as qg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no HIP device")
    return t


def _weights(torch, codec, n, k, seed):
    return qg.QWeight.from_canonical(codec, n, k, synth.gen_weight(codec, n, k, seed), device="cuda")


def _x(torch, m, k, seed):
    return torch.from_numpy(synth.gen_x(m, k, seed)).cuda()


def test_side_stream_matches_default_stream(torch):
    n, k = 200, 512
    w, wu = _weights(torch, 2, n, k, 41), _weights(torch, 2, n, k, 42)
    calls = [lambda x: qg.qgemm_prefill(w, x), lambda x: qg.qgemv_decode(w, x[:3]),
             lambda x: qg.qgemm_swiglu(w, wu, x)]
    x = _x(torch, 150, k, 43)
    ref = [f(x) for f in calls]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()              # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = [f(x) for f in calls]         # the binding passes the current stream
    got.append(qg.qgemm_prefill(w, x, stream=side))   # and an explicit one
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r, g in zip(ref + [ref[0]], got):
        assert torch.equal(r, g)


def test_graph_capture_and_replay(torch):
    """Capture the prefill, the decode GEMV and the gated GEMM once; replay
    the graph three times with new X between the replays and eager launches
    in between, and compare every replay with eager results."""
    n, k = 136, 256
    w, wu = _weights(torch, 1, n, k, 51), _weights(torch, 1, n, k, 52)
    x_static = _x(torch, 96, k, 53)
    y_pre = torch.empty((96, n), dtype=torch.float16, device="cuda")
    y_gemv = torch.empty((2, n), dtype=torch.float16, device="cuda")
    y_glu = torch.empty((96, n), dtype=torch.float16, device="cuda")

    def body():
        qg.qgemm_prefill(w, x_static, out=y_pre)
        qg.qgemv_decode(w, x_static[:2], out=y_gemv)
        qg.qgemm_swiglu(w, wu, x_static, out=y_glu)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()                              # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    for rep in range(3):
        x_new = _x(torch, 96, k, 60 + rep)
        x_static.copy_(x_new)
        graph.replay()
        eager = (qg.qgemm_prefill(w, x_new), qg.qgemv_decode(w, x_new[:2]), qg.qgemm_swiglu(w, wu, x_new))
        torch.cuda.synchronize()
        for g, e in zip((y_pre, y_gemv, y_glu), eager):
            assert torch.equal(g, e), f"replay {rep} differs from the eager call"
        assert np.all(np.isfinite(y_pre.cpu().numpy().astype(np.float32)))
