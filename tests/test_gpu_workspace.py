"""GPU tests of the library workspace (q4_workspace_reserve, capture safety).

* a stack token captured into a HIP graph on a stream whose workspace was only
  reserved (no eager call on it before) replays bit-identical to eager tokens;
* without a reservation a call during capture fails with Q4_ERANGE and
  enqueues nothing (the capture stays valid);
* a graph captured against the stream's workspace still replays correctly
  after a later, larger call on the same stream grew the workspace (the
  replaced buffer is kept until q4_workspace_release).
"""
import numpy as np
import pytest

import bench
from gpu_common import bits

pytestmark = pytest.mark.gpu

SMALL = dict(d=256, f=512, n_qkv=768, v_off=512, dv=256, layers=4, eps=1e-5)


@pytest.fixture(scope="module")
def q4():
    import int4_weight_only_q4_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def small(q4):
    import torch
    return bench.build_stack(q4, torch, SMALL)


def _eager_tokens(torch, stack, h0, n):
    """n chained eager tokens on the current stream: [h_1 .. h_n], [r_1 .. r_n]."""
    hs, rs = [], []
    h = h0
    for _ in range(n):
        r_out = torch.empty_like(h0)
        h_out = torch.empty_like(h0)
        stack.decode(h, h, r_out, h_out)
        hs.append(h_out)
        rs.append(r_out)
        h = h_out
    torch.cuda.synchronize()
    return [bits(x) for x in hs], [bits(x) for x in rs]


def _capture_pair(torch, stack, s, hs, r_out):
    graphs = []
    for a in (0, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            stack.decode(hs[a], hs[a], r_out, hs[1 - a])
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def test_capture_on_reserved_stream_replays_equal_eager(q4, small):
    import torch
    stack, st = small
    need = q4.stack_workspace_bytes(stack)
    assert need > 0
    s = torch.cuda.Stream()
    q4.workspace_reserve(need, stream=s)  # the stream's only preparation
    hs = [st["h0"].clone(), torch.empty_like(st["h0"])]
    r_out = torch.empty_like(st["h0"])
    graphs = _capture_pair(torch, stack, s, hs, r_out)
    ref_h, ref_r = _eager_tokens(torch, stack, st["h0"], 4)
    for i in range(4):
        graphs[i & 1].replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(hs[(i + 1) & 1]), ref_h[i]), ("h", i)
        assert np.array_equal(bits(r_out), ref_r[i]), ("r", i)
        # eager work and a synchronisation between replays
        _eager_tokens(torch, stack, st["h0"], 1)
    del graphs
    q4.workspace_release(stream=s)


def test_capture_without_reservation_fails_cleanly(q4, small):
    import torch
    stack, st = small
    s = torch.cuda.Stream()
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda")
    r_out = torch.empty_like(st["h0"])
    h_out = torch.empty_like(st["h0"])
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=s):
        dummy.add_(1.0)
        try:
            stack.decode(st["h0"], st["h0"], r_out, h_out)
        except q4.Q4Error as e:
            err = e
    assert err is not None and err.status == q4.Q4_ERANGE, err
    assert "q4_workspace_reserve" in str(err)
    g.replay()
    torch.cuda.synchronize()
    assert torch.all(dummy == 1.0)  # the capture held the one add and nothing else
    # the same call outside capture works on that stream (it allocates)
    with torch.cuda.stream(s):
        stack.decode(st["h0"], st["h0"], r_out, h_out)
    torch.cuda.synchronize()
    ref_h, ref_r = _eager_tokens(torch, stack, st["h0"], 1)
    assert np.array_equal(bits(h_out), ref_h[0])
    q4.workspace_release(stream=s)


def test_graph_survives_workspace_growth(q4, small):
    """Capture against a just-large-enough workspace, then grow it with a larger
    call on the same stream (a split prefill matmul), then replay."""
    import torch
    import datagen
    stack, st = small
    s = torch.cuda.Stream()
    need = q4.stack_workspace_bytes(stack)
    q4.workspace_reserve(need, stream=s)
    hs = [st["h0"].clone(), torch.empty_like(st["h0"])]
    r_out = torch.empty_like(st["h0"])
    graphs = _capture_pair(torch, stack, s, hs, r_out)
    # a prefill matmul whose K-split partials exceed the reserved bytes
    n, k, m = 4096, 8192, 64
    assert q4.workspace_bytes(n, k, m) > max(need, 1 << 20)
    W = torch.from_numpy(datagen.words(datagen.seed_for(4, 40), n, k).view(np.int32)).cuda()
    S = torch.from_numpy(datagen.scales(datagen.seed_for(4, 41), n, k)).cuda()
    X = torch.from_numpy(datagen.activations(datagen.seed_for(4, 42), m, k)).cuda()
    with torch.cuda.stream(s):
        Y = q4.gemm(W, S, X)
    torch.cuda.synchronize()
    Y_ref = q4.gemm(W, S, X)  # the default stream's own workspace
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y), bits(Y_ref))
    ref_h, ref_r = _eager_tokens(torch, stack, st["h0"], 2)
    for i in range(2):
        graphs[i & 1].replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(hs[(i + 1) & 1]), ref_h[i]), ("h", i)
        assert np.array_equal(bits(r_out), ref_r[i]), ("r", i)
    del graphs
    q4.workspace_release(stream=s)
