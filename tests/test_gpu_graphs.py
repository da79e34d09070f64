"""The library's calls captured in HIP graphs (through torch.cuda.CUDAGraph on
the capturing stream) give the eager results bit for bit: decode attention
replayed several times with eager work between the replays, and decode-loop
steps (append, with a page packed in place inside a graph, then decode)
replayed step by step against an eager twin cache."""
import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_srht_amd as tq
    tq.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().cpu().numpy()


@pytest.mark.parametrize("index", [3, 4])
def test_decode_graph_replays_match_eager(dev, index):
    """Workload 3's per-head widths (all three page classes) and workload 4's
    QJL keys, 9 pages and a ragged tail."""
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(index, {"n_tokens": 64 * 9 + 5, "batch": 2, "n_layers": 1})
    S = W.qjl_matrix(42, 0)
    layer = tq.Layer(W.rotation_signs(42, 0), dev, S)
    cache = tq.Cache(w.formats[0], [w.n_tokens] * w.batch, dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    tq.encode_kv(layer, cache, k, v)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.workspace_bytes(cache, w.n_q_heads), dtype=torch.uint8, device=dev)
    tq.decode_attention(layer, cache, q, out=out, workspace=ws)
    torch.cuda.synchronize()
    eager = _np(out).copy()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):   # warm-up on the side stream, as capture asks
        tq.decode_attention(layer, cache, q, out=out, workspace=ws)
    torch.cuda.current_stream(dev).wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tq.decode_attention(layer, cache, q, out=out, workspace=ws)
    for r in range(3):
        out.fill_(float("nan"))
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_np(out), eager), f"replay {r}"
        # eager work between replays
        tq.decode_attention(layer, cache, q * 2, out=torch.empty_like(out))
        torch.cuda.synchronize()


def test_decode_loop_steps_in_graphs_match_eager(dev):
    """70 steps from 100 tokens: the pending page that fills at token 128 is
    packed inside a replayed graph."""
    import kv_cache_vector_srht_amd as tq
    B, H, G = 2, 2, 4
    T = 64 * 3
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 64})
    targets = [W.FP16, (3, 2, False, True), (2, 2, True, True)]
    fm = [[list(targets) for _ in range(H)] for _ in range(B)]
    S = W.qjl_matrix(42, 0)
    layer = tq.Layer(W.rotation_signs(42, 0), dev, S)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    caches = [tq.Cache(fm, [100, 100], dev) for _ in range(2)]
    for c in caches:
        tq.encode_kv(layer, c, k[:, :, :100], v[:, :, :100], tok0=0)
    outs = [torch.empty((B, H * G, 128), dtype=torch.float32, device=dev) for _ in range(2)]
    wss = [torch.empty(tq.workspace_bytes(c, H * G), dtype=torch.uint8, device=dev) for c in caches]
    steps = 70
    news = [(k[:, :, 100 + i].contiguous(), v[:, :, 100 + i].contiguous()) for i in range(steps)]
    torch.cuda.synchronize()
    graphs = []
    for i in range(steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            tq.append_kv(layer, caches[1], news[i][0], news[i][1])
            tq.decode_attention(layer, caches[1], q, out=outs[1], workspace=wss[1])
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(steps):
        tq.append_kv(layer, caches[0], news[i][0], news[i][1])
        tq.decode_attention(layer, caches[0], q, out=outs[0], workspace=wss[0])
        graphs[i].replay()
        torch.cuda.synchronize()
        assert np.array_equal(_np(outs[0]), _np(outs[1])), f"step {i}"
        assert np.array_equal(_np(caches[0].n_tokens), _np(caches[1].n_tokens))
    assert _np(caches[1].n_tokens).tolist() == [100 + steps] * B
    assert np.array_equal(_np(caches[0].pool), _np(caches[1].pool))
    assert np.array_equal(_np(caches[0].pages), _np(caches[1].pages))
