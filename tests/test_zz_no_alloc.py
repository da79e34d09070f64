"""tq_decode_attention_noalloc (decode attention with the library's built-in
device scratch, for callers that cannot allocate) against tq_decode_attention
with a workspace: bit for bit, on two calls in a row, the second on a smaller
cache (the scratch keeps the first call's contents), and its refusal of a
cache whose scratch need exceeds the built-in size."""
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


def _case(dev, n_tokens, batch, layer_index):
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(3, {"n_tokens": n_tokens, "batch": batch})
    fm = w.formats[layer_index]
    layer = tq.Layer(W.rotation_signs(42, layer_index), dev)
    cache = tq.Cache(fm, [n_tokens] * batch, dev)
    k, v = W.make_kv(w, layer_index, device=dev)
    q = W.make_query(w, layer_index, device=dev)
    tq.encode_kv(layer, cache, k, v)
    return layer, cache, q


def test_noalloc_matches_workspace_decode(dev):
    import kv_cache_vector_srht_amd as tq
    for n_tokens, batch, l in ((64 * 40 + 17, 3, 2), (64 * 9 + 5, 2, 0)):   # the second call is smaller
        layer, cache, q = _case(dev, n_tokens, batch, l)
        print(f"noalloc decode: {batch} sessions x {n_tokens} tokens, layer {l}", flush=True)
        assert tq.workspace_bytes(cache, q.shape[1]) <= tq.NOALLOC_SCRATCH_BYTES
        ref = tq.decode_attention(layer, cache, q)
        out = torch.full_like(ref, float("nan"))
        tq.decode_attention_noalloc(layer, cache, q, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())
        out2 = torch.full_like(ref, float("nan"))
        tq.decode_attention_noalloc(layer, cache, q, out2, softmax_scale=0.05)
        ref2 = tq.decode_attention(layer, cache, q, softmax_scale=0.05)
        torch.cuda.synchronize()
        assert np.array_equal(out2.cpu().numpy(), ref2.cpu().numpy())


def test_noalloc_refuses_a_cache_past_its_scratch(dev):
    import kv_cache_vector_srht_amd as tq
    # 64 sessions x 8 KV heads x 1024 pages, 64 query heads: the split
    # partials need about 67 MB, past the 32 MiB scratch
    fm = [[[(3, 2, False)] * 1024 for _ in range(8)] for _ in range(64)]
    cache = tq.Cache(fm, [64] * 64, dev)
    q = torch.zeros((64, 64, 128), dtype=torch.float16, device=dev)
    assert tq.workspace_bytes(cache, 64) > tq.NOALLOC_SCRATCH_BYTES
    layer = tq.Layer(W.rotation_signs(42, 0), dev)
    out = torch.zeros((64, 64, 128), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError, match="scratch"):
        tq.decode_attention_noalloc(layer, cache, q, out)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
