"""GPU parity of the QJL key encode on the matrix cores at a size where every
wave of the persistent kernel takes several pages in turn (8192 QJL key pages
over at most 2048 waves), with the key width changing from page to page, so the
per-wave tables are staged again between the pages a wave takes."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_parity import Tally, compare_attention, compare_unit_full

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


def test_qjl_keys_many_pages_per_wave(dev):
    import kv_cache_vector_srht_amd as tq
    B, H, G, P = 1, 8, 4, 1024
    w = W.make_workload(2, {"n_tokens": 64 * P, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 0, "dtype": "float16"})
    # key widths cycle 1..8 along the pages (a different start per head), all QJL
    fm = [[[W.packed(1 + (p + 3 * h) % 8, 2, True) for p in range(P)] for h in range(H)]]
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, [64 * P], dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    print("encode 8192 QJL pages", flush=True)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    out = _np(tq.decode_attention(layer, cache, q))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    pool = _np(cache.pool)
    t = Tally()
    for h in (0, 5):
        kh = _np(k[0, h]).astype(np.float64)
        vh = _np(v[0, h]).astype(np.float64)
        Kh, Vh = compare_unit_full(pool, cache.offsets, 0, h, kh, vh, fm[0][h], signs, S, t)
        compare_attention(out[0, h * G:(h + 1) * G], _np(q[0, h * G:(h + 1) * G]).astype(np.float64), Kh, Vh, t)
    t.check()
