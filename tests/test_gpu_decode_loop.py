"""GPU parity of the decode loop (tq_append_kv): one token per session per
step into fp16 tail pages that are packed in place when their 64th token
arrives, with decode attention between steps.  The oracle's view of the cache
at each checked step: the sink page and the partial tail page fp16, every
complete page encoded in its target format from its 64 fp16 rows."""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import Tally, compare_attention, compare_unit_full, layer_args

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


def _effective(targets, n):
    """Formats decode sees for a unit holding n tokens: page 0 (sink) fp16,
    complete pages packed in their target, the partial tail fp16."""
    out = []
    for p in range((n + 63) // 64):
        full = 64 * (p + 1) <= n
        out.append(W.FP16 if p == 0 or not full else targets[p])
    return out


@pytest.mark.parametrize("dtype,kinds", [("float16", (O.LLOYD_MAX, O.LLOYD_MAX)),
                                         ("float32", (O.LLOYD_MAX, O.LLOYD_MAX)),
                                         ("float16", (O.POLAR, O.POLAR)),
                                         ("float16", (O.PolarSplit(1), O.PolarSplit(-1)))])
def test_decode_loop_append_and_pack(dev, dtype, kinds):
    import kv_cache_vector_srht_amd as tq
    B, H, G, T = 2, 2, 4, 64 * 5 + 20
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 64, "dtype": dtype})
    # head 0: K3/V2; head 1: K2 + QJL / V2; pages past the sink are pending
    targets = [[W.FP16] + [W.packed(3, 2, False)] * 5, [W.FP16] + [W.packed(2, 2, True)] * 5]
    fm = [[[f if p == 0 else (f[0], f[1], f[2], True) for p, f in enumerate(targets[h])]
           for h in range(H)] for _ in range(B)]
    signs = W.rotation_signs(42, 0)
    S = W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S, **layer_args(kinds[0], kinds[1]))
    k, v = W.make_kv(w, 0, device=dev)          # [B, H, T, 128], the tokens in order
    q = W.make_query(w, 0, device=dev)
    start = [100, 90]                            # ragged sessions
    cache = tq.Cache(fm, start, dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k[:, :, :100], v[:, :, :100], tok0=0, error_flags=flags)
    kh = _np(k).astype(np.float64)
    vh = _np(v).astype(np.float64)
    if dtype == "float32":   # the tail pages hold fp16 rows; packing encodes those
        kh = kh.astype(np.float16).astype(np.float64)
        vh = vh.astype(np.float16).astype(np.float64)
    qh = _np(q).astype(np.float64)
    t = Tally()
    steps = T - start[0]
    checks = {0, 27, 28, 37, 38, 91, 101, steps - 1}
    for step in range(steps):
        n = [s + step for s in start]
        k_new = torch.stack([k[b, :, n[b]] for b in range(B)]).contiguous()
        v_new = torch.stack([v[b, :, n[b]] for b in range(B)]).contiguous()
        tq.append_kv(layer, cache, k_new, v_new, error_flags=flags)
        if step not in checks:
            continue
        out = _np(tq.decode_attention(layer, cache, q))
        torch.cuda.synchronize()
        pool = _np(cache.pool)
        n1 = [x + 1 for x in n]
        assert _np(cache.n_tokens).tolist() == n1
        desc = _np(cache.pages).view(np.uint64)
        for b in range(B):
            for h in range(H):
                eff = _effective(targets[h], n1[b])
                for p in range(1, len(eff)):
                    pending = bool(int(desc[b, h, p]) >> 57 & 1)
                    assert pending == (eff[p] == W.FP16), (step, b, h, p)
                Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n1[b]], vh[b, h, :n1[b]],
                                           eff, signs, S, t, kinds[0], kinds[1])
                compare_attention(out[b, h * G:(h + 1) * G], qh[b, h * G:(h + 1) * G], Kh, Vh, t)
    assert int(flags.item()) == 0
    t.check()


def test_append_into_a_packed_page_is_flagged(dev):
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(2, {"n_tokens": 128, "batch": 1, "n_kv_heads": 1, "n_q_heads": 4, "sink_tokens": 0})
    fm = [[[W.packed(3, 2, False), W.packed(3, 2, False)]]]
    layer = tq.Layer(W.rotation_signs(42, 0), dev)
    cache = tq.Cache(fm, [64], dev)
    k, v = W.make_kv(w, 0, device=dev)
    tq.encode_kv(layer, cache, k, v)
    before = _np(cache.pool).copy()
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.append_kv(layer, cache, k[:, :, 64].contiguous(), v[:, :, 64].contiguous(), error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 32
    assert np.array_equal(_np(cache.pool), before)
    assert _np(cache.n_tokens).tolist() == [65]
