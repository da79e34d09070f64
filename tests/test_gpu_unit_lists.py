"""Decode attention with the per-unit class record (tq_cache.unit_classes):
each class's split launch covers only the (session, KV head) units that hold
it.  With an exact record the output and the page mass are bit-identical to
the launch over every unit (NULL record) and match the oracle; a record that
leaves a class out of one unit drops exactly that unit's pages of the class."""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
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


C3, C1, W6, W8, Q2 = W.packed(3, 2), W.packed(1, 1), W.packed(6, 6), W.packed(8, 7), W.packed(2, 2, True)
P = 6
# units (session, KV head): common only, wide only, QJL only, fp16 + common,
# then mixes of all three classes
PLAN = [
    [[C3] * P, [W6] * P, [Q2] * P, [W.FP16] + [C1] * (P - 1)],
    [[C3, W8, C1, W6, W.FP16, C3], [W8] * P, [W.FP16, C3, C3, C3, C3, Q2], [C1, W6, Q2, C3, W8, C1]],
]


def _setup(dev):
    import kv_cache_vector_srht_amd as tq
    B, H, G = 2, 4, 4
    n_tokens = [P * 64 - 10, 5 * 64]
    fm = [[list(r) for r in row] for row in PLAN]
    for b in range(B):   # a partial last page is fp16
        if n_tokens[b] % 64:
            for h in range(H):
                fm[b][h][(n_tokens[b] - 1) // 64] = W.FP16
    w = W.make_workload(2, {"n_tokens": P * 64, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 0, "dtype": "float16"})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, n_tokens, dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    return tq, layer, cache, fm, n_tokens, k, v, q, signs, S


def _decode(tq, layer, cache, q):
    B, Hq = q.shape[0], q.shape[1]
    mass = torch.full((B, Hq, cache.max_pages), 7.0, dtype=torch.float32, device=q.device)
    out = tq.decode_attention(layer, cache, q, page_mass=mass)
    torch.cuda.synchronize()
    return _np(out).copy(), _np(mass).copy()


def test_unit_lists_match_full_grid_and_oracle(dev):
    tq, layer, cache, fm, n_tokens, k, v, q, signs, S = _setup(dev)
    # session 0's partial last page is fp16 (class 2) in every unit
    assert cache.unit_classes.tolist() == [[3, 6, 2, 3], [7, 4, 3, 7]]
    print("decode with unit lists", flush=True)
    out_l, mass_l = _decode(tq, layer, cache, q)
    cache.struct.unit_classes = None
    print("decode over every unit", flush=True)
    out_f, mass_f = _decode(tq, layer, cache, q)
    assert np.array_equal(out_l, out_f)
    assert np.array_equal(mass_l, mass_f)
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    G = 4
    for b in range(2):
        n = n_tokens[b]
        for h in range(4):
            rows = slice(h * G, (h + 1) * G)
            Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n], vh[b, h, :n],
                                       fm[b][h], signs, S, t)
            compare_attention(out_l[b, rows], qh[b, rows], Kh, Vh, t)
    t.check()


def test_unit_record_drops_one_units_class(dev):
    tq, layer, cache, fm, n_tokens, k, v, q, signs, S = _setup(dev)
    out0, mass0 = _decode(tq, layer, cache, q)
    # unit (1, 0) loses its wide pages (pages 1 and 3); every other unit keeps all
    cache.unit_classes[1, 0] &= ~np.uint8(tq.CACHE_WIDE_PAGES)
    print("decode with one unit's wide class left out", flush=True)
    out1, mass1 = _decode(tq, layer, cache, q)
    G = 4
    for b in range(2):
        for h in range(4):
            rows = slice(h * G, (h + 1) * G)
            if (b, h) == (1, 0):
                continue
            assert np.array_equal(out1[b, rows], out0[b, rows]), (b, h)
            assert np.array_equal(mass1[b, rows], mass0[b, rows]), (b, h)
    rows = slice(0, G)
    assert np.all(mass1[1, rows, 1] == 0) and np.all(mass1[1, rows, 3] == 0)
    assert np.allclose(mass1[1, rows].sum(axis=1), 1.0, atol=1e-5)
    # the unit's output is attention over its remaining pages (the oracle's)
    n = n_tokens[1]
    keep = np.concatenate([np.arange(64 * p, min(n, 64 * p + 64)) for p in range(P)
                           if p not in (1, 3) and 64 * p < n])
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    Kh, Vh = compare_unit_full(pool, cache.offsets, 1, 0, kh[1, 0, :n], vh[1, 0, :n], fm[1][0], signs, S, t)
    compare_attention(out1[1, rows], qh[1, rows], Kh[keep], Vh[keep], t)
    t.check()
    ref = O.page_attention_mass(qh[1, rows], Kh)
    assert not np.allclose(mass0[1, rows, 1], 0) and np.allclose(mass0[1, rows, :5], ref, rtol=1e-3, atol=1e-6)


def test_admitted_class_held_by_no_unit(dev):
    """page_classes admits every class, the record lists only common pages:
    the wide and other launches are left out and their partials count as
    empty, so the output is that of the exact hint."""
    import kv_cache_vector_srht_amd as tq
    B, H, G = 2, 4, 4
    fm = [[[C3, C1, W.packed(4, 4), C3] for _ in range(H)] for _ in range(B)]
    w = W.make_workload(2, {"n_tokens": 256, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 0, "dtype": "float16"})
    layer = tq.Layer(W.rotation_signs(42, 0), dev)
    cache = tq.Cache(fm, [256, 200], dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    tq.encode_kv(layer, cache, k, v)
    assert cache.page_classes == tq.CACHE_COMMON_PAGES and (cache.unit_classes == 1).all()
    out1, mass1 = _decode(tq, layer, cache, q)
    cache.struct.page_classes = 7
    print("decode with every class admitted", flush=True)
    out7, mass7 = _decode(tq, layer, cache, q)
    assert np.array_equal(out1, out7) and np.array_equal(mass1, mass7)



def test_more_units_than_listed(dev):
    """528 (session, KV head) units, above the 512 a launch can list: the
    record is ignored and every class's grid covers every unit; sampled units
    against the oracle."""
    import kv_cache_vector_srht_amd as tq
    B, H, G = 66, 8, 1
    plans = [[C3, W6], [Q2, C1], [W8, W.FP16], [C1, C3]]
    fm = [[list(plans[(b * H + h) % 4]) for h in range(H)] for b in range(B)]
    n_tokens = [128 if b % 3 else 100 for b in range(B)]
    for b in range(B):
        if n_tokens[b] % 64:
            for h in range(H):
                fm[b][h][1] = W.FP16
    w = W.make_workload(2, {"n_tokens": 128, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 0, "dtype": "float16"})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, n_tokens, dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    tq.encode_kv(layer, cache, k, v)
    print("decode over 528 units", flush=True)
    out = _np(tq.decode_attention(layer, cache, q))
    torch.cuda.synchronize()
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    for b, h in [(0, 0), (0, 1), (1, 2), (33, 7), (64, 5), (65, 3), (65, 6)]:
        n = n_tokens[b]
        Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n], vh[b, h, :n], fm[b][h], signs, S, t)
        compare_attention(out[b, h:h + 1], qh[b, h:h + 1], Kh, Vh, t)
    t.check()
