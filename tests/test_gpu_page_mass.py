"""GPU parity of the page attention mass that tq_decode_attention_mass exports
(the signal attention-weighted tier demotion reads): per (session, query
head), the softmax weights summed over each page, against the oracle's
weights over its reconstruction of the cache."""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import Tally, compare_attention, compare_unit_full

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MASS_RTOL = 1e-3
MASS_ATOL = 1e-6


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_srht_amd as tq
    tq.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().cpu().numpy()


def test_page_mass_parity(dev):
    import kv_cache_vector_srht_amd as tq
    B, H, G, P = 4, 2, 4, 8
    T = P * 64
    n_tokens = [T - 20, 5 * 64 + 3, T, 0]           # ragged, full, and an empty session
    base = [W.FP16, W.packed(3, 2), W.packed(6, 6), W.packed(2, 2, True), W.packed(1, 1),
            W.packed(8, 7), W.packed(4, 4), W.packed(2, 3)]
    fm = []
    for b in range(B):
        last = (n_tokens[b] - 1) // 64 if n_tokens[b] else -1
        partial = n_tokens[b] % 64 != 0
        fm.append([[W.FP16 if (p == last and partial) else f for p, f in enumerate(base[h:] + base[:h])]
                   for h in range(H)])
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 64, "dtype": "float16"})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, n_tokens, dev)
    assert cache.page_classes == 7
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    mass = torch.full((B, H * G, P), 7.0, dtype=torch.float32, device=dev)   # every entry is written
    print("decode with page mass", flush=True)
    out_m = _np(tq.decode_attention(layer, cache, q, page_mass=mass)).copy()
    out = _np(tq.decode_attention(layer, cache, q))
    got = _np(mass).copy()
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    # exporting the mass does not change the attention output
    assert np.array_equal(out_m, out)
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    for b in range(B):
        n = n_tokens[b]
        npg = (n + 63) // 64
        for h in range(H):
            rows = slice(h * G, (h + 1) * G)
            assert np.all(got[b, rows, npg:] == 0)
            if n == 0:
                assert np.all(out[b, rows] == 0)
                continue
            Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n], vh[b, h, :n], fm[b][h],
                                       signs, S, t)
            compare_attention(out[b, rows], qh[b, rows], Kh, Vh, t)
            ref = O.page_attention_mass(qh[b, rows], Kh)
            err = np.abs(got[b, rows, :npg] - ref)
            assert np.all(err <= MASS_RTOL * ref + MASS_ATOL), \
                f"session {b} head {h}: mass error {err.max():.3e}"
            assert np.allclose(got[b, rows].sum(axis=1), 1.0, atol=1e-5)
    t.check()

    # a class the hint leaves out is not attended: its pages get no mass
    cache.struct.page_classes = tq.CACHE_COMMON_PAGES | tq.CACHE_OTHER_PAGES
    mass.fill_(7.0)
    tq.decode_attention(layer, cache, q, page_mass=mass)
    got2 = _np(mass)
    for b in range(B):
        for h in range(H):
            for p, f in enumerate(fm[b][h]):
                if f[0] >= 5 and f[1] >= 5 and not f[2]:
                    assert np.all(got2[b, h * G:(h + 1) * G, p] == 0)
            if n_tokens[b]:
                assert np.allclose(got2[b, h * G:(h + 1) * G].sum(axis=1), 1.0, atol=1e-5)


def test_token_mass_parity(dev):
    """tq_decode_attention_token_mass: every token's softmax weight against the
    oracle's over its reconstruction of the cache (every page class, ragged and
    empty sessions), zeros past n_tokens, page sums equal to the page masses,
    and the attention output unchanged."""
    import kv_cache_vector_srht_amd as tq
    B, H, G, P = 3, 2, 4, 6
    T = P * 64
    n_tokens = [T - 20, 3 * 64, 0]
    base = [W.FP16, W.packed(3, 2), W.packed(6, 6), W.packed(2, 2, True), W.packed(1, 1), W.packed(8, 7)]
    fm = []
    for b in range(B):
        last = (n_tokens[b] - 1) // 64 if n_tokens[b] else -1
        partial = n_tokens[b] % 64 != 0
        fm.append([[W.FP16 if (p == last and partial) else f for p, f in enumerate(base[h:] + base[:h])]
                   for h in range(H)])
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 64, "dtype": "float16"})
    signs, S = W.rotation_signs(42, 1), W.qjl_matrix(42, 1)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, n_tokens, dev)
    k, v = W.make_kv(w, 1, device=dev)
    q = W.make_query(w, 1, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    tmass = torch.full((B, H * G, P * 64), 7.0, dtype=torch.float32, device=dev)   # every entry is written
    pmass = torch.full((B, H * G, P), 7.0, dtype=torch.float32, device=dev)
    print("decode with token mass", flush=True)
    out_t = _np(tq.decode_attention(layer, cache, q, token_mass=tmass)).copy()
    out_p = _np(tq.decode_attention(layer, cache, q, page_mass=pmass)).copy()
    out = _np(tq.decode_attention(layer, cache, q))
    got, gotp = _np(tmass).copy(), _np(pmass).copy()
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert np.array_equal(out_t, out) and np.array_equal(out_p, out)
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    for b in range(B):
        n = n_tokens[b]
        assert np.all(got[b, :, n:] == 0)
        if n == 0:
            continue
        for h in range(H):
            rows = slice(h * G, (h + 1) * G)
            Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n], vh[b, h, :n], fm[b][h],
                                       signs, S, t)
            ref = O.token_attention_weights(qh[b, rows], Kh)
            err = np.abs(got[b, rows, :n] - ref)
            assert np.all(err <= MASS_RTOL * ref + MASS_ATOL), \
                f"session {b} head {h}: token weight error {err.max():.3e}"
            assert np.allclose(got[b, rows].sum(axis=1), 1.0, atol=1e-5)
            npg = (n + 63) // 64
            sums = got[b, rows, :npg * 64].reshape(G, npg, 64).sum(axis=2)
            assert np.allclose(sums, gotp[b, rows, :npg], rtol=1e-4, atol=1e-7)
    t.check()
