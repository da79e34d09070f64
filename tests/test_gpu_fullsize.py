"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: one encode call and one decode-attention call per layer over every
session and KV head.  The oracle checks sampled (session, KV head) units page
by page and their query heads' attention rows, plus dequantised windows; the
reduced cases in test_gpu_parity.py cover every unit of smaller shapes and the
edge cases."""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import Tally, compare_attention, compare_dequant, compare_unit_full

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


def _units_per_format(fm, limit):
    """One (session, KV head) unit per distinct set of page formats (the widths
    are per (layer, head)), sessions rotated."""
    seen, units = set(), []
    for h in range(len(fm[0])):
        b = h % len(fm)
        key = frozenset(fm[b][h])
        if key not in seen:
            seen.add(key)
            units.append((b, h))
    return units[:limit]


def run_full(w, layer_ids, units_of, windows, dev, tally=None):
    import kv_cache_vector_srht_amd as tq
    t = tally or Tally()
    G = w.n_q_heads // w.n_kv_heads
    for l in layer_ids:
        fm = w.formats[l]
        has_qjl = any(f[2] for row in fm for r in row for f in r)
        signs = W.rotation_signs(W.ROTATION_SEED, l)
        S = W.qjl_matrix(W.ROTATION_SEED, l) if has_qjl else None
        layer = tq.Layer(signs, dev, S, w.k_codebook, w.v_codebook)
        cache = tq.Cache(fm, [w.n_tokens] * w.batch, dev)
        k, v = W.make_kv(w, l, device=dev)
        q = W.make_query(w, l, device=dev)
        ws = torch.empty(tq.workspace_bytes(cache, w.n_q_heads), dtype=torch.uint8, device=dev)
        out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
        tq.encode_kv(layer, cache, k, v, tok0=0, error_flags=flags)
        tq.decode_attention(layer, cache, q, out=out, workspace=ws)
        deq = [(t0, n, _np(tq.dequantize(layer, cache, 0, t0, n)), _np(tq.dequantize(layer, cache, 1, t0, n)))
               for t0, n in windows]
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, f"encode error flags {int(flags.item())}"
        pool = _np(cache.pool)
        out_h = _np(out)
        qh = _np(q).astype(np.float64)
        units = units_of(fm)
        print(f"layer {l}: units {units}", flush=True)
        for (b, h) in units:
            kh = _np(k[b, h]).astype(np.float64)
            vh = _np(v[b, h]).astype(np.float64)
            Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh, vh, fm[b][h], signs, S, t,
                                       w.k_codebook, w.v_codebook)
            compare_attention(out_h[b, h * G:(h + 1) * G], qh[b, h * G:(h + 1) * G], Kh, Vh, t)
            for t0, n, dk, dv in deq:
                compare_dequant(dk[b, h], Kh[t0:t0 + n], t)
                compare_dequant(dv[b, h], Vh[t0:t0 + n], t)
        del k, v, cache
    t.check()
    return t


@pytest.mark.timeout(240)
def test_fullsize_qwen3_8b_stack_32k(dev):
    w = W.make_workload(3)
    # layers with hub (6-8 bit), peripheral (1-2 bit) and base K3/V2 heads
    layers = [0, 2, 3, 21, 35]
    for l in layers[1:]:
        kinds = {f for row in w.formats[l] for r in row for f in r}
        assert any(f[0] >= 6 for f in kinds) and (3, 2, False) in kinds
    T = w.n_tokens
    run_full(w, layers, lambda fm: _units_per_format(fm, 3), [(0, 256), (T // 2 - 128, 256), (T - 256, 256)],
             dev)


@pytest.mark.timeout(240)
def test_fullsize_long_context_128k_qjl(dev):
    w = W.make_workload(4)
    T = w.n_tokens
    run_full(w, [0], lambda fm: [(0, 0), (7, 3), (w.batch - 1, w.n_kv_heads - 1)],
             [(0, 256), (T - 256, 256)], dev)


@pytest.mark.timeout(240)
def test_fullsize_tiers_256k(dev):
    w = W.make_workload(5)
    T = w.n_tokens
    fm = w.formats[0]
    assert len({f for f in fm[0][0] if f[0]}) >= 3
    # oldest tier, the K4/V4 tier, and the boundary into the fp16 tier
    run_full(w, [0], lambda fm: [(0, 0), (3, 5), (w.batch - 1, w.n_kv_heads - 2)],
             [(0, 256), (T - 4096, 256), (T - 1024 - 128, 256)], dev)


@pytest.mark.timeout(300)
def test_fullsize_tiers_256k_reached_by_retiering(dev):
    """The 256K tiered workload built the way the pages' tiering runs: every
    packed page encoded at its head's warm tier (K4/V4 plus the head's offset),
    then one tq_retier_pages call demotes the older and the masked pages to
    their tiers in place.  Sampled units against the oracle: demoted pages hold
    the oracle's warm-tier codes requantised to the target widths with the
    warm-tier norms; attention over the re-tiered cache."""
    import math
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(5)
    fm = w.formats[0]
    B, H, T = w.batch, w.n_kv_heads, w.n_tokens
    offs = [int(math.floor(5 * s)) - 2 for s in W._score_rng(5, 0, 11).random(H)]
    warm = [W.packed(min(8, max(1, 4 + o)), min(8, max(1, 4 + o))) for o in offs]
    init = [[[f if f[0] == 0 else warm[h] for f in fm[b][h]] for h in range(H)] for b in range(B)]
    signs = W.rotation_signs(W.ROTATION_SEED, 0)
    layer = tq.Layer(signs, dev)
    cache = tq.Cache(init, [T] * B, dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    pages = [(b, h, p) for b in range(B) for h in range(H) for p in range(len(fm[b][h]))
             if tuple(fm[b][h][p]) != tuple(init[b][h][p])]
    print(f"demoting {len(pages)} of {B * H * len(fm[0][0])} pages", flush=True)
    tq.retier_pages(layer, cache, pages, [fm[b][h][p] for b, h, p in pages], error_flags=flags)
    out = _np(tq.decode_attention(layer, cache, q))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert cache.page_classes == tq.page_classes(fm)
    assert np.array_equal(_np(cache.pages).view(np.uint64), cache.host_pages)
    pool = _np(cache.pool)
    qh = _np(q).astype(np.float64)
    G = w.n_q_heads // H
    t = Tally()
    for (b, h) in [(0, 0), (3, 5), (B - 1, H - 2)]:
        kh = _np(k[b, h]).astype(np.float64)
        vh = _np(v[b, h]).astype(np.float64)
        demoted = {p for (bb, hh, p) in pages if (bb, hh) == (b, h)}
        Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, kh, vh, fm[b][h], signs, None, t,
                                   skip=demoted)
        # demoted pages, one oracle pass per (warm, target) group
        groups = {}
        for p in sorted(demoted):
            groups.setdefault(tuple(fm[b][h][p]), []).append(p)
        (kb, vb, _) = warm[h]
        for (nkb, nvb, _), plist in groups.items():
            rows = np.concatenate([np.arange(64 * p, 64 * p + 64) for p in plist])
            sec = O.page_sections((nkb, nvb, False))
            raws = [pool[int(cache.offsets[b, h, p]):int(cache.offsets[b, h, p]) + O.page_bytes((nkb, nvb, False))]
                    for p in plist]

            def part(name):
                o, n = sec[name]
                return b"".join(r[o:o + n].tobytes() for r in raws)
            recon = {}
            for which, X, ob, nb in (("k", kh, kb, nkb), ("v", vh, vb, nvb)):
                e = O.encode(X[rows], signs, ob)
                exp = O.requantize_codes(e["codes"], ob, nb)
                if which == "k":
                    g = np.concatenate([O.unpack_block(r[sec["k_codes"][0]:sec["k_codes"][0] + sec["k_codes"][1]]
                                                       .tobytes(), nb) for r in raws])
                else:
                    g = np.concatenate([O.v_codes_from_streams(O.unpack_block(
                        r[sec["v_codes"][0]:sec["v_codes"][0] + sec["v_codes"][1]].tobytes(), nb)) for r in raws])
                diff = g != exp
                t.coords += g.size
                if diff.any():
                    c = e["codes"][diff]
                    lo = O.requantize_codes(np.maximum(c - 1, 0), ob, nb)
                    hi = O.requantize_codes(np.minimum(c + 1, (1 << ob) - 1), ob, nb)
                    assert np.all(e["near"][diff] & ((g[diff] == lo) | (g[diff] == hi)))
                    t.mismatches += int(diff.sum())
                norm = np.frombuffer(part(f"{which}_norm"), dtype="<f4")
                assert np.allclose(norm, e["norm"], rtol=1e-5, atol=0)
                recon[which] = O.dequantize(e["norm"], g, signs, nb)
            Kh[rows], Vh[rows] = recon["k"], recon["v"]
        compare_attention(out[b, h * G:(h + 1) * G], qh[b, h * G:(h + 1) * G], Kh, Vh, t)
    t.check()
