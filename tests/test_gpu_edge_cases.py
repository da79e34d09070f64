"""GPU parity on the method's degenerate cases, through every GPU encoder:
zero-norm rows and rows whose rotated coordinates sit exactly on a decision
boundary (the zero vector gives u = 0; sums of a few basis vectors and the
scaled sign vector give exact zeros, the middle boundary of every even number
of levels).  The codes of those rows must be the oracle's bit for bit, not
merely within the boundary allowance: the tie rule code = #{t_k <= u} is a
reading of the pages' silence, and a tie is a tie on both sides.  Paths: the
bulk encoder (tq_encode_kv, fp16 and fp32 inputs), the decode loop's packing of
a full tail page (tq_append_kv) and fp16-to-packed re-tiering
(tq_retier_pages).  Also decode attention with a caller's softmax scale and
with a zero query (uniform weights: the mean of the values)."""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import (NORM_ULPS, Tally, _cmp_codes, compare_attention, compare_unit_full, ulps32)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_SPECIAL = 8


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_srht_amd as tq
    tq.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().cpu().numpy()


def _inputs(w, signs, dev):
    """The workload's keys and values with the degenerate rows in the first
    N_SPECIAL tokens of every page (as keys and as values)."""
    k, v = W.make_kv(w, 0, device=dev)
    X = torch.as_tensor(W.degenerate_rows(signs), dtype=k.dtype, device=dev)
    for p in range(w.n_tokens // 64):
        k[:, :, 64 * p:64 * p + N_SPECIAL] = X
        v[:, :, 64 * p:64 * p + N_SPECIAL] = X.flip(0)
    return k, v


def check_page_exact(raw, fmt, K64, V64, signs, S, k_kind, v_kind, t, what):
    """One packed page against the oracle: the degenerate rows bit for bit
    (codes, norms, and for keys with QJL the sketch of the zero rows: every
    sign +1 and gamma 0), the other rows under the usual allowance."""
    kb, vb, qjl = fmt
    sec = O.page_sections(fmt)

    def part(name):
        o, n = sec[name]
        return raw[o:o + n].tobytes()
    sp = slice(0, N_SPECIAL)
    for which, X, bits, kind, codes in (
            ("K", K64, kb, k_kind, O.unpack_block(part("k_codes"), kb)),
            ("V", V64, vb, v_kind, O.v_codes_from_streams(O.unpack_block(part("v_codes"), vb)))):
        e = O.encode(X, signs, bits, kind)
        exact = np.ones((N_SPECIAL, O.HEAD_DIM), dtype=bool)
        if kind == O.POLAR:
            # angle codes: exact only for a pair that is exactly zero (the
            # angle of (0, 0) is atan2(+0, +0) = 0, sector L/2); a nonzero pair
            # on an axis or diagonal lies on a sector edge, whose side float
            # rounding decides on both sides (the angle allowance)
            U = e["u"][sp]
            exact[:, 1::2] = (U[:, 0::2] == 0) & (U[:, 1::2] == 0)
        got_sp = np.where(exact, codes[sp], -1)
        want_sp = np.where(exact, e["codes"][sp], -1)
        # (edge pairs are structural ties, not rare rounding cases: they are
        # held to the one-level rule but kept out of the mismatch fraction)
        _cmp_codes(codes[sp], e["codes"][sp], e["near"][sp] & ~exact, Tally(), f"{what} {which} (edge pairs)",
                   0, [], kind, bits)
        bad = np.argwhere(got_sp != want_sp)
        assert bad.size == 0, (f"{what} {which}: degenerate rows differ at {bad[:4].tolist()} "
                               f"(got {got_sp[tuple(bad[:4].T)]}, want {want_sp[tuple(bad[:4].T)]})")
        _cmp_codes(codes[N_SPECIAL:], e["codes"][N_SPECIAL:], e["near"][N_SPECIAL:], t,
                   f"{what} {which}", 0, [], kind, bits)
        t.coords += codes[sp].size
        norm = np.frombuffer(part("k_norm" if which == "K" else "v_norm"), dtype="<f4")
        assert np.array_equal(norm[sp], e["norm"][sp]), f"{what} {which}: norms {norm[sp]} vs {e['norm'][sp]}"
        t.worst_norm_ulp = max(t.worst_norm_ulp, ulps32(norm, e["norm"]))
        assert ulps32(norm, e["norm"]) <= NORM_ULPS, f"{what} {which} norms"
        if which == "K" and qjl:
            kh = O.dequantize(e["norm"], e["codes"], signs, bits, kind)
            qj = O.qjl_encode(X, kh, S)
            z = O.unpack_signs(part("qjl_signs"))
            g = np.frombuffer(part("qjl_gamma"), dtype="<f4")
            zero = np.linalg.norm(X, axis=1) == 0
            assert np.all(z[zero]) and np.all(g[zero] == 0), f"{what}: sketch of a zero row"
            assert np.all(qj["z"][zero]) and np.all(qj["gamma"][zero] == 0)
            ok = ~zero
            assert not ((z[ok] != qj["z"][ok]) & ~qj["near"][ok]).any(), f"{what}: QJL signs"


def _formats_all_widths(qjl_head1, polar=False):
    widths = range(1, 5) if polar else range(1, 9)
    combos = [(kb, vb) for kb in widths for vb in widths]
    P = len(combos) // 2 + 2
    return [[[W.packed(*combos[(p + 7 * h) % len(combos)], qjl_head1 and h == 1)
              for p in range(P)] for h in range(2)]]


@pytest.mark.parametrize("dtype,kind,qjl", [("float16", O.LLOYD_MAX, True), ("float32", O.LLOYD_MAX, True),
                                            ("float16", O.UNIFORM, False), ("float16", O.BETA, True),
                                            ("float16", O.POLAR, False)])
def test_degenerate_rows_bulk_encoder(dev, dtype, kind, qjl):
    import kv_cache_vector_srht_amd as tq
    fm = _formats_all_widths(qjl, polar=kind == O.POLAR)
    P = len(fm[0][0])
    w = W.make_workload(2, {"n_tokens": 64 * P, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8,
                            "sink_tokens": 0, "dtype": dtype})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S if qjl else None, kind, kind)
    cache = tq.Cache(fm, [w.n_tokens], dev)
    k, v = _inputs(w, signs, dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"bulk encode {dtype} kind {kind} qjl {qjl}: {P} pages x 2 heads", flush=True)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    pool = _np(cache.pool)
    kh, vh = _np(k).astype(np.float64), _np(v).astype(np.float64)
    t = Tally()
    for h in range(2):
        for p, fmt in enumerate(fm[0][h]):
            off = int(cache.offsets[0, h, p])
            rows = slice(64 * p, 64 * p + 64)
            check_page_exact(pool[off:off + O.page_bytes(fmt)], fmt, kh[0, h, rows], vh[0, h, rows], signs, S,
                             kind, kind, t, f"page (0,{h},{p}) fmt {fmt}")
    t.check()


def test_degenerate_rows_decode_loop_packing(dev):
    """Tail pages filled one token per step by tq_append_kv; each is packed in
    place (per-token encoder) when its 64th token arrives."""
    import kv_cache_vector_srht_amd as tq
    targets = [[W.packed(3, 2), W.packed(1, 1), W.packed(8, 8), W.packed(4, 4)],
               [W.packed(2, 2, True), W.packed(5, 3, True), W.packed(2, 1), W.packed(6, 6)]]
    P = 1 + len(targets[0])
    fm = [[[W.FP16] + [(f[0], f[1], f[2], True) for f in targets[h]] for h in range(2)]]
    w = W.make_workload(2, {"n_tokens": 64 * P, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8,
                            "sink_tokens": 64, "dtype": "float16"})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, [64], dev)
    k, v = _inputs(w, signs, dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k[:, :, :64], v[:, :, :64], error_flags=flags)
    print(f"append {64 * (P - 1)} tokens", flush=True)
    for n in range(64, 64 * P):
        tq.append_kv(layer, cache, k[:, :, n].contiguous(), v[:, :, n].contiguous(), error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    desc = _np(cache.pages).view(np.uint64)
    assert not any(int(desc[0, h, p]) >> 57 & 1 for h in range(2) for p in range(P))
    pool = _np(cache.pool)
    kh, vh = _np(k).astype(np.float64), _np(v).astype(np.float64)
    t = Tally()
    for h in range(2):
        for p in range(1, P):
            fmt = targets[h][p - 1]
            off = int(cache.offsets[0, h, p])
            rows = slice(64 * p, 64 * p + 64)
            check_page_exact(pool[off:off + O.page_bytes(fmt)], fmt, kh[0, h, rows], vh[0, h, rows], signs, S,
                             O.LLOYD_MAX, O.LLOYD_MAX, t, f"appended page (0,{h},{p}) fmt {fmt}")
    t.check()


def test_degenerate_rows_retier_from_fp16(dev):
    """fp16 pages (copies of the rows) encoded into packed formats by
    tq_retier_pages, as the pages' tiering moves a chunk out of fp16."""
    import kv_cache_vector_srht_amd as tq
    targets = [[W.packed(4, 4), W.packed(2, 1, True), W.packed(7, 5), W.packed(1, 2)],
               [W.packed(3, 3, True), W.packed(1, 1), W.packed(8, 6, True), W.packed(2, 4)]]
    P = len(targets[0])
    fm = [[[W.FP16] * P for _ in range(2)]]
    w = W.make_workload(2, {"n_tokens": 64 * P, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8,
                            "sink_tokens": 0, "dtype": "float16"})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, [w.n_tokens], dev)
    k, v = _inputs(w, signs, dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    pages = [(0, h, p) for h in range(2) for p in range(P)]
    print(f"retier {len(pages)} fp16 pages", flush=True)
    tq.retier_pages(layer, cache, pages, [targets[h][p] for _, h, p in pages], error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    pool = _np(cache.pool)
    kh, vh = _np(k).astype(np.float64), _np(v).astype(np.float64)
    t = Tally()
    for _, h, p in pages:
        fmt = targets[h][p]
        off = int(cache.offsets[0, h, p])
        rows = slice(64 * p, 64 * p + 64)
        check_page_exact(pool[off:off + O.page_bytes(fmt)], fmt, kh[0, h, rows], vh[0, h, rows], signs, S,
                         O.LLOYD_MAX, O.LLOYD_MAX, t, f"re-tiered page (0,{h},{p}) fmt {fmt}")
    t.check()


def _decode_setup(dev, zero_query=False):
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(2, {"n_tokens": 64 * 7 + 21, "batch": 2, "n_kv_heads": 2, "n_q_heads": 8,
                            "sink_tokens": 64})
    fm = w.formats[0]
    for h in range(2):   # head 1 carries QJL keys and a wide page
        fm[0][h] = [f if f[0] == 0 else (W.packed(2, 2, True) if h == 1 else f) for f in fm[0][h]]
        fm[1][h] = [f if (f[0] == 0 or p != 3) else W.packed(6, 7) for p, f in enumerate(fm[1][h])]
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    n_tok = [w.n_tokens, 64 * 5]           # a ragged pair of sessions
    cache = tq.Cache(fm, n_tok, dev)
    k, v = _inputs(w, signs, dev)
    q = W.make_query(w, 0, device=dev)
    if zero_query:
        q.zero_()
    tq.encode_kv(layer, cache, k, v)
    return w, fm, signs, S, layer, cache, k, v, q, n_tok


def _reference_units(w, fm, signs, S, cache, k, v, n_tok, t):
    pool = _np(cache.pool)
    kh, vh = _np(k).astype(np.float64), _np(v).astype(np.float64)
    out = {}
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            n = n_tok[b]
            out[b, h] = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n], vh[b, h, :n], fm[b][h],
                                          signs, S, t)
    return out


@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_decode_with_softmax_scale(dev, scale):
    """out = softmax(scale q . k) . v for a caller's scale (0 selects 1/sqrt(d)),
    and the page masses with the same scale."""
    import kv_cache_vector_srht_amd as tq
    w, fm, signs, S, layer, cache, k, v, q, n_tok = _decode_setup(dev)
    mass = torch.zeros((w.batch, w.n_q_heads, cache.max_pages), dtype=torch.float32, device=dev)
    print(f"decode softmax_scale {scale}", flush=True)
    out = _np(tq.decode_attention(layer, cache, q, softmax_scale=scale))
    out_m = _np(tq.decode_attention(layer, cache, q, softmax_scale=scale, page_mass=mass))
    torch.cuda.synchronize()
    assert np.array_equal(out, out_m)
    t = Tally()
    ref = _reference_units(w, fm, signs, S, cache, k, v, n_tok, t)
    qh = _np(q).astype(np.float64)
    m = _np(mass)
    G = w.n_q_heads // w.n_kv_heads
    for (b, h), (Kh, Vh) in ref.items():
        rows = slice(h * G, (h + 1) * G)
        exp = np.stack([O.attention(qq, Kh, Vh, scale) for qq in qh[b, rows]])
        err = np.abs(out[b, rows] - exp).max(axis=1) / np.abs(exp).max(axis=1)
        t.worst_attn = max(t.worst_attn, float(err.max()))
        pm = O.page_attention_mass(qh[b, rows], Kh, scale)
        got = m[b, rows, :pm.shape[1]]
        assert np.all(np.abs(got - pm) <= 1e-3 * pm + 1e-6), f"page mass ({b},{h})"
    t.check()


def test_decode_zero_query(dev):
    """q = 0: every score is 0, the weights are uniform and the output is the
    mean of the values (fp16 rows, dequantised packed rows)."""
    import kv_cache_vector_srht_amd as tq
    w, fm, signs, S, layer, cache, k, v, q, n_tok = _decode_setup(dev, zero_query=True)
    print("decode zero query", flush=True)
    out = _np(tq.decode_attention(layer, cache, q))
    torch.cuda.synchronize()
    t = Tally()
    ref = _reference_units(w, fm, signs, S, cache, k, v, n_tok, t)
    G = w.n_q_heads // w.n_kv_heads
    for (b, h), (Kh, Vh) in ref.items():
        mean = Vh.mean(axis=0)
        rows = out[b, h * G:(h + 1) * G]
        err = np.abs(rows - mean[None, :]).max(axis=1) / np.abs(mean).max()
        t.worst_attn = max(t.worst_attn, float(err.max()))
        compare_attention(rows, np.zeros((G, 128)), Kh, Vh, t)
    t.check()


@pytest.mark.parametrize("qjl", [False, True])
def test_subnormal_rows_bulk_encoder(dev, qjl):
    """Rows whose fp16 values all lie in fp16's subnormal range (multiples of
    2^-24 below 2^-14): their norms and codes follow the oracle under the usual
    allowance, so no step of the encoders (the norm's products included)
    flushes them to zero."""
    import kv_cache_vector_srht_amd as tq
    fm = _formats_all_widths(qjl)
    P = len(fm[0][0])
    w = W.make_workload(2, {"n_tokens": 64 * P, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8, "sink_tokens": 0})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S if qjl else None)
    cache = tq.Cache(fm, [w.n_tokens], dev)
    k, v = W.make_kv(w, 0, device=dev)
    rng = np.random.default_rng(7)
    for p in range(P):
        for x in (k, v):
            sub = rng.integers(-1000, 1001, size=(1, 2, N_SPECIAL, 128)).astype(np.float64) * 2.0 ** -24
            x[:, :, 64 * p:64 * p + N_SPECIAL] = torch.as_tensor(sub, dtype=x.dtype, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"bulk encode of subnormal rows, qjl {qjl}: {P} pages x 2 heads", flush=True)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    kh, vh = _np(k).astype(np.float64), _np(v).astype(np.float64)
    assert np.all(np.abs(kh[0, :, :N_SPECIAL]) < 2.0 ** -14) and np.any(kh[0, :, :N_SPECIAL] != 0)
    pool = _np(cache.pool)
    t = Tally()
    for h in range(2):
        compare_unit_full(pool, cache.offsets, 0, h, kh[0, h], vh[0, h], fm[0][h], signs, S if qjl else None, t)
    t.check()
