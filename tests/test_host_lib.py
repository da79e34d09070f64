"""libtq host-side behaviour, no GPU needed: exports, codebooks, layer
randomness, sizes and argument validation (every device call here fails its
host validation before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_srht_amd as tq
import workloads as W
from oracle import tq_oracle as O

HDR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tq.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tq.LIB_PATH):
        from kv_cache_vector_srht_amd import build
        build.build()
    return tq.lib()


def test_exports_every_declared_symbol(L):
    decl = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(tq_[a-z_0-9]+)\s*\(", open(HDR).read(), re.M)
    assert set(decl) == set(tq.EXPORTS)
    for name in decl:
        assert hasattr(L, name)


def test_checked_build_exports_every_declared_symbol(L):
    # the checked build (device index checks) is the same library
    import ctypes
    C = ctypes.CDLL(tq.CHECKED_LIB_PATH)
    for name in tq.EXPORTS:
        assert hasattr(C, name)


def test_release_build_has_no_device_checks(L):
    # no HIP call: a release build answers TQ_ERR_UNSUPPORTED and zero flags
    assert tq.device_checks() is None
    assert L.tq_device_checks(None, 0) == -1   # TQ_ERR_INVALID_ARG: null flags


def test_shaped_encode_rejects_bad_shapes(L):
    # launch shapes are checked on the host before anything else
    for ppb, qw in ((17, 0), (-1, 0), (0, -1)):
        st = L.tq_encode_kv_shaped(None, None, None, ppb, qw, None)
        assert st == -1, (ppb, qw, st)   # TQ_ERR_INVALID_ARG
        assert b"pages_per_block" in tq.lib().tq_last_error() or b"qjl_workgroups" in tq.lib().tq_last_error()


@pytest.mark.parametrize("kind", [tq.LLOYD_MAX, tq.UNIFORM, tq.BETA, tq.POLAR])
@pytest.mark.parametrize("bits", range(1, 9))
def test_codebook_bit_equal_to_oracle(L, bits, kind):
    c, t = tq.build_codebook(bits, kind)
    oc, ot = O.codebook(bits, kind)
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(t.view(np.uint32), ot.view(np.uint32))


@pytest.fixture(scope="module")
def fit_samples():
    """Keys (with outlier channels) and values of a small workload, and the
    oracle's fitted codebooks of each."""
    w = W.make_workload(2, {"n_tokens": 128})
    k, v = W.make_kv(w, 0)
    signs = W.rotation_signs(42, 0)
    out = []
    for x in (k, v):
        X = x.float().numpy().reshape(-1, 128)
        out.append((X, O.fit_codebooks(X, signs)))
    return signs, out


@pytest.mark.parametrize("which", [0, 1])
def test_fitted_codebooks_bit_equal_to_oracle(L, fit_samples, which):
    signs, samples = fit_samples
    X, fc = samples[which]
    tab = tq.calibrated_table(X, signs)
    for b in range(1, 9):
        c, t = tq.fit_codebook(X, signs, b)
        oc, ot = fc.tables[b]
        assert np.array_equal(c.view(np.uint32), oc.view(np.uint32)), b
        assert np.array_equal(t.view(np.uint32), ot.view(np.uint32)), b
        co, to = (1 << b) - 2, 510 + (1 << b) - b - 1
        assert np.array_equal(tab[co:co + (1 << b)], c) and np.array_equal(tab[to:to + (1 << b) - 1], t)
    # zero vectors are skipped; all-zero samples are refused
    Xz = np.concatenate([X, np.zeros((5, 128), np.float32)])
    assert np.array_equal(tq.fit_codebook(Xz, signs, 3)[0], fc.tables[3][0])
    with pytest.raises(tq.TQError):
        tq.fit_codebook(np.zeros((4, 128), np.float32), signs, 2)


@pytest.mark.parametrize("kind", [tq.LLOYD_MAX, tq.UNIFORM, tq.BETA, tq.POLAR, "fitted"])
def test_codebook_table_layout(L, kind, fit_samples):
    if kind == "fitted":
        signs, samples = fit_samples
        X, kind = samples[0]
        tab = tq.calibrated_table(X, signs)
    else:
        tab = tq.codebook_table(kind)
    for b in range(1, 9):
        c, t = O.codebook(b, kind)
        co, to = (1 << b) - 2, 510 + (1 << b) - b - 1
        assert np.array_equal(tab[co:co + (1 << b)], c) and np.array_equal(tab[to:to + (1 << b) - 1], t)
    assert np.all(tab[1012:1024] == 0)
    # pair tables of widths 1..4: (c[lo], c[hi]), or PolarQuant's pair levels
    for b, first in ((1, 0), (2, 4), (3, 20), (4, 84)):
        Lb = 1 << b
        pt = tab[1056 + 2 * first:1056 + 2 * (first + Lb * Lb)].reshape(Lb * Lb, 2)
        lo, hi = np.arange(Lb * Lb) % Lb, np.arange(Lb * Lb) >> b
        if kind is tq.POLAR or (isinstance(kind, int) and kind == tq.POLAR):
            want = O.polar_pairs(b)[lo, hi]
            ulp = np.abs(pt.view(np.int32).astype(np.int64) - want.astype(np.float32).view(np.int32))
            assert np.all((ulp <= 1) | (np.abs(pt - want) < 1e-12)), b
        else:
            c = O.codebook(b, kind)[0]
            assert np.array_equal(pt[:, 0], c[lo]) and np.array_equal(pt[:, 1], c[hi]), b
    # lookup grids: with g = fl32(u S + O) (one fma), code(u) = base + [g >=
    # boundary] at bin floor(g), or at the nearest integer for 256-bin grids
    # (their O carries the -1/2); the boundary is stored as fl32(t S + O)
    words = tab.view(np.uint32)
    rng = np.random.default_rng(0)
    for b in range(1, 5 if kind is tq.POLAR or (isinstance(kind, int) and kind == tq.POLAR) else 9):
        gS, gO = tab[1024 + 4 * (b - 1)], tab[1024 + 4 * (b - 1) + 1]
        nb, off = int(words[1024 + 4 * (b - 1) + 2]), int(words[1024 + 4 * (b - 1) + 3])
        ent = words[off:off + 2 * nb].reshape(nb, 2)
        c, t = O.codebook(b, kind)
        # bin edges of the grid (integer and half-integer index points) and their neighbours
        edges = ((np.arange(-2, nb + 2, 0.5) - np.float64(gO)) / np.float64(gS)).astype(np.float32)
        u = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 2,
                            t, np.nextafter(t, np.float32(-np.inf)), np.nextafter(t, np.float32(np.inf)),
                            edges, np.nextafter(edges, np.float32(-np.inf)), np.nextafter(edges, np.float32(np.inf)),
                            np.float32([-50, 50, 0, -0.0, -11.32, 11.32])]).astype(np.float32)
        # one rounding of the exact u S + O, as the device's fma
        x = (u.astype(np.longdouble) * np.longdouble(gS) + np.longdouble(gO)).astype(np.float32)
        xb = x.astype(np.float64)
        if nb == 256:   # byte grid: round half to even, saturate to [0, 255]
            bins = np.clip(np.rint(xb), 0, 255).astype(np.int64)
        else:
            bins = np.clip(np.trunc(xb).astype(np.int64), 0, nb - 1)
        got = ent[bins, 0] + (x >= ent[bins, 1].view(np.float32))
        want = np.searchsorted(t, u, side="right")
        # the stored boundary is the grid coordinate of t rounded the same way
        nz = ent[:, 1].view(np.float32) < 1e38
        tw = (t.astype(np.longdouble) * np.longdouble(gS) + np.longdouble(gO)).astype(np.float32)
        assert np.all(np.isin(ent[nz, 1].view(np.float32), tw)), b
        # exact on the boundaries themselves (a tie is a tie) and away from
        # them; within 1e-6 of a boundary (the parity allowance) the rounding
        # of g may take the neighbouring level
        diff = got != want
        assert not diff[np.isin(u, t)].any(), b
        dist = np.min(np.abs(u[:, None].astype(np.float64) - t[None, :].astype(np.float64)), axis=1)
        assert np.all(~diff | ((dist <= 1e-6) & (np.abs(got.astype(np.int64) - want) == 1))), b


@pytest.mark.parametrize("shift", [-3, -1, 0, 1, 2, 3])
def test_polar_table_with_angle_shift(L, shift):
    """tq_polar_table: Rayleigh levels at every width, pair tables of widths
    1..4 indexed by the pair field rc | tc << (b - shift) equal to the oracle's
    (to 1 ulp: both round the exact product), the shift in the last entry, and
    radius lookup grids at the widths the pages use."""
    tab = tq.polar_table(shift)
    assert tab[-1] == shift
    if shift == 0:
        assert np.array_equal(tab, tq.codebook_table(tq.POLAR))
    for b in range(1, 9):
        c, t = O.codebook(b, O.POLAR)
        co, to = (1 << b) - 2, 510 + (1 << b) - b - 1
        assert np.array_equal(tab[co:co + (1 << b)], c) and np.array_equal(tab[to:to + (1 << b) - 1], t)
    for b, first in ((1, 0), (2, 4), (3, 20), (4, 84)):
        n = 1 << (2 * b)
        pt = tab[1056 + 2 * first:1056 + 2 * (first + n)].reshape(n, 2)
        try:
            want = O.polar_pair_table(b, shift)
        except ValueError:          # this width cannot carry the shift: no table
            assert np.all(pt == 0)
            continue
        ulp = np.abs(pt.view(np.int32).astype(np.int64) - want.view(np.int32))
        assert np.all((ulp <= 1) | (np.abs(pt - want) < 1e-12)), b
    words = tab.view(np.uint32)
    for r in range(1, 5 - min(shift, 0)):
        assert int(words[1024 + 4 * (r - 1) + 2]) > 0, r       # a radius grid at width r
    with pytest.raises(tq.TQError):
        tq.polar_table(4)


@pytest.mark.parametrize("layer", [0, 1, 35])
def test_layer_params_match_generator(L, layer):
    s, S = tq.layer_params(42, layer)
    assert np.array_equal(s, W.rotation_signs(42, layer))
    assert np.array_equal(S.view(np.uint32), W.qjl_matrix(42, layer).view(np.uint32))


def test_sign_mask(L):
    s = W.rotation_signs(42, 0)
    m = tq.sign_mask(s)
    for j in range(128):
        assert ((int(m[j // 32]) >> (j % 32)) & 1) == (1 if s[j] < 0 else 0)
    with pytest.raises(tq.TQError):
        tq.sign_mask(np.zeros(128, np.int8))


def test_page_sizes_match_oracle(L):
    for fmt in [(0, 0, False), (1, 1, False), (3, 2, False), (2, 2, True), (8, 8, True), (4, 4, False)]:
        assert tq.page_bytes(fmt) == O.page_bytes(fmt)
    assert L.tq_page_bytes(9, 1, 0) == 0 and L.tq_page_bytes(0, 1, 0) == 0 and L.tq_page_bytes(2, 0, 0) == 0


def test_page_descriptor_bits(L):
    d = L.tq_page_descriptor(256 * 7, 3, 2, 1)
    assert d == (256 * 7) | (3 << 48) | (2 << 52) | (1 << 56) | (1 << 63)
    assert L.tq_page_descriptor(100, 3, 2, 0) == 0          # not 256-aligned
    assert L.tq_page_descriptor(1 << 48, 3, 2, 0) == 0      # past 48 bits
    assert L.tq_page_descriptor(0, 0, 0, 0) == 1 << 63      # fp16 page at offset 0


def test_cache_bytes_and_workspace(L):
    fm = [[[W.FP16, (3, 2, False), (2, 2, True)]]]
    desc = np.array([L.tq_page_descriptor(0, 0, 0, 0), L.tq_page_descriptor(32768, 3, 2, 0),
                     L.tq_page_descriptor(32768 + 5632, 2, 2, 1), 0], dtype=np.uint64)
    assert L.tq_cache_bytes(desc.ctypes.data, 4) == O.cache_bytes(fm[0][0])
    c = tq.tq_cache(4, 8, 512, 0, None, None, None, 0)
    n = L.tq_decode_workspace_bytes(ctypes.byref(c), 32)
    # 32 units x 512 pages over ~1024 groups: 16 pages per split, 32 splits;
    # room for wide ranges down to a quarter of that (a merged launch may
    # shorten them), other ranges half as long
    assert n == 4 * (4 * 32 * 384 + 4 * 32 * (32 + 128 + 64) * 132)
    # one unit of 300000 pages: ranges are capped at 256 pages (the split
    # kernel keeps a range's descriptors in LDS): 1172 common, 4688 wide
    # (64-page) and 2344 other (128-page) ranges
    big = tq.tq_cache(1, 1, 300000, 0, None, None, None, 0)
    assert L.tq_decode_workspace_bytes(ctypes.byref(big), 1) == 4 * (384 + (1172 + 4688 + 2344) * 132)
    c0 = tq.tq_cache(0, 8, 512, 0, None, None, None, 0)
    assert L.tq_decode_workspace_bytes(ctypes.byref(c0), 32) == 0


def _fake_layer(**kw):
    base = dict(head_dim=128, k_codebook=0, v_codebook=0, jl_dim=128, sign_mask=0x1000,
                k_table=0x2000, v_table=0x3000, qjl_s=None)
    base.update(kw)
    return tq.tq_layer(**base)


def _fake_cache(**kw):
    base = dict(n_sessions=1, n_kv_heads=8, max_pages=4, page_classes=0, n_tokens=0x4000,
                pages=0x5000, pool=0x100000, pool_bytes=1 << 20)
    base.update(kw)
    return tq.tq_cache(**base)


def _encode(L, layer, cache, **kw):
    base = dict(k=0x10000, v=0x20000, dtype=1, tok0=0, ntok=64, reserved=0, stride_b=8 * 64 * 128,
                stride_h=64 * 128, stride_t=128, error_flags=None)
    base.update(kw)
    inp = tq.tq_kv_input(**base)
    return L.tq_encode_kv(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(inp), None)


def test_encode_validation(L):
    bad = [
        (dict(layer=_fake_layer(head_dim=64)), -2),
        (dict(layer=_fake_layer(k_codebook=5)), -1),
        (dict(layer=_fake_layer(sign_mask=0x1004)), -3),
        (dict(layer=_fake_layer(qjl_s=0x6000, jl_dim=64)), -2),
        (dict(cache=_fake_cache(n_sessions=0)), -1),
        (dict(cache=_fake_cache(pool=0x100010)), -3),
        (dict(cache=_fake_cache(pages=None)), -1),
        (dict(inp=dict(tok0=32)), -1),
        (dict(inp=dict(ntok=0)), -1),
        (dict(inp=dict(ntok=4 * 64 + 1)), -1),
        (dict(inp=dict(dtype=7)), -1),
        (dict(inp=dict(k=0x10002)), -3),
        (dict(inp=dict(stride_t=100)), -3),
        (dict(inp=dict(stride_t=-128)), -1),
        (dict(inp=dict(v=None)), -1),
    ]
    for case, want in bad:
        layer = case.get("layer", _fake_layer())
        cache = case.get("cache", _fake_cache())
        st = _encode(L, layer, cache, **case.get("inp", {}))
        assert st == want, (case, st, L.tq_last_error())
        assert L.tq_last_error()
    assert L.tq_encode_kv(None, None, None, None) == -1


def _decode(L, layer, cache, ws_bytes=1 << 30, **kw):
    base = dict(q=0x30000, dtype=1, n_q_heads=32, stride_b=32 * 128, stride_h=128, softmax_scale=0.0,
                qjl_scoring=0)
    base.update(kw)
    qq = tq.tq_query(**base)
    return L.tq_decode_attention(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(qq),
                                 ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000), ws_bytes, None)


def test_decode_validation(L):
    cases = [
        (dict(kw=dict(n_q_heads=12)), -1),     # not a multiple of 8 KV heads
        (dict(kw=dict(n_q_heads=8 * 16)), -2),  # group 16
        (dict(kw=dict(dtype=5)), -1),
        (dict(kw=dict(softmax_scale=float("nan"))), -1),
        (dict(kw=dict(qjl_scoring=2)), -1),
        (dict(kw=dict(q=None)), -1),
        (dict(ws=16), -4),
        (dict(layer=_fake_layer(head_dim=256)), -2),
        (dict(cache=_fake_cache(page_classes=8)), -1),
    ]
    # a per-unit class record with an unknown bit (unit 7 of 8)
    bad_units = (ctypes.c_uint8 * 8)(1, 1, 2, 4, 7, 0, 1, 8)
    cases.append((dict(cache=_fake_cache(unit_classes=ctypes.addressof(bad_units))), -1))
    for case, want in cases:
        st = _decode(L, case.get("layer", _fake_layer()), case.get("cache", _fake_cache()),
                     case.get("ws", 1 << 30), **case.get("kw", {}))
        assert st == want, (case, st, L.tq_last_error())
    assert b"unit 7" in L.tq_last_error()


def test_decode_mass_validation(L):
    """tq_decode_attention_mass: its own argument errors, then the decode ones."""
    lay, cac = _fake_layer(), _fake_cache()
    qq = tq.tq_query(q=0x30000, dtype=1, n_q_heads=32, stride_b=32 * 128, stride_h=128,
                     softmax_scale=0.0, qjl_scoring=0)

    def call(mass, ws_bytes=1 << 30, query=qq):
        return L.tq_decode_attention_mass(ctypes.byref(lay), ctypes.byref(cac), ctypes.byref(query),
                                          ctypes.c_void_p(0x40000), mass, ctypes.c_void_p(0x50000),
                                          ws_bytes, None)
    assert call(None) == -1
    assert call(ctypes.c_void_p(0x60002)) == -3
    assert call(ctypes.c_void_p(0x60000), ws_bytes=16) == -4
    bad = tq.tq_query(q=0x30000, dtype=1, n_q_heads=12, stride_b=0, stride_h=128, softmax_scale=0.0,
                      qjl_scoring=0)
    assert call(ctypes.c_void_p(0x60000), query=bad) == -1


def _append(L, layer, cache, **kw):
    base = dict(k=0x10000, v=0x20000, dtype=1, reserved=0, stride_b=8 * 128, stride_h=128, error_flags=None)
    base.update(kw)
    inp = tq.tq_token_input(**base)
    return L.tq_append_kv(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(inp), None)


def test_append_validation(L):
    cases = [
        (dict(kw=dict(dtype=3)), -1),
        (dict(kw=dict(k=None)), -1),
        (dict(kw=dict(v=0x20008)), -3),
        (dict(kw=dict(stride_h=100)), -3),
        (dict(kw=dict(stride_b=-128)), -1),
        (dict(kw=dict(error_flags=0x70002)), -3),
        (dict(layer=_fake_layer(head_dim=64)), -2),
        (dict(cache=_fake_cache(pool=None)), -1),
    ]
    for case, want in cases:
        st = _append(L, case.get("layer", _fake_layer()), case.get("cache", _fake_cache()), **case.get("kw", {}))
        assert st == want, (case, st, L.tq_last_error())
    assert L.tq_append_kv(None, None, None, None) == -1


def test_retier_validation(L):
    """tq_retier_pages: argument errors found on the host (no launch)."""
    lay, cac = _fake_layer(), _fake_cache()
    idx, desc = ctypes.c_void_p(0x70000), ctypes.c_void_p(0x71000)

    def call(layer=lay, cache=cac, i=idx, d=desc, n=4, err=None, sources=0):
        return L.tq_retier_pages(ctypes.byref(layer) if layer is not None else None,
                                 ctypes.byref(cache) if cache is not None else None, i, d, n, sources,
                                 err, None)
    assert call(n=-1) == -1
    assert call(sources=4) == -1
    assert call(n=0) == 0                      # nothing to do, nothing launched
    assert call(i=None) == -1 and call(d=None) == -1
    assert call(i=ctypes.c_void_p(0x70004)) == -3
    assert call(d=ctypes.c_void_p(0x71004)) == -3
    assert call(err=ctypes.c_void_p(0x72002)) == -3
    assert call(layer=_fake_layer(head_dim=64)) == -2
    assert call(cache=_fake_cache(page_classes=16)) == -1
    assert call(layer=None) == -1 and call(cache=None) == -1


def test_pending_pages_in_the_footprint(L):
    d = [L.tq_page_descriptor(0, 3, 2, 0), L.tq_page_descriptor(256 * 128, 3, 2, 0) | tq.PAGE_PENDING]
    arr = np.array(d, dtype=np.uint64)
    assert L.tq_cache_bytes(arr.ctypes.data, 2) == tq.page_bytes((3, 2, False)) + tq.page_bytes((0, 0, False))
    assert tq.page_bytes((3, 2, False, True)) == tq.page_bytes((0, 0, False))
    with pytest.raises(tq.TQError):
        tq.page_bytes((0, 0, False, True))


def test_dequantize_validation(L):
    out = ctypes.c_void_p(0x60000)
    lay, cac = _fake_layer(), _fake_cache()
    assert L.tq_dequantize(ctypes.byref(lay), ctypes.byref(cac), 2, 1, 0, 64, out, None) == -1
    assert L.tq_dequantize(ctypes.byref(lay), ctypes.byref(cac), 0, 1, 0, 0, out, None) == -1
    assert L.tq_dequantize(ctypes.byref(lay), ctypes.byref(cac), 0, 1, 0, 4 * 64 + 1, out, None) == -1
    assert L.tq_dequantize(ctypes.byref(lay), ctypes.byref(cac), 0, 1, 0, 64, ctypes.c_void_p(0x60004), None) == -3
    assert L.tq_dequantize(ctypes.byref(lay), ctypes.byref(cac), 0, 1, 0, 64, None, None) == -1


def test_status_strings(L):
    assert L.tq_status_string(0) == b"ok" and L.tq_status_string(-4) == b"workspace too small"


def test_page_classes_bits():
    import kv_cache_vector_srht_amd as tq
    assert tq.page_classes([[[W.packed(3, 2, False), W.packed(1, 1, False)]]]) == tq.CACHE_COMMON_PAGES
    assert tq.page_classes([[[W.FP16, W.packed(2, 2, True)]]]) == tq.CACHE_OTHER_PAGES
    assert tq.page_classes([[[W.packed(4, 4, False)], [W.packed(8, 8, False)]]]) == \
        tq.CACHE_COMMON_PAGES | tq.CACHE_WIDE_PAGES
    assert tq.page_classes([[[W.packed(4, 6, False), W.packed(6, 6, True)]]]) == tq.CACHE_OTHER_PAGES
    assert tq.page_classes([[[(3, 2, False, True)]]]) == tq.CACHE_COMMON_PAGES | tq.CACHE_OTHER_PAGES
    w3 = W.make_workload(3, {"n_tokens": 128, "batch": 1})
    assert tq.page_classes(w3.formats[0]) == tq.CACHE_COMMON_PAGES
    assert tq.page_classes(w3.formats[2]) == tq.CACHE_COMMON_PAGES | tq.CACHE_WIDE_PAGES


def test_unit_classes_record():
    """Per (session, KV head) classes; their union is the cache's page classes."""
    import numpy as np
    import kv_cache_vector_srht_amd as tq
    fm = [[[W.packed(3, 2)], [W.packed(8, 6), W.FP16], [W.packed(2, 2, True)], [(3, 2, False, True)]]]
    got = tq.unit_classes(fm)
    assert got.dtype == np.uint8 and got.shape == (1, 4)
    assert got.tolist() == [[tq.CACHE_COMMON_PAGES, tq.CACHE_WIDE_PAGES | tq.CACHE_OTHER_PAGES,
                             tq.CACHE_OTHER_PAGES, tq.CACHE_COMMON_PAGES | tq.CACHE_OTHER_PAGES]]
    w3 = W.make_workload(3, {"n_tokens": 128, "batch": 2})
    for l in range(w3.n_layers):
        u = tq.unit_classes(w3.formats[l])
        assert int(np.bitwise_or.reduce(u.reshape(-1))) == tq.page_classes(w3.formats[l])
        # the hub heads hold the wide pages, the same heads in every session
        assert (u[0] == u[1]).all()

