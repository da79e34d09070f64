"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Sizes here span several pages, heads and sessions with
ragged tails; tests/test_gpu_fullsize.py covers the full workload sizes on
sampled units."""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import (Tally, compare_attention, compare_dequant, compare_unit_full, compare_unit_pages,
                               layer_args)

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


def run_case(w, layers, dev, units=None, n_tokens=None, dequant=True, chunks=None, tally=None,
             query_dtype=None, layer_kw=None, qjl_s=None, query_scale=None):
    """Encode + decode every listed layer of workload w on the GPU; compare the
    listed units (all by default) with the oracle.  ``qjl_s`` replaces the
    seeded QJL matrix of layers with QJL pages; ``query_scale`` multiplies the
    query (after its cast to ``query_dtype``)."""
    import kv_cache_vector_srht_amd as tq
    t = tally or Tally()
    G = w.n_q_heads // w.n_kv_heads
    for l in layers:
        fm = w.formats[l]
        has_qjl = any(f[2] for row in fm for r in row for f in r)
        signs = W.rotation_signs(W.ROTATION_SEED, l)
        S = (qjl_s if qjl_s is not None else W.qjl_matrix(W.ROTATION_SEED, l)) if has_qjl else None
        if layer_kw is None:
            layer = tq.Layer(signs, dev, S, **layer_args(w.k_codebook, w.v_codebook))
        else:
            layer = tq.Layer(signs, dev, S, **layer_kw)
        ntoks = n_tokens or [w.n_tokens] * w.batch
        cache = tq.Cache(fm, ntoks, dev)
        k, v = W.make_kv(w, l, device=dev)
        q = W.make_query(w, l, device=dev)
        if query_dtype is not None:
            q = q.to(query_dtype)
        if query_scale is not None:
            q = q * query_scale
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
        if chunks:
            for t0, t1 in chunks:
                tq.encode_kv(layer, cache, k[:, :, t0:t1], v[:, :, t0:t1], tok0=t0, error_flags=flags)
        else:
            tq.encode_kv(layer, cache, k, v, tok0=0, error_flags=flags)
        out = _np(tq.decode_attention(layer, cache, q))
        dk = _np(tq.dequantize(layer, cache, 0, 0, w.n_tokens)) if dequant else None
        dv = _np(tq.dequantize(layer, cache, 1, 0, w.n_tokens)) if dequant else None
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, f"encode error flags {int(flags.item())}"
        kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
        pool = _np(cache.pool)
        for (b, h) in (units or [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]):
            T = ntoks[b]
            k_ok, v_ok, k_alt, v_alt, z_alt = compare_unit_pages(cache, b, h, kh[b, h], vh[b, h], fm[b][h],
                                                          signs, S, t, w.k_codebook, w.v_codebook,
                                                          n_tokens=w.n_tokens, pool_host=pool)
            # the oracle's encoding under the admissible boundary tie-breaks and
            # near-zero QJL signs taken above
            Kh, Vh = O.reconstruct_unit(kh[b, h, :T], vh[b, h, :T], fm[b][h], signs, S,
                                        w.k_codebook, w.v_codebook, k_alt, v_alt, z_alt)
            rows = out[b, h * G:(h + 1) * G]
            if T == 0:
                assert np.all(rows == 0)
            else:
                compare_attention(rows, qh[b, h * G:(h + 1) * G], Kh, Vh, t)
            if dequant and T > 0:
                Kf, Vf = O.reconstruct_unit(kh[b, h], vh[b, h], fm[b][h], signs, S,
                                            w.k_codebook, w.v_codebook, k_alt, v_alt, z_alt)
                compare_dequant(dk[b, h], Kf, t)
                compare_dequant(dv[b, h], Vf, t)
    t.check()
    return t


def test_workload1_single_head_fp32(dev):
    run_case(W.make_workload(1), [0], dev)


def test_workload2_llama_layer_chunked(dev):
    w = W.make_workload(2)
    chunks = [(0, 128)] + [(t0, t0 + 64) for t0 in range(128, 4096, 64)]
    run_case(w, [0], dev, chunks=chunks)


def test_workload3_per_head_bits_ragged(dev):
    w = W.make_workload(3, {"n_tokens": 64 * 9 + 17, "batch": 2})
    # layers whose heads cover hub (6-8), peripheral (1-2) and base (3/2) widths
    run_case(w, [0, 1, 2], dev)


def test_workload4_qjl_sink_ragged(dev):
    w = W.make_workload(4, {"n_tokens": 64 * 6 + 5, "batch": 2})
    run_case(w, [0], dev)


def test_workload5_tiers_demotion(dev):
    w = W.make_workload(5, {"n_tokens": 64 * 1100 + 33, "batch": 1})
    fm = w.formats[0][0][0]
    # fp16 newest tier, three packed tiers (some pages demoted), ragged fp16 tail
    assert len({f for f in fm if f[0]}) >= 3 and fm[-1] == W.FP16 and fm[-17] == W.FP16
    run_case(w, [0], dev, units=[(0, h) for h in range(8)], dequant=False)


def _all_bits_workload(G=4, dtype="float16", kind=O.LLOYD_MAX, pages=66, qjl=False):
    w = W.make_workload(2, {"n_tokens": 64 * pages, "batch": 1, "n_kv_heads": 2,
                            "n_q_heads": 2 * G, "sink_tokens": 0, "dtype": dtype})
    combos = [(kb, vb) for kb in range(1, 9) for vb in range(1, 9)]
    w.k_codebook = w.v_codebook = kind
    w.formats = [[[[W.packed(*combos[(p + 7 * h) % 64], qjl) if p > 0 else W.FP16
                    for p in range(pages)] for h in range(2)]]]
    return w


def test_every_bit_width_pair(dev):
    run_case(_all_bits_workload(), [0], dev)


def test_every_bit_width_with_qjl_uniform_codebook(dev):
    run_case(_all_bits_workload(kind=O.UNIFORM, qjl=True), [0], dev)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_gqa_groups(dev, G):
    run_case(_all_bits_workload(G=G, pages=12), [0], dev, dequant=False)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_gqa_groups_qjl(dev, G):
    # every packed page carries the QJL sketch: the layer runs the other
    # class's own launch, whose QJL term reads the per-workgroup sign table
    run_case(_all_bits_workload(G=G, pages=12, qjl=True), [0], dev, dequant=False)


def test_fp32_inputs_and_fp32_query(dev):
    run_case(_all_bits_workload(dtype="float32", pages=10), [0], dev, query_dtype=torch.float32)


def test_fp32_inputs_with_qjl(dev):
    # float32 rows into the QJL key kernel (its second input instantiation)
    run_case(_all_bits_workload(dtype="float32", pages=10, qjl=True), [0], dev, query_dtype=torch.float32)


def test_qjl_matrix_rows_of_any_scale(dev):
    # the sketch's signs do not depend on the scale of S's rows; the key kernel
    # rescales each row of S D H D before splitting it into float16 parts, so
    # rows far outside float16's range, tiny rows and a zero row (every sign +)
    # must all match the oracle
    S = W.qjl_matrix(W.ROTATION_SEED, 0).astype(np.float64)
    scale = np.ones(S.shape[0])
    scale[0::16] = 4e3      # S D H D entries past float16's largest value
    scale[3::7] = 1e-6      # entries in float16's subnormal range
    scale[9] = 0.0
    S = (S * scale[:, None]).astype(np.float32)
    run_case(_all_bits_workload(pages=8, qjl=True), [0], dev, qjl_s=S)


def test_short_and_empty_sessions(dev):
    w = W.make_workload(2, {"n_tokens": 64 * 3, "batch": 3, "sink_tokens": 64})
    # session 0: 1 token (partial fp16 page); session 1: none; session 2: all 192
    run_case(w, [0], dev, n_tokens=[1, 0, 192], dequant=False)


def test_partial_packed_page_is_flagged_and_untouched(dev):
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(2, {"n_tokens": 128, "batch": 1, "sink_tokens": 0})
    layer = tq.Layer(W.rotation_signs(42, 0), dev)
    cache = tq.Cache(w.formats[0], [128], dev)
    k, v = W.make_kv(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k[:, :, :100], v[:, :, :100], tok0=0, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 1
    assert int(cache.page_view(0, 0, 1).to(torch.int32).sum()) == 0


def test_deterministic(dev):
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(4, {"n_tokens": 64 * 8, "batch": 2})
    S = W.qjl_matrix(42, 0)
    layer = tq.Layer(W.rotation_signs(42, 0), dev, S)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    res = []
    for _ in range(2):
        cache = tq.Cache(w.formats[0], [w.n_tokens] * w.batch, dev)
        tq.encode_kv(layer, cache, k, v)
        out = tq.decode_attention(layer, cache, q)
        torch.cuda.synchronize()
        res.append((_np(cache.pool).copy(), _np(out).copy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_page_class_hint(dev):
    """Decode with the page-class bits the binding derives equals decode with
    the bits cleared (0 = unknown: every class runs), bit for bit, for tables
    with common pages only, other pages only, and common and wide pages."""
    import kv_cache_vector_srht_amd as tq
    cases = [(W.make_workload(3, {"n_tokens": 64 * 5, "batch": 2}), l) for l in (0, 2)]
    cases.append((W.make_workload(4, {"n_tokens": 64 * 4 + 9, "batch": 2}), 0))
    seen = set()
    for w, l in cases:
        fm = w.formats[l]
        S = W.qjl_matrix(42, l) if any(f[2] for row in fm for r in row for f in r) else None
        layer = tq.Layer(W.rotation_signs(42, l), dev, S)
        cache = tq.Cache(fm, [w.n_tokens] * w.batch, dev)
        k, v = W.make_kv(w, l, device=dev)
        q = W.make_query(w, l, device=dev)
        tq.encode_kv(layer, cache, k, v)
        hinted = _np(tq.decode_attention(layer, cache, q)).copy()
        seen.add(cache.page_classes)
        cache.struct.page_classes = 0
        unknown = _np(tq.decode_attention(layer, cache, q))
        assert np.array_equal(hinted, unknown)
    assert seen == {1, 2, 5}


@pytest.mark.parametrize("mode", [O.QJL_SCORE_SIGN, O.QJL_SCORE_UNBIASED])
def test_qjl_scoring_modes(dev, mode):
    """Decode with either QJL score form against the oracle's scores: the keys
    without their sketch plus ``O.qjl_score_term``.  Every width with QJL keys,
    an fp16 first page, GQA 4, a full and a ragged session."""
    import kv_cache_vector_srht_amd as tq
    w = _all_bits_workload(pages=20, qjl=True)
    n_tok = [w.n_tokens, 64 * 17 + 9]
    w.batch = 2
    fm = [w.formats[0][0], [[W.FP16 if p == 17 else f for p, f in enumerate(row)] for row in w.formats[0][0]]]
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    cache = tq.Cache(fm, n_tok, dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    qh = _np(q).astype(np.float64)
    # the sign of S q is decided in float32 on the device: the seeded queries
    # keep every projection clear of zero by far more than its rounding
    qf = qh.reshape(-1, 128)
    ratio = np.abs(qf @ S.astype(np.float64).T) / (np.linalg.norm(S, axis=1)[None, :] *
                                                   np.linalg.norm(qf, axis=1)[:, None])
    assert ratio.min() > 1e-5
    tq.encode_kv(layer, cache, k, v)
    print(f"decode, qjl_scoring {mode}", flush=True)
    out = _np(tq.decode_attention(layer, cache, q, qjl_scoring=mode))
    pool = _np(cache.pool)
    kh, vh = _np(k).astype(np.float64), _np(v).astype(np.float64)
    t = Tally()
    G = w.n_q_heads // w.n_kv_heads
    for b in range(2):
        n = n_tok[b]
        for h in range(w.n_kv_heads):
            parts = {}
            _, Vh = compare_unit_full(pool, cache.offsets, b, h, kh[b, h, :n], vh[b, h, :n], fm[b][h],
                                      signs, S, t, parts=parts)
            rows = slice(h * G, (h + 1) * G)
            ref = O.decode_attention_unit_qjl(qh[b, rows], parts["kbase"], Vh, parts["z"], parts["gamma"],
                                              S, mode)
            err = np.abs(out[b, rows] - ref).max(axis=1) / np.abs(ref).max(axis=1)
            t.worst_attn = max(t.worst_attn, float(err.max()))
    t.check()


def test_every_bit_width_pair_beta_codebook(dev):
    run_case(_all_bits_workload(kind=O.BETA, pages=40), [0], dev)


def test_beta_keys_lloyd_max_values_with_qjl(dev):
    w = _all_bits_workload(pages=24, qjl=True)
    w.k_codebook, w.v_codebook = O.BETA, O.LLOYD_MAX
    run_case(w, [0], dev)


def test_fitted_codebooks(dev):
    """Codebooks fitted to a sample of another layer's keys and values (in this
    layer's rotation), the library's tables on the GPU, the oracle's own fit
    on the CPU; every width pair, QJL on half the heads."""
    import kv_cache_vector_srht_amd as tq
    w = _all_bits_workload(pages=34)
    w.formats = [[[[f if (h == 0 or f[0] == 0) else (f[0], f[1], True) for f in row]
                   for h, row in enumerate(w.formats[0][0])]]]
    cal = W.make_workload(2, {"n_tokens": 256})
    kc, vc = W.make_kv(cal, 1)
    signs = W.rotation_signs(42, 0)
    Xk = kc.float().numpy().reshape(-1, 128)
    Xv = vc.float().numpy().reshape(-1, 128)
    w.k_codebook, w.v_codebook = O.fit_codebooks(Xk, signs), O.fit_codebooks(Xv, signs)
    layer_kw = dict(k_codebook=tq.FITTED, v_codebook=tq.FITTED,
                    k_table=tq.calibrated_table(Xk, signs), v_table=tq.calibrated_table(Xv, signs))
    run_case(w, [0], dev, layer_kw=layer_kw)


def _narrow_workload(pages=24, qjl=False, G=4):
    """Every (K, V) width pair within 1..4 bits, an fp16 first page."""
    w = W.make_workload(2, {"n_tokens": 64 * pages, "batch": 1, "n_kv_heads": 2,
                            "n_q_heads": 2 * G, "sink_tokens": 0, "dtype": "float16"})
    combos = [(kb, vb) for kb in range(1, 5) for vb in range(1, 5)]
    w.formats = [[[[W.packed(*combos[(p + 5 * h) % 16], qjl) if p > 0 else W.FP16
                    for p in range(pages)] for h in range(2)]]]
    return w


def _packed_narrow_workload(pages=40, G=4):
    """Every (K, V) width pair within 1..4 bits and no fp16 page, so that the
    layer takes the common class's own launch (four query heads: 3- and 4-bit
    keys scored on the matrix cores, 1- and 2-bit keys from the query's key
    table, both kinds in one range)."""
    w = W.make_workload(2, {"n_tokens": 64 * pages, "batch": 1, "n_kv_heads": 2,
                            "n_q_heads": 2 * G, "sink_tokens": 0, "dtype": "float16"})
    combos = [(kb, vb) for kb in range(1, 5) for vb in range(1, 5)]
    w.formats = [[[[W.packed(*combos[(p + 5 * h) % 16], False) for p in range(pages)] for h in range(2)]]]
    return w


@pytest.mark.parametrize("kind", [O.LLOYD_MAX, O.UNIFORM, O.BETA, O.POLAR])
def test_common_launch_every_narrow_width_pair(dev, kind):
    w = _packed_narrow_workload()
    w.k_codebook = w.v_codebook = kind
    run_case(w, [0], dev)


@pytest.mark.parametrize("scale", [0.0, 2.0 ** -40, 16.0])
def test_common_launch_query_scales(dev, scale):
    """The matrix-core key scores stage the query times a power of two that
    puts its largest magnitude near 2^10 (and undo it): a zero query (uniform
    weights), a tiny one and a large one."""
    run_case(_packed_narrow_workload(pages=20), [0], dev, query_dtype=torch.float32, query_scale=scale)


def test_polar_every_narrow_width_pair(dev):
    """PolarQuant keys and values at every width pair up to 4 bits."""
    w = _narrow_workload(pages=34)
    w.k_codebook = w.v_codebook = O.POLAR
    run_case(w, [0], dev)


def test_polar_keys_with_qjl_and_scalar_values(dev):
    w = _narrow_workload(pages=18, qjl=True)
    w.k_codebook, w.v_codebook = O.POLAR, O.LLOYD_MAX
    run_case(w, [0], dev)


def test_split_polar_keys_with_qjl_fp32_inputs(dev):
    # float32 rows into the PolarQuant instantiation of the QJL key kernel, at
    # an angle shift (key widths 2-4, the ones that carry it), scalar values
    combos = [(kb, vb) for kb in range(2, 5) for vb in range(1, 5)]
    pages = 1 + len(combos)
    w = W.make_workload(2, {"n_tokens": 64 * pages, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8,
                            "sink_tokens": 0, "dtype": "float32"})
    w.formats = [[[[W.packed(*combos[(p + 5 * h) % len(combos)], True) if p > 0 else W.FP16
                    for p in range(pages)] for h in range(2)]]]
    w.k_codebook, w.v_codebook = O.PolarSplit(-1), O.LLOYD_MAX
    run_case(w, [0], dev, query_dtype=torch.float32)


@pytest.mark.parametrize("k_shift,v_shift", [(1, -1), (2, 3), (-2, -3)])
def test_polar_split_widths(dev, k_shift, v_shift):
    """PolarQuant with radius and angle widths of their own: every width pair
    whose widths can carry the shifts (radius b - t, angle b + t bits),
    encoded by the bulk encoder, decoded and dequantised, against the oracle's
    PolarSplit (2-bit and 3-bit angles take the tangent tests, wider ones the
    arctangent)."""
    ks = [b for b in range(1, 5) if 1 <= b - k_shift and 1 <= b + k_shift <= 8]
    vs = [b for b in range(1, 5) if 1 <= b - v_shift and 1 <= b + v_shift <= 8]
    combos = [(kb, vb) for kb in ks for vb in vs]
    pages = 1 + 2 * len(combos)
    w = W.make_workload(2, {"n_tokens": 64 * pages, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8,
                            "sink_tokens": 64})
    w.formats = [[[[W.packed(*combos[(p + 3 * h) % len(combos)]) if p > 0 else W.FP16
                    for p in range(pages)] for h in range(2)]]]
    w.k_codebook, w.v_codebook = O.PolarSplit(k_shift), O.PolarSplit(v_shift)
    run_case(w, [0], dev)


def test_polar_split_refuses_widths_without_a_split(dev):
    """A page too narrow for the angle shift (no radius bit left) is refused by
    encode (flag 4, page untouched)."""
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(2, {"n_tokens": 128, "batch": 1, "n_kv_heads": 1, "n_q_heads": 4,
                            "sink_tokens": 0})
    fm = [[[W.packed(3, 2), W.packed(2, 2)]]]
    layer = tq.Layer(W.rotation_signs(42, 0), dev, None, **layer_args(O.PolarSplit(2), O.LLOYD_MAX))
    cache = tq.Cache(fm, [128], dev)
    k, v = W.make_kv(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 4
    kpart = cache.page_view(0, 0, 1)[:1024 * 2 + 256]
    assert int(kpart.to(torch.int32).abs().sum()) == 0


def test_polar_refuses_wide_pages(dev):
    """A PolarQuant part wider than 4 bits is refused by encode (flag 4, page
    untouched) and skipped by decode and dequantise."""
    import kv_cache_vector_srht_amd as tq
    w = W.make_workload(2, {"n_tokens": 128, "batch": 1, "n_kv_heads": 1, "n_q_heads": 4,
                            "sink_tokens": 0})
    fm = [[[W.packed(3, 2), W.packed(6, 2)]]]
    layer = tq.Layer(W.rotation_signs(42, 0), dev, None, tq.POLAR, tq.LLOYD_MAX)
    cache = tq.Cache(fm, [128], dev)
    k, v = W.make_kv(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 4
    # the K part of the refused page stays zero
    kpart = cache.page_view(0, 0, 1)[:1024 * 6 + 256]
    assert int(kpart.to(torch.int32).abs().sum()) == 0
