"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes a part of ``oracle/tq_oracle.py`` with a closed form, an
invariant, a textbook table (tests/golden/max1960_gaussian.json), a figure the
pages print (tests/golden/pages_figures.json), an independent numerical routine
(quadrature) or a brute-force loop, chosen so that a plausible slip in the
oracle (a dropped D, a transposed operand, a wrong constant, an off-by-one
code) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import tq_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _signs(seed=5):
    return W.rotation_signs(seed, 0)


# ----------------------------------------------------------------- rotation
def test_hadamard_closed_form_and_orthogonality():
    d = 128
    H = O.sylvester_hadamard(d)
    i = np.arange(d)
    pop = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(H, np.where(pop % 2 == 0, 1, -1))
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))


def test_rotation_two_by_two_by_hand():
    # D = diag(1, -1): D H D = [[1, -1], [-1, -1]]
    R = O.rotation_matrix([1, -1])
    assert np.allclose(R, np.array([[1.0, -1.0], [-1.0, -1.0]]) / math.sqrt(2), atol=1e-15)


def test_rotation_orthogonal_symmetric_involutory():
    s = _signs()
    R = O.rotation_matrix(s)
    I = np.eye(128)
    assert np.max(np.abs(R @ R.T - I)) < 1e-12
    assert np.max(np.abs(R - R.T)) == 0.0
    # one D on both sides: R is its own inverse (D H D D H D = D H H D = d I)
    assert np.max(np.abs(R @ R - I)) < 1e-12
    x = np.random.default_rng(1).standard_normal((16, 128))
    assert np.allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(np.abs(R[:, 0]), 1 / math.sqrt(128), atol=1e-15)
    # all-plus signs reduce to the normalised Sylvester matrix
    assert np.allclose(O.rotation_matrix(np.ones(128)), O.sylvester_hadamard(128) / math.sqrt(128))


def test_rotation_gaussianises_outliers():
    # TurboQuant-MLX v2.0, How It Works > Pipeline: the rotation brings heavy
    # outlier channels to a near-Gaussian coordinate distribution (kurtosis ~3).
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4000, 128))
    x[:, [7, 31, 64, 100]] *= 20.0
    k_before = np.mean(x ** 4) / np.mean(x ** 2) ** 2
    u = x @ O.rotation_matrix(_signs()).T
    k_after = np.mean(u ** 4) / np.mean(u ** 2) ** 2
    assert k_before > 50 and 1.5 < k_after < 3.5


# ----------------------------------------------------------------- codebooks
def test_one_bit_lloyd_max_closed_form():
    c, t = O.lloyd_max_gaussian(1)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-15 and c[0] == -c[1]
    assert t[0] == 0.0
    c32, _ = O.codebook(1)
    assert c32[1] == np.float32(math.sqrt(2 / math.pi))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960(bits):
    g = _golden("max1960_gaussian.json")["lloyd_max"][str(bits)]
    c, t = O.lloyd_max_gaussian(bits)
    L = 1 << bits
    assert np.allclose(c[L // 2:], g["levels"], atol=6e-4, rtol=0)
    assert np.allclose(t[L // 2:], g["endpoints"], atol=6e-4, rtol=0)
    assert abs(O.gaussian_mse(c, t) / g["mse"] - 1) < 1e-3


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_lloyd_max_conditions_by_quadrature(bits):
    """Centroid condition re-derived by numerical integration (not the oracle's
    closed-form phi differences), symmetric, strictly increasing."""
    c, t = O.lloyd_max_gaussian(bits)
    L = 1 << bits
    assert np.all(np.diff(c) > 0) and np.allclose(c, -c[::-1], atol=0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    pdf = lambda z: math.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    for k in range(L // 2, L):   # symmetric: check the positive half
        a, b = edges[k], edges[k + 1]
        num = integrate.quad(lambda z: z * pdf(z), a, b, epsabs=0, epsrel=1e-13, limit=200)[0]
        den = integrate.quad(pdf, a, b, epsabs=0, epsrel=1e-13, limit=200)[0]
        assert abs(num / den - c[k]) < 1e-8 * max(1.0, abs(c[k]))


def test_lloyd_max_high_rate_panter_dite():
    # D(b) ~ (pi sqrt(3) / 2) 4^-b for a Gaussian at high rate (Panter & Dite 1951).
    c, t = O.lloyd_max_gaussian(8)
    assert abs(O.gaussian_mse(c, t) / (math.pi * math.sqrt(3) / 2 * 4.0 ** -8) - 1) < 0.02


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_uniform_grid_matches_max_1960(bits):
    g = _golden("max1960_gaussian.json")["uniform"][str(bits)]
    c, t = O.uniform_gaussian(bits)
    assert abs(O.uniform_step(bits) - g["step"]) < 6e-4
    assert abs(O.gaussian_mse(c, t) / g["mse"] - 1) < 2e-3
    assert np.allclose(np.diff(c), O.uniform_step(bits), rtol=1e-12)


@pytest.mark.parametrize("bits", [2, 5, 8])
def test_uniform_step_is_stationary(bits):
    delta = O.uniform_step(bits)
    L = 1 << bits

    def mse(dl):
        c = (np.arange(L) - (L - 1) / 2) * dl
        return O.gaussian_mse(c, 0.5 * (c[:-1] + c[1:]))
    h = delta * 1e-4
    assert mse(delta) < mse(delta - h) and mse(delta) < mse(delta + h)


def test_mse_formula_by_quadrature():
    c, t = O.lloyd_max_gaussian(3)
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    pdf = lambda z: math.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    q = sum(integrate.quad(lambda z, ck=ck: (z - ck) ** 2 * pdf(z), a, b, epsrel=1e-12)[0]
            for a, b, ck in zip(edges[:-1], edges[1:], c))
    assert abs(q - O.gaussian_mse(c, t)) < 1e-10


# ------------------------------------------------------------------- encode
@pytest.mark.parametrize("bits", [1, 3, 8])
def test_encode_rotated_basis_vector(bits):
    s = _signs()
    R = O.rotation_matrix(s)
    L = 1 << bits
    x = 3.5 * R[:, 9]                      # R x = 3.5 e_9, so u = sqrt(d) e_9
    e = O.encode(x[None, :], s, bits)
    assert e["codes"][0, 9] == L - 1
    # the other coordinates are 0 up to rounding: they sit on either side of
    # the boundary t = 0 (exact ties are pinned by test_encode_zero_vector)
    others = np.delete(e["codes"][0], 9)
    assert np.all(np.abs(np.delete(e["u"][0], 9)) < 1e-12)
    assert np.all((others == L // 2) | (others == L // 2 - 1))
    assert abs(float(e["norm"][0]) - 3.5) < 1e-6


def test_encode_zero_vector():
    e = O.encode(np.zeros((1, 128)), _signs(), 3)
    assert e["norm"][0] == 0 and np.all(e["codes"] == 4)
    assert np.all(O.dequantize(e["norm"], e["codes"], _signs(), 3) == 0)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_cosine_matches_distortion(bits):
    """For Gaussian rows the rotated coordinates are ~N(0,1), so with Lloyd-Max
    levels E cos(x, xhat) ~ sqrt(1 - D_b), D_b the Gaussian distortion (Max 1960)."""
    g = _golden("max1960_gaussian.json")["lloyd_max"][str(bits)]
    x = W.gaussian_rows(11, 3000)
    s = _signs()
    e = O.encode(x, s, bits)
    xh = O.dequantize(e["norm"], e["codes"], s, bits)
    cos = np.sum(x * xh, 1) / np.linalg.norm(x, axis=1) / np.linalg.norm(xh, axis=1)
    assert abs(cos.mean() - math.sqrt(1 - g["mse"])) < 0.005


def test_one_bit_cosine_figure():
    fig = _golden("pages_figures.json")["one_bit_cosine"]["cosine"]
    x = W.gaussian_rows(12, 3000)
    s = _signs()
    e = O.encode(x, s, 1)
    xh = O.dequantize(e["norm"], e["codes"], s, 1)
    cos = np.sum(x * xh, 1) / np.linalg.norm(x, axis=1) / np.linalg.norm(xh, axis=1)
    assert abs(cos.mean() - fig) < 0.01


def test_tier_quality_figures():
    s = _signs()
    x = W.gaussian_rows(13, 2000)
    for row in _golden("pages_figures.json")["tier_quality"]["rows"]:
        cs = []
        for b in (row["k_bits"], row["v_bits"]):
            e = O.encode(x, s, b)
            xh = O.dequantize(e["norm"], e["codes"], s, b)
            cs.append(np.mean(np.sum(x * xh, 1) / np.linalg.norm(x, axis=1) / np.linalg.norm(xh, axis=1)))
        assert abs(np.mean(cs) - row["cosine"]) < 0.03


def test_eight_bit_is_near_lossless():
    x = W.gaussian_rows(14, 200) * 3
    s = _signs()
    e = O.encode(x, s, 8)
    xh = O.dequantize(e["norm"], e["codes"], s, 8)
    rel = np.linalg.norm(x - xh, axis=1) / np.linalg.norm(x, axis=1)
    # sqrt(D_8) = 0.0064 on average; overload of a rare |u| > 4.6 lifts the worst row
    assert rel.mean() < 0.0075 and rel.max() < 0.04


def test_boundary_flags():
    s = _signs()
    R = O.rotation_matrix(s)
    _, t32 = O.codebook(2)
    u = np.zeros(128)
    u[3] = float(t32[2]) + 1e-9           # within 1e-6 of a boundary
    u[4] = float(t32[2]) + 1e-3           # clear of it
    rest = math.sqrt((128 - u[3] ** 2 - u[4] ** 2) / 126)
    u[[j for j in range(128) if j not in (3, 4)]] = rest
    x = R @ u                              # ||x|| = sqrt(d), so sqrt(d) R x / ||x|| = u
    e = O.encode(x[None, :], s, 2)
    assert abs(e["u"][0, 3] - u[3]) < 1e-12
    assert e["near"][0, 3] and not e["near"][0, 4]
    assert e["codes"][0, 4] == 3


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_pack_round_trip_and_bijection(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(64, 128))
    blk = O.pack_block(codes, bits)
    assert len(blk) == 1024 * bits
    assert np.array_equal(O.unpack_block(blk, bits), codes)
    base = np.frombuffer(blk, dtype=np.uint8)
    seen = set()
    for _ in range(60):
        s, n, k = rng.integers(64), rng.integers(128), rng.integers(bits)
        c2 = codes.copy()
        c2[s, n] ^= 1 << k
        diff = np.unpackbits(np.frombuffer(O.pack_block(c2, bits), dtype=np.uint8) ^ base)
        pos = np.nonzero(diff)[0]
        assert pos.size == 1
        seen.add((int(pos[0]), (int(s), int(n), int(k))))
    # distinct code bits land on distinct storage bits
    assert len({p for p, _ in seen}) == len({key for _, key in seen})
    full = np.full((64, 128), (1 << bits) - 1)
    assert O.pack_block(full, bits) == b"\xff" * (1024 * bits)


def test_v_stream_order_is_a_permutation():
    codes = np.arange(64 * 128).reshape(64, 128)
    st = O.v_stream_codes(codes)
    assert sorted(st.ravel().tolist()) == list(range(64 * 128))
    assert np.array_equal(O.v_codes_from_streams(st), codes)
    # stream s holds one coordinate pair (c0, c0 + 1) over the 64 tokens:
    # position 2t (2t + 1) is token t, coordinate c0 (c0 + 1); hand-worked:
    # stream 0: coordinates 0, 1; stream 5 (n = 5: bit 2 set, n & 3 = 1):
    # 64 + 2 = 66, 67; stream 43 (n = 11: n >> 3 = 1, n & 3 = 3; P = 1):
    # 32 + 8 + 6 = 46, 47
    for s_, c0 in ((0, 0), (5, 66), (43, 46)):
        for t in (0, 17, 63):
            assert st[s_, 2 * t] == codes[t, c0] and st[s_, 2 * t + 1] == codes[t, c0 + 1]
    pairs = {(O.v_stream_coord(s_, 0), O.v_stream_coord(s_, 1)) for s_ in range(64)}
    assert sorted(c for pr in pairs for c in pr) == list(range(128))
    assert all(b == a + 1 and a % 2 == 0 for a, b in pairs)


def test_sign_words_round_trip():
    z = np.random.default_rng(3).random((64, 128)) < 0.5
    raw = O.pack_signs(z)
    assert len(raw) == 1024 and np.array_equal(O.unpack_signs(raw), z)


def test_footprint_matches_pages_table():
    fig = _golden("pages_figures.json")["footprint_fp16_vs_3bit"]
    vpt = fig["values_per_token"]
    vectors_per_token = vpt // 128
    for row in fig["rows"]:
        pages = row["tokens"] // 64
        codes = pages * vectors_per_token * len(O.pack_block(np.zeros((64, 128), int), 3)) // 64 * 64
        # one 3-bit code block holds 64 vectors: bytes per vector = 48
        code_bytes = row["tokens"] * vectors_per_token * (1024 * 3 // 64)
        fp16_bytes = row["tokens"] * vpt * 2
        assert code_bytes == row["tq3_mb"] * 2 ** 20
        assert fp16_bytes == row["fp16_mb"] * 2 ** 20
        assert round(fp16_bytes / code_bytes, 1) == row["ratio"]


def test_page_ratio_matches_pages_table():
    fp16 = O.page_bytes((0, 0, False))
    for row in _golden("pages_figures.json")["compression_by_bits"]["rows"]:
        b = row["bits"]
        assert round(fp16 / O.page_bytes((b, b, False)), 1) == row["ratio"]


# ---------------------------------------------------------------------- QJL
def test_qjl_estimator_unbiased_with_closed_form_variance():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128)
    r = rng.standard_normal(128) * 0.3
    m, trials = 128, 3000
    est = np.empty(trials)
    for k in range(trials):
        S = rng.standard_normal((m, 128))
        z = (S @ r) >= 0
        rhat = O.qjl_reconstruct(z[None, :], np.float32([np.linalg.norm(r)]), S)[0]
        est[k] = q @ rhat
    truth = q @ r
    g32 = float(np.float32(np.linalg.norm(r)))
    var = ((math.pi / 2) * (q @ q) * g32 ** 2 - truth ** 2 * (g32 / np.linalg.norm(r)) ** 2) / m
    assert abs(est.mean() - truth * g32 / np.linalg.norm(r)) < 4 * math.sqrt(var / trials)
    assert abs(est.var() / var - 1) < 0.15


def test_qjl_key_estimate_unbiased_through_encode_and_reconstruct():
    """The whole QJL key path of the oracle, composed: x_hat from the codec,
    (z, gamma) = qjl_encode(x, x_hat, S), r_hat = qjl_reconstruct(z, gamma, S).
    Over Gaussian S the attended key x_hat + r_hat is an unbiased estimate of
    x along any q ("TurboMOQ", QJL residual correction: the sign sketch
    corrects the residual), with variance ((pi/2) |q|^2 |r|^2 - (q.r)^2) / m
    for r = x - x_hat (the sign of a Gaussian projection: E[sign(s.r) s] =
    sqrt(2/pi) r/|r|).  A residual taken the other way round (x_hat - x) would
    centre the estimate on 2 q.x_hat - q.x instead."""
    rng = np.random.default_rng(41)
    signs = W.rotation_signs(42, 3)
    x = rng.standard_normal((1, 128))
    e = O.encode(x, signs, 2)
    xh = O.dequantize(e["norm"], e["codes"], signs, 2)
    r = (x - xh)[0]
    q = rng.standard_normal(128)
    m, trials = 128, 4000
    est = np.empty(trials)
    for k in range(trials):
        S = rng.standard_normal((m, 128))
        qj = O.qjl_encode(x, xh, S)
        est[k] = q @ (xh[0] + O.qjl_reconstruct(qj["z"], qj["gamma"], S)[0])
    g32 = float(np.float32(np.linalg.norm(r)))
    scale = g32 / np.linalg.norm(r)          # gamma is stored in float32
    mean = q @ xh[0] + scale * (q @ r)
    var = ((math.pi / 2) * (q @ q) * g32 ** 2 - (scale * (q @ r)) ** 2) / m
    assert abs(mean - q @ x[0]) < 1e-6 * abs(q @ x[0]) + 1e-9
    assert abs(est.mean() - mean) < 4 * math.sqrt(var / trials)
    assert abs(est.var() / var - 1) < 0.15
    wrong = 2 * (q @ xh[0]) - q @ x[0]
    assert abs(est.mean() - wrong) > 8 * math.sqrt(var / trials)


def test_qjl_orientation_with_a_permutation_sketch():
    """S a permutation matrix (row i selects coordinate pi(i)): the sketch is
    z_i = [r_pi(i) >= 0] and the reconstruction sqrt(pi/2)/m gamma S^T (2z - 1)
    is sqrt(pi/2)/m gamma sign(r), coordinate by coordinate.  S^T in place of
    S would select pi^-1(i) instead."""
    rng = np.random.default_rng(43)
    perm = rng.permutation(128)
    assert np.any(perm[perm] != np.arange(128))      # not an involution: S != S^T
    S = np.zeros((128, 128))
    S[np.arange(128), perm] = 1.0
    x = rng.standard_normal((3, 128))
    xh = 0.7 * x + 0.2 * rng.standard_normal((3, 128))
    r = x - xh
    qj = O.qjl_encode(x, xh, S)
    assert np.array_equal(qj["z"], r[:, perm] >= 0)
    assert np.array_equal(qj["gamma"], np.linalg.norm(r, axis=1).astype(np.float32))
    rh = O.qjl_reconstruct(qj["z"], qj["gamma"], S)
    expect = math.sqrt(math.pi / 2) / 128 * qj["gamma"].astype(np.float64)[:, None] * np.where(r >= 0, 1.0, -1.0)
    assert np.allclose(rh, expect, rtol=1e-14, atol=0)


def test_qjl_encode_scale_and_signs():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 128))
    xh = x * 0.9
    S = rng.standard_normal((128, 128))
    qj = O.qjl_encode(x, xh, S)
    assert np.allclose(qj["gamma"], np.linalg.norm(0.1 * x, axis=1), rtol=1e-6)
    assert np.array_equal(qj["z"], (0.1 * x) @ S.T >= 0)


# ---------------------------------------------------------------- attention
def test_attention_special_cases():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((9, 128))
    V = rng.standard_normal((9, 128))
    assert np.allclose(O.attention(rng.standard_normal(128), K[:1], V[:1]), V[0])
    assert np.allclose(O.attention(np.zeros(128), K, V), V.mean(axis=0))
    # two tokens, closed form
    q = rng.standard_normal(128)
    s1, s2 = K[0] @ q / math.sqrt(128), K[1] @ q / math.sqrt(128)
    w1 = 1 / (1 + math.exp(s2 - s1))
    assert np.allclose(O.attention(q, K[:2], V[:2]), w1 * V[0] + (1 - w1) * V[1])


def test_attention_brute_force_loops():
    rng = np.random.default_rng(7)
    for n, d in ((1, 4), (5, 8), (8, 16)):
        q = rng.standard_normal(d)
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        scores = []
        for t in range(n):
            acc = 0.0
            for j in range(d):
                acc += K[t][j] * q[j]
            scores.append(acc / math.sqrt(d))
        w = [math.exp(s) for s in scores]
        tot = sum(w)
        ref = [sum(w[t] * V[t][j] for t in range(n)) / tot for j in range(d)]
        assert np.allclose(O.attention(q, K, V), ref, rtol=1e-12)


def test_reconstruct_unit_fp16_sink_and_lossless_limit():
    rng = np.random.default_rng(8)
    T = 64 * 3 + 20
    K = rng.standard_normal((T, 128)).astype(np.float16)
    V = rng.standard_normal((T, 128)).astype(np.float16)
    fmts = [W.FP16, (8, 8, False), (8, 8, False), W.FP16]
    Kh, Vh = O.reconstruct_unit(K, V, fmts, _signs())
    assert np.array_equal(Kh[:64], K[:64].astype(np.float64))
    assert np.array_equal(Vh[192:], V[192:].astype(np.float64))
    rel = np.linalg.norm(Kh[64:192] - K[64:192], axis=1) / np.linalg.norm(K[64:192].astype(float), axis=1)
    assert rel.max() < 0.02
    q = rng.standard_normal((4, 128))
    out = O.decode_attention_unit(q, Kh, Vh)
    exact = np.stack([O.attention(qq, K.astype(float), V.astype(float)) for qq in q])
    assert np.max(np.abs(out - exact)) / np.max(np.abs(exact)) < 0.05


def test_page_bytes_round_trip_through_decode_page():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((64, 128))
    V = rng.standard_normal((64, 128))
    S = W.qjl_matrix(42, 0)
    s = _signs()
    fmt = (2, 3, True)
    enc = O.encode_page(K, V, fmt, s, S)
    assert len(enc["bytes"]) == O.page_bytes(fmt)
    Kd, Vd = O.decode_page(enc["bytes"], fmt, s, S)
    Kh, Vh = O.reconstruct_unit(K, V, [fmt], s, S)
    assert np.allclose(Kd, Kh, atol=1e-12) and np.allclose(Vd, Vh, atol=1e-12)


def test_overrides_only_within_the_boundary_allowance():
    s = _signs()
    R = O.rotation_matrix(s)
    _, t32 = O.codebook(2)
    u = np.zeros(128)
    u[3] = float(t32[2]) + 1e-9
    u[4] = float(t32[2]) + 1e-3
    rest = math.sqrt((128 - u[3] ** 2 - u[4] ** 2) / 126)
    u[[j for j in range(128) if j not in (3, 4)]] = rest
    x = (R @ u)[None, :]
    base = O.encode(x, s, 2)["codes"][0]
    alt = O.encode(x, s, 2, overrides=([0], [3], [base[3] - 1]))["codes"][0]
    assert alt[3] == base[3] - 1 and np.array_equal(np.delete(alt, 3), np.delete(base, 3))
    with pytest.raises(ValueError):
        O.encode(x, s, 2, overrides=([0], [4], [base[4] - 1]))   # not near a boundary
    with pytest.raises(ValueError):
        O.encode(x, s, 2, overrides=([0], [3], [base[3] - 2]))   # two levels away


# ---------------------------------------------------------------- re-tiering
def test_requantize_codes_pins():
    # same width: the identity (each centroid lies strictly inside its own cell)
    for b in range(1, 9):
        c = np.arange(1 << b)
        assert np.array_equal(O.requantize_codes(c, b, b), c)
    # to 1 bit: the sign of the centroid (boundary 0): the lower half of the levels -> 0
    for b in range(2, 9):
        c = np.arange(1 << b)
        assert np.array_equal(O.requantize_codes(c, b, 1), (c >= (1 << (b - 1))).astype(np.int64))
    # 2 -> 1 by hand with Max (1960): levels -1.5104, -0.4528, 0.4528, 1.5104 -> 0, 0, 1, 1
    assert O.requantize_codes(np.array([0, 1, 2, 3]), 2, 1).tolist() == [0, 0, 1, 1]
    # 3 -> 2: the 3-bit levels +-0.2451, +-0.7560, +-1.3439, +-2.1519 against the 2-bit
    # boundaries 0, +-0.9816 (Max 1960, Table I)
    assert O.requantize_codes(np.arange(8), 3, 2).tolist() == [0, 0, 1, 1, 2, 2, 3, 3]
    # monotone and symmetric (code L-1-c maps to L'-1 minus the map of c) for every pair
    # of widths; a demotion reaches both end levels
    for b in range(1, 9):
        for nb in range(1, 9):
            m = O.requantize_codes(np.arange(1 << b), b, nb)
            assert np.all(np.diff(m) >= 0)
            assert np.array_equal(m[::-1], (1 << nb) - 1 - m)
            if nb <= b:
                assert m[0] == 0 and m[-1] == (1 << nb) - 1


def test_retier_page_keeps_norms_and_reconstructs_nearest_levels():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((64, 128))
    V = rng.standard_normal((64, 128))
    signs = W.rotation_signs(42, 1)
    page = O.encode_page(K, V, (4, 4, False), signs)
    new = O.retier_page(page["bytes"], (4, 4, False), (2, 1, False), signs)
    assert len(new) == O.page_bytes((2, 1, False))
    sec_o, sec_n = O.page_sections((4, 4, False)), O.page_sections((2, 1, False))
    for name in ("k_norm", "v_norm"):
        (oo, on), (no, nn) = sec_o[name], sec_n[name]
        assert page["bytes"][oo:oo + on] == new[no:no + nn]
    # the demoted codes are the encoder's codes of the old reconstruction's rotated
    # coordinates (u = centroids), which requantize_codes states directly
    kc = O.unpack_block(new[sec_n["k_codes"][0]:sec_n["k_codes"][0] + sec_n["k_codes"][1]], 2)
    assert np.array_equal(kc, O.requantize_codes(page["k"]["codes"], 4, 2))
    Kd, Vd = O.decode_page(new, (2, 1, False), signs)
    K4, V4 = O.decode_page(page["bytes"], (4, 4, False), signs)
    # re-encoding the 4-bit reconstruction at 2 bits gives the same codes (u = centroids
    # up to rounding, never within 1e-6 of a 2-bit boundary here)
    e2 = O.encode(K4, signs, 2)
    assert not e2["near"].any() and np.array_equal(e2["codes"], kc)
    assert np.corrcoef(Kd.ravel(), K.ravel())[0, 1] > 0.9
    # an fp16 page is encoded from its rows
    raw16 = O.fp16_page_bytes(K, V)
    K16 = K.astype(np.float16).astype(np.float64)
    V16 = V.astype(np.float16).astype(np.float64)
    assert O.retier_page(raw16, W.FP16, (3, 2, False), signs) == \
        O.encode_page(K16, V16, (3, 2, False), signs)["bytes"]


def test_page_attention_mass_pins():
    rng = np.random.default_rng(3)
    T = 150
    K = rng.standard_normal((T, 128)) * 2
    qs = rng.standard_normal((3, 128))
    m = O.page_attention_mass(qs, K)
    assert m.shape == (3, 3)
    assert np.allclose(m.sum(axis=1), 1.0, atol=1e-12)
    # the page masses are attention over values that indicate each token's page
    ind = np.zeros((T, 3))
    ind[np.arange(T), np.arange(T) // 64] = 1.0
    for g in range(3):
        assert np.allclose(m[g], O.attention(qs[g], K, ind), atol=1e-12)
    # identical keys: mass in proportion to the tokens a page holds
    same = np.tile(rng.standard_normal(128), (T, 1))
    assert np.allclose(O.page_attention_mass(qs[:1], same)[0], [64 / T, 64 / T, 22 / T], atol=1e-12)
    # closed form: page 0 scores 0, page 1 scores c
    q = np.zeros(128)
    q[0] = 1.0
    K2 = np.zeros((128, 128))
    K2[64:, 0] = 3.0
    c = 3.0 / math.sqrt(128)
    want1 = math.exp(c) / (1 + math.exp(c))
    assert np.allclose(O.page_attention_mass(q[None], K2)[0], [1 - want1, want1], atol=1e-12)
    # a key that dominates every other score takes all the mass
    K3 = rng.standard_normal((T, 128)) * 0.01
    K3[140] = 1e3 * qs[0] / np.linalg.norm(qs[0])
    assert O.page_attention_mass(qs[:1], K3)[0, 2] > 1 - 1e-12


def test_token_attention_weights_pins():
    rng = np.random.default_rng(5)
    T = 150
    K = rng.standard_normal((T, 128)) * 2
    qs = rng.standard_normal((3, 128))
    w = O.token_attention_weights(qs, K)
    assert w.shape == (3, T) and np.all(w >= 0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    # the weights are attention over one-hot values: value t picks token t
    for g in range(3):
        assert np.allclose(w[g], O.attention(qs[g], K, np.eye(T)), atol=1e-12)
    # a page's tokens sum to its page mass
    pm = O.page_attention_mass(qs, K)
    for p in range(3):
        assert np.allclose(w[:, 64 * p:64 * p + 64].sum(axis=1), pm[:, p], atol=1e-12)
    # closed form: two scores 0 and c
    q = np.zeros(128)
    q[0] = 1.0
    K2 = np.zeros((2, 128))
    K2[1, 0] = 3.0
    c = 3.0 / math.sqrt(128)
    assert np.allclose(O.token_attention_weights(q[None], K2)[0], [1 / (1 + math.exp(c)), 1 / (1 + math.exp(-c))],
                       atol=1e-12)
    # a softmax scale multiplies every score
    assert np.allclose(O.token_attention_weights(q[None], K2, scale=0.5)[0],
                       [1 / (1 + math.exp(1.5)), 1 / (1 + math.exp(-1.5))], atol=1e-12)


def test_requantize_decisions_are_far_from_ties():
    """Every centroid sits at least 1e-4 from every boundary of a narrower or
    equal width, so the map is the same whether it is decided in float32 or
    float64."""
    for kind in (O.LLOYD_MAX, O.UNIFORM):
        for b in range(1, 9):
            c, _ = O.codebook(b, kind)
            for nb in range(1, b + 1):
                _, t = O.codebook(nb, kind)
                gap = np.abs(c[:, None] - t[None, :]).min()
                assert gap > 1e-4, (kind, b, nb, gap)
                m32 = np.searchsorted(t.astype(np.float32), c.astype(np.float32), side="right")
                assert np.array_equal(m32, O.requantize_codes(np.arange(1 << b), b, nb, kind))


def test_qjl_sign_scoring_pins():
    """The sign-agreement score of the sketch: exact at parallel and
    antiparallel residuals, q . rhat in the unbiased mode, and a mean of
    ||q|| ||r|| asin(rho) over draws of S (Grothendieck's identity
    P[sign(g.x) = sign(g.y)] = 1 - angle / pi for Gaussian g)."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal(128)
    S = rng.standard_normal((128, 128))
    for sgn in (1.0, -1.0):
        r = sgn * 0.4 * q
        z = (S @ r >= 0)[None, :]
        g = np.float32([np.linalg.norm(r)])
        want = sgn * (math.pi / 2) * np.linalg.norm(q) * float(g[0])
        assert np.isclose(O.qjl_score_term(q, z, g, S, O.QJL_SCORE_SIGN)[0], want, rtol=1e-12)
    # unbiased mode is the score against the reconstructed residual
    r = rng.standard_normal(128) * 0.2
    z = (S @ r >= 0)[None, :]
    g = np.float32([np.linalg.norm(r)])
    assert np.isclose(O.qjl_score_term(q, z, g, S, O.QJL_SCORE_UNBIASED)[0],
                      q @ O.qjl_reconstruct(z, g, S)[0], rtol=1e-12)
    # mean over S: ||q|| ||r|| asin(rho), at an oblique and a small correlation
    u = q / np.linalg.norm(q)
    w = rng.standard_normal(128)
    w -= (w @ u) * u
    w /= np.linalg.norm(w)
    for rho in (0.6, 0.1):
        r = 0.3 * (rho * u + math.sqrt(1 - rho * rho) * w)
        g = np.float32([np.linalg.norm(r)])
        est = np.empty(2000)
        for k in range(est.size):
            Sk = rng.standard_normal((128, 128))
            est[k] = O.qjl_score_term(q, (Sk @ r >= 0)[None, :], g, Sk, O.QJL_SCORE_SIGN)[0]
        want = np.linalg.norm(q) * float(g[0]) * math.asin(rho)
        assert abs(est.mean() - want) < 4 * est.std() / math.sqrt(est.size)


def test_decode_attention_unit_qjl_matches_reconstruction_in_unbiased_mode():
    rng = np.random.default_rng(22)
    T = 70
    Kb = rng.standard_normal((T, 128))
    V = rng.standard_normal((T, 128))
    S = rng.standard_normal((128, 128))
    r = rng.standard_normal((T, 128)) * 0.3
    qj = O.qjl_encode(Kb + r, Kb, S)
    g = qj["gamma"].copy()
    g[:10] = 0          # tokens without a sketch
    qs = rng.standard_normal((4, 128))
    got = O.decode_attention_unit_qjl(qs, Kb, V, qj["z"], g, S, O.QJL_SCORE_UNBIASED)
    Kh = Kb + O.qjl_reconstruct(qj["z"], g, S)
    assert np.allclose(got, O.decode_attention_unit(qs, Kh, V), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------ Beta codebook
def _sphere_density(u, d=128):
    # written out directly from the law of sqrt(d) x_1, x uniform on the unit sphere
    c = math.gamma(d / 2) / (math.sqrt(math.pi * d) * math.gamma((d - 1) / 2))
    y = 1.0 - u * u / d
    return c * y ** ((d - 3) / 2) if y > 0 else 0.0


def test_beta_codebook_pins():
    from scipy import integrate
    d = 128
    end = math.sqrt(d)
    # the density is a probability law with unit variance
    assert abs(integrate.quad(_sphere_density, -end, end, epsabs=1e-13)[0] - 1) < 1e-10
    assert abs(integrate.quad(lambda u: u * u * _sphere_density(u), -end, end, epsabs=1e-13)[0] - 1) < 1e-10
    # 1 bit: the centroid is E|U| = sqrt(d) Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c1, t1 = O.codebook(1, O.BETA)
    want = math.sqrt(d) * math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert np.float32(want) == c1[1] and c1[0] == -c1[1] and t1[0] == 0
    # centroid condition by quadrature, cell by cell
    for bits in (2, 3, 4, 5):
        c, t = O.codebook(bits, O.BETA)
        edges = np.concatenate(([-end], t.astype(np.float64), [end]))
        for k in range(c.size):
            a, b = edges[k], edges[k + 1]
            P = integrate.quad(_sphere_density, a, b, epsabs=1e-15, limit=200)[0]
            M = integrate.quad(lambda u: u * _sphere_density(u), a, b, epsabs=1e-15, limit=200)[0]
            assert abs(M / P - c[k]) < 2e-6 * max(1.0, abs(c[k])), (bits, k, M / P, c[k])
        assert np.array_equal(c, -c[::-1])
    # optimal for its law: a lower MSE under the sphere density than the
    # Gaussian Lloyd-Max codebook of the same width
    def mse(c, t):
        edges = np.concatenate(([-end], t.astype(np.float64), [end]))
        return sum(integrate.quad(lambda u: (u - c[k]) ** 2 * _sphere_density(u), edges[k], edges[k + 1],
                                  epsabs=1e-15, limit=200)[0] for k in range(c.size))
    for bits in (1, 2, 3, 4):
        assert mse(*O.codebook(bits, O.BETA)) < mse(*O.codebook(bits, O.LLOYD_MAX))
    # as d grows the law tends to N(0,1) and so does the codebook
    for bits in (1, 2, 3):
        big, _ = O.lloyd_max_sphere(bits, d=10 ** 7)
        gauss, _ = O.lloyd_max_gaussian(bits)
        assert np.allclose(big, gauss, atol=1e-6)


def test_beta_codebook_law_matches_random_directions():
    """The law the codebook is built for is that of rotated, normalised
    coordinates of random directions: empirical tails of sqrt(d) x_1."""
    from scipy import integrate
    rng = np.random.default_rng(23)
    X = rng.standard_normal((200000, 128))
    u = math.sqrt(128) * X[:, 0] / np.linalg.norm(X, axis=1)
    for t in (0.5, 1.0, 2.0):
        p = integrate.quad(_sphere_density, t, math.sqrt(128), epsabs=1e-14)[0]
        emp = np.mean(u >= t)
        assert abs(emp - p) < 5 * math.sqrt(p * (1 - p) / u.size)


# -------------------------------------------------------- fitted codebooks
def test_fit_levels_hand_example():
    mags = np.array([0.1, 0.2, 0.3, 2.0, 2.2])
    c, t = O.fit_levels(mags, 2)
    assert np.allclose(c, [-2.1, -0.2, 0.2, 2.1], atol=1e-7) and np.allclose(t, [-1.15, 0.0, 1.15], atol=1e-7)
    c1, t1 = O.fit_levels(mags, 1)
    assert np.allclose(c1, [-mags.mean(), mags.mean()]) and t1[0] == 0
    # symmetric at every width, and exactly so in float32
    for b in range(1, 6):
        c, t = O.fit_levels(np.sort(np.random.default_rng(b).exponential(size=3000)), b)
        assert np.array_equal(c, -c[::-1]) and np.array_equal(t, -t[::-1])


def test_sample_magnitudes_rotate_and_normalise():
    signs = W.rotation_signs(42, 3)
    R = O.rotation_matrix(signs)
    Y = np.zeros((3, 128))
    Y[0, :2] = [3.0, 4.0]
    Y[2, 5] = -2.0            # row 1 is zero: skipped
    X = Y @ R                  # R is symmetric and its own inverse, so R x = y
    m = O.sample_magnitudes(X, signs)
    want = np.sort(np.concatenate(([0.6 * math.sqrt(128), 0.8 * math.sqrt(128)], np.zeros(126),
                                   [math.sqrt(128)], np.zeros(127))))
    assert m.size == 256 and np.allclose(m, want, atol=1e-9)


def test_fit_levels_is_a_fixed_point_of_k_means():
    rng = np.random.default_rng(24)
    mags = np.sort(np.abs(rng.standard_t(5, size=4000)))
    for bits in (2, 3):
        c, t = O.fit_levels(mags, bits, sweeps=10000)
        h = c.size // 2
        # brute force: each positive level is the mean of the magnitudes closer
        # to it than to its neighbours
        for k in range(h):
            lo = 0.0 if k == 0 else (float(c[h + k - 1]) + float(c[h + k])) / 2
            hi = math.inf if k == h - 1 else (float(c[h + k]) + float(c[h + k + 1])) / 2
            cell = [x for x in mags if lo <= x < hi]
            assert abs(sum(cell) / len(cell) - float(c[h + k])) < 1e-6
        # k-means never raises its objective: below the Gaussian start's
        def obj(levels):
            pos = levels[levels.size // 2:].astype(np.float64)
            return np.min((mags[:, None] - pos[None, :]) ** 2, axis=1).sum()
        assert obj(c) <= obj(O.codebook(bits, O.LLOYD_MAX)[0])


def test_fitted_codebooks_approach_the_laws_they_sample():
    """Fitted to many samples of a law, the codebook approaches that law's
    Lloyd-Max codebook: Gaussian magnitudes give the Gaussian one; rotated,
    normalised Gaussian vectors (random directions) give the Beta one."""
    rng = np.random.default_rng(25)
    g = np.sort(np.abs(rng.standard_normal(2_000_000)))
    m = O.sample_magnitudes(rng.standard_normal((20000, 128)), W.rotation_signs(42, 0))
    for b in (1, 2, 3):
        assert np.allclose(O.fit_levels(g, b)[0], O.codebook(b, O.LLOYD_MAX)[0], atol=0.005)
        assert np.allclose(O.fit_levels(m, b)[0], O.codebook(b, O.BETA)[0], atol=0.005)


# ------------------------------------------------------------- PolarQuant
def test_rayleigh_radius_codebook_pins():
    from scipy import integrate
    f = lambda r: r * math.exp(-r * r / 2)
    for bits in (1, 2, 3, 4):
        c, t = O.codebook(bits, O.POLAR)
        assert np.all(np.diff(c) > 0) and c[0] > 0 and np.allclose(t, (c[:-1] + c[1:]) / 2, rtol=1e-6)
        edges = np.concatenate(([0.0], t.astype(np.float64), [np.inf]))
        for k in range(c.size):
            P = integrate.quad(f, edges[k], edges[k + 1], epsabs=1e-14)[0]
            M = integrate.quad(lambda r: r * f(r), edges[k], edges[k + 1], epsabs=1e-14)[0]
            assert abs(M / P - c[k]) < 2e-6 * c[k], (bits, k)
    # the pair table is radius level times the sector middle's direction
    for bits in (1, 2, 3):
        L = 1 << bits
        c, _ = O.codebook(bits, O.POLAR)
        P = O.polar_pairs(bits)
        for j in range(L):
            a = -math.pi + (2 * j + 1) * math.pi / L
            assert np.allclose(P[:, j, 0], c * math.cos(a), rtol=1e-6, atol=1e-7)
            assert np.allclose(P[:, j, 1], c * math.sin(a), rtol=1e-6, atol=1e-7)


def _vectors_with_rotated(U, signs):
    """Rows x with sqrt(d) R x / ||x|| = U for rows U of squared norm d."""
    return U @ O.rotation_matrix(signs) / math.sqrt(U.shape[1])


def test_polar_encode_hand_example():
    signs = W.rotation_signs(42, 2)
    r = math.sqrt(2.0)                    # every pair at radius sqrt(2): ||u||^2 = 128
    th = np.array([0.1, 1.7, -2.0, 3.0, -0.4] + [0.5] * 59)
    U = np.zeros((1, 128))
    U[0, 0::2], U[0, 1::2] = r * np.cos(th), r * np.sin(th)
    X = _vectors_with_rotated(U, signs)
    e = O.encode(X, signs, 2, O.POLAR)
    assert np.allclose(e["u"], U, atol=1e-12)
    # 2 bits: radius boundaries ~ (0.822, 1.420, 2.127): sqrt(2) is level 1;
    # angle sectors of pi/2 from -pi: 0.1 -> 2, 1.7 -> 3, -2.0 -> 0, 3.0 -> 3, -0.4 -> 1
    assert np.all(e["codes"][0, 0::2] == 1)
    assert e["codes"][0, 1::2][:5].tolist() == [2, 3, 0, 3, 1]
    # reconstruction: the norm times the pair levels, rotated back
    xh = O.dequantize(e["norm"], e["codes"], signs, 2, O.POLAR)
    P = O.polar_pairs(2)
    uh = np.empty(128)
    uh[0::2] = P[1, e["codes"][0, 1::2], 0]
    uh[1::2] = P[1, e["codes"][0, 1::2], 1]
    assert np.allclose(math.sqrt(128) * (xh @ O.rotation_matrix(signs).T) / float(e["norm"][0]), uh, atol=1e-9)


def test_polar_angle_wraps_and_flags_sector_edges():
    assert O.polar_angle_code(np.array([math.pi, -math.pi, 0.0, -1e-12]), 3).tolist() == [0, 0, 4, 3]
    signs = W.rotation_signs(42, 2)
    L = 8
    th = np.array([-math.pi + 2 * math.pi * 3 / L + 1e-7, 0.3] + [0.7] * 62)
    U = np.zeros((1, 128))
    U[0, 0::2], U[0, 1::2] = math.sqrt(2) * np.cos(th), math.sqrt(2) * np.sin(th)
    e = O.encode(_vectors_with_rotated(U, signs), signs, 3, O.POLAR)
    assert e["near"][0, 1] and not e["near"][0, 3]
    # a cyclic neighbour is an admissible override at a flagged angle; 2 steps are not
    O.encode(_vectors_with_rotated(U, signs), signs, 3, O.POLAR, overrides=([0], [1], [2]))
    with pytest.raises(ValueError):
        O.encode(_vectors_with_rotated(U, signs), signs, 3, O.POLAR, overrides=([0], [1], [5]))


def test_polar_distortion_matches_closed_form():
    """For Gaussian pairs the mean squared pair error of independent radius
    (Lloyd-Max) and angle (uniform) quantisers is
    2 + (1 - 2 sinc(pi/L)) sum_k P_k c_k^2, sinc x = sin x / x (the Lloyd-Max
    centroid condition gives E[R; cell k] = c_k P_k).  Checked against the
    oracle's encode and dequantise of vectors whose rotated coordinates are
    Gaussian up to the normalisation (d = 128, so within a few per cent)."""
    rng = np.random.default_rng(26)
    signs = W.rotation_signs(42, 0)
    R = O.rotation_matrix(signs)
    X = rng.standard_normal((3000, 128))
    for bits in (2, 3, 4):
        L = 1 << bits
        c, t = O.codebook(bits, O.POLAR)
        e = np.concatenate(([0.0], t.astype(np.float64), [np.inf]))
        Pk = np.exp(-0.5 * e[:-1] ** 2) - np.exp(-0.5 * np.where(np.isinf(e[1:]), np.inf, e[1:]) ** 2)
        x = math.pi / L
        D = 2 + (1 - 2 * math.sin(x) / x) * np.sum(Pk * c.astype(np.float64) ** 2)
        enc = O.encode(X, signs, bits, O.POLAR)
        xh = O.dequantize(enc["norm"], enc["codes"], signs, bits, O.POLAR)
        uh = math.sqrt(128) * (xh @ R.T) / enc["norm"][:, None].astype(np.float64)
        mse_pair = np.mean(np.sum((enc["u"] - uh) ** 2, axis=1)) / 64
        assert abs(mse_pair / D - 1) < 0.03, (bits, mse_pair, D)


def test_polar_split_shift0_is_polar():
    rng = np.random.default_rng(31)
    signs = W.rotation_signs(42, 1)
    X = rng.standard_normal((40, 128))
    for bits in (1, 2, 3, 4):
        a = O.encode(X, signs, bits, O.POLAR)
        b = O.encode(X, signs, bits, O.PolarSplit(0))
        assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["near"], b["near"])
        assert np.array_equal(O.dequantize(a["norm"], a["codes"], signs, bits, O.POLAR),
                              O.dequantize(b["norm"], b["codes"], signs, bits, O.PolarSplit(0)))
        P, T = O.polar_pairs(bits), O.polar_pair_table(bits, 0)
        L = 1 << bits
        for rc in range(L):
            for tc in range(L):
                assert np.array_equal(P[rc, tc], T[rc | (tc << bits)])


def test_polar_split_packing_hand_example():
    """Width 3 with shift 2: a 1-bit radius and a 5-bit angle.  Pairs at radius
    sqrt(2) and angles 0.1 and -2.0: sectors of 2 pi / 32 from -pi give
    floor((0.1 + pi) 32 / (2 pi)) = 16 and floor((-2.0 + pi) 32 / (2 pi)) = 5;
    the field F = rc | tc << 1 is stored as F & 7 (even position) and F >> 3."""
    signs = W.rotation_signs(42, 2)
    th = np.array([0.1, -2.0] + [0.5] * 62)
    U = np.zeros((1, 128))
    U[0, 0::2], U[0, 1::2] = math.sqrt(2) * np.cos(th), math.sqrt(2) * np.sin(th)
    e = O.encode(_vectors_with_rotated(U, signs), signs, 3, O.PolarSplit(2))
    _, t1 = O.codebook(1, O.POLAR)
    rc = int(math.sqrt(2) >= float(t1[0]))
    for i, tc in ((0, 16), (1, 5)):
        F = rc | (tc << 1)
        assert e["codes"][0, 2 * i] == F & 7 and e["codes"][0, 2 * i + 1] == F >> 3
    assert np.all(e["codes"] < 8)
    # the reconstruction is radius level rc in the middle of the sector
    xh = O.dequantize(e["norm"], e["codes"], signs, 3, O.PolarSplit(2))
    uh = math.sqrt(128) * (xh @ O.rotation_matrix(signs).T) / float(e["norm"][0])
    c1, _ = O.codebook(1, O.POLAR)
    for i, tc in ((0, 16), (1, 5)):
        mid = -math.pi + (2 * tc + 1) * math.pi / 32
        assert np.allclose(uh[0, 2 * i:2 * i + 2], [c1[rc] * math.cos(mid), c1[rc] * math.sin(mid)], atol=1e-6)


def test_polar_split_overrides_move_one_level_or_sector():
    signs = W.rotation_signs(42, 2)
    L = 32                                  # width 3, shift 2: 5 angle bits
    th = np.array([-math.pi + 2 * math.pi * 7 / L + 1e-7, 0.3] + [0.7] * 62)
    U = np.zeros((1, 128))
    U[0, 0::2], U[0, 1::2] = math.sqrt(2) * np.cos(th), math.sqrt(2) * np.sin(th)
    X = _vectors_with_rotated(U, signs)
    kind = O.PolarSplit(2)
    e = O.encode(X, signs, 3, kind)
    assert e["near"][0, 1] and not e["near"][0, 3]
    F = e["codes"][0, 0] | (e["codes"][0, 1] << 3)
    assert F >> 1 == 7
    G = (F & 1) | (6 << 1)                  # one sector down: admissible at the flagged edge
    O.encode(X, signs, 3, kind, overrides=([0, 0], [0, 1], [G & 7, G >> 3]))
    H = (F & 1) | (5 << 1)                  # two sectors: not
    with pytest.raises(ValueError):
        O.encode(X, signs, 3, kind, overrides=([0, 0], [0, 1], [H & 7, H >> 3]))
    with pytest.raises(ValueError):
        O.polar_widths(2, 2)                # no radius bit left


def test_polar_split_distortion_matches_closed_form():
    """The closed form of the polar distortion above, with the radius levels of
    r = b - t bits and 2^(b + t) angle sectors, for shifts of either sign."""
    rng = np.random.default_rng(27)
    signs = W.rotation_signs(42, 0)
    R = O.rotation_matrix(signs)
    X = rng.standard_normal((3000, 128))
    for bits, shift in ((2, 1), (3, 1), (3, -1), (4, 2), (4, -2)):
        rb, ab = O.polar_widths(bits, shift)
        c, t = O.codebook(rb, O.POLAR)
        e = np.concatenate(([0.0], t.astype(np.float64), [np.inf]))
        Pk = np.exp(-0.5 * e[:-1] ** 2) - np.exp(-0.5 * np.where(np.isinf(e[1:]), np.inf, e[1:]) ** 2)
        x = math.pi / (1 << ab)
        D = 2 + (1 - 2 * math.sin(x) / x) * np.sum(Pk * c.astype(np.float64) ** 2)
        kind = O.PolarSplit(shift)
        enc = O.encode(X, signs, bits, kind)
        xh = O.dequantize(enc["norm"], enc["codes"], signs, bits, kind)
        uh = math.sqrt(128) * (xh @ R.T) / enc["norm"][:, None].astype(np.float64)
        mse_pair = np.mean(np.sum((enc["u"] - uh) ** 2, axis=1)) / 64
        assert abs(mse_pair / D - 1) < 0.03, (bits, shift, mse_pair, D)
