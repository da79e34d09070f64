"""CPU check of the arithmetic the QJL key kernel uses for the sketch: each
float32 operand y split as hi + lo = fp16(y) + fp16(y - hi), and a product
taken as hi_a hi_b + hi_a lo_b + lo_a hi_b (float16 products are exact in
float32).  The error against the exact product is far inside the band in
which a QJL sign may differ (1e-5 ||S_i|| ||r||), for rows scaled to a largest
magnitude of 8 and residuals scaled to norm sqrt(d), as the kernel scales
them (the signs do not depend on either scale)."""
import numpy as np


def _split(y):
    y = np.asarray(y, dtype=np.float32)
    hi = y.astype(np.float16)
    lo = (y - hi.astype(np.float32)).astype(np.float16)
    return hi, lo


def _split_dot(a, b):
    """sum over the last axis of the three float16 products, accumulated in
    float32 in order (as one lane's accumulator would)."""
    ah, al = _split(a)
    bh, bl = _split(b)
    acc = np.zeros(a.shape[:-1], dtype=np.float32)
    for j in range(a.shape[-1]):
        for x, y in ((al[..., j], bh[..., j]), (ah[..., j], bl[..., j]), (ah[..., j], bh[..., j])):
            acc = (acc + x.astype(np.float32) * y.astype(np.float32)).astype(np.float32)
    return acc


def test_split_products_error_within_the_sign_band():
    rng = np.random.default_rng(3)
    d = 128
    S = rng.standard_normal((64, d)) * np.exp(rng.uniform(-12, 12, size=(64, 1)))   # rows of any scale
    S = S / np.abs(S).max(axis=1, keepdims=True) * 8.0
    for width_scale in (1.0, 1e-3, 1e-6):   # residuals of wide and narrow codes
        v = rng.standard_normal((32, d)) * width_scale
        v[:, rng.integers(0, d, 8)] *= 40.0          # outlier coordinates
        v = v / np.linalg.norm(v, axis=1, keepdims=True) * np.sqrt(d)
        S32, v32 = S.astype(np.float32), v.astype(np.float32)
        exact = v32.astype(np.float64) @ S32.astype(np.float64).T
        got = np.stack([_split_dot(np.broadcast_to(v32[t], S32.shape), S32) for t in range(v32.shape[0])])
        band = 1e-5 * np.linalg.norm(S32, axis=1)[None, :] * np.linalg.norm(v32, axis=1)[:, None]
        # split error (2^-21 per term) plus the float32 accumulation's own
        err = np.abs(got.astype(np.float64) - exact)
        terms = np.abs(v32.astype(np.float64)) @ np.abs(S32.astype(np.float64)).T
        assert np.all(err <= 2.0 ** -21 * terms + d * 2.0 ** -24 * terms), width_scale
        assert np.all(err <= 0.05 * band), width_scale


def test_split_is_exact_for_float16_values():
    # values already in float16 have lo = 0 and their products are exact
    rng = np.random.default_rng(4)
    a = rng.standard_normal((4, 32)).astype(np.float16).astype(np.float32)
    b = rng.standard_normal((4, 32)).astype(np.float16).astype(np.float32)
    ah, al = _split(a)
    assert np.all(al == 0) and np.array_equal(ah.astype(np.float32), a)
    got = _split_dot(a, b)
    want = np.zeros(4, dtype=np.float32)
    for j in range(32):
        want = (want + a[:, j] * b[:, j]).astype(np.float32)
    assert np.array_equal(got, want)
