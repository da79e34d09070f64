"""CPU checks of the GPU-parity helpers: fed pages that the oracle itself
wrote, the one-pass unit comparison must find no mismatch and return exactly
the oracle's reconstruction."""
import numpy as np

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import Tally, compare_unit_full


def _pool_from_oracle(K, V, formats, signs, S):
    offsets = np.zeros((1, 1, len(formats)), dtype=np.int64)
    blobs, off = [], 0
    for p, fmt in enumerate(formats):
        lo, hi = 64 * p, min(K.shape[0], 64 * p + 64)
        raw = (O.fp16_page_bytes(K[lo:hi], V[lo:hi]) if fmt[0] == 0
               else O.encode_page(K[lo:hi], V[lo:hi], fmt, signs, S)["bytes"])
        offsets[0, 0, p] = off
        blobs.append(raw + bytes((-len(raw)) % 256))
        off += len(blobs[-1])
    return np.frombuffer(b"".join(blobs), dtype=np.uint8), offsets


def test_compare_unit_full_matches_reconstruct_unit():
    rng = np.random.default_rng(5)
    T = 64 * 7 + 20
    K = rng.standard_normal((T, 128)).astype(np.float16).astype(np.float64)
    V = rng.standard_normal((T, 128)).astype(np.float16).astype(np.float64)
    K[:, 3] *= 25
    formats = [W.FP16, W.packed(3, 2, False), W.packed(2, 2, True), W.packed(3, 2, False),
               W.packed(7, 6, False), W.packed(2, 2, True), W.packed(1, 1, False), W.FP16]
    signs = W.rotation_signs(42, 3)
    S = W.qjl_matrix(42, 3)
    pool, offsets = _pool_from_oracle(K, V, formats, signs, S)
    t = Tally()
    Kh, Vh = compare_unit_full(pool, offsets, 0, 0, K, V, formats, signs, S, t)
    Kr, Vr = O.reconstruct_unit(K, V, formats, signs, S)
    assert t.mismatches == 0 and t.sign_mismatches == 0 and t.coords == 2 * 6 * 64 * 128
    assert np.array_equal(Kh, Kr) and np.array_equal(Vh, Vr)


def test_reconstruct_unit_takes_an_admissible_sign_override():
    # a sketch row orthogonal to token 5's residual puts (S r)_0 at zero, where
    # either sign is admissible: the other sign moves that key by exactly
    # -/+ 2 sqrt(pi/2) / m * gamma * S_0, and no other row
    rng = np.random.default_rng(11)
    K = rng.standard_normal((64, 128)).astype(np.float16).astype(np.float64)
    V = rng.standard_normal((64, 128)).astype(np.float16).astype(np.float64)
    signs = W.rotation_signs(42, 1)
    fmt = W.packed(2, 2, True)
    S = W.qjl_matrix(42, 1).astype(np.float64)
    kh = O.dequantize(O.encode(K, signs, 2)["norm"], O.encode(K, signs, 2)["codes"], signs, 2)
    r = K[5] - kh[5]
    S[0] -= (S[0] @ r) / (r @ r) * r
    qj = O.qjl_encode(K, kh, S)
    assert qj["near"][5, 0]
    base, _ = O.reconstruct_unit(K, V, [fmt], signs, S)
    flip = not qj["z"][5, 0]
    got, _ = O.reconstruct_unit(K, V, [fmt], signs, S, sign_overrides=([5], [0], [flip]))
    step = np.sqrt(np.pi / 2) / 128 * float(qj["gamma"][5]) * 2.0 * S[0]
    want = base.copy()
    want[5] += step if flip else -step
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    assert np.array_equal(np.delete(got, 5, axis=0), np.delete(base, 5, axis=0))
    # an override away from zero is not admissible
    far = int(np.argmax(np.abs(qj["residual"][3] @ S.T)))
    try:
        O.reconstruct_unit(K, V, [fmt], signs, S, sign_overrides=([3], [far], [not qj["z"][3, far]]))
    except AssertionError:
        pass
    else:
        raise AssertionError("a sign override away from zero was accepted")
