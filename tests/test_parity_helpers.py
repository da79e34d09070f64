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
