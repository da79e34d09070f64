"""The seeded workload recipes and random draws (shared by both sides)."""
import json
import math
import os

import numpy as np

import workloads as W


def test_splitmix64_reference_vector():
    with open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64_reference.json")) as f:
        g = json.load(f)
    assert W.splitmix64(g["seed"], 5) == g["outputs"]


def test_layer_randomness_shapes_and_statistics():
    s = W.rotation_signs(42, 0)
    assert s.dtype == np.int8 and set(np.unique(s).tolist()) <= {-1, 1}
    assert not np.array_equal(s, W.rotation_signs(42, 1))   # per-layer seeds differ
    S = W.qjl_matrix(42, 0)
    assert S.shape == (128, 128) and S.dtype == np.float32
    assert abs(S.mean()) < 0.03 and abs(S.std() - 1) < 0.03
    # Box-Muller of the published definition: first pair by hand
    z = W.splitmix64(42, 2, start=128)
    u1, u2 = (z[0] >> 11) * 2.0 ** -53, (z[1] >> 11) * 2.0 ** -53
    r = math.sqrt(-2 * math.log(1 - u1))
    assert S[0, 0] == np.float32(r * math.cos(2 * math.pi * u2))
    assert S[0, 1] == np.float32(r * math.sin(2 * math.pi * u2))


def test_workload_plans():
    w2 = W.make_workload(2)
    f = w2.formats[0][0][0]
    assert f[:2] == [W.FP16, W.FP16] and all(x == (4, 4, False) for x in f[2:]) and len(f) == 64
    w3 = W.make_workload(3, {"n_tokens": 640})
    bits = {w3.formats[l][0][h][0] for l in range(36) for h in range(8)}
    assert all(1 <= kb <= 8 for kb, vb, q in bits) and (3, 2, False) in bits
    hub = [kb for kb, vb, q in bits if kb >= 6]
    per = [kb for kb, vb, q in bits if kb <= 2]
    assert hub and per
    w4 = W.make_workload(4, {"n_tokens": 640, "batch": 2})
    assert w4.formats[0][1][3][2] == (2, 2, True) and w4.formats[0][1][3][0] == W.FP16
    w5 = W.make_workload(5)
    row = w5.formats[0][0][0]
    assert len(row) == 4096 and all(x == W.FP16 for x in row[-16:])
    assert all(x != W.FP16 for x in row[:-16])


def test_tier_by_age():
    assert [W.tier_of_age(a) for a in (0, 1023, 1024, 8191, 8192, 65535, 65536)] == [0, 0, 1, 1, 2, 2, 3]


def test_generated_tensors_are_seeded():
    w = W.make_workload(2)
    k1, v1 = W.make_kv(w, 0, tokens=64)
    k2, v2 = W.make_kv(w, 0, tokens=64)
    assert (k1 == k2).all() and (v1 == v2).all()
    ch, sc = W.outlier_channels(2, 0, 8)[0]
    assert 2 <= len(ch) <= 6 and np.all((sc >= 10) & (sc <= 30))
    big = k1[0, 0].float().abs().mean(0)
    assert float(big[ch].min()) > 3 * float(np.delete(big.numpy(), ch).mean())
