"""The kernels' own checks, on the GPU.

* The checked build (libtq_checked.so, compiled with TQ_DEVICE_CHECKS=1: every
  kernel verifies its index invariants as it runs, records a violated one and
  keeps the access in bounds) records nothing and computes the release
  build's results bit for bit: encode at every width (Lloyd-Max with QJL
  keys, PolarQuant keys with QJL, uniform keys with Beta values), decode
  attention, dequantisation, and a decode loop (appends with in-place packing)
  followed by re-tiering.
* LDS barrier discipline: the encoders reuse their LDS across the pages a
  workgroup takes in turn and across the passes of a page, with barriers in
  between; the pages they write do not depend on the launch shape (pages per
  workgroup of the bulk encoder, persistent workgroups of the QJL key
  encoder), byte for byte.
"""
import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import layer_args

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


def _same_bytes(a, b, what):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape, what
    diff = np.flatnonzero(a.view(np.uint8) != b.view(np.uint8))
    assert diff.size == 0, f"{what}: {diff.size} bytes differ, first at {diff[:4].tolist()}"


def _formats(qjl, widths):
    combos = [(kb, vb) for kb in widths for vb in widths]
    P = len(combos) // 2 + 2
    return [[[W.packed(*combos[(p + 7 * h) % len(combos)], qjl and h == 1) for p in range(P)] for h in range(2)]]


def _encode_decode(tq, kinds, qjl, widths, dev, shape=(0, 0)):
    fm = _formats(qjl, widths)
    P = len(fm[0][0])
    w = W.make_workload(2, {"n_tokens": 64 * P, "batch": 1, "n_kv_heads": 2, "n_q_heads": 8, "sink_tokens": 0})
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S if qjl else None, **layer_args(*kinds))
    cache = tq.Cache(fm, [w.n_tokens], dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags, pages_per_block=shape[0], qjl_workgroups=shape[1])
    out = tq.decode_attention(layer, cache, q)
    dk = tq.dequantize(layer, cache, 0, 0, w.n_tokens)
    dv = tq.dequantize(layer, cache, 1, 0, w.n_tokens)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0, f"encode error flags {int(flags.item())}"
    return {"pool": _np(cache.pool), "out": _np(out), "dk": _np(dk), "dv": _np(dv)}


CASES = [((O.LLOYD_MAX, O.LLOYD_MAX), True, range(1, 9)),
         ((O.POLAR, O.LLOYD_MAX), True, range(1, 5)),
         ((O.UNIFORM, O.BETA), False, range(1, 9))]


@pytest.mark.parametrize("kinds,qjl,widths", CASES)
def test_checked_build_encode_decode(dev, kinds, qjl, widths):
    import kv_cache_vector_srht_amd as tq
    print(f"checked build: encode/decode/dequantize, kinds {kinds}, qjl {qjl}", flush=True)
    ref = _encode_decode(tq, kinds, qjl, widths, dev)
    with tq.library():
        assert tq.device_checks(reset=True) is not None
        got = _encode_decode(tq, kinds, qjl, widths, dev)
        flags = tq.device_checks(reset=True)
    assert flags == 0, f"device checks recorded {flags:#x}"
    for name in ref:
        _same_bytes(got[name], ref[name], name)


def _loop_and_retier(tq, dev):
    B, H, G, T = 2, 2, 4, 64 * 3 + 20
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G, "sink_tokens": 64})
    targets = [[W.FP16] + [W.packed(3, 2, False)] * 3, [W.FP16] + [W.packed(2, 2, True)] * 3]
    fm = [[[f if p == 0 else (f[0], f[1], f[2], True) for p, f in enumerate(targets[h])] for h in range(H)]
          for _ in range(B)]
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    start = [100, 90]
    cache = tq.Cache(fm, start, dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    # the first 100 tokens by the bulk encoder (the sink page, a pending page's
    # rows), then one token per session and step; packing fires at every 64th
    tq.encode_kv(layer, cache, k[:, :, :100], v[:, :, :100], tok0=0, error_flags=flags)
    outs = []
    for step in range(T - max(start)):
        kk = torch.stack([k[b, :, start[b] + step] for b in range(B)]).contiguous()
        vv = torch.stack([v[b, :, start[b] + step] for b in range(B)]).contiguous()
        tq.append_kv(layer, cache, kk, vv, error_flags=flags)
        if step % 16 == 0:
            outs.append(_np(tq.decode_attention(layer, cache, q)))
    # demote head 0's packed pages (K3/V2) to K1/V1 in place (QJL pages are no
    # re-tiering source)
    pages = [(b, 0, p) for b in range(B) for p in (1, 2)]
    tq.retier_pages(layer, cache, pages, [(1, 1, False)] * len(pages), error_flags=flags)
    outs.append(_np(tq.decode_attention(layer, cache, q)))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0, f"error flags {int(flags.item())}"
    return {"pool": _np(cache.pool), "n_tokens": _np(cache.n_tokens), "out": np.stack(outs)}


def test_checked_build_decode_loop_and_retier(dev):
    import kv_cache_vector_srht_amd as tq
    print("checked build: decode loop (append, pack in place) and re-tiering", flush=True)
    ref = _loop_and_retier(tq, dev)
    with tq.library():
        tq.device_checks(reset=True)
        got = _loop_and_retier(tq, dev)
        flags = tq.device_checks(reset=True)
    assert flags == 0, f"device checks recorded {flags:#x}"
    for name in ref:
        _same_bytes(got[name], ref[name], name)


@pytest.mark.parametrize("kinds,qjl,widths", CASES[:2])
def test_encoder_launch_shapes_write_the_same_pages(dev, kinds, qjl, widths):
    import kv_cache_vector_srht_amd as tq
    ref = _encode_decode(tq, kinds, qjl, widths, dev)
    for shape in ((1, 0), (2, 1), (3, 3), (8, 2), (16, 0), (5, 64)):
        print(f"launch shape {shape}: pages per workgroup, QJL workgroups", flush=True)
        got = _encode_decode(tq, kinds, qjl, widths, dev, shape)
        _same_bytes(got["pool"], ref["pool"], f"pool at launch shape {shape}")
        _same_bytes(got["out"], ref["out"], f"decode after launch shape {shape}")
