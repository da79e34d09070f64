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
