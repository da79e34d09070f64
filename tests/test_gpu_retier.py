"""GPU parity of page re-tiering (tq_retier_pages): packed pages demoted to
narrower widths through the code-to-code table, fp16 pages encoded into packed
formats, in place and into other slots, followed by decode attention over the
re-tiered cache.  The oracle's view: a demoted page holds the oracle's codes of
the original rows requantised to the new widths (``O.requantize_codes``) with
the original norms; an fp16-sourced page holds the oracle's encoding of its
fp16 rows."""
import ctypes

import numpy as np
import pytest

import workloads as W
from oracle import tq_oracle as O
from tests.gpu_parity import NORM_ULPS, Tally, compare_attention, compare_unit_full, ulps32

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


def _plan(B, H, P, seed):
    """Old formats [B][H][P] and the re-tiering list {(b, h, p): new format}.
    Covers every (old width, new width) demotion pair for keys and for values,
    fp16 pages into plain and QJL formats, and untouched pages of each kind."""
    rng = np.random.default_rng(seed)
    pairs = [(ob, nb) for ob in range(1, 9) for nb in range(1, ob + 1)]
    kp, vp = rng.permutation(len(pairs)), rng.permutation(len(pairs))
    slots = []
    for i in range(len(pairs)):
        (kb, nkb), (vb, nvb) = pairs[kp[i]], pairs[vp[i]]
        slots.append((W.packed(kb, vb), W.packed(nkb, nvb)))
    for tgt in [(4, 4, False), (3, 2, False), (2, 1, False), (1, 1, False), (8, 8, False),
                (2, 2, True), (5, 3, True), (1, 1, True)]:
        slots.append((W.FP16, tgt))
    for keep in [W.FP16, W.FP16, W.packed(2, 2, True), W.packed(4, 4), W.packed(6, 7)]:
        slots.append((keep, None))
    while len(slots) < B * H * P:
        slots.append((W.packed(int(rng.integers(1, 9)), int(rng.integers(1, 9))), None))
    assert len(slots) == B * H * P
    order = rng.permutation(len(slots))
    old = [[[None] * P for _ in range(H)] for _ in range(B)]
    todo = {}
    for n, i in enumerate(order):
        b, h, p = n // (H * P), (n // P) % H, n % P
        old[b][h][p], new = slots[i]
        if new is not None:
            todo[(b, h, p)] = new
    return old, todo


def compare_demoted(raw, old, new, K, V, signs, t, k_kind, v_kind, what):
    """One demoted page against the oracle; returns its reconstruction."""
    (kb, vb, _), (nkb, nvb, _) = old, new
    ek, ev = O.encode(K, signs, kb, k_kind), O.encode(V, signs, vb, v_kind)
    sec = O.page_sections(new)

    def part(name):
        o, n = sec[name]
        return raw[o:o + n].tobytes()
    got = {"k": O.unpack_block(part("k_codes"), nkb),
           "v": O.v_codes_from_streams(O.unpack_block(part("v_codes"), nvb))}
    recon = {}
    for which, e, ob, nb, kind in (("k", ek, kb, nkb, k_kind), ("v", ev, vb, nvb, v_kind)):
        exp = O.requantize_codes(e["codes"], ob, nb, kind)
        g = got[which]
        diff = g != exp
        t.coords += g.size
        if diff.any():
            # an admissible boundary tie-break of the encode, carried through the
            # map: the GPU's old code was a neighbour of the oracle's
            c = e["codes"][diff]
            lo = O.requantize_codes(np.maximum(c - 1, 0), ob, nb, kind)
            hi = O.requantize_codes(np.minimum(c + 1, (1 << ob) - 1), ob, nb, kind)
            ok = e["near"][diff] & ((g[diff] == lo) | (g[diff] == hi))
            assert ok.all(), f"{what} {which}: {int((~ok).sum())} requantised codes differ away from a boundary"
            t.mismatches += int(diff.sum())
        norm = np.frombuffer(part(f"{which}_norm"), dtype="<f4")
        assert ulps32(norm, e["norm"]) <= NORM_ULPS, f"{what} {which} norms"
        recon[which] = O.dequantize(e["norm"], g, signs, nb, kind)
    return recon["k"], recon["v"]


@pytest.mark.parametrize("kinds", [(O.LLOYD_MAX, O.LLOYD_MAX), (O.UNIFORM, O.LLOYD_MAX)])
def test_retier_pages_parity(dev, kinds):
    import kv_cache_vector_srht_amd as tq
    kk, vk = kinds
    B, H, G, P = 2, 4, 2, 8
    T = P * 64
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 0, "dtype": "float32"})
    old, todo = _plan(B, H, P, seed=7 + kk)
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S, kk, vk)
    listed = sorted(todo)
    # every third listed page moves to a new slot past the pages
    moved = listed[::3]
    spare = sum((tq.page_bytes(todo[p]) + 255) // 256 * 256 for p in moved)
    cache = tq.Cache(old, [T] * B, dev, spare_bytes=spare)
    new_off, at = [], cache.spare_offset
    for p in listed:
        if p in moved:
            new_off.append(at)
            at += (tq.page_bytes(todo[p]) + 255) // 256 * 256
        else:
            new_off.append(int(cache.offsets[p]))
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, tok0=0, error_flags=flags)
    torch.cuda.synchronize()
    before = _np(cache.pool).copy()
    old_offsets = cache.offsets.copy()
    print(f"re-tiering {len(listed)} pages ({len(moved)} moved), codebooks {kinds}", flush=True)
    tq.retier_pages(layer, cache, listed, [todo[p] for p in listed], new_offsets=new_off, error_flags=flags)
    out = _np(tq.decode_attention(layer, cache, q))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0, f"error flags {int(flags.item())}"
    assert np.array_equal(_np(cache.pages).view(np.uint64), cache.host_pages)
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    for b in range(B):
        for h in range(H):
            for p in range(P):
                o = int(old_offsets[b, h, p])
                n = tq.page_bytes(old[b][h][p])
                if (b, h, p) not in todo or (b, h, p) in moved:
                    assert np.array_equal(pool[o:o + n], before[o:o + n]), f"page {(b, h, p)} changed"
            demoted = [p for p in range(P) if (b, h, p) in todo and old[b][h][p][0] != 0]
            Keff, Veff = kh[b, h].copy(), vh[b, h].copy()
            for p in range(P):
                if (b, h, p) in todo and old[b][h][p][0] == 0:
                    r = slice(64 * p, 64 * p + 64)
                    Keff[r] = Keff[r].astype(np.float16)
                    Veff[r] = Veff[r].astype(np.float16)
            Kh, Vh = compare_unit_full(pool, cache.offsets, b, h, Keff, Veff, cache.formats[b][h], signs, S,
                                       t, kk, vk, skip=set(demoted))
            for p in demoted:
                r = slice(64 * p, 64 * p + 64)
                off = int(cache.offsets[b, h, p])
                raw = pool[off:off + tq.page_bytes(todo[(b, h, p)])]
                Kh[r], Vh[r] = compare_demoted(raw, old[b][h][p], todo[(b, h, p)], kh[b, h, r], vh[b, h, r],
                                               signs, t, kk, vk, f"page {(b, h, p)}")
            compare_attention(out[b, h * G:(h + 1) * G], qh[b, h * G:(h + 1) * G], Kh, Vh, t)
    t.check()


def _raw_retier(cache, layer, idx, descs, flags, sources=0):
    import kv_cache_vector_srht_amd as tq
    i = torch.tensor(idx, dtype=torch.int64, device=cache.device)
    d = torch.from_numpy(np.array(descs, dtype=np.uint64).view(np.int64)).to(cache.device)
    st = tq.lib().tq_retier_pages(ctypes.byref(layer.struct), ctypes.byref(cache.struct), i.data_ptr(),
                                  d.data_ptr(), len(idx), sources, flags.data_ptr(), None)
    tq.check(st, "tq_retier_pages")
    torch.cuda.synchronize()


def test_retier_rejects_unsupported_changes(dev):
    """Each refused change raises its flag and leaves the page and its
    descriptor as they were."""
    import kv_cache_vector_srht_amd as tq
    L = tq.lib()
    fm = [[[W.FP16, W.packed(4, 4), W.packed(2, 2, True), (3, 2, False, True), W.packed(3, 3)]]]
    signs = W.rotation_signs(42, 0)
    layer = tq.Layer(signs, dev, None)           # no S: a QJL target is refused
    cache = tq.Cache(fm, [5 * 64], dev)
    w = W.make_workload(2, {"n_tokens": 5 * 64, "batch": 1, "n_kv_heads": 1, "n_q_heads": 1,
                            "sink_tokens": 0})
    k, v = W.make_kv(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k[:, :, :64 * 3], v[:, :, :64 * 3], tok0=0, error_flags=flags)
    tq.encode_kv(layer, cache, k[:, :, 64 * 4:], v[:, :, 64 * 4:], tok0=64 * 4, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    off = cache.offsets[0, 0]

    def desc(p, kb, vb, q=0, o=None):
        return L.tq_page_descriptor(int(off[p] if o is None else o), kb, vb, q)
    cases = [
        ([1], [desc(1, 5, 4)], 64),                  # a packed width that grows
        ([2], [desc(2, 1, 1)], 64),                  # a QJL page as the source
        ([1], [desc(1, 2, 2, 1)], 64),               # QJL target from a packed page
        ([3], [desc(3, 2, 2)], 64),                  # a pending page
        ([0], [desc(0, 2, 2, 1)], 8),                # QJL target, the layer has no S
        ([5], [desc(0, 2, 2)], 16),                  # past the page table
        ([-1], [desc(0, 2, 2)], 16),
        ([1], [desc(1, 2, 2) & ~tq_present()], 2),   # target not present
        ([4], [desc(4, 2, 2, o=off[4] + 256)], 4),   # overlaps its old slot
        ([4], [desc(4, 2, 2, o=cache.pool_bytes)], 4),   # outside the pool
    ]
    for idx, ds, want in cases:
        pool0, pages0 = _np(cache.pool).copy(), _np(cache.pages).copy()
        flags.zero_()
        print(f"case {idx} -> flag {want}", flush=True)
        _raw_retier(cache, layer, idx, ds, flags)
        assert int(flags.item()) == want, (idx, int(flags.item()), want)
        assert np.array_equal(_np(cache.pool), pool0) and np.array_equal(_np(cache.pages), pages0)
    # a source kind the hint leaves out is refused (page 1 is packed, page 0 fp16)
    for idx, ds, src in (([1], [desc(1, 2, 2)], 2), ([0], [desc(0, 2, 2)], 1)):
        pool0, pages0 = _np(cache.pool).copy(), _np(cache.pages).copy()
        flags.zero_()
        _raw_retier(cache, layer, idx, ds, flags, sources=src)
        assert int(flags.item()) == 64
        assert np.array_equal(_np(cache.pool), pool0) and np.array_equal(_np(cache.pages), pages0)
    # a good entry next to a refused one still goes through
    flags.zero_()
    _raw_retier(cache, layer, [1, 2], [desc(1, 2, 1), desc(2, 1, 1)], flags)
    assert int(flags.item()) == 64
    assert _np(cache.pages).view(np.uint64)[0, 0, 1] == desc(1, 2, 1)


def tq_present():
    return 1 << 63


def test_retier_fp16_into_polar_and_refuse_polar_demotion(dev):
    """With PolarQuant parts an fp16 page is encoded into a polar format of at
    most 4 bits; a packed polar page is not re-coded (flag 64) and a polar
    target wider than 4 bits is refused (flag 4)."""
    import kv_cache_vector_srht_amd as tq
    B, H, G, P = 1, 2, 4, 4
    T = P * 64
    w = W.make_workload(2, {"n_tokens": T, "batch": B, "n_kv_heads": H, "n_q_heads": H * G,
                            "sink_tokens": 0, "dtype": "float16"})
    fm = [[[W.FP16, W.FP16, W.packed(3, 2), W.FP16] for _ in range(H)]]
    signs, S = W.rotation_signs(42, 0), W.qjl_matrix(42, 0)
    layer = tq.Layer(signs, dev, S, tq.POLAR, tq.POLAR)
    cache = tq.Cache(fm, [T], dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    tq.encode_kv(layer, cache, k, v, error_flags=flags)
    tq.retier_pages(layer, cache, [(0, 0, 0), (0, 1, 1), (0, 1, 0)],
                    [(4, 4, False), (2, 1, True), (3, 3, False)], error_flags=flags)
    out = _np(tq.decode_attention(layer, cache, q))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    pool = _np(cache.pool)
    kh, vh, qh = _np(k).astype(np.float64), _np(v).astype(np.float64), _np(q).astype(np.float64)
    t = Tally()
    for h in range(H):
        Keff, Veff = kh[0, h].copy(), vh[0, h].copy()
        Kh, Vh = compare_unit_full(pool, cache.offsets, 0, h, Keff, Veff, cache.formats[0][h], signs, S, t,
                                   O.POLAR, O.POLAR)
        compare_attention(out[0, h * G:(h + 1) * G], qh[0, h * G:(h + 1) * G], Kh, Vh, t)
    t.check()
    L = tq.lib()
    off = cache.offsets[0, 0]
    for idx, d, want in (([2], [L.tq_page_descriptor(int(off[2]), 2, 1, 0)], 64),
                         ([3], [L.tq_page_descriptor(int(off[3]), 6, 2, 0)], 4)):
        pool0 = _np(cache.pool).copy()
        flags.zero_()
        _raw_retier(cache, layer, idx, d, flags)
        assert int(flags.item()) == want
        assert np.array_equal(_np(cache.pool), pool0)
