"""Helpers of the GPU parity tests: run the HIP path through the binding, run
the CPU oracle on the same seeded inputs, and compare unit by unit.

Acceptance bars for this method, applied here:
* codes bit-exact, except coordinates whose float64 u lies within 1e-6 of a
  boundary, which may differ by one level; such mismatches must stay
  <= 1e-5 of the coordinates compared (with one coordinate of slack for tiny
  cases);
* QJL sign bits equal except where |(S r)_i| < 1e-5 ||S_i|| ||r|| (float32
  evaluation of the projection), compared on keys whose codes all match;
* QJL sign flips (all of them near zero) at most 1e-5 of the signs compared,
  the same fraction as the codes;
* norms within NORM_ULPS float32 ulp of the oracle's (the float32 rounding of
  the exact norm): the device sums 128 float32 squares, each addition
  rounding, before the square root (worst seen 8 ulp); gamma within a
  relative 1e-5 plus GAMMA_ULPS_OF_X float32 ulp of ||x|| (see below);
* dequantised vectors: cosine >= 0.999999 against the oracle's;
* decode attention: per (session, query head) row,
  max_j |o - o_ref| / max_j |o_ref| <= 1e-3.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from oracle import tq_oracle as O
import workloads as W

BOUNDARY_EPS = 1e-6
MISMATCH_FRACTION = 1e-5
NORM_RTOL = 1e-5          # gamma's relative part
NORM_ULPS = 16
SIGN_FRACTION = 1e-5
# gamma = (n / sqrt(d)) ||u - c||: u - c is formed in float32 from a vector of
# norm sqrt(d), so its error is a few ulp of ||u||, not of ||u - c||; at high
# widths (||u - c|| ~ ||u|| / 150 at 8 bits) that exceeds NORM_RTOL of gamma.
# Bound: |dgamma| <= NORM_RTOL gamma + GAMMA_ULPS_OF_X * 2^-24 ||x||.
GAMMA_ULPS_OF_X = 4
COS_MIN = 0.999999
ATTN_RTOL = 1e-3


def ulps32(got, exp) -> float:
    """Largest |got - exp| in float32 ulp of exp (0 for empty input)."""
    got = np.asarray(got, dtype=np.float32)
    exp = np.asarray(exp, dtype=np.float32)
    if got.size == 0:
        return 0.0
    d = np.abs(got.astype(np.float64) - exp.astype(np.float64))
    return float(np.max(d / np.spacing(np.abs(exp)).astype(np.float64)))


@dataclass
class Tally:
    coords: int = 0
    mismatches: int = 0            # admissible boundary tie-breaks the GPU took
    sign_bits: int = 0
    sign_mismatches: int = 0
    worst_attn: float = 0.0
    worst_cos: float = 1.0
    worst_norm_ulp: float = 0.0
    worst_gamma_rel: float = 0.0
    notes: List[str] = field(default_factory=list)

    def report(self) -> str:
        return (f"parity: {self.coords} codes, {self.mismatches} admissible tie-breaks; "
                f"{self.sign_bits} QJL signs, {self.sign_mismatches} flipped near zero; "
                f"norms within {self.worst_norm_ulp:.2f} ulp, gamma within {self.worst_gamma_rel:.2e} rel; "
                f"attention rel err {self.worst_attn:.2e}; dequantised cosine {self.worst_cos:.9f}")

    def check(self):
        print(self.report(), flush=True)
        allowed = max(1, int(MISMATCH_FRACTION * self.coords))
        assert self.mismatches <= allowed, f"{self.mismatches} code mismatches > {allowed} ({self.coords} coords)"
        if self.sign_bits:
            assert self.sign_mismatches <= max(1, int(SIGN_FRACTION * self.sign_bits)), \
                f"{self.sign_mismatches} QJL sign mismatches of {self.sign_bits}"
        assert self.worst_attn <= ATTN_RTOL, f"attention relative error {self.worst_attn:.3e}"
        assert self.worst_cos >= COS_MIN, f"dequantised cosine {self.worst_cos:.9f}"


def layer_args(k_kind, v_kind) -> dict:
    """tq.Layer codebook arguments for the oracle's kinds: a PolarSplit is kind
    POLAR with the library's table for its shift."""
    import kv_cache_vector_srht_amd as tq
    kw = {}
    for part, kind in (("k", k_kind), ("v", v_kind)):
        if isinstance(kind, O.PolarSplit):
            kw[part + "_codebook"] = tq.POLAR
            kw[part + "_table"] = tq.polar_table(kind.shift)
        else:
            kw[part + "_codebook"] = kind
    return kw


def _cmp_codes(got: np.ndarray, exp: np.ndarray, near: np.ndarray, t: Tally, what: str, lo: int,
               alt: list, kind=O.LLOYD_MAX, bits: int = 0):
    diff = got != exp
    t.coords += got.size
    if diff.any():
        shift = O.polar_shift(kind)
        if shift is None:
            step = np.abs(got - exp)
            bad = diff & ~(near & (step == 1))
        else:
            # PolarQuant: a pair's radius may move one level near a radius
            # boundary and its angle one sector, cyclically, near a sector edge
            rb, ab = O.polar_widths(bits, shift)
            Fg = got[:, 0::2] | (got[:, 1::2] << bits)
            Fe = exp[:, 0::2] | (exp[:, 1::2] << bits)
            m = (1 << rb) - 1
            dr = np.abs((Fg & m) - (Fe & m))
            dt = np.abs((Fg >> rb) - (Fe >> rb))
            dt = np.minimum(dt, (1 << ab) - dt)
            ok = ((dr == 0) | ((dr == 1) & near[:, 0::2])) & ((dt == 0) | ((dt == 1) & near[:, 1::2]))
            bad = diff & ~np.repeat(ok, 2, axis=1)
        assert not bad.any(), f"{what}: {int(bad.sum())} code mismatches away from a boundary " \
                              f"(first at {np.argwhere(bad)[0].tolist()}, got {got[bad][:4]}, want {exp[bad][:4]})"
        t.mismatches += int(diff.sum())
        r, c = np.nonzero(diff)
        alt.append((r + lo, c, got[r, c]))
    return ~diff.any(axis=1)   # rows (tokens) whose codes all match


def _stack(alt):
    if not alt:
        return None
    return tuple(np.concatenate([a[i] for a in alt]) for i in range(3))


def compare_unit_pages(cache, b: int, h: int, K: np.ndarray, V: np.ndarray, formats, signs, S,
                       t: Tally, k_kind=O.LLOYD_MAX, v_kind=O.LLOYD_MAX, n_tokens=None,
                       pool_host: Optional[np.ndarray] = None):
    """Compare every page of unit (b, h) with the oracle's encoding of K, V.

    Returns (k_ok, v_ok, k_alt, v_alt, z_alt): boolean arrays [T] marking
    tokens whose K (resp. V) codes all match, the admissible boundary
    tie-breaks the GPU took, as (tokens, coordinates, codes), and its
    admissible near-zero QJL signs, as (tokens, rows of S, signs), for
    ``reconstruct_unit``.
    """
    T = K.shape[0] if n_tokens is None else n_tokens
    k_ok = np.ones(T, dtype=bool)
    v_ok = np.ones(T, dtype=bool)
    k_alt, v_alt, z_alt = [], [], []
    for p, fmt in enumerate(formats):
        lo, hi = p * 64, min(T, (p + 1) * 64)
        if lo >= T:
            break
        off = int(cache.offsets[b, h, p])
        nbytes = O.page_bytes(fmt)
        raw = (pool_host[off:off + nbytes] if pool_host is not None
               else cache.page_view(b, h, p).cpu().numpy()).tobytes()
        assert len(raw) == nbytes
        if fmt[0] == 0:
            exp = O.fp16_page_bytes(K[lo:hi], V[lo:hi])
            assert raw == exp, f"fp16 page ({b},{h},{p}) differs"
            continue
        enc = O.encode_page(K[lo:hi], V[lo:hi], fmt, signs, S, k_kind, v_kind)
        kb, vb, qjl = fmt
        sec = O.page_sections(fmt)

        def part(name):
            o, n = sec[name]
            return raw[o:o + n]
        kc = O.unpack_block(part("k_codes"), kb)
        ok_rows = _cmp_codes(kc, enc["k"]["codes"], enc["k"]["near"], t, f"K page ({b},{h},{p}) fmt {fmt}",
                             lo, k_alt, k_kind, kb)
        vc = O.v_codes_from_streams(O.unpack_block(part("v_codes"), vb))
        v_rows = _cmp_codes(vc, enc["v"]["codes"], enc["v"]["near"], t, f"V page ({b},{h},{p}) fmt {fmt}",
                            lo, v_alt, v_kind, vb)
        k_ok[lo:hi] = ok_rows
        v_ok[lo:hi] = v_rows
        for name, ref in (("k_norm", enc["k"]["norm"]), ("v_norm", enc["v"]["norm"])):
            got = np.frombuffer(part(name), dtype="<f4")
            t.worst_norm_ulp = max(t.worst_norm_ulp, ulps32(got, ref))
            assert ulps32(got, ref) <= NORM_ULPS, f"{name} page ({b},{h},{p}): {ulps32(got, ref)} ulp"
        if qjl:
            z = O.unpack_signs(part("qjl_signs"))
            g = np.frombuffer(part("qjl_gamma"), dtype="<f4")
            qj = enc["qjl"]
            rows = np.nonzero(ok_rows)[0]
            dz = (z[rows] != qj["z"][rows])
            assert not (dz & ~qj["near"][rows]).any(), f"QJL signs page ({b},{h},{p})"
            t.sign_bits += dz.size
            t.sign_mismatches += int(dz.sum())
            if dz.any():
                r, c = np.nonzero(dz)
                z_alt.append((lo + rows[r], c, z[rows[r], c]))
            assert np.allclose(g[rows], qj["gamma"][rows], rtol=NORM_RTOL, atol=1e-30), \
                f"QJL gamma page ({b},{h},{p})"
            gr = np.abs(g[rows] - qj["gamma"][rows]) / np.maximum(qj["gamma"][rows], 1e-30)
            t.worst_gamma_rel = max(t.worst_gamma_rel, float(gr.max()) if gr.size else 0.0)
            k_ok[lo + rows[dz.any(axis=1)]] = False
    return k_ok, v_ok, _stack(k_alt), _stack(v_alt), _stack(z_alt)


def compare_attention(out_rows: np.ndarray, q_rows: np.ndarray, Kh: np.ndarray, Vh: np.ndarray,
                      t: Tally):
    ref = O.decode_attention_unit(q_rows, Kh, Vh)
    err = np.abs(out_rows - ref).max(axis=1) / np.abs(ref).max(axis=1)
    t.worst_attn = max(t.worst_attn, float(err.max()))
    return ref


def compare_dequant(got: np.ndarray, ref: np.ndarray, t: Tally):
    """Row-wise cosine of the GPU reconstruction against the oracle's."""
    num = np.sum(got * ref, axis=1)
    den = np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1)
    nz = den > 0
    if nz.any():
        t.worst_cos = min(t.worst_cos, float(np.min(num[nz] / den[nz])))
    assert np.all(np.linalg.norm(got[~nz], axis=1) == 0) and np.all(np.linalg.norm(ref[~nz], axis=1) == 0)


def compare_unit_full(pool_host: np.ndarray, offsets: np.ndarray, b: int, h: int, K: np.ndarray,
                      V: np.ndarray, formats, signs, S, t: Tally, k_kind=O.LLOYD_MAX,
                      v_kind=O.LLOYD_MAX, skip=(), parts=None):
    """Compare every page of unit (b, h) with the oracle, encoding the pages of
    one format together (one oracle pass over the unit), and return the
    oracle's reconstruction (Kh, Vh) under the admissible boundary tie-breaks
    and near-zero QJL signs the GPU took: the same composition of oracle steps as
    ``O.reconstruct_unit`` with overrides, without encoding twice.  Pages in
    ``skip`` are left to the caller (their rows of Kh, Vh stay zero).  With a
    ``parts`` dict, also returns there the keys without their QJL term
    ("kbase") and the oracle's sketch ("z" [T, 128] bool, "gamma" [T], zero
    on rows without one)."""
    T = K.shape[0]
    Kh = np.zeros((T, O.HEAD_DIM))
    Vh = np.zeros((T, O.HEAD_DIM))
    if parts is not None:
        parts["kbase"] = np.zeros((T, O.HEAD_DIM))
        parts["z"] = np.zeros((T, O.HEAD_DIM), dtype=bool)
        parts["gamma"] = np.zeros(T, dtype=np.float32)
    groups = {}
    for p, fmt in enumerate(formats):
        lo, hi = p * 64, min(T, (p + 1) * 64)
        if lo >= T:
            break
        if p in skip:
            continue
        off = int(offsets[b, h, p])
        if fmt[0] == 0:
            # the rows the session holds (rows past its tokens are unspecified)
            raw = pool_host[off:off + O.page_bytes(fmt)]
            n = hi - lo
            exp = np.frombuffer(O.fp16_page_bytes(K[lo:hi], V[lo:hi]), dtype=np.uint8)
            half = 64 * O.HEAD_DIM * 2
            assert np.array_equal(raw[:n * 256], exp[:n * 256]) and \
                np.array_equal(raw[half:half + n * 256], exp[half:half + n * 256]), f"fp16 page ({b},{h},{p}) differs"
            Kh[lo:hi] = K[lo:hi].astype(np.float16)
            Vh[lo:hi] = V[lo:hi].astype(np.float16)
            if parts is not None:
                parts["kbase"][lo:hi] = Kh[lo:hi]
        else:
            assert hi - lo == 64, "a packed page must be full"
            groups.setdefault(tuple(fmt), []).append(p)
    for fmt, plist in groups.items():
        kb, vb, qjl = fmt
        sec = O.page_sections(fmt)
        rows = np.concatenate([np.arange(p * 64, (p + 1) * 64) for p in plist])
        raws = [pool_host[int(offsets[b, h, p]):int(offsets[b, h, p]) + O.page_bytes(fmt)] for p in plist]

        def part(name):
            o, n = sec[name]
            return [r[o:o + n].tobytes() for r in raws]
        gk = np.concatenate([O.unpack_block(x, kb) for x in part("k_codes")])
        gv = np.concatenate([O.v_codes_from_streams(O.unpack_block(x, vb)) for x in part("v_codes")])
        what = f"unit ({b},{h}) fmt {fmt}"
        ek = O.encode(K[rows], signs, kb, k_kind)
        ev = O.encode(V[rows], signs, vb, v_kind)
        for name, e in (("k_norm", ek), ("v_norm", ev)):
            got = np.frombuffer(b"".join(part(name)), dtype="<f4")
            t.worst_norm_ulp = max(t.worst_norm_ulp, ulps32(got, e["norm"]))
            assert ulps32(got, e["norm"]) <= NORM_ULPS, f"{name} {what}: {ulps32(got, e['norm'])} ulp"
        k_alt, v_alt = [], []
        _cmp_codes(gk, ek["codes"], ek["near"], t, "K " + what, 0, k_alt, k_kind, kb)
        _cmp_codes(gv, ev["codes"], ev["near"], t, "V " + what, 0, v_alt, v_kind, vb)
        kc, vc = ek["codes"].copy(), ev["codes"].copy()
        for codes, alt in ((kc, k_alt), (vc, v_alt)):
            for r, c, code in alt:
                codes[r, c] = code
        kh = O.dequantize(ek["norm"], kc, signs, kb, k_kind)
        if parts is not None:
            parts["kbase"][rows] = kh
        if qjl:
            qj = O.qjl_encode(K[rows], kh, S)
            z = np.concatenate([O.unpack_signs(x) for x in part("qjl_signs")])
            g = np.frombuffer(b"".join(part("qjl_gamma")), dtype="<f4")
            dz = z != qj["z"]
            assert not (dz & ~qj["near"]).any(), f"QJL signs {what}"
            t.sign_bits += dz.size
            t.sign_mismatches += int(dz.sum())
            dg = np.abs(g - qj["gamma"])
            t.worst_gamma_rel = max(t.worst_gamma_rel, float(np.max(dg / np.maximum(qj["gamma"], 1e-30))))
            xn = np.linalg.norm(K[rows], axis=1)
            assert np.all(dg <= NORM_RTOL * qj["gamma"] + GAMMA_ULPS_OF_X * 2.0 ** -24 * xn + 1e-30), \
                (f"QJL gamma {what}: max rel {np.max(dg / np.maximum(qj['gamma'], 1e-30)):.3e}, "
                 f"max |dgamma| / ||x|| {np.max(dg / np.maximum(xn, 1e-30)):.3e}")
            # the GPU's sign where it is admissible (every difference is, above)
            za = np.where(dz, z, qj["z"])
            kh = kh + O.qjl_reconstruct(za, qj["gamma"], S)
            if parts is not None:
                parts["z"][rows] = za
                parts["gamma"][rows] = qj["gamma"]
        Kh[rows] = kh
        Vh[rows] = O.dequantize(ev["norm"], vc, signs, vb, v_kind)
    return Kh, Vh
