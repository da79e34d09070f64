"""CPU oracle for the SRHT KV-cache codec and compressed-domain decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it: the only code both sides share is the seeded
input generator module ``workloads``.

Everything is plain numpy in float64 (scipy/mpmath only as root finders), written
to be read against the source pages:

* "TurboQuant-MLX v2.0", What's New > Walsh-Hadamard Rotation and
  How It Works > Pipeline: the randomized rotation is the SRHT ``D @ H @ D``
  (sign diagonal, Walsh-Hadamard, the same sign diagonal), O(n log n),
  orthogonal and invertible; the norm of each vector is kept and no per-block
  constants are stored; QJL corrects keys only with ``sign(S . residual)``.
* "TurboMOQ", Architecture and Full Feature Set: Lloyd-Max codebooks,
  symmetric/grid quantisation, per-head bit widths 1-8; QJL residual
  correction section: 1-bit sign-encoded JL projection with a per-vector scale.
* "TurboQuant-MLX v2.0", What's New > FP16 Attention Sinks and Dynamic Chunk
  Buffering: the first 128 tokens stay fp16, compression fires on 64-token chunks.

Readings where the pages are silent (each also listed in the design notes):
  R1 one sign diagonal D on both sides of H, so R = D H D / sqrt(d) is symmetric
     and its own inverse; H in Sylvester (natural) order.
  R2 the scalar quantiser sees u = sqrt(d) R x / ||x||, which is ~N(0,1) per
     coordinate; the norm is stored as float32.
  R3 code = #{k : t_k <= u} with t the float32 boundaries (ties round up) and the
     decision taken in float32 on both sides: u is rounded to float32 first.
  R4 code 0 is the most negative centroid; codes are packed LSB-first in
     128-code streams (layout below).
  R5 QJL: r = x - xhat in the original domain, z = sign(S r) with sign(0) = +1,
     gamma = ||r|| (float32), rhat = sqrt(pi/2)/m * gamma * S^T z.
  R6 attention: scores q.k / sqrt(d), softmax over every cached token of the
     session, query head h reads KV head floor(h / G).

Parity pins live in ``tests/test_oracle_pins.py``.  The packing layout itself is
a convention (the pages name bit packing only as a utility module); it is pinned by
the bijection/round-trip/footprint checks there.
"""
from __future__ import annotations

import math
from functools import lru_cache
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy import optimize
from scipy.special import ndtr

HEAD_DIM = 128
PAGE_TOKENS = 64
STREAM_CODES = 128
LLOYD_MAX = 0
UNIFORM = 1
BETA = 2
POLAR = 4      # PolarQuant: coordinate pairs as (radius, angle)


# ----------------------------------------------------------------------------
# Rotation ("TurboQuant-MLX v2.0", What's New > Walsh-Hadamard Rotation).
# ----------------------------------------------------------------------------
def sylvester_hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H, H], [H, -H]] (int64)."""
    assert d >= 1 and (d & (d - 1)) == 0
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def rotation_matrix(signs: Sequence[int]) -> np.ndarray:
    """R = D H D / sqrt(d) with D = diag(signs) (reading R1), float64."""
    return _rotation_cached(tuple(int(v) for v in np.asarray(signs).ravel())).copy()


def signed_hadamard(signs: Sequence[int]) -> np.ndarray:
    """D H D with D = diag(signs), the unnormalised rotation: entries +-1
    (float64, exact).  u = sqrt(d) R x / n = (D H D x) / n, since the sqrt(d)
    of R = D H D / sqrt(d) cancels."""
    s = np.asarray(signs, dtype=np.float64).ravel()
    return s[:, None] * sylvester_hadamard(s.shape[0]).astype(np.float64) * s[None, :]


@lru_cache(maxsize=64)
def _rotation_cached(signs: Tuple[int, ...]) -> np.ndarray:
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    Dm = np.diag(s)
    return Dm @ sylvester_hadamard(d).astype(np.float64) @ Dm / math.sqrt(d)


# ----------------------------------------------------------------------------
# Codebooks ("TurboMOQ", Architecture: Lloyd-Max codebook; symmetric grid).
# ----------------------------------------------------------------------------
def _phi(x):
    with np.errstate(over="ignore"):
        return np.exp(-0.5 * np.square(x)) / math.sqrt(2.0 * math.pi)


def _mass(a, b):
    """P(a <= Z < b) for Z ~ N(0,1), evaluated on the tail side (no cancellation)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.where(a >= 0, ndtr(-a) - ndtr(-b), ndtr(b) - ndtr(a))


def _centroids_of_cells(edges):
    """E[Z | edges_k <= Z < edges_k+1] for every cell."""
    return (_phi(edges[:-1]) - _phi(edges[1:])) / _mass(edges[:-1], edges[1:])


def _lloyd_map(cpos: np.ndarray) -> np.ndarray:
    """One Lloyd-Max update of the positive half of a symmetric codebook.

    Boundaries are midpoints of neighbouring centroids; centroids are the
    conditional means of N(0,1) over their cells.
    """
    c = np.concatenate((-cpos[::-1], cpos))
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    return _centroids_of_cells(edges)[cpos.size:]


@lru_cache(maxsize=None)
def lloyd_max_gaussian(bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """MSE-optimal 2^bits-level scalar quantiser for N(0,1) (Lloyd-Max).

    The quantiser is the unique fixed point (N(0,1) is log-concave) of the two
    Lloyd-Max conditions; it is symmetric, so only the positive half is solved.
    Steps: Lloyd iterations from a spread start, a library root finder on the
    conditions in float64, then Newton steps in 40-digit arithmetic (the fixed
    point is ill-conditioned at 8 bits: the Lloyd map contracts by 0.99985).

    Returns (centroids, boundaries) in float64, ascending; boundaries are the
    midpoints of neighbouring centroids.
    """
    import mpmath as mp
    L = 1 << bits
    h = L // 2
    k = np.arange(h)
    cpos = math.sqrt(3.0) * np.sqrt(2.0) * np.array(
        [float(mp.erfinv((2 * (h + i) + 1) / L - 1)) for i in k])
    for _ in range(200):
        cpos = _lloyd_map(cpos)
    sol = optimize.root(lambda c: c - _lloyd_map(c), cpos, method="hybr", tol=1e-15)
    cpos = np.sort(sol.x)

    with mp.workdps(40):
        def cond_mean(a, b):
            pa = mp.npdf(a) if a != -mp.inf else mp.mpf(0)
            pb = mp.npdf(b) if b != mp.inf else mp.mpf(0)
            if a >= 0:
                m = mp.ncdf(-a) - mp.ncdf(-b)
            else:
                m = mp.ncdf(b) - mp.ncdf(a)
            return (pa - pb) / m

        def F(*cp):
            c = [-x for x in reversed(cp)] + list(cp)
            t = [(c[i] + c[i + 1]) / 2 for i in range(len(c) - 1)]
            e = [-mp.inf] + t + [mp.inf]
            return [cp[i] - cond_mean(e[h + i], e[h + i + 1]) for i in range(h)]

        x0 = [mp.mpf(float(v)) for v in cpos]
        if h == 1:
            root = [mp.findroot(lambda x: F(x)[0], x0[0])]
        else:
            root = mp.findroot(F, x0, tol=mp.mpf(10) ** -30)
            root = [root[i] for i in range(h)]
        root = [+r for r in root]   # round to the working precision first
        cfull = [-x for x in reversed(root)] + list(root)
        tfull = [(cfull[i] + cfull[i + 1]) / 2 for i in range(L - 1)]
        c = np.array([float(x) for x in cfull])
        t = np.array([float(x) for x in tfull])
        # float32 rounding taken from the high-precision values
        c32 = np.array([_round_f32(x) for x in cfull], dtype=np.float32)
        t32 = np.array([_round_f32(x) for x in tfull], dtype=np.float32)
    _F32_TABLES[(bits, LLOYD_MAX)] = (c32, t32)
    return c, t


def _round_f32(x) -> np.float32:
    """float32 nearest to the mpmath number x (checked against both neighbours)."""
    import mpmath as mp
    f = np.float32(float(x))
    cands = (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf)))
    return min(cands, key=lambda c: abs(mp.mpf(float(c)) - x))


_F32_TABLES: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = {}


@lru_cache(maxsize=None)
def uniform_gaussian(bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric mid-rise uniform grid with the MSE-optimal step for N(0,1).

    Levels c_k = (k - (L-1)/2) * delta, boundaries at their midpoints
    (k - L/2) * delta.  delta solves d MSE / d delta = 0, i.e.
    delta * sum_k m_k^2 P_k = sum_k m_k (phi(a_k) - phi(b_k)) with m_k the
    level multipliers and [a_k, b_k) the cells (the cell edges move with delta,
    but the squared error is continuous across them, so no edge terms appear).
    """
    import mpmath as mp
    L = 1 << bits
    m = [mp.mpf(2 * k - (L - 1)) / 2 for k in range(L)]

    with mp.workdps(40):
        def g(delta):
            num = mp.mpf(0)
            den = mp.mpf(0)
            for k in range(L):
                a = -mp.inf if k == 0 else (k - mp.mpf(L) / 2) * delta
                b = mp.inf if k == L - 1 else (k + 1 - mp.mpf(L) / 2) * delta
                pa = mp.mpf(0) if a == -mp.inf else mp.npdf(a)
                pb = mp.mpf(0) if b == mp.inf else mp.npdf(b)
                P = mp.ncdf(b) - mp.ncdf(a) if (a == -mp.inf or a < 0) else mp.ncdf(-a) - mp.ncdf(-b)
                num += m[k] * (pa - pb)
                den += m[k] ** 2 * P
            return delta * den - num

        # bracket from the 1-bit closed form downward
        delta = mp.findroot(g, (mp.mpf(0.5) * 4 / L, mp.mpf(4.0) * 4 / L), solver="anderson")
        cfull = [mk * delta for mk in m]
        tfull = [(k + 1 - mp.mpf(L) / 2) * delta for k in range(L - 1)]
        c = np.array([float(x) for x in cfull])
        t = np.array([float(x) for x in tfull])
        _F32_TABLES[(bits, UNIFORM)] = (
            np.array([_round_f32(x) for x in cfull], dtype=np.float32),
            np.array([_round_f32(x) for x in tfull], dtype=np.float32))
        _UNIFORM_DELTA[bits] = float(delta)
    return c, t


_UNIFORM_DELTA: Dict[int, float] = {}


# The Beta codebook ("TurboMOQ", Head-to-Head Comparison: Beta-CDF; Project
# Structure: Beta-distribution codebooks): Lloyd-Max for the law of one
# coordinate of sqrt(d) times a uniformly random unit vector of R^d,
#   f(u) = C (1 - u^2/d)^((d-3)/2) on |u| < sqrt(d),
#   C = Gamma(d/2) / (sqrt(pi d) Gamma((d-1)/2)),
# i.e. u^2/d ~ Beta(1/2, (d-1)/2).  For x >= 0 the upper tail is
# (1/2) I_{1-x^2/d}((d-1)/2, 1/2) and the partial first moment
# int_x^sqrt(d) u f(u) du = C d/(d-1) (1 - x^2/d)^((d-1)/2).
def _sphere_c(d: int) -> float:
    return math.exp(math.lgamma(d / 2) - math.lgamma((d - 1) / 2)) / math.sqrt(math.pi * d)


def _sphere_lloyd_map(cpos: np.ndarray, d: int) -> np.ndarray:
    """One Lloyd-Max update of the positive half under the sphere marginal."""
    from scipy.special import betainc
    C = _sphere_c(d)
    c = np.concatenate((-cpos[::-1], cpos))
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([0.0], t[cpos.size:], [math.sqrt(d)]))
    y = np.clip(1.0 - edges * edges / d, 0.0, 1.0)
    tail = 0.5 * betainc((d - 1) / 2, 0.5, y)
    mom = C * d / (d - 1) * y ** ((d - 1) / 2)
    return (mom[:-1] - mom[1:]) / (tail[:-1] - tail[1:])


@lru_cache(maxsize=None)
def lloyd_max_sphere(bits: int, d: int = HEAD_DIM) -> Tuple[np.ndarray, np.ndarray]:
    """MSE-optimal 2^bits-level quantiser of the sphere marginal above.

    Steps as for the Gaussian: Lloyd iterations from the Gaussian codebook, a
    library root finder in float64, then Newton steps in 40-digit arithmetic
    whose Jacobian is the tridiagonal one of the conditions
    c_i = E[U | a_i <= U < b_i] with a_i, b_i the midpoints next to c_i:
    d mean / d a = f(a) (mean - a) / P and d mean / d b = f(b) (b - mean) / P.
    Returns (centroids, boundaries) in float64, ascending.
    """
    import mpmath as mp
    L = 1 << bits
    h = L // 2
    cpos = lloyd_max_gaussian(bits)[0][h:].copy()
    for _ in range(200):
        cpos = _sphere_lloyd_map(cpos, d)
    sol = optimize.root(lambda c: c - _sphere_lloyd_map(c, d), cpos, method="hybr", tol=1e-15)
    cpos = np.sort(sol.x)
    with mp.workdps(40):
        D = mp.mpf(d)
        C = mp.gamma(D / 2) / (mp.sqrt(mp.pi * D) * mp.gamma((D - 1) / 2))
        end = mp.sqrt(D)

        def dens(x):
            y = 1 - x * x / D
            return C * y ** ((D - 3) / 2) if y > 0 else mp.mpf(0)

        def tail(x):
            y = 1 - x * x / D
            return mp.betainc((D - 1) / 2, mp.mpf(1) / 2, 0, y, regularized=True) / 2 if y > 0 else mp.mpf(0)

        def mom(x):
            y = 1 - x * x / D
            return C * D / (D - 1) * y ** ((D - 1) / 2) if y > 0 else mp.mpf(0)

        c = [mp.mpf(float(v)) for v in cpos]
        for _ in range(30):
            a = [mp.mpf(0)] + [(c[i - 1] + c[i]) / 2 for i in range(1, h)]
            b = a[1:] + [end]
            ta = [tail(x) for x in a] + [mp.mpf(0)]
            ma = [mom(x) for x in a] + [mp.mpf(0)]
            P = [ta[i] - ta[i + 1] for i in range(h)]
            mean = [(ma[i] - ma[i + 1]) / P[i] for i in range(h)]
            da = [dens(a[i]) * (mean[i] - a[i]) / P[i] for i in range(h)]
            db = [dens(b[i]) * (b[i] - mean[i]) / P[i] if i < h - 1 else mp.mpf(0) for i in range(h)]
            # J step = -F, J tridiagonal: lower -da_i/2, diagonal 1 - (da_i + db_i)/2, upper -db_i/2
            rhs = [-(c[i] - mean[i]) for i in range(h)]
            diag = [1 - (da[i] if i > 0 else 0) / 2 - db[i] / 2 for i in range(h)]
            low = [-da[i] / 2 if i > 0 else mp.mpf(0) for i in range(h)]
            up = [-db[i] / 2 for i in range(h)]
            for i in range(1, h):
                w = low[i] / diag[i - 1]
                diag[i] -= w * up[i - 1]
                rhs[i] -= w * rhs[i - 1]
            step = [mp.mpf(0)] * h
            step[h - 1] = rhs[h - 1] / diag[h - 1]
            for i in range(h - 2, -1, -1):
                step[i] = (rhs[i] - up[i] * step[i + 1]) / diag[i]
            c = [c[i] + step[i] for i in range(h)]
            if max(abs(x) for x in step) < mp.mpf(10) ** -34:
                break
        cfull = [-x for x in reversed(c)] + list(c)
        tfull = [(cfull[i] + cfull[i + 1]) / 2 for i in range(L - 1)]
        if d == HEAD_DIM:
            _F32_TABLES[(bits, BETA)] = (
                np.array([_round_f32(x) for x in cfull], dtype=np.float32),
                np.array([_round_f32(x) for x in tfull], dtype=np.float32))
        return np.array([float(x) for x in cfull]), np.array([float(x) for x in tfull])


def uniform_step(bits: int) -> float:
    uniform_gaussian(bits)
    return _UNIFORM_DELTA[bits]


# PolarQuant ("TurboQuant-MLX v2.0", How It Works > Pipeline and Architecture
# Notes; the cache's r_bits / theta_bits, Quick Start): after the rotation each
# coordinate pair (u_2i, u_2i+1) becomes a radius and an angle, quantised
# independently, with no per-block constants.  Readings: the pair of a
# rotated, normalised vector is close to a standard 2-D Gaussian pair, whose
# radius is Rayleigh(1) and angle uniform; the radius takes the Lloyd-Max
# quantiser of Rayleigh(1) and the angle the uniform grid of L = 2^b sectors
# [-pi + 2 pi k / L, -pi + 2 pi (k+1) / L) with level at the sector's middle;
# r_bits = theta_bits = the page width b, so a polar page has the size and
# stream layout of a scalar one: stream position 2i holds pair i's radius
# code, position 2i+1 its angle code.
def _rayleigh_lloyd_map(c: np.ndarray) -> np.ndarray:
    """One Lloyd-Max update for Rayleigh(1): cells between midpoints, from 0 to inf."""
    e = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    tail = np.exp(-0.5 * e * e)                                       # P(R >= x)
    mom = np.where(np.isinf(e), 0.0, np.nan_to_num(e) * tail) + math.sqrt(2 * math.pi) * ndtr(-e)
    return (mom[:-1] - mom[1:]) / (tail[:-1] - tail[1:])


@lru_cache(maxsize=None)
def lloyd_max_rayleigh(bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """MSE-optimal 2^bits-level quantiser of the Rayleigh(1) radius.

    f(r) = r exp(-r^2/2), P(R >= x) = exp(-x^2/2), and
    E[R; R >= x] = x exp(-x^2/2) + sqrt(2 pi) Q(x) with Q the Gaussian upper
    tail.  Lloyd iterations, a float64 root finder, then Newton steps in
    40-digit arithmetic with the tridiagonal Jacobian of the conditions
    c_k = E[R | t_k <= R < t_k+1] (t the midpoints; the first cell starts at 0).
    Returns (levels, boundaries) in float64.
    """
    import mpmath as mp
    L = 1 << bits
    c = np.sqrt(-2.0 * np.log(1.0 - (np.arange(L) + 0.5) / L))      # equal-probability start
    for _ in range(300):
        c = _rayleigh_lloyd_map(c)
    sol = optimize.root(lambda x: x - _rayleigh_lloyd_map(x), c, method="hybr", tol=1e-15)
    c = np.sort(sol.x)
    with mp.workdps(40):
        dens = lambda x: x * mp.exp(-x * x / 2)
        tail = lambda x: mp.exp(-x * x / 2)
        mom = lambda x: x * mp.exp(-x * x / 2) + mp.sqrt(2 * mp.pi) * mp.ncdf(-x)
        cm = [mp.mpf(float(v)) for v in c]
        for _ in range(30):
            a = [mp.mpf(0)] + [(cm[i - 1] + cm[i]) / 2 for i in range(1, L)]
            ta = [tail(x) for x in a] + [mp.mpf(0)]
            ma = [mom(x) for x in a] + [mp.mpf(0)]
            P = [ta[i] - ta[i + 1] for i in range(L)]
            mean = [(ma[i] - ma[i + 1]) / P[i] for i in range(L)]
            da = [dens(a[i]) * (mean[i] - a[i]) / P[i] if i > 0 else mp.mpf(0) for i in range(L)]
            db = [dens(a[i + 1]) * (a[i + 1] - mean[i]) / P[i] if i < L - 1 else mp.mpf(0) for i in range(L)]
            rhs = [-(cm[i] - mean[i]) for i in range(L)]
            diag = [1 - da[i] / 2 - db[i] / 2 for i in range(L)]
            low = [-da[i] / 2 for i in range(L)]
            up = [-db[i] / 2 for i in range(L)]
            for i in range(1, L):
                w = low[i] / diag[i - 1]
                diag[i] -= w * up[i - 1]
                rhs[i] -= w * rhs[i - 1]
            step = [mp.mpf(0)] * L
            step[L - 1] = rhs[L - 1] / diag[L - 1]
            for i in range(L - 2, -1, -1):
                step[i] = (rhs[i] - up[i] * step[i + 1]) / diag[i]
            cm = [cm[i] + step[i] for i in range(L)]
            if max(abs(x) for x in step) < mp.mpf(10) ** -34:
                break
        tm = [(cm[i] + cm[i + 1]) / 2 for i in range(L - 1)]
        _RAYLEIGH_LEVELS[bits] = list(cm)
        _F32_TABLES[(bits, POLAR)] = (np.array([_round_f32(x) for x in cm], dtype=np.float32),
                                      np.array([_round_f32(x) for x in tm], dtype=np.float32))
        # pair values (r_k cos a_j, r_k sin a_j), a_j the sector middles
        pair = np.zeros((L, L, 2), dtype=np.float32)
        for k in range(L):
            for j in range(L):
                ang = -mp.pi + (2 * j + 1) * mp.pi / L
                pair[k, j, 0] = _round_f32(cm[k] * mp.cos(ang))
                pair[k, j, 1] = _round_f32(cm[k] * mp.sin(ang))
        _POLAR_PAIRS[bits] = pair
        return np.array([float(x) for x in cm]), np.array([float(x) for x in tm])


_POLAR_PAIRS: Dict[int, np.ndarray] = {}
_RAYLEIGH_LEVELS: Dict[int, list] = {}   # 40-digit levels of lloyd_max_rayleigh


def polar_pairs(bits: int) -> np.ndarray:
    """[L, L, 2] float32: the reconstructed pair of radius code k, angle code j."""
    lloyd_max_rayleigh(bits)
    return _POLAR_PAIRS[bits]


class PolarSplit:
    """PolarQuant with the radius and the angle at widths of their own
    ("TurboQuant-MLX v2.0", Quick Start: r_bits and theta_bits are separate
    settings; "turboquant-mlx" README, apply_turboquant_cache: k/v_theta_bits
    and k/v_radius_bits).  Reading: a part keeps the page width b of the
    scalar layout (a pair has 2b bits); ``shift`` t moves bits from the
    radius to the angle, r = b - t and theta = b + t (both 1..8), and the
    pair's 2b-bit field F = radius code | angle code << r is stored as two
    b-bit codes, F's low bits at stream position 2i and its high bits at
    2i + 1.  Shift 0 is POLAR itself.  Pass one wherever a codebook kind goes."""

    def __init__(self, shift: int):
        self.shift = int(shift)

    def __eq__(self, other):
        return isinstance(other, PolarSplit) and other.shift == self.shift

    def __hash__(self):
        return hash(("polar", self.shift))

    def __repr__(self):
        return f"PolarSplit({self.shift})"


def polar_shift(kind):
    """The angle shift of a PolarQuant kind (0 for POLAR), None for others."""
    if isinstance(kind, PolarSplit):
        return kind.shift
    if isinstance(kind, (int, np.integer)) and not isinstance(kind, bool) and kind == POLAR:
        return 0
    return None


def polar_widths(bits: int, shift: int) -> Tuple[int, int]:
    """(radius bits, angle bits) of a page width under an angle shift."""
    r, a = bits - shift, bits + shift
    if not (1 <= r <= 8 and 1 <= a <= 8):
        raise ValueError(f"width {bits} cannot carry an angle shift of {shift}")
    return r, a


def polar_pair_table(bits: int, shift: int = 0) -> np.ndarray:
    """[2^(2 bits), 2] float32: entry F = rc | tc << r is the pair of radius
    level rc (Lloyd-Max of Rayleigh(1) at r bits) in the middle direction of
    angle sector tc of 2^theta, each value the float32 nearest the exact one."""
    import mpmath as mp
    r, a = polar_widths(bits, shift)
    lloyd_max_rayleigh(r)
    lv = _RAYLEIGH_LEVELS[r]
    out = np.zeros((1 << (2 * bits), 2), dtype=np.float32)
    with mp.workdps(40):
        for tc in range(1 << a):
            ang = -mp.pi + (2 * tc + 1) * mp.pi / (1 << a)
            cs, sn = mp.cos(ang), mp.sin(ang)
            for rc in range(1 << r):
                out[rc | (tc << r)] = (_round_f32(lv[rc] * cs), _round_f32(lv[rc] * sn))
    return out


def polar_angle_code(theta: np.ndarray, bits: int) -> np.ndarray:
    """Sector index of angles in [-pi, pi] (pi is the direction of -pi: sector 0)."""
    L = 1 << bits
    return np.floor((np.asarray(theta, dtype=np.float64) + math.pi) * L / (2 * math.pi)).astype(np.int64) % L


# Codebooks fitted to sample data ("TurboMOQ", Quick Start: calibrate codebooks
# from sample data; Architecture: Lloyd-Max codebook (k-means)).
class FittedCodebook:
    """Fitted codebooks for every width: pass one wherever a codebook kind goes."""

    def __init__(self, tables: Dict[int, Tuple[np.ndarray, np.ndarray]]):
        self.tables = tables


def sample_magnitudes(X: np.ndarray, signs) -> np.ndarray:
    """|u| for every coordinate of u = sqrt(d) R x / ||x|| of the nonzero rows
    of X, sorted (the samples and their mirror images -u share them)."""
    X = np.asarray(X, dtype=np.float64).reshape(-1, HEAD_DIM)
    n = np.sqrt(np.sum(X * X, axis=1))
    X = X[n > 0]
    n = n[n > 0]
    R = rotation_matrix(signs)
    U = math.sqrt(HEAD_DIM) * (X @ R.T) / n[:, None]
    return np.sort(np.abs(U).ravel())


def fit_levels(mags: np.ndarray, bits: int, sweeps: int = 200) -> Tuple[np.ndarray, np.ndarray]:
    """Lloyd's iteration (k-means in one dimension) for a symmetric codebook.

    The positive levels c_0 < ... < c_{h-1} start at the Gaussian Lloyd-Max
    ones.  A sweep puts each magnitude in the cell between the midpoints of its
    neighbouring levels (the first cell starts at 0, the last is open) and moves
    every level to the mean of its cell; an empty cell keeps its level.  Stops
    when no magnitude changes cell, or after `sweeps` sweeps.  Returns float32
    (centroids, boundaries): the levels mirrored, and the midpoints taken in
    float64.
    """
    L = 1 << bits
    h = L // 2
    c = codebook(bits, LLOYD_MAX)[0][h:].astype(np.float64)
    prev = None
    for _ in range(sweeps):
        t = 0.5 * (c[:-1] + c[1:])
        pos = np.concatenate(([0], np.searchsorted(mags, t, side="left"), [mags.size]))
        if prev is not None and np.array_equal(pos, prev):
            break
        for k in range(h):
            if pos[k + 1] > pos[k]:
                c[k] = mags[pos[k]:pos[k + 1]].mean()
        prev = pos
    full = np.concatenate((-c[::-1], c))
    return full.astype(np.float32), (0.5 * (full[:-1] + full[1:])).astype(np.float32)


def fit_codebooks(X: np.ndarray, signs) -> FittedCodebook:
    """Fitted codebooks of every width 1..8 from the sample vectors X [n, 128]."""
    mags = sample_magnitudes(X, signs)
    return FittedCodebook({b: fit_levels(mags, b) for b in range(1, 9)})


def codebook(bits: int, kind: int = LLOYD_MAX) -> Tuple[np.ndarray, np.ndarray]:
    """(centroids, boundaries) as float32 arrays, the values both sides compare with."""
    if isinstance(kind, FittedCodebook):
        return kind.tables[bits]
    if isinstance(kind, PolarSplit):
        return codebook(polar_widths(bits, kind.shift)[0], POLAR)
    if kind == LLOYD_MAX:
        lloyd_max_gaussian(bits)
    elif kind == UNIFORM:
        uniform_gaussian(bits)
    elif kind == BETA:
        lloyd_max_sphere(bits)
    elif kind == POLAR:
        lloyd_max_rayleigh(bits)
    else:
        raise ValueError(kind)
    return _F32_TABLES[(bits, kind)]


def gaussian_mse(centroids, boundaries) -> float:
    """E[(Z - Q(Z))^2] for Z ~ N(0,1) of a scalar quantiser (float64 closed form).

    Over a cell [a, b) with level c: E[(Z-c)^2 1_cell] =
    P (1 + c^2) + (a phi(a) - b phi(b)) - 2 c (phi(a) - phi(b)).
    """
    c = np.asarray(centroids, dtype=np.float64)
    e = np.concatenate(([-np.inf], np.asarray(boundaries, dtype=np.float64), [np.inf]))
    a, b = e[:-1], e[1:]
    P = _mass(a, b)
    aphi = np.where(np.isinf(a), 0.0, np.nan_to_num(a) * _phi(np.nan_to_num(a)))
    bphi = np.where(np.isinf(b), 0.0, np.nan_to_num(b) * _phi(np.nan_to_num(b)))
    dphi = _phi(a) - _phi(b)
    return float(np.sum(P * (1 + c * c) + (aphi - bphi) - 2 * c * dphi))


# ----------------------------------------------------------------------------
# Encode / dequantise one batch of head vectors.
# ----------------------------------------------------------------------------
def encode(X: np.ndarray, signs, bits: int, kind: int = LLOYD_MAX,
           boundary_eps: float = 1e-6, overrides=None) -> Dict[str, np.ndarray]:
    """Encode rows of X (values as stored, upcast to float64).

    n = ||x||_2 (stored float32); u = sqrt(d) R x / n (u = 0 when n = 0);
    code_j = #{k : t_k <= float32(u_j)} (readings R2, R3).
    ``near`` flags coordinates whose float64 u lies within ``boundary_eps`` of
    a boundary: there the float32 decision may legitimately differ by one level.
    ``overrides`` = (rows, cols, codes) selects that other admissible level at
    flagged coordinates (any other override raises ValueError).
    """
    X = np.asarray(X, dtype=np.float64)
    n = np.sqrt(np.sum(X * X, axis=-1))
    # D H D x with the integer matrix: the products are exact and, for fp16
    # inputs, so are the sums, so a coordinate that cancels is exactly 0 (a
    # tie at the middle boundary) rather than a rounding residue of either sign
    Y = X @ signed_hadamard(signs).T
    safe = np.where(n > 0, n, 1.0)
    U = np.where(n[:, None] > 0, Y / safe[:, None], 0.0)
    c32, t32 = codebook(bits, kind)
    t64 = t32.astype(np.float64)
    L = 1 << bits
    ps = polar_shift(kind)
    if ps is not None:
        # radius and angle of each coordinate pair; the radius decision in
        # float32 like the scalar codes, the angle sector from float64 (the
        # device's float32 angle may differ within ANGLE_EPS of a sector edge).
        # The radius takes rb bits and the angle ab (rb = ab = bits unless the
        # kind is a PolarSplit); the pair field rc | tc << rb is stored as two
        # bits-wide codes, low half at the even position.
        rb, ab = polar_widths(bits, ps)
        LA = 1 << ab
        r = np.hypot(U[:, 0::2], U[:, 1::2])
        th = np.arctan2(U[:, 1::2], U[:, 0::2])
        rc = np.searchsorted(t32, r.astype(np.float32), side="right").astype(np.int64)
        near_r = np.minimum(np.abs(r - t64[np.clip(rc - 1, 0, t64.size - 1)]),
                            np.abs(r - t64[np.clip(rc, 0, t64.size - 1)])) < boundary_eps
        tc = polar_angle_code(th, ab)
        edge = (th + math.pi) * LA / (2 * math.pi)
        near_t = np.abs(edge - np.rint(edge)) * (2 * math.pi / LA) < ANGLE_EPS
        F = rc | (tc << rb)
        codes = np.empty(U.shape, dtype=np.int64)
        near = np.empty(U.shape, dtype=bool)
        codes[:, 0::2], codes[:, 1::2] = F & (L - 1), F >> bits
        near[:, 0::2], near[:, 1::2] = near_r, near_t
    else:
        U32 = U.astype(np.float32)
        # the number of boundaries <= u (t32 is ascending)
        codes = np.searchsorted(t32, U32, side="right").astype(np.int64)
        below = np.abs(U - t64[np.clip(codes - 1, 0, t64.size - 1)])
        above = np.abs(U - t64[np.clip(codes, 0, t64.size - 1)])
        near = np.minimum(below, above) < boundary_eps
    if overrides is not None:
        rows, cols, alt = (np.asarray(v, dtype=np.int64) for v in overrides)
        if rows.size:
            if ps is None:
                step = np.abs(alt - codes[rows, cols])
                if not np.all(near[rows, cols]) or not np.all(step == 1):
                    raise ValueError("override outside the boundary allowance")
                codes = codes.copy()
                codes[rows, cols] = alt
            else:
                # a pair may move one radius level (near a radius boundary)
                # and one angle sector, cyclically (near a sector edge)
                new = codes.copy()
                new[rows, cols] = alt
                pr, pc = np.unique(np.stack([rows, cols // 2]), axis=1)
                F0 = codes[pr, 2 * pc] | (codes[pr, 2 * pc + 1] << bits)
                F1 = new[pr, 2 * pc] | (new[pr, 2 * pc + 1] << bits)
                m = (1 << rb) - 1
                dr = np.abs((F1 & m) - (F0 & m))
                dt = np.abs((F1 >> rb) - (F0 >> rb))
                dt = np.minimum(dt, LA - dt)
                ok = ((dr == 0) | ((dr == 1) & near[pr, 2 * pc])) & ((dt == 0) | ((dt == 1) & near[pr, 2 * pc + 1]))
                if not np.all(ok) or not np.all((F1 >> rb) < LA):
                    raise ValueError("override outside the boundary allowance")
                codes = new
    return {"norm": n.astype(np.float32), "u": U, "codes": codes, "near": near}


ANGLE_EPS = 1e-5   # radians: the angle-sector allowance of polar codes


def dequantize(norm32: np.ndarray, codes: np.ndarray, signs, bits: int,
               kind: int = LLOYD_MAX) -> np.ndarray:
    """xhat = (n / sqrt(d)) R^T c[code], from the stored float32 values."""
    c32, _ = codebook(bits, kind)
    R = rotation_matrix(signs)
    d = R.shape[0]
    codes = np.asarray(codes, dtype=np.int64)
    ps = polar_shift(kind)
    if ps is not None:
        P = polar_pair_table(bits, ps).astype(np.float64)
        F = codes[:, 0::2] | (codes[:, 1::2] << bits)
        C = np.empty(codes.shape)
        C[:, 0::2] = P[F, 0]
        C[:, 1::2] = P[F, 1]
    else:
        C = c32.astype(np.float64)[codes]
    return (np.asarray(norm32, dtype=np.float64)[:, None] / math.sqrt(d)) * (C @ R)


def qjl_encode(X: np.ndarray, Xhat: np.ndarray, S: np.ndarray,
               sign_eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """QJL residual sketch of keys ("TurboMOQ", QJL residual correction).

    r = x - xhat; z_i = +1 if (S r)_i >= 0 else -1; gamma = ||r|| (float32).
    ``near`` flags projections with |(S r)_i| < sign_eps * ||S_i|| ||r||, where
    float32 evaluation may flip the sign.
    """
    r = np.asarray(X, dtype=np.float64) - np.asarray(Xhat, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    P = r @ S.T
    z = P >= 0
    g = np.sqrt(np.sum(r * r, axis=-1))
    bound = np.sqrt(np.sum(S * S, axis=-1))[None, :] * g[:, None]
    return {"z": z, "gamma": g.astype(np.float32), "near": np.abs(P) < sign_eps * bound,
            "residual": r}


def qjl_reconstruct(z: np.ndarray, gamma32: np.ndarray, S: np.ndarray) -> np.ndarray:
    """rhat = sqrt(pi/2) / m * gamma * S^T z, z in {-1, +1}."""
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    zs = np.where(z, 1.0, -1.0)
    return math.sqrt(math.pi / 2.0) / m * np.asarray(gamma32, dtype=np.float64)[:, None] * (zs @ S)


# ----------------------------------------------------------------------------
# Packed page layout (reading R4).
#
# A page holds 64 tokens of one (session, KV head).  Each b-bit code block is
# 64 streams of 128 codes; a stream is its codes LSB-first (code n at bits
# n*b .. n*b+b-1), i.e. b little-endian 128-bit words, and word w of stream s
# sits at byte (w*64 + s)*16 of the block.
#   K block: stream t = token t, codes of coordinates 0..127 in order.
#   V block: stream s = n + 32 P (n < 32, P in {0, 1}) holds, for every token
#            t, the codes of coordinates c0 and c0 + 1 at stream positions 2t
#            and 2t + 1, c0 = 64 bit2(n) + 32 P + 8 (n >> 3) + 2 (n & 3) (so one
#            stream is one coordinate pair over the page).
# Page = K block (1024 bK B) | K norms (64 x f32) | [QJL signs 64 x 16 B,
#        bit i of token t's 128-bit word = z_i, | QJL gamma 64 x f32] |
#        V block (1024 bV B) | V norms (64 x f32).
# An fp16 page is the 64 K rows then the 64 V rows, fp16, 128 per row.
# ----------------------------------------------------------------------------
def k_stream_codes(codes: np.ndarray) -> np.ndarray:
    """[64 tokens][128 coords] -> [64 streams][128 codes] for a K block."""
    assert codes.shape == (PAGE_TOKENS, HEAD_DIM)
    return np.array(codes, copy=True)


def v_stream_coord(s: int, k: int) -> int:
    """Coordinate k (0 or 1) of V stream s (layout above)."""
    n = s & 31
    return 64 * ((n >> 2) & 1) + 32 * (s >> 5) + 8 * (n >> 3) + 2 * (n & 3) + k


# token and coordinate of every (stream, position) of a V block
_V_TOKEN = np.array([[p >> 1 for p in range(STREAM_CODES)] for _ in range(64)])
_V_COORD = np.array([[v_stream_coord(s, p & 1) for p in range(STREAM_CODES)] for s in range(64)])


def v_stream_codes(codes: np.ndarray) -> np.ndarray:
    """[64 tokens][128 coords] -> [64 streams][128 codes] for a V block:
    stream s, position p holds token p >> 1, coordinate v_stream_coord(s, p & 1)."""
    codes = np.asarray(codes)
    assert codes.shape == (PAGE_TOKENS, HEAD_DIM)
    return codes[_V_TOKEN, _V_COORD]


def v_codes_from_streams(streams: np.ndarray) -> np.ndarray:
    """Inverse of v_stream_codes."""
    streams = np.asarray(streams)
    out = np.empty((PAGE_TOKENS, HEAD_DIM), dtype=streams.dtype)
    out[_V_TOKEN, _V_COORD] = streams
    return out


def pack_block(streams: np.ndarray, bits: int) -> bytes:
    """64 streams of 128 codes -> 1024*bits bytes (layout above).

    Bit n*bits+k of a stream is bit k of its code n; the stream's bits are
    gathered into little-endian bytes, cut into 16-byte words, and word w of
    stream s is written at byte (w*64 + s)*16.
    """
    streams = np.asarray(streams, dtype=np.int64)
    assert streams.shape == (64, STREAM_CODES)
    assert streams.min() >= 0 and streams.max() < (1 << bits)
    k = np.arange(bits)
    stream_bits = ((streams[:, :, None] >> k[None, None, :]) & 1).astype(np.uint8)  # [s][n][k]
    stream_bytes = np.packbits(stream_bits.reshape(64, STREAM_CODES * bits), axis=1,
                               bitorder="little")                                   # [s][16*bits]
    words = stream_bytes.reshape(64, bits, 16).transpose(1, 0, 2)                      # [w][s][16]
    return words.tobytes()


def unpack_block(block: bytes, bits: int) -> np.ndarray:
    """Inverse of pack_block: 1024*bits bytes -> [64 streams][128 codes]."""
    assert len(block) == 1024 * bits
    words = np.frombuffer(block, dtype=np.uint8).reshape(bits, 64, 16).transpose(1, 0, 2)
    stream_bits = np.unpackbits(words.reshape(64, 16 * bits), axis=1, bitorder="little")
    stream_bits = stream_bits.reshape(64, STREAM_CODES, bits).astype(np.int64)
    return np.sum(stream_bits << np.arange(bits)[None, None, :], axis=2)


def pack_signs(z: np.ndarray) -> bytes:
    """[T][128] booleans -> T x 16 bytes; bit i of token t's word is z[t, i]."""
    z = np.asarray(z, dtype=np.uint8)
    return np.packbits(z, axis=1, bitorder="little").tobytes()


def unpack_signs(raw: bytes) -> np.ndarray:
    b = np.frombuffer(raw, dtype=np.uint8).reshape(-1, 16)
    return np.unpackbits(b, axis=1, bitorder="little").astype(bool)


def page_bytes(fmt) -> int:
    """Bytes one page of this format occupies."""
    kb, vb, qjl = fmt
    if kb == 0:
        return 2 * PAGE_TOKENS * HEAD_DIM * 2
    return 1024 * (kb + vb) + 2 * 256 + (1024 + 256 if qjl else 0)


def page_sections(fmt) -> Dict[str, Tuple[int, int]]:
    kb, vb, qjl = fmt
    off = 0
    sec = {}
    for name, size in (("k_codes", 1024 * kb), ("k_norm", 256),
                       ("qjl_signs", 1024 if qjl else 0), ("qjl_gamma", 256 if qjl else 0),
                       ("v_codes", 1024 * vb), ("v_norm", 256)):
        sec[name] = (off, size)
        off += size
    return sec


def encode_page(K64: np.ndarray, V64: np.ndarray, fmt, signs, S=None,
                k_kind: int = LLOYD_MAX, v_kind: int = LLOYD_MAX) -> Dict:
    """Encode one full packed page; returns the page bytes and the pieces."""
    kb, vb, qjl = fmt
    assert kb > 0 and K64.shape == (PAGE_TOKENS, HEAD_DIM)
    ek = encode(K64, signs, kb, k_kind)
    ev = encode(V64, signs, vb, v_kind)
    sec = page_sections(fmt)
    buf = bytearray(page_bytes(fmt))

    def put(name, data):
        o, n = sec[name]
        assert len(data) == n
        buf[o:o + n] = data

    put("k_codes", pack_block(k_stream_codes(ek["codes"]), kb))
    put("k_norm", ek["norm"].astype("<f4").tobytes())
    res = {"k": ek, "v": ev}
    if qjl:
        khat = dequantize(ek["norm"], ek["codes"], signs, kb, k_kind)
        qj = qjl_encode(K64, khat, S)
        put("qjl_signs", pack_signs(qj["z"]))
        put("qjl_gamma", qj["gamma"].astype("<f4").tobytes())
        res["qjl"] = qj
    put("v_codes", pack_block(v_stream_codes(ev["codes"]), vb))
    put("v_norm", ev["norm"].astype("<f4").tobytes())
    res["bytes"] = bytes(buf)
    return res


def fp16_page_bytes(K: np.ndarray, V: np.ndarray) -> bytes:
    """An fp16 page: 64 K rows then 64 V rows (tokens past the end stay zero)."""
    buf = np.zeros((2, PAGE_TOKENS, HEAD_DIM), dtype="<f2")
    buf[0, :K.shape[0]] = np.asarray(K, dtype=np.float16)
    buf[1, :V.shape[0]] = np.asarray(V, dtype=np.float16)
    return buf.tobytes()


def decode_page(raw: bytes, fmt, signs, S=None, k_kind: int = LLOYD_MAX,
                v_kind: int = LLOYD_MAX, add_qjl: bool = True):
    """Reconstructed (keys, values) float64 [64, 128] of one page's bytes."""
    kb, vb, qjl = fmt
    if kb == 0:
        a = np.frombuffer(raw, dtype="<f2").reshape(2, PAGE_TOKENS, HEAD_DIM).astype(np.float64)
        return a[0], a[1]
    sec = page_sections(fmt)

    def get(name):
        o, n = sec[name]
        return raw[o:o + n]
    kc = unpack_block(get("k_codes"), kb)
    kn = np.frombuffer(get("k_norm"), dtype="<f4")
    vc = v_codes_from_streams(unpack_block(get("v_codes"), vb))
    vn = np.frombuffer(get("v_norm"), dtype="<f4")
    K = dequantize(kn, kc, signs, kb, k_kind)
    if qjl and add_qjl:
        z = unpack_signs(get("qjl_signs"))
        g = np.frombuffer(get("qjl_gamma"), dtype="<f4")
        K = K + qjl_reconstruct(z, g, S)
    V = dequantize(vn, vc, signs, vb, v_kind)
    return K, V


# ----------------------------------------------------------------------------
# Re-tiering a page in place ("TurboMOQ", Progressive temporal tiering and
# Attention-weighted tier demotion: a page moves to a tier with fewer bits).
#
# Reading: a packed page keeps its rotation and its norms; every stored code c
# of width b becomes the code of its own centroid under the new width b':
# code' = #{k : t'_k <= c_b[c]} (the same float32 decision as encode).  The
# original vectors are gone, so this is the only information the page still
# holds.  An fp16 page is encoded from its rows (as encode would).
# ----------------------------------------------------------------------------
def requantize_codes(codes: np.ndarray, bits: int, new_bits: int, kind: int = LLOYD_MAX) -> np.ndarray:
    """Codes of width `bits` mapped to width `new_bits` through their centroids."""
    if polar_shift(kind) is not None:
        raise ValueError("polar pages are not re-coded by a scalar map")
    c_old, _ = codebook(bits, kind)
    _, t_new = codebook(new_bits, kind)
    return np.searchsorted(t_new, c_old[np.asarray(codes, dtype=np.int64)], side="right").astype(np.int64)


def retier_page(raw: bytes, fmt, new_fmt, signs, S=None, k_kind: int = LLOYD_MAX,
                v_kind: int = LLOYD_MAX) -> bytes:
    """The bytes of a page re-tiered from `fmt` to the packed `new_fmt`."""
    nkb, nvb, nqjl = new_fmt
    assert nkb > 0
    kb, vb, qjl = fmt
    if kb == 0:
        a = np.frombuffer(raw, dtype="<f2").reshape(2, PAGE_TOKENS, HEAD_DIM).astype(np.float64)
        return encode_page(a[0], a[1], new_fmt, signs, S, k_kind, v_kind)["bytes"]
    assert not qjl and not nqjl, "a QJL residual cannot be recomputed without the original keys"
    sec = page_sections(fmt)

    def get(name):
        o, n = sec[name]
        return raw[o:o + n]
    # stream order is kept: only the codes change width
    ks = requantize_codes(unpack_block(get("k_codes"), kb), kb, nkb, k_kind)
    vs = requantize_codes(unpack_block(get("v_codes"), vb), vb, nvb, v_kind)
    out = bytearray(page_bytes(new_fmt))
    nsec = page_sections(new_fmt)

    def put(name, data):
        o, n = nsec[name]
        assert len(data) == n
        out[o:o + n] = data
    put("k_codes", pack_block(ks, nkb))
    put("k_norm", get("k_norm"))
    put("v_codes", pack_block(vs, nvb))
    put("v_norm", get("v_norm"))
    return bytes(out)


# ----------------------------------------------------------------------------
# Scoring a QJL-sketched key ("TurboQuant-MLX v2.0", RaBitQ vs QJL correction).
# ----------------------------------------------------------------------------
QJL_SCORE_UNBIASED = 0
QJL_SCORE_SIGN = 1


def qjl_score_term(q: np.ndarray, z: np.ndarray, gamma32: np.ndarray, S: np.ndarray,
                   mode: int = QJL_SCORE_UNBIASED) -> np.ndarray:
    """The sketch's share of q . k for keys with signs z [T, m] (True = +1, as
    qjl_encode gives them) and scales gamma.

    UNBIASED: the query stays real, sqrt(pi/2)/m gamma z . (S q), which is
    q . rhat (the QJL estimator of q . r).
    SIGN: the query is reduced to signs as well and the agreement is scaled by
    pi/2 (the RaBitQ-style correction): pi/2 / m gamma ||q|| z . sign(S q),
    sign(0) = +1; its mean over S is ||q|| ||r|| asin(cos(q, r)).
    """
    q = np.asarray(q, dtype=np.float64)
    z = np.where(np.asarray(z, dtype=bool), 1.0, -1.0)
    g = np.asarray(gamma32, dtype=np.float64)
    Sq = np.asarray(S, dtype=np.float64) @ q
    m = Sq.size
    if mode == QJL_SCORE_UNBIASED:
        return math.sqrt(math.pi / 2) / m * g * (z @ Sq)
    if mode == QJL_SCORE_SIGN:
        sq = np.where(Sq >= 0, 1.0, -1.0)
        return (math.pi / 2) / m * g * np.linalg.norm(q) * (z @ sq)
    raise ValueError(mode)


def decode_attention_unit_qjl(q_heads: np.ndarray, Kbase: np.ndarray, Vh: np.ndarray,
                              z: np.ndarray, gamma32: np.ndarray, S: np.ndarray,
                              mode: int = QJL_SCORE_UNBIASED) -> np.ndarray:
    """Outputs [G, 128]: scores (q . kbase_t + the sketch term of token t) / sqrt(d),
    softmax, values.  Tokens without a sketch have gamma = 0."""
    Kbase = np.asarray(Kbase, dtype=np.float64)
    Vh = np.asarray(Vh, dtype=np.float64)
    out = []
    for q in np.asarray(q_heads, dtype=np.float64):
        s = (Kbase @ q + qjl_score_term(q, z, gamma32, S, mode)) / math.sqrt(q.size)
        p = np.exp(s - np.max(s))
        out.append((p[:, None] * Vh).sum(axis=0) / p.sum())
    return np.stack(out)


# ----------------------------------------------------------------------------
# Attention over the reconstructed cache (reading R6).
# ----------------------------------------------------------------------------
def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
              scale: float | None = None) -> np.ndarray:
    """softmax(keys q * scale) . values for one query vector (float64)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = keys @ q * scale
    p = np.exp(s - np.max(s))
    return (p[:, None] * values).sum(axis=0) / p.sum()


def reconstruct_unit(K: np.ndarray, V: np.ndarray, formats, signs, S=None,
                     k_kind: int = LLOYD_MAX, v_kind: int = LLOYD_MAX,
                     k_overrides=None, v_overrides=None, sign_overrides=None):
    """Keys/values as decode attention sees them for one (session, KV head).

    K, V: the stored input rows [T, 128] of this unit; formats: page formats.
    fp16 pages keep the fp16 values; packed pages are encoded then dequantised
    (keys plus the QJL residual when the page carries one).  Pages of one
    format are encoded together (rows are independent).  ``k_overrides`` /
    ``v_overrides`` = (tokens, cols, codes) pick the other admissible level at
    boundary coordinates (see ``encode``); ``sign_overrides`` = (tokens, rows
    of S, signs) the other admissible QJL sign where (S r)_i is within
    rounding of zero (``qjl_encode``'s ``near``).
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    T = K.shape[0]
    Kh = np.zeros((T, HEAD_DIM))
    Vh = np.zeros((T, HEAD_DIM))
    groups: Dict[Tuple, List[int]] = {}
    for p, fmt in enumerate(formats):
        lo, hi = p * PAGE_TOKENS, min(T, (p + 1) * PAGE_TOKENS)
        if lo >= T:
            break
        if fmt[0] == 0:
            Kh[lo:hi] = K[lo:hi].astype(np.float16).astype(np.float64)
            Vh[lo:hi] = V[lo:hi].astype(np.float16).astype(np.float64)
        else:
            assert hi - lo == PAGE_TOKENS, "a packed page must be full"
            groups.setdefault(tuple(fmt), []).append(p)
    def local(ov, rows):
        if ov is None:
            return None
        tok, col, code = (np.asarray(v, dtype=np.int64) for v in ov)
        pos = np.full(T, -1, dtype=np.int64)
        pos[rows] = np.arange(rows.size)
        sel = pos[tok] >= 0 if tok.size else np.zeros(0, dtype=bool)
        return pos[tok[sel]], col[sel], code[sel]

    for fmt, plist in groups.items():
        kb, vb, qjl = fmt
        rows = np.concatenate([np.arange(p * PAGE_TOKENS, (p + 1) * PAGE_TOKENS) for p in plist])
        ek = encode(K[rows], signs, kb, k_kind, overrides=local(k_overrides, rows))
        ev = encode(V[rows], signs, vb, v_kind, overrides=local(v_overrides, rows))
        kh = dequantize(ek["norm"], ek["codes"], signs, kb, k_kind)
        if qjl:
            qj = qjl_encode(K[rows], kh, S)
            z = qj["z"].copy()
            so = local(sign_overrides, rows)
            if so is not None:
                assert np.all(qj["near"][so[0], so[1]]), "a sign override away from zero"
                z[so[0], so[1]] = so[2].astype(bool)
            kh = kh + qjl_reconstruct(z, qj["gamma"], S)
        Kh[rows] = kh
        Vh[rows] = dequantize(ev["norm"], ev["codes"], signs, vb, v_kind)
    return Kh, Vh


def decode_attention_unit(q_heads: np.ndarray, Kh: np.ndarray, Vh: np.ndarray) -> np.ndarray:
    """Outputs [G, 128] for the G query heads that read one KV head."""
    return np.stack([attention(q, Kh, Vh) for q in np.asarray(q_heads, dtype=np.float64)])


def page_attention_mass(q_heads: np.ndarray, Kh: np.ndarray, scale: float | None = None) -> np.ndarray:
    """[G, n_pages]: for each query head, the softmax weights of the keys Kh
    ("TurboMOQ", Attention-weighted tier demotion: tiers follow the attention
    tokens receive) summed over each 64-token page."""
    Kh = np.asarray(Kh, dtype=np.float64)
    T = Kh.shape[0]
    n_pages = (T + PAGE_TOKENS - 1) // PAGE_TOKENS
    out = np.zeros((len(q_heads), n_pages))
    for g, q in enumerate(np.asarray(q_heads, dtype=np.float64)):
        sc = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        s = Kh @ q * sc
        w = np.exp(s - np.max(s))
        w /= w.sum()
        for p in range(n_pages):
            out[g, p] = w[p * PAGE_TOKENS:(p + 1) * PAGE_TOKENS].sum()
    return out


def token_attention_weights(q_heads: np.ndarray, Kh: np.ndarray, scale: float | None = None) -> np.ndarray:
    """[G, T]: for each query head, the softmax weight of every key of Kh, the
    per-position importance an attention-weighted tier policy reads
    ("TurboMOQ", Attention-weighted tier demotion: tiers are kept per
    position).  Computed on its own from the scores (not from
    page_attention_mass), so that the two can be checked against each other."""
    Kh = np.asarray(Kh, dtype=np.float64)
    out = np.zeros((len(q_heads), Kh.shape[0]))
    for g, q in enumerate(np.asarray(q_heads, dtype=np.float64)):
        sc = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        s = np.array([float(np.dot(k, q)) for k in Kh]) * sc
        e = np.exp(s - s.max())
        out[g] = e / e.sum()
    return out


# ----------------------------------------------------------------------------
# Footprint.
# ----------------------------------------------------------------------------
def cache_bytes(formats_flat: Sequence) -> int:
    """Bytes of a cache whose pages have these formats."""
    return int(sum(page_bytes(f) for f in formats_flat))
