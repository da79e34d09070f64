"""Seeded synthetic workloads for the SRHT KV-cache codec.

This module is the only code shared between the CPU oracle (``oracle/``) and the
HIP library's Python binding.  It holds no part of the method's arithmetic
(no rotation, no quantisation, no packing, no attention): only

* the random draws the method consumes -- the sign diagonal D of the randomized
  Walsh-Hadamard rotation and the Gaussian JL matrix S of the QJL residual --
  produced by a counter-based SplitMix64 stream (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) followed by
  the Box-Muller transform (Box & Muller, 1958);
* the five workload recipes (shapes, dtypes, bit-width plans, sink/tier/demotion
  layout of the 64-token pages);
* seeded tensor generators for keys, values and queries.

Page formats are described as tuples and never as byte layouts: each side
derives sizes and offsets with its own code.

Sources for the recipes (pages cited by title and section):
* "TurboQuant-MLX v2.0", What's New (SRHT rotation ``D @ H @ D`` with seed 42;
  fp16 attention sinks of 128 tokens; 64-token chunk buffering).
* MLX TurboQuant skill page, Standalone Benchmark (one cache per layer seeded
  ``42 + layer``).
* "TurboMOQ", Architecture (per-head bit widths 1-8; progressive temporal tiers
  Active/Warm/Cold/Archive by token age) and Attention-weighted tier demotion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
PAGE_TOKENS = 64
JL_DIM = 128
ROTATION_SEED = 42

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


# ----------------------------------------------------------------------------
# Counter-based SplitMix64 (the published mixing function, evaluated at
# state = seed + i * golden_gamma for i = 1, 2, ...).
# ----------------------------------------------------------------------------
def splitmix64(seed: int, count: int, start: int = 0) -> List[int]:
    """Outputs ``start+1 .. start+count`` of SplitMix64 seeded with ``seed``."""
    out = []
    s = (seed + start * _GAMMA) & _MASK64
    for _ in range(count):
        s = (s + _GAMMA) & _MASK64
        z = s
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def layer_seed(seed: int, layer: int) -> int:
    """Per-layer seed: one cache per layer seeded ``seed + layer``."""
    return (seed + layer) & _MASK64


def rotation_signs(seed: int, layer: int, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Sign diagonal D of the rotation for one layer, as int8 values +1/-1.

    Draw j (j = 0..head_dim-1) of the layer's stream gives D_j = -1 when its
    top bit is set, else +1.  Keys and values of every head of the layer share D.
    """
    draws = splitmix64(layer_seed(seed, layer), head_dim)
    return np.array([-1 if (z >> 63) else 1 for z in draws], dtype=np.int8)


def qjl_matrix(seed: int, layer: int, head_dim: int = HEAD_DIM,
               jl_dim: int = JL_DIM) -> np.ndarray:
    """Gaussian JL matrix S (jl_dim x head_dim, row-major, float32) for one layer.

    Continues the layer's stream after the head_dim sign draws.  Uniforms are
    u = (z >> 11) * 2^-53; each pair (u1, u2) gives the two Box-Muller normals
    sqrt(-2 ln(1-u1)) cos(2 pi u2) and sqrt(-2 ln(1-u1)) sin(2 pi u2), in that
    order, filling S row by row; each is rounded to float32.
    """
    n = jl_dim * head_dim
    draws = splitmix64(layer_seed(seed, layer), n + (n & 1), start=head_dim)
    vals = []
    two_pi = 2.0 * math.pi
    for i in range(0, len(draws), 2):
        u1 = (draws[i] >> 11) * (1.0 / 9007199254740992.0)
        u2 = (draws[i + 1] >> 11) * (1.0 / 9007199254740992.0)
        r = math.sqrt(-2.0 * math.log(1.0 - u1))
        a = two_pi * u2
        vals.append(r * math.cos(a))
        vals.append(r * math.sin(a))
    return np.array(vals[:n], dtype=np.float64).astype(np.float32).reshape(jl_dim, head_dim)


# ----------------------------------------------------------------------------
# Page formats.  A format is FP16 (the page is stored uncompressed) or a tuple
# (k_bits, v_bits, qjl) for a packed page.
# ----------------------------------------------------------------------------
FP16 = (0, 0, False)
LLOYD_MAX = 0
UNIFORM = 1


def packed(k_bits: int, v_bits: int, qjl: bool = False) -> Tuple[int, int, bool]:
    assert 1 <= k_bits <= 8 and 1 <= v_bits <= 8
    return (int(k_bits), int(v_bits), bool(qjl))


@dataclass
class Workload:
    """One synthetic workload: shapes, dtype and the page-format plan."""
    name: str
    index: int                      # 1..5, as listed below
    n_layers: int
    batch: int                      # sessions B
    n_kv_heads: int
    n_q_heads: int
    n_tokens: int                   # cached tokens per session
    dtype: str                      # "float32" or "float16"
    sink_tokens: int
    k_codebook: int = LLOYD_MAX
    v_codebook: int = LLOYD_MAX
    chunked_encode: bool = False    # encode the body in 64-token calls
    note: str = ""
    # formats[layer][session][head][page]
    formats: List = field(default_factory=list)

    @property
    def n_pages(self) -> int:
        return (self.n_tokens + PAGE_TOKENS - 1) // PAGE_TOKENS


def _score_rng(index: int, layer: int, salt: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, index, layer, salt])))


def _uniform_plan(w: Workload, fmt_of_page) -> None:
    w.formats = [[[[fmt_of_page(l, b, h, p) for p in range(w.n_pages)]
                   for h in range(w.n_kv_heads)]
                  for b in range(w.batch)]
                 for l in range(w.n_layers)]


def _sink_or_tail(w: Workload, p: int) -> bool:
    """Sink pages, and a final partial page, stay fp16."""
    if p * PAGE_TOKENS < w.sink_tokens:
        return True
    return (p + 1) * PAGE_TOKENS > w.n_tokens


def head_bits_plan(index: int, layer: int, n_kv_heads: int,
                   base: Tuple[int, int]) -> List[Tuple[int, int]]:
    """Per-head (k_bits, v_bits) from a seeded importance score s ~ U(0,1).

    Hub heads (s >= 0.9) take 6-8 bits, peripheral heads (s < 0.25) 1-2 bits,
    the rest keep the base widths (the topology-aware allocation of "TurboMOQ",
    Full Feature Set: hub heads 6-8 bit, peripheral 1-2 bit).
    """
    s = _score_rng(index, layer, 7).random(n_kv_heads)
    out = []
    for v in s:
        if v >= 0.9:
            b = 6 + min(2, int((v - 0.9) / 0.1 * 3))
            out.append((b, b))
        elif v < 0.25:
            b = 1 + min(1, int(v / 0.25 * 2))
            out.append((b, b))
        else:
            out.append(base)
    return out


TIER_FORMATS = [None, (4, 4), (3, 2), (2, 1)]   # Active (fp16), Warm, Cold, Archive
TIER_AGE_LIMITS = [1024, 8192, 65536]           # token-age bounds of Active/Warm/Cold


def tier_of_age(age: int) -> int:
    for t, lim in enumerate(TIER_AGE_LIMITS):
        if age < lim:
            return t
    return 3


def make_workload(index: int, scale: Optional[Dict] = None) -> Workload:
    """Build workload ``index`` (1..5).  ``scale`` overrides sizes (tests only)."""
    scale = dict(scale or {})
    if index == 1:
        w = Workload("single-head-4k-fp32", 1, n_layers=1, batch=1, n_kv_heads=1,
                     n_q_heads=1, n_tokens=4096, dtype="float32", sink_tokens=0,
                     note="1 head, d=128, 4096 tokens, fp32, K4/V4 Lloyd-Max, no sink")
    elif index == 2:
        w = Workload("llama3-8b-layer-4k", 2, n_layers=1, batch=1, n_kv_heads=8,
                     n_q_heads=32, n_tokens=4096, dtype="float16", sink_tokens=128,
                     chunked_encode=True,
                     note="8 KV / 32 Q heads, 4096 tokens, fp16, K4/V4, 128-token fp16 sink, 64-token chunks")
    elif index == 3:
        w = Workload("qwen3-8b-stack-32k", 3, n_layers=36, batch=4, n_kv_heads=8,
                     n_q_heads=32, n_tokens=32768, dtype="float16", sink_tokens=0,
                     note="36 layers x 8 KV heads, 32K context, batch 4, base K3/V2, per-head 1-8 bits")
    elif index == 4:
        w = Workload("long-ctx-128k-qjl", 4, n_layers=1, batch=16, n_kv_heads=8,
                     n_q_heads=32, n_tokens=131072, dtype="float16", sink_tokens=128,
                     note="128K context, 16 sessions, K2+QJL(m=128)/V2, 128-token fp16 sink")
    elif index == 5:
        w = Workload("tiers-256k", 5, n_layers=1, batch=8, n_kv_heads=8,
                     n_q_heads=32, n_tokens=262144, dtype="float16", sink_tokens=0,
                     note="256K context, 8 sessions, age tiers fp16/K4V4/K3V2/K2V1, per-head +-2, demotion mask")
    else:
        raise ValueError(f"unknown workload {index}")
    for k, v in scale.items():
        setattr(w, k, v)
    _plan(w)
    return w


def _plan(w: Workload) -> None:
    if w.index in (1, 2):
        _uniform_plan(w, lambda l, b, h, p: FP16 if _sink_or_tail(w, p) else packed(4, 4))
    elif w.index == 3:
        per_layer = [head_bits_plan(3, l, w.n_kv_heads, (3, 2)) for l in range(w.n_layers)]
        _uniform_plan(w, lambda l, b, h, p: FP16 if _sink_or_tail(w, p)
                      else packed(*per_layer[l][h]))
    elif w.index == 4:
        _uniform_plan(w, lambda l, b, h, p: FP16 if _sink_or_tail(w, p) else packed(2, 2, True))
    elif w.index == 5:
        offs = [int(math.floor(5 * s)) - 2 for s in _score_rng(5, 0, 11).random(w.n_kv_heads)]
        demote = _score_rng(5, 0, 13).random((w.batch, w.n_pages)) < 0.25

        def fmt(l, b, h, p):
            if _sink_or_tail(w, p):
                return FP16
            newest = min(w.n_tokens, (p + 1) * PAGE_TOKENS) - 1
            tier = tier_of_age(w.n_tokens - 1 - newest)
            if tier == 0:
                return FP16
            if demote[b, p]:
                tier = min(3, tier + 1)
            kb, vb = TIER_FORMATS[tier]
            return packed(min(8, max(1, kb + offs[h])), min(8, max(1, vb + offs[h])))
        _uniform_plan(w, fmt)


# ----------------------------------------------------------------------------
# Tensor generators.
# ----------------------------------------------------------------------------
def _tensor_seed(index: int, layer: int, which: int) -> int:
    return int(np.random.SeedSequence([2026, index, layer, which]).generate_state(1)[0])


def outlier_channels(index: int, layer: int, n_kv_heads: int) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Per-head outlier channels of the keys and their scale factors.

    Workload 1: channels {7, 31, 64, 100} scaled x20.  Others: per head 2-6
    distinct channels, each scaled by U[10, 30].
    """
    if index == 1:
        return [(np.array([7, 31, 64, 100]), np.full(4, 20.0))] * n_kv_heads
    rng = _score_rng(index, layer, 17)
    out = []
    for _ in range(n_kv_heads):
        n = int(rng.integers(2, 7))
        ch = np.sort(rng.choice(HEAD_DIM, size=n, replace=False))
        out.append((ch, rng.uniform(10.0, 30.0, size=n)))
    return out


def make_kv(w: Workload, layer: int, device="cpu", tokens: Optional[int] = None):
    """Keys and values ``[B, H_kv, T, 128]`` in the workload dtype, seeded.

    Draws are N(0,1) in float32 from a torch generator seeded per (workload,
    layer, K/V); key outlier channels are scaled in float32; then the tensor is
    rounded to the workload dtype.  Both sides consume the rounded values.
    """
    import torch
    T = w.n_tokens if tokens is None else tokens
    shape = (w.batch, w.n_kv_heads, T, HEAD_DIM)
    dt = torch.float16 if w.dtype == "float16" else torch.float32
    out = []
    for which in (0, 1):
        g = torch.Generator(device=device)
        g.manual_seed(_tensor_seed(w.index, layer, which))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if which == 0:
            for h, (ch, sc) in enumerate(outlier_channels(w.index, layer, w.n_kv_heads)):
                idx = torch.as_tensor(ch, device=device, dtype=torch.long)
                x[:, h, :, idx] *= torch.as_tensor(sc, device=device, dtype=torch.float32)
        out.append(x.to(dt))
    return out[0], out[1]


def make_query(w: Workload, layer: int, device="cpu"):
    """One decode query per session: ``[B, H_q, 128]`` N(0,1) in the workload dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_tensor_seed(w.index, layer, 2))
    q = torch.randn((w.batch, w.n_q_heads, HEAD_DIM), generator=g, device=device,
                    dtype=torch.float32)
    return q.to(torch.float16 if w.dtype == "float16" else torch.float32)


def gaussian_rows(seed: int, n: int, dim: int = HEAD_DIM) -> np.ndarray:
    """Plain N(0,1) float64 rows for small statistical checks."""
    return np.random.Generator(np.random.PCG64(seed)).standard_normal((n, dim))


def degenerate_rows(signs) -> np.ndarray:
    """Eight head vectors [8, 128] (float64, exactly representable in fp16)
    for the degenerate cases of the codec: exact ties and the zero vector.

    Row 0 is the zero vector and row 1 the zero vector of negative zeros
    (their norm is 0).  Rows 2-4 are sums and differences of two or four basis
    vectors and row 5 a scaled basis vector: under a Walsh-Hadamard rotation
    with any sign diagonal their coordinates are sums of a few +-1 terms, many
    of which cancel exactly, so those coordinates sit exactly on the middle
    decision boundary 0 of every even number of levels.  Row 6 is the sign
    vector itself scaled, x = c D: D H D x = c D H 1 is zero outside its first
    coordinate.  Row 7 is a basis vector scaled by -2.
    """
    s = np.asarray(signs, dtype=np.float64)
    X = np.zeros((8, HEAD_DIM))
    X[1] = -0.0
    X[2, [0, 1]] = 1.0
    X[3, 5], X[3, 77] = 3.5, -3.5
    X[4, [9, 10, 40, 100]] = 0.75
    X[5, 64] = 0.5
    X[6] = 0.25 * s
    X[7, 127] = -2.0
    return X
