"""Benchmark of the SRHT KV-cache hot path on one MI355X.

One step = encode every layer's keys and values into packed pages, then one
decode-attention query per session over every layer's cache (all rows of the
hot path), on the Qwen3-8B-shaped workload: 36 layers x 8 KV heads x
head_dim 128, 32K context, batch 4, fp16 inputs, base K3/V2 with per-head
widths 1-8.  Inputs are synthetic, seeded, and resident in HBM before timing.

Prints one JSON line.  ``value`` is decode-attention effective bandwidth
(algorithmic bytes per decode step / decode time); the encode rate is in
``encode_mtokens_per_s``.  The ``roofline`` object describes the kernel that
dominates the step, timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn effective HBM GB/s (% of peak) + encode Mtokens/s at 32K ctx"
HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3   # dense float32 matrix-core peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="workload index 1..5 (default 3)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--codecs", type=int, default=1,
                    help="compare the scalar codec with PolarQuant on one layer (1, default) or skip (0)")
    ap.add_argument("--qjl", type=int, default=1,
                    help="also time one layer of the QJL workload's encode (1 = yes)")
    ap.add_argument("--tiering", type=int, default=1,
                    help="measure page-mass export and page re-tiering (1, default) or skip (0)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--loop-steps", type=int, default=64,
                    help="decode-loop steps (append one token per session + decode attention, "
                         "every layer) measured after the main step; 0 skips")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (calibrates "
                         "the HBM byte counters) and exit")
    return ap.parse_args()


def decode_bytes(w, formats, n_q_heads):
    """Algorithmic bytes one decode step reads/writes for one layer: packed
    pages (codes + norms [+ QJL]), fp16 pages, q and out."""
    import kv_cache_vector_srht_amd as tq
    total = 0
    for row in formats:
        for fm in row:
            for p, f in enumerate(fm):
                ntok = min(64, w.n_tokens - 64 * p)
                if ntok <= 0:
                    break
                if f[0] == 0:
                    total += ntok * 512
                else:
                    total += tq.page_bytes(f)
    qbytes = 2 if w.dtype == "float16" else 4
    total += w.batch * n_q_heads * 128 * (qbytes + 4)
    return total


def encode_bytes(w, formats):
    """Algorithmic bytes of one layer's encode call: K and V inputs plus the
    pages written."""
    import kv_cache_vector_srht_amd as tq
    ebytes = 2 if w.dtype == "float16" else 4
    inp = 2 * w.batch * w.n_kv_heads * w.n_tokens * 128 * ebytes
    out = 0
    for row in formats:
        for fm in row:
            for p, f in enumerate(fm):
                ntok = min(64, w.n_tokens - 64 * p)
                if ntok <= 0:
                    break
                out += ntok * 512 if f[0] == 0 else tq.page_bytes(f)
    return inp + out


def traffic_record(kernel: str, workload: str):
    """Measured HBM traffic of `kernel` from profiles/, if taken on this workload
    and on the current source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    sha = hashlib.sha256()
    for f in rec.get("sources", []):
        sha.update(open(os.path.join(ROOT, f), "rb").read())
    sha = sha.hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def valu_record(workload: str):
    """VALU issue per kernel (fraction of SIMD cycles issuing VALU) from the
    committed SQ counter record, if taken on this workload and on the current
    kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"valu_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    sha = hashlib.sha256()
    for f in rec.get("sources", []):
        sha.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("source_sha256") != sha.hexdigest():
        return None
    return rec.get("valu_issue")


def cpu_baseline(w, layers_data, seconds: float):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole (layer, session, KV head) units, encode then decode attention."""
    import numpy as np
    from oracle import tq_oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
    G = w.n_q_heads // w.n_kv_heads
    enc_t = dec_t = 0.0
    tokens = dec_bytes = 0
    units = 0
    t_start = time.perf_counter()
    l = b = h = 0
    while time.perf_counter() - t_start < seconds and units < 64:
        k, v, q, signs, S = layers_data(l, b, h)
        fm = w.formats[l][b][h]
        t0 = time.perf_counter()
        groups = {}
        for p, f in enumerate(fm):
            if f[0]:
                groups.setdefault(tuple(f), []).append(p)
        encs = {}
        for f, plist in groups.items():
            rows = np.concatenate([np.arange(64 * p, 64 * p + 64) for p in plist])
            ek = O.encode(k[rows], signs, f[0], w.k_codebook)
            ev = O.encode(v[rows], signs, f[1], w.v_codebook)
            qj = None
            if f[2]:
                kh0 = O.dequantize(ek["norm"], ek["codes"], signs, f[0], w.k_codebook)
                qj = O.qjl_encode(k[rows], kh0, S)
            encs[f] = (rows, ek, ev, qj)
        t1 = time.perf_counter()
        Kh = np.zeros_like(k)
        Vh = np.zeros_like(v)
        for p, f in enumerate(fm):
            if f[0] == 0:
                Kh[64 * p:64 * p + 64] = k[64 * p:64 * p + 64].astype(np.float16)
                Vh[64 * p:64 * p + 64] = v[64 * p:64 * p + 64].astype(np.float16)
        for f, (rows, ek, ev, qj) in encs.items():
            kh = O.dequantize(ek["norm"], ek["codes"], signs, f[0], w.k_codebook)
            if qj is not None:
                kh = kh + O.qjl_reconstruct(qj["z"], qj["gamma"], S)
            Kh[rows] = kh
            Vh[rows] = O.dequantize(ev["norm"], ev["codes"], signs, f[1], w.v_codebook)
        O.decode_attention_unit(q[h * G:(h + 1) * G], Kh, Vh)
        t2 = time.perf_counter()
        enc_t += t1 - t0
        dec_t += t2 - t1
        tokens += w.n_tokens
        one = type(w)(**{**w.__dict__})
        one.batch, one.n_kv_heads, one.n_q_heads = 1, 1, G
        dec_bytes += decode_bytes(one, [[fm]], G)
        units += 1
        h += 1
        if h == w.n_kv_heads:
            h, b = 0, b + 1
            if b == w.batch:
                b, l = 0, (l + 1) % w.n_layers
    unit_count = w.n_layers * w.batch * w.n_kv_heads
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": dec_bytes / dec_t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model, "affinity_cpus": len(os.sched_getaffinity(0)),
        "sample": (f"{units} of {unit_count} (layer, session, KV head) units, "
                   f"{w.n_tokens} tokens each: encode then decode attention for the "
                   f"{G} query heads; numpy float64"),
        # one whole-stack session-token = one vector per (layer, KV head)
        "encode_mtokens_per_s": tokens / (w.n_layers * w.n_kv_heads) / enc_t / 1e6,
        "seconds": enc_t + dec_t,
    }


def hbm_stream(dev, mib: int = 4096, reps: int = 20):
    """Plain streaming references on the same GPU, each over buffers far larger
    than the 256 MB last-level cache: a device-to-device copy (bytes read plus
    bytes written) and a float32 sum (bytes read).  Median of ``reps`` HIP-event
    timed repetitions after two untimed ones."""
    import numpy as np
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))

    t_copy = timed(lambda: dst.copy_(src))
    t_read = timed(lambda: torch.sum(src, dim=0, out=acc))
    nbytes = n * 4
    del src, dst
    torch.cuda.synchronize()
    return {"copy_gbs": round(2 * nbytes / t_copy / 1e9, 1), "read_gbs": round(nbytes / t_read / 1e9, 1),
            "buffer_bytes": nbytes, "reps": reps,
            "what": "device copy (read + write bytes) and float32 sum (read bytes), median"}


def decode_graph(w, layers, caches, queries, outs, wss, dec_bytes, dev, reps: int = 50):
    """The decode step of every layer captured once in a HIP graph and replayed
    ``reps`` times (after three untimed replays); median step time.  The layers'
    pages together far exceed the last-level cache, so every replay streams HBM."""
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    stream = torch.cuda.current_stream(dev)
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for l in range(w.n_layers):
            tq.decode_attention(layers[l], caches[l], queries[l], out=outs[l], workspace=wss[l])
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    del g
    med = float(np.median(ts))
    return {"reps": reps, "median_ms": round(med * 1e3, 4), "min_ms": round(min(ts) * 1e3, 4),
            "gbs": round(dec_bytes / med / 1e9, 1),
            "frac_of_peak": round(dec_bytes / med / 1e9 / HBM_PEAK_GBS, 4)}


def qjl_encode(dev, sessions: int = 4, reps: int = 3):
    """Encode of one layer of the 128K QJL workload's shape at ``sessions`` of
    its 16 sessions (keys K2 + QJL sketch, values V2, 128-token fp16 sink):
    HIP-event time of tq_encode_kv, median of ``reps`` after one untimed call.
    The sketch (2 x 128 x 128 flops per key, on the float32 matrix cores) is
    the dominant part; its rate is bounded below by sketch flops / call time."""
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    import workloads as W
    w = W.make_workload(4, {"batch": sessions})
    S = W.qjl_matrix(W.ROTATION_SEED, 0)
    layer = tq.Layer(W.rotation_signs(W.ROTATION_SEED, 0), dev, S, w.k_codebook, w.v_codebook)
    cache = tq.Cache(w.formats[0], [w.n_tokens] * w.batch, dev)
    k, v = W.make_kv(w, 0, device=dev)
    stream = torch.cuda.current_stream(dev)
    tq.encode_kv(layer, cache, k, v)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        tq.encode_kv(layer, cache, k, v)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    t = float(np.median(ts))
    qjl_keys = sum(64 for row in w.formats[0] for r in row for f in r if f[2])
    flops = qjl_keys * 2.0 * 128 * 128
    out = {"workload": w.name, "sessions": sessions, "encode_ms": round(t * 1e3, 3),
           "mtokens_per_s": round(w.batch * w.n_tokens / t / 1e6, 2),
           "qjl_keys": qjl_keys, "sketch_tflops_lower_bound": round(flops / t / 1e12, 2),
           "fp32_mfma_peak_tflops": FP32_MFMA_PEAK_TFLOPS}
    del cache, k, v
    torch.cuda.synchronize()
    return out


def decode_loop(w, layers, inputs, queries, outs, wss, steps, dev, graph=False):
    """The decode loop the cache serves: every step appends one token per
    session to every layer (tq_append_kv into a pending fp16 tail page, packed
    in place when its 64th token arrives) and runs decode attention over every
    layer.  Each layer's cache is the workload's, prefilled by encode, plus one
    pending tail page per (session, KV head) in the format of its last page.

    With ``graph``, one step (append + decode over every layer, reading the new
    tokens from a fixed staging buffer) is captured once in a HIP graph and
    replayed every step after one copy of that step's tokens into the buffer;
    the copy is inside the timed region."""
    import torch
    import kv_cache_vector_srht_amd as tq
    caches, wss = [], []
    for l in range(w.n_layers):
        fm = [[list(r) + [tuple(r[-1][:3]) + (True,)] for r in row] for row in w.formats[l]]
        c = tq.Cache(fm, [w.n_tokens] * w.batch, dev)
        k, v = inputs[l]
        tq.encode_kv(layers[l], c, k, v, tok0=0)
        caches.append(c)
        # the tail page adds a page to every row: the split plan, and so the
        # workspace, is this cache's own
        wss.append(torch.empty(tq.workspace_bytes(c, w.n_q_heads), dtype=torch.uint8, device=dev))
    g = torch.Generator(device=dev).manual_seed(7)
    dtype = inputs[0][0].dtype
    news = torch.randn((steps, w.n_layers, w.batch, w.n_kv_heads, 2, 128), generator=g,
                       device=dev).to(dtype)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_append = t_decode = 0.0
    if graph:
        stage = torch.empty_like(news[0])
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        hg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(hg, stream=cap):
            for l in range(w.n_layers):
                tq.append_kv(layers[l], caches[l], stage[l, :, :, 0], stage[l, :, :, 1])
            for l in range(w.n_layers):
                tq.decode_attention(layers[l], caches[l], queries[l], out=outs[l], workspace=wss[l])
        torch.cuda.synchronize()
        for i in range(steps):
            ev[0].record(stream)
            stage.copy_(news[i])
            hg.replay()
            ev[2].record(stream)
            ev[2].synchronize()
            t_decode += ev[0].elapsed_time(ev[2])
        ms = t_decode / steps
        del hg
        return {"steps": steps, "ms_per_step": round(ms, 3),
                "us_per_layer": round(ms / w.n_layers * 1e3, 2),
                "tokens_per_s": round(w.batch / (ms / 1e3), 1),
                "context": f"{w.n_tokens} + 1..{steps} tokens, every layer, one HIP graph per step"}
    for i in range(steps):
        ev[0].record(stream)
        for l in range(w.n_layers):
            tq.append_kv(layers[l], caches[l], news[i, l, :, :, 0], news[i, l, :, :, 1])
        ev[1].record(stream)
        for l in range(w.n_layers):
            tq.decode_attention(layers[l], caches[l], queries[l], out=outs[l], workspace=wss[l])
        ev[2].record(stream)
        ev[2].synchronize()
        t_append += ev[0].elapsed_time(ev[1])
        t_decode += ev[1].elapsed_time(ev[2])
    ms = (t_append + t_decode) / steps
    return {"steps": steps, "ms_per_step": round(ms, 3),
            "append_us_per_layer": round(t_append / steps / w.n_layers * 1e3, 2),
            "decode_us_per_layer": round(t_decode / steps / w.n_layers * 1e3, 2),
            "tokens_per_s": round(w.batch / (ms / 1e3), 1),
            "context": f"{w.n_tokens} + 1..{steps} tokens, every layer, one new token per session per step"}


def tiering(w, layers, inputs, queries, outs, wss, dev):
    """The mechanisms attention-weighted tier demotion runs on: decode with the
    page attention mass exported (every layer, against plain decode), and
    tq_retier_pages calls that each demote every packed page of a layer by one
    bit in K and in V (floor 1) in place."""
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    stream = torch.cuda.current_stream(dev)
    caches = []
    for l in range(w.n_layers):
        c = tq.Cache(w.formats[l], [w.n_tokens] * w.batch, dev)
        k, v = inputs[l]
        tq.encode_kv(layers[l], c, k, v, tok0=0)
        caches.append(c)
    masses = [torch.empty((w.batch, w.n_q_heads, c.max_pages), dtype=torch.float32, device=dev) for c in caches]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_plain = t_mass = 0.0
    reps = 3
    for r in range(reps + 1):
        ev[0].record(stream)
        for l in range(w.n_layers):
            tq.decode_attention(layers[l], caches[l], queries[l], out=outs[l], workspace=wss[l])
        ev[1].record(stream)
        for l in range(w.n_layers):
            tq.decode_attention(layers[l], caches[l], queries[l], out=outs[l], workspace=wss[l],
                                page_mass=masses[l])
        ev[2].record(stream)
        ev[2].synchronize()
        if r:   # the first round warms up
            t_plain += ev[0].elapsed_time(ev[1])
            t_mass += ev[1].elapsed_time(ev[2])
    # one-bit demotion of every packed page of a layer, in place: a warm-up
    # call on the last layer, then one timed call on each of the first eight
    # (the median is reported)
    def demotions(c):
        pages, fmts, moved = [], [], 0
        for b in range(c.n_sessions):
            for h in range(c.n_kv_heads):
                for p, f in enumerate(c.formats[b][h]):
                    if f[0] >= 1 and not f[2]:
                        nf = (max(1, f[0] - 1), max(1, f[1] - 1), False)
                        pages.append((b, h, p))
                        fmts.append(nf)
                        moved += tq.page_bytes(f) + tq.page_bytes(nf)
        return pages, fmts, moved
    import ctypes
    L = tq.lib()
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    runs = []
    for l in [w.n_layers - 1] + list(range(min(8, w.n_layers - 1))):
        c = caches[l]
        pages, fmts, moved = demotions(c)
        H, P = c.n_kv_heads, c.max_pages
        # the page list is built and copied before the timed region
        idx = torch.tensor([(b * H + h) * P + p for b, h, p in pages], dtype=torch.int64, device=dev)
        desc = torch.from_numpy(np.array([L.tq_page_descriptor(int(c.offsets[pg]), f[0], f[1], 0)
                                          for pg, f in zip(pages, fmts)], dtype=np.uint64).view(np.int64)).to(dev)
        torch.cuda.synchronize()
        ev[0].record(stream)
        tq.check(L.tq_retier_pages(ctypes.byref(layers[l].struct), ctypes.byref(c.struct), idx.data_ptr(),
                                   desc.data_ptr(), len(pages), tq.RETIER_FROM_PACKED, flags.data_ptr(),
                                   ctypes.c_void_p(stream.cuda_stream)), "tq_retier_pages")
        ev[1].record(stream)
        ev[1].synchronize()
        if l != w.n_layers - 1:
            runs.append((ev[0].elapsed_time(ev[1]), len(pages), moved))
    assert int(flags.item()) == 0
    rt_ms, n_pages, moved = sorted(runs)[len(runs) // 2]
    return {"decode_us_per_layer": round(t_plain / reps / w.n_layers * 1e3, 2),
            "decode_with_mass_us_per_layer": round(t_mass / reps / w.n_layers * 1e3, 2),
            "retier_pages": n_pages, "retier_us": round(rt_ms * 1e3, 2),
            "retier_gbs": round(moved / (rt_ms / 1e3) / 1e9, 1),
            "retier": "every packed page of a layer demoted by one bit in K and V, in place; "
                      "median of the first eight layers, one call each"}


def codecs(w, inputs, queries, dev, reps=5):
    """Scalar Lloyd-Max against PolarQuant on one layer of the workload's shape
    with every page at 4 + 4 bits (the pages' default of 4-bit radius and
    4-bit angle): encode and decode attention time per layer (median of
    `reps` after a warm-up) and the effective GB/s of each."""
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    import workloads as W
    stream = torch.cuda.current_stream(dev)
    k, v = inputs[0]
    q = queries[0]
    fm = [[[W.packed(4, 4)] * w.n_pages for _ in range(w.n_kv_heads)] for _ in range(w.batch)]
    page = tq.page_bytes(W.packed(4, 4))
    n_pages = w.batch * w.n_kv_heads * w.n_pages
    enc_bytes = k.numel() * k.element_size() * 2 + n_pages * page
    dec_bytes = n_pages * page + q.numel() * q.element_size() + w.batch * w.n_q_heads * 128 * 4
    res = {}
    for name, kind in (("lloyd_max", tq.LLOYD_MAX), ("polar", tq.POLAR)):
        layer = tq.Layer(W.rotation_signs(W.ROTATION_SEED, 0), dev, None, kind, kind)
        c = tq.Cache(fm, [w.n_tokens] * w.batch, dev)
        out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
        ws = torch.empty(tq.workspace_bytes(c, w.n_q_heads), dtype=torch.uint8, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        te, td = [], []
        for r in range(reps + 1):
            ev[0].record(stream)
            tq.encode_kv(layer, c, k, v, tok0=0)
            ev[1].record(stream)
            tq.decode_attention(layer, c, q, out=out, workspace=ws)
            ev[2].record(stream)
            ev[2].synchronize()
            if r:
                te.append(ev[0].elapsed_time(ev[1]))
                td.append(ev[1].elapsed_time(ev[2]))
        e_ms, d_ms = float(np.median(te)), float(np.median(td))
        res[name] = {"encode_us": round(e_ms * 1e3, 2), "encode_gbs": round(enc_bytes / e_ms / 1e6, 1),
                     "decode_us": round(d_ms * 1e3, 2), "decode_gbs": round(dec_bytes / d_ms / 1e6, 1)}
    res["shape"] = (f"one layer, {w.batch} sessions x {w.n_kv_heads} KV heads x {w.n_tokens} tokens, "
                    f"every page K4/V4")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; a deployment shards sessions and KV heads across GPUs, each GPU "
              "running this single-GPU path on its share", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return
    w = W.make_workload(args.workload)
    if args.layers:
        w.n_layers = args.layers
        w.formats = w.formats[:args.layers]
    G = w.n_q_heads // w.n_kv_heads
    print(f"# bench: workload {w.index} ({w.name}), {w.n_layers} layers, B={w.batch}, "
          f"T={w.n_tokens}", file=sys.stderr, flush=True)

    layers, caches, inputs, queries, outs, wss = [], [], [], [], [], []
    enc_bytes = dec_bytes = 0
    for l in range(w.n_layers):
        fm = w.formats[l]
        has_qjl = any(f[2] for row in fm for r in row for f in r)
        signs = W.rotation_signs(W.ROTATION_SEED, l)
        S = W.qjl_matrix(W.ROTATION_SEED, l) if has_qjl else None
        layers.append(tq.Layer(signs, dev, S, w.k_codebook, w.v_codebook))
        caches.append(tq.Cache(fm, [w.n_tokens] * w.batch, dev))
        inputs.append(W.make_kv(w, l, device=dev))
        queries.append(W.make_query(w, l, device=dev))
        outs.append(torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev))
        wss.append(torch.empty(tq.workspace_bytes(caches[-1], w.n_q_heads), dtype=torch.uint8,
                               device=dev))
        enc_bytes += encode_bytes(w, fm)
        dec_bytes += decode_bytes(w, fm, w.n_q_heads)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(ev_enc=None, ev_dec=None):
        if ev_enc:
            ev_enc[0].record(stream)
        for l in range(w.n_layers):
            k, v = inputs[l]
            tq.encode_kv(layers[l], caches[l], k, v, tok0=0)
        if ev_enc:
            ev_enc[1].record(stream)
        for l in range(w.n_layers):
            tq.decode_attention(layers[l], caches[l], queries[l], out=outs[l], workspace=wss[l])
        if ev_dec:
            ev_dec[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step((e[0], e[1]), (None, e[2]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    dec_ms = np.array([b.elapsed_time(c) for _, b, c in evs])
    enc_s = float(np.mean(enc_ms)) / 1e3
    dec_s = float(np.mean(dec_ms)) / 1e3
    ms_per_step = wall / args.steps * 1e3
    dec_gbs = dec_bytes / dec_s / 1e9
    enc_gbs = enc_bytes / enc_s / 1e9
    enc_mtok = w.batch * w.n_tokens / enc_s / 1e6

    # the kernel that dominates the step
    # (encode is one encode_pages_kernel launch per layer, plus qjl_keys_kernel
    # when a layer has QJL keys; decode is four launches per layer, reported as
    # one call)
    if enc_s >= dec_s:
        name, per_launch_bytes, per_launch_s = ("encode_pages_kernel", enc_bytes / w.n_layers,
                                                enc_s / w.n_layers)
    else:
        name, per_launch_bytes, per_launch_s = ("decode_attention", dec_bytes / w.n_layers,
                                                dec_s / w.n_layers)
    achieved = per_launch_bytes / per_launch_s / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_record(name, w.name),
            "kernel": name, "bytes_per_launch": int(per_launch_bytes),
            "launch_us": round(per_launch_s * 1e6, 2)}
    qjl_keys = sum(64 for fm in w.formats for row in fm for r in row for f in r if f[2])
    if qjl_keys and enc_s >= dec_s:
        # With QJL key pages the encode call is dominated by qjl_keys_kernel, the
        # sketch z = sign(S r) as a float32 matrix-core product (2 x 128 x 128
        # flops per key).  Its own duration is not separable from the call's
        # encode_pages_kernel with events around the call, so the rate is a
        # lower bound: sketch flops / whole call time.
        flops = qjl_keys * 2.0 * 128 * 128 / w.n_layers
        tflops = flops / per_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "qjl_keys_kernel", "flops_per_launch": int(flops),
                "launch_us": round(per_launch_s * 1e6, 2),
                "timed": "whole tq_encode_kv call (qjl_keys_kernel + encode_pages_kernel): lower bound",
                "hbm_gbs_of_call": round(achieved, 1)}
    line = {
        "metric": METRIC, "value": round(dec_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "batch": w.batch,
                   "kv_heads": w.n_kv_heads, "q_heads": w.n_q_heads, "head_dim": 128,
                   "context": w.n_tokens, "input_dtype": w.dtype},
        "decode_frac_of_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_ms_per_step": round(dec_s * 1e3, 3),
        "encode_mtokens_per_s": round(enc_mtok, 3),
        "encode_gbs": round(enc_gbs, 1),
        "encode_ms_per_step": round(enc_s * 1e3, 3),
        "decode_bytes_per_step": int(dec_bytes), "encode_bytes_per_step": int(enc_bytes),
        "roofline": roof,
        # from profiles/ (rocprofv3 SQ counters), when taken on these sources
        "valu_issue": valu_record(w.name),
    }
    line["decode_graph"] = decode_graph(w, layers, caches, queries, outs, wss, dec_bytes, dev)
    hs = hbm_stream(dev)
    best = max(hs["copy_gbs"], hs["read_gbs"])
    hs["decode_frac_of_stream"] = round(dec_gbs / best, 4)
    hs["encode_frac_of_copy"] = round(achieved / hs["copy_gbs"], 4)
    line["hbm_stream"] = hs
    if args.loop_steps > 0:
        line["decode_loop"] = decode_loop(w, layers, inputs, queries, outs, wss, args.loop_steps, dev)
        line["decode_loop_graph"] = decode_loop(w, layers, inputs, queries, outs, wss, args.loop_steps,
                                                dev, graph=True)
    if args.qjl:
        line["qjl_encode"] = qjl_encode(dev)
    if args.tiering:
        line["tiering"] = tiering(w, layers, inputs, queries, outs, wss, dev)
    if args.codecs:
        line["codecs"] = codecs(w, inputs, queries, dev)
    if not args.no_cpu_baseline:
        kv_host = {}

        def layer_unit(l, b, h):
            if l not in kv_host:
                k, v = inputs[l]
                kv_host[l] = (k.cpu().numpy(), v.cpu().numpy(), queries[l].cpu().numpy())
            k, v, q = kv_host[l]
            signs = W.rotation_signs(W.ROTATION_SEED, l)
            S = W.qjl_matrix(W.ROTATION_SEED, l) if any(f[2] for f in w.formats[l][b][h]) else None
            return (k[b, h].astype(np.float64), v[b, h].astype(np.float64),
                    q[b].astype(np.float64), signs, S)
        cb = cpu_baseline(w, layer_unit, args.cpu_seconds)
        line["cpu_baseline"] = {k2: (round(v2, 4) if isinstance(v2, float) else v2)
                                for k2, v2 in cb.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
