"""Benchmark of the SRHT KV-cache hot path on one MI355X.

One step = encode every layer's keys and values into packed pages, then one
decode-attention query per session over every layer's cache (all rows of the
hot path), on the Qwen3-8B-shaped workload: 36 layers x 8 KV heads x
head_dim 128, 32K context, batch 4, fp16 inputs, base K3/V2 with per-head
widths 1-8.  Inputs are synthetic, seeded, and resident in HBM before timing.

Prints one JSON line.  ``value`` is decode-attention effective bandwidth
(algorithmic bytes per decode step / decode time); the encode rate is in
``encode_mtokens_per_s``.  The ``roofline`` object describes the kernel that
dominates the step and ``decode_roofline`` the decode-attention call, both
timed with HIP events on the stream they run on.  Beside the step the line
carries: the small single-head and Llama-3-8B-layer configurations as
latency (``latency``), one full-size layer of the 128K QJL and 256K tier
workloads (``one_layer``), the decode loop, the tiering mechanisms, a codec
comparison, plain HBM stream rates, and the CPU oracle on a bounded sample
(``cpu_baseline``: one core and a process pool over every core).
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
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense float16 matrix-core peak


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
    ap.add_argument("--subworkloads", type=int, default=1,
                    help="also time one full-size layer of the 128K QJL and 256K tier workloads (1 = yes)")
    ap.add_argument("--latency", type=int, default=1,
                    help="also time the single-head and Llama-3-8B-layer configurations as latency (1 = yes)")
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


def _oracle_unit(job):
    """One (layer, session, KV head) unit through the CPU oracle: encode every
    packed page group, rebuild K and V (fp16 pages as stored), then decode
    attention for the unit's query heads.  Returns (encode s, decode s)."""
    import numpy as np
    from oracle import tq_oracle as O
    fm, k, v, q, signs, S, k_codebook, v_codebook = job
    k, v, q = k.astype(np.float64), v.astype(np.float64), q.astype(np.float64)
    t0 = time.perf_counter()
    groups = {}
    for p, f in enumerate(fm):
        if f[0]:
            groups.setdefault(tuple(f), []).append(p)
    encs = {}
    for f, plist in groups.items():
        rows = np.concatenate([np.arange(64 * p, 64 * p + 64) for p in plist])
        ek = O.encode(k[rows], signs, f[0], k_codebook)
        ev = O.encode(v[rows], signs, f[1], v_codebook)
        qj = None
        if f[2]:
            kh0 = O.dequantize(ek["norm"], ek["codes"], signs, f[0], k_codebook)
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
        kh = O.dequantize(ek["norm"], ek["codes"], signs, f[0], k_codebook)
        if qj is not None:
            kh = kh + O.qjl_reconstruct(qj["z"], qj["gamma"], S)
        Kh[rows] = kh
        Vh[rows] = O.dequantize(ev["norm"], ev["codes"], signs, f[1], v_codebook)
    O.decode_attention_unit(q, Kh, Vh)
    return t1 - t0, time.perf_counter() - t1


_ONE_THREAD = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def _one_thread_pool(n):
    """A pool of ``n`` fresh interpreters (spawned, so nothing of this
    process's GPU state is inherited), each with single-threaded BLAS."""
    import multiprocessing as mp
    saved = {k: os.environ.get(k) for k in _ONE_THREAD}
    os.environ.update({k: "1" for k in _ONE_THREAD})
    try:
        pool = mp.get_context("spawn").Pool(n)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return pool


def cpu_baseline(w, unit_job, seconds: float):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole (layer, session, KV head) units, encode then decode attention, each
    unit in one single-threaded process.  Two legs: one core (units one after
    another, ``seconds / 2`` of work) and every core of this process's CPU
    share (capped at 16) running units side by side in a process pool, for
    about ``seconds / 2`` of wall time.  ``value`` is the all-core leg."""
    import numpy as np
    G = w.n_q_heads // w.n_kv_heads
    unit_count = w.n_layers * w.batch * w.n_kv_heads
    units = [(l, b, h) for l in range(w.n_layers) for b in range(w.batch) for h in range(w.n_kv_heads)]
    one = type(w)(**{**w.__dict__})
    one.batch, one.n_kv_heads, one.n_q_heads = 1, 1, G

    def unit_bytes(u):
        l, b, h = u
        return decode_bytes(one, [[w.formats[l][b][h]]], G)

    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(affinity, 16))
    # one core
    pool = _one_thread_pool(1)
    done, enc_t, dec_t, nbytes = 0, 0.0, 0.0, 0
    try:
        while enc_t + dec_t < seconds / 2 and done < len(units):
            e, d = pool.apply(_oracle_unit, (unit_job(*units[done]),))
            enc_t, dec_t, nbytes = enc_t + e, dec_t + d, nbytes + unit_bytes(units[done])
            done += 1
    finally:
        pool.terminate()
        pool.join()
    single = {"value": nbytes / dec_t / 1e9, "unit": "GB/s", "cores": 1, "units": done,
              "encode_mtokens_per_s": done * w.n_tokens / (w.n_layers * w.n_kv_heads) / enc_t / 1e6,
              "seconds": enc_t + dec_t}
    # every core: rounds of `cores` units side by side until the budget is used;
    # the rate is bytes over wall time, process start-up excluded
    pool = _one_thread_pool(cores)
    n_all, p_bytes, p_enc, p_dec = 0, 0, 0.0, 0.0
    try:
        pool.map(abs, range(cores))          # the workers are up
        t_start = time.perf_counter()
        nxt = done
        while time.perf_counter() - t_start < seconds / 2:
            batch = [units[(nxt + i) % len(units)] for i in range(cores)]
            nxt += cores
            res = pool.map(_oracle_unit, [unit_job(*u) for u in batch], chunksize=1)
            for u, (e, d) in zip(batch, res):
                p_enc, p_dec, p_bytes = p_enc + e, p_dec + d, p_bytes + unit_bytes(u)
            n_all += len(batch)
        wall = time.perf_counter() - t_start
    finally:
        pool.terminate()
        pool.join()
    # the pool's wall time holds encode and decode; split it as their CPU time splits
    dec_wall = wall * p_dec / (p_enc + p_dec)
    enc_wall = wall - dec_wall
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
        "value": p_bytes / dec_wall / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model, "affinity_cpus": affinity,
        "sample": (f"{n_all} (all cores) and {done} (one core) of {unit_count} (layer, session, "
                   f"KV head) units, {w.n_tokens} tokens each: encode then decode attention for "
                   f"the {G} query heads; numpy float64, one BLAS thread per process"),
        # one whole-stack session-token = one vector per (layer, KV head)
        "encode_mtokens_per_s": n_all * w.n_tokens / (w.n_layers * w.n_kv_heads) / enc_wall / 1e6,
        "seconds": wall,
        "single_core": single,
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


def _median_us(ts):
    import numpy as np
    return round(float(np.median(ts)) * 1e6, 2)


def latency(dev, reps: int = 60):
    """The two small configurations as latency, each figure a median of
    ``reps`` calls after warm-up calls: device time between HIP events around
    the call on its stream, and host time from the call's start to the end of a
    stream synchronize after it (argument marshalling and launches included).

    single-head-4k-fp32: one tq_encode_kv of all 4096 tokens, then one
    tq_decode_attention.  llama3-8b-layer-4k: the 4096-token prefill as 64
    tq_encode_kv calls of 64 tokens each (every chunk call is one sample; the
    first two chunks are the fp16 sink), the whole chunked prefill, and one
    tq_decode_attention for the 32 query heads."""
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    import workloads as W
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        t0 = time.perf_counter()
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3, time.perf_counter() - t0

    out = {"reps": reps}
    for idx in (1, 2):
        w = W.make_workload(idx)
        fm = w.formats[0]
        layer = tq.Layer(W.rotation_signs(W.ROTATION_SEED, 0), dev, None, w.k_codebook, w.v_codebook)
        cache = tq.Cache(fm, [w.n_tokens] * w.batch, dev)
        k, v = W.make_kv(w, 0, device=dev)
        q = W.make_query(w, 0, device=dev)
        o = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
        ws = torch.empty(tq.workspace_bytes(cache, w.n_q_heads), dtype=torch.uint8, device=dev)
        rec = {"tokens": w.n_tokens, "kv_heads": w.n_kv_heads, "q_heads": w.n_q_heads,
               "input_dtype": w.dtype}
        if w.chunked_encode:
            chunks = w.n_tokens // 64

            def prefill():
                for c in range(chunks):
                    tq.encode_kv(layer, cache, k[:, :, 64 * c:64 * c + 64], v[:, :, 64 * c:64 * c + 64],
                                 tok0=64 * c)
            prefill()
            torch.cuda.synchronize()
            dev_t, host_t = [], []
            for r in range(max(1, reps // chunks) + 1):
                for c in range(chunks):
                    d, h = timed(lambda: tq.encode_kv(layer, cache, k[:, :, 64 * c:64 * c + 64],
                                                      v[:, :, 64 * c:64 * c + 64], tok0=64 * c))
                    dev_t.append(d)
                    host_t.append(h)
            rec["chunk_encode_us"] = {"device": _median_us(dev_t), "host": _median_us(host_t),
                                      "samples": len(dev_t), "tokens_per_call": 64}
            pre = [timed(prefill) for _ in range(max(3, reps // 10))]
            rec["chunked_prefill_us"] = {"device": _median_us([a for a, _ in pre]),
                                         "host": _median_us([b for _, b in pre]), "calls": chunks,
                                         "samples": len(pre)}
        else:
            enc = lambda: tq.encode_kv(layer, cache, k, v, tok0=0)
            for _ in range(3):
                enc()
            ts = [timed(enc) for _ in range(reps)]
            rec["encode_us"] = {"device": _median_us([a for a, _ in ts]),
                                "host": _median_us([b for _, b in ts]), "tokens_per_call": w.n_tokens}
        dec = lambda: tq.decode_attention(layer, cache, q, out=o, workspace=ws)
        for _ in range(3):
            dec()
        ts = [timed(dec) for _ in range(reps)]
        rec["decode_us"] = {"device": _median_us([a for a, _ in ts]), "host": _median_us([b for _, b in ts])}
        rec["decode_bytes"] = decode_bytes(w, fm, w.n_q_heads)
        out[w.name] = rec
        del cache, k, v, q, o, ws
    torch.cuda.synchronize()
    return out


def one_layer(idx, dev, enc_reps: int = 5, dec_reps: int = 30):
    """One layer of a long-context workload at its full size (every session,
    every KV head, the whole context): encode then decode attention, each
    timed with HIP events on the launch stream, median of ``enc_reps`` /
    ``dec_reps`` calls after warm-up calls, as effective GB/s of the
    algorithmic bytes.  For the QJL workload the call's sketch rate, sketch
    flops (2 x 128 x 128 per key) over the whole encode call, is a lower bound
    of qjl_quad_kernel's."""
    import numpy as np
    import torch
    import kv_cache_vector_srht_amd as tq
    import workloads as W
    w = W.make_workload(idx)
    fm = w.formats[0]
    has_qjl = any(f[2] for row in fm for r in row for f in r)
    S = W.qjl_matrix(W.ROTATION_SEED, 0) if has_qjl else None
    layer = tq.Layer(W.rotation_signs(W.ROTATION_SEED, 0), dev, S, w.k_codebook, w.v_codebook)
    cache = tq.Cache(fm, [w.n_tokens] * w.batch, dev)
    k, v = W.make_kv(w, 0, device=dev)
    q = W.make_query(w, 0, device=dev)
    o = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.workspace_bytes(cache, w.n_q_heads), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def times(fn, warm, reps):
        for _ in range(warm):
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

    t_enc = times(lambda: tq.encode_kv(layer, cache, k, v, tok0=0), 1, enc_reps)
    t_dec = times(lambda: tq.decode_attention(layer, cache, q, out=o, workspace=ws), 3, dec_reps)
    eb, db = encode_bytes(w, fm), decode_bytes(w, fm, w.n_q_heads)
    rec = {"workload": w.name, "layers": 1, "batch": w.batch, "context": w.n_tokens,
           "decode_us": round(t_dec * 1e6, 2), "decode_bytes": db,
           "decode_gbs": round(db / t_dec / 1e9, 1), "decode_frac_of_peak": round(db / t_dec / 1e9 / HBM_PEAK_GBS, 4),
           "encode_us": round(t_enc * 1e6, 2), "encode_bytes": eb, "encode_gbs": round(eb / t_enc / 1e9, 1),
           "encode_mtokens_per_s": round(w.batch * w.n_tokens / t_enc / 1e6, 2)}
    if has_qjl:
        keys = sum(64 for row in fm for r in row for f in r if f[2])
        tf = keys * 2.0 * 128 * 128 / t_enc / 1e12
        rec["qjl_sketch_tflops_lower_bound"] = round(tf, 2)
        rec["qjl_sketch_frac_lower_bound"] = round(tf / FP32_MFMA_PEAK_TFLOPS, 4)
    del cache, k, v, q, o, ws
    torch.cuda.synchronize()
    return rec


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
    # (encode is one encode_pages_kernel launch per layer, plus qjl_quad_kernel
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
    # the headline kernel: the decode-attention call of one layer (qprep_kernel,
    # the split kernel(s) of the layer's page classes, combine_kernel), timed
    # with HIP events around each step's decode calls on the launch stream
    dec_roof = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_record("decode_attention", w.name),
                "kernel": "decode_attention (qprep_kernel + split_kernel + combine_kernel)",
                "bytes_per_launch": int(dec_bytes / w.n_layers),
                "launch_us": round(dec_s / w.n_layers * 1e6, 2)}
    qjl_keys = sum(64 for fm in w.formats for row in fm for r in row for f in r if f[2])
    if qjl_keys and enc_s >= dec_s:
        # With QJL key pages the encode call is dominated by qjl_quad_kernel,
        # whose contraction is the sketch z = sign(S r), 2 x 128 x 128 flops per
        # key at float32 accuracy, executed as three float16 products (hi/lo
        # split of both operands) on the matrix cores.  achieved/peak take the
        # float32 flops against the float32 matrix peak; the executed float16
        # flops (3x) against the float16 peak are given beside them.  Its own
        # duration is not separable from the call's encode_pages_kernel with
        # events around the call, so the rates are lower bounds: flops / whole
        # call time.
        flops = qjl_keys * 2.0 * 128 * 128 / w.n_layers
        tflops = flops / per_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "qjl_quad_kernel", "flops_per_launch": int(flops),
                "launch_us": round(per_launch_s * 1e6, 2),
                "executed": "3 float16 products per float32 product (v_mfma_f32_16x16x32_f16)",
                "fp16_executed_tflops": round(3 * tflops, 2), "fp16_peak": FP16_MFMA_PEAK_TFLOPS,
                "fp16_frac": round(3 * tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                "timed": "whole tq_encode_kv call (qjl_quad_kernel + encode_pages_kernel): lower bound",
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
        "decode_roofline": dec_roof,
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
    if args.latency:
        line["latency"] = latency(dev)
    if args.subworkloads:
        line["one_layer"] = {W.make_workload(i).name: one_layer(i, dev) for i in (4, 5)}
    if args.tiering:
        line["tiering"] = tiering(w, layers, inputs, queries, outs, wss, dev)
    if args.codecs:
        line["codecs"] = codecs(w, inputs, queries, dev)
    if not args.no_cpu_baseline:
        kv_host = {}

        def unit_job(l, b, h):
            if l not in kv_host:
                k, v = inputs[l]
                kv_host[l] = (k.cpu().numpy(), v.cpu().numpy(), queries[l].cpu().numpy())
            k, v, q = kv_host[l]
            signs = W.rotation_signs(W.ROTATION_SEED, l)
            S = W.qjl_matrix(W.ROTATION_SEED, l) if any(f[2] for f in w.formats[l][b][h]) else None
            return (w.formats[l][b][h], k[b, h], v[b, h], q[b, h * G:(h + 1) * G], signs, S,
                    w.k_codebook, w.v_codebook)

        def rounded(d):
            return {k2: (round(v2, 4) if isinstance(v2, float) else rounded(v2) if isinstance(v2, dict)
                         else v2) for k2, v2 in d.items()}
        line["cpu_baseline"] = rounded(cpu_baseline(w, unit_job, args.cpu_seconds))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
