"""Python binding of libtq (SRHT KV-cache compression + compressed decode attention).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of encode, decode attention and dequantisation runs in
the library's HIP kernels.  Importing this module does not touch the GPU; the
first call loads ``lib/libtq.so`` and raises ``TQError`` if it is missing or a
call fails.  There is no fallback path.

Names follow ``include/tq.h``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

HEAD_DIM = 128
PAGE_TOKENS = 64
JL_DIM = 128
CODEBOOK_TABLE_FLOATS = 12288
LLOYD_MAX = 0
UNIFORM = 1
BETA = 2
FITTED = 3
POLAR = 4
DTYPE_F32 = 0
DTYPE_F16 = 1
QJL_SCORE_UNBIASED = 0
QJL_SCORE_SIGN = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtq.so")
# the same library built with TQ_DEVICE_CHECKS=1 (device index checks)
CHECKED_LIB_PATH = os.path.join(_PKG, "lib", "libtq_checked.so")
EXPORTS = ("tq_page_bytes", "tq_page_descriptor", "tq_build_codebook", "tq_codebook_table",
           "tq_layer_params", "tq_sign_mask", "tq_decode_workspace_bytes", "tq_cache_bytes",
           "tq_status_string", "tq_last_error", "tq_encode_kv", "tq_decode_attention",
           "tq_dequantize", "tq_append_kv", "tq_retier_pages", "tq_decode_attention_mass",
           "tq_fit_codebook", "tq_calibrated_table", "tq_decode_attention_noalloc",
           "tq_decode_attention_token_mass", "tq_polar_table", "tq_encode_kv_shaped",
           "tq_device_checks")
NOALLOC_SCRATCH_BYTES = 32 << 20     # TQ_NOALLOC_SCRATCH_BYTES
ERR_UNSUPPORTED = -2                 # TQ_ERR_UNSUPPORTED


class TQError(RuntimeError):
    pass


# ------------------------------------------------------------------ structs
class tq_layer(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("k_codebook", ctypes.c_int32),
                ("v_codebook", ctypes.c_int32), ("jl_dim", ctypes.c_int32),
                ("sign_mask", ctypes.c_void_p), ("k_table", ctypes.c_void_p),
                ("v_table", ctypes.c_void_p), ("qjl_s", ctypes.c_void_p)]


class tq_cache(ctypes.Structure):
    _fields_ = [("n_sessions", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("page_classes", ctypes.c_int32),
                ("n_tokens", ctypes.c_void_p), ("pages", ctypes.c_void_p),
                ("pool", ctypes.c_void_p), ("pool_bytes", ctypes.c_uint64),
                ("unit_classes", ctypes.c_void_p)]


class tq_kv_input(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("tok0", ctypes.c_int32), ("ntok", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_t", ctypes.c_int64), ("error_flags", ctypes.c_void_p)]


class tq_token_input(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("error_flags", ctypes.c_void_p)]


class tq_query(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float), ("qjl_scoring", ctypes.c_int32)]


_lib = None


def _open(path: str) -> ctypes.CDLL:
    """Loads a build of libtq and declares its calls' argument types."""
    if not os.path.exists(path):
        raise TQError(f"{path} is missing: build it with __graft_entry__.build() "
                      "or python kv_cache_vector_srht_amd/build.py")
    L = ctypes.CDLL(path)
    L.tq_page_bytes.restype = ctypes.c_size_t
    L.tq_page_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.tq_page_descriptor.restype = ctypes.c_uint64
    L.tq_page_descriptor.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.tq_build_codebook.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.tq_codebook_table.argtypes = [ctypes.c_int, ctypes.c_void_p]
    L.tq_polar_table.argtypes = [ctypes.c_int, ctypes.c_void_p]
    L.tq_fit_codebook.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    L.tq_calibrated_table.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.tq_layer_params.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    L.tq_sign_mask.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.tq_decode_workspace_bytes.restype = ctypes.c_size_t
    L.tq_decode_workspace_bytes.argtypes = [ctypes.POINTER(tq_cache), ctypes.c_int]
    L.tq_cache_bytes.restype = ctypes.c_size_t
    L.tq_cache_bytes.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.tq_status_string.restype = ctypes.c_char_p
    L.tq_status_string.argtypes = [ctypes.c_int]
    L.tq_last_error.restype = ctypes.c_char_p
    L.tq_encode_kv.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                               ctypes.POINTER(tq_kv_input), ctypes.c_void_p]
    L.tq_encode_kv_shaped.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                                      ctypes.POINTER(tq_kv_input), ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    L.tq_device_checks.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.tq_decode_attention.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                                      ctypes.POINTER(tq_query), ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.tq_decode_attention_mass.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                                           ctypes.POINTER(tq_query), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.tq_decode_attention_token_mass.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                                                 ctypes.POINTER(tq_query), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.tq_decode_attention_noalloc.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                                              ctypes.POINTER(tq_query), ctypes.c_void_p, ctypes.c_void_p]
    L.tq_append_kv.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache),
                               ctypes.POINTER(tq_token_input), ctypes.c_void_p]
    L.tq_retier_pages.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache), ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.tq_dequantize.argtypes = [ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache), ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
    return L


def lib() -> ctypes.CDLL:
    """The loaded libtq (raises TQError when it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


class library:
    """Context manager: every call of this module inside the block goes to the
    build of libtq at ``path`` (the checked build, by default), loaded beside
    the release one; device memory and streams are shared."""

    def __init__(self, path: str = None):
        self.path = path or CHECKED_LIB_PATH

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _open(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def device_checks(reset: bool = True):
    """tq_device_checks: the check bits the kernels recorded (a checked build),
    or None for a release build."""
    flags = ctypes.c_uint32(0)
    st = lib().tq_device_checks(ctypes.byref(flags), 1 if reset else 0)
    if st == ERR_UNSUPPORTED:
        return None
    check(st, "tq_device_checks")
    return int(flags.value)


def check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise TQError(f"{what}: {L.tq_status_string(status).decode()} ({status}): "
                      f"{L.tq_last_error().decode()}")


# ------------------------------------------------------------- host helpers
def build_codebook(bits: int, kind: int = LLOYD_MAX):
    """(centroids, boundaries) float32 numpy arrays from tq_build_codebook."""
    import numpy as np
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(max(L - 1, 1), np.float32)
    check(lib().tq_build_codebook(bits, kind, c.ctypes.data, t.ctypes.data), "tq_build_codebook")
    return c, t[:L - 1]


def codebook_table(kind: int = LLOYD_MAX):
    import numpy as np
    tab = np.zeros(CODEBOOK_TABLE_FLOATS, np.float32)
    check(lib().tq_codebook_table(kind, tab.ctypes.data), "tq_codebook_table")
    return tab


def polar_table(angle_shift: int = 0):
    """tq_polar_table: the table of a PolarQuant part whose page width b gives
    b - angle_shift radius bits and b + angle_shift angle bits (use with kind
    POLAR as Layer's k_table / v_table)."""
    import numpy as np
    tab = np.zeros(CODEBOOK_TABLE_FLOATS, np.float32)
    check(lib().tq_polar_table(int(angle_shift), tab.ctypes.data), "tq_polar_table")
    return tab


def _samples(vectors, signs):
    import numpy as np
    X = np.ascontiguousarray(np.asarray(vectors, dtype=np.float32).reshape(-1, HEAD_DIM))
    sg = np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
    if sg.size != HEAD_DIM:
        raise TQError("signs must hold 128 entries")
    return X, sg


def fit_codebook(vectors, signs, bits: int):
    """tq_fit_codebook: (centroids, boundaries) fitted to sample vectors [n, 128]."""
    import numpy as np
    X, sg = _samples(vectors, signs)
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(max(L - 1, 1), np.float32)
    check(lib().tq_fit_codebook(X.ctypes.data, X.shape[0], sg.ctypes.data, bits, c.ctypes.data,
                                t.ctypes.data), "tq_fit_codebook")
    return c, t[:L - 1]


def calibrated_table(vectors, signs):
    """tq_calibrated_table: a codebook table fitted to sample vectors [n, 128]."""
    import numpy as np
    X, sg = _samples(vectors, signs)
    tab = np.zeros(CODEBOOK_TABLE_FLOATS, np.float32)
    check(lib().tq_calibrated_table(X.ctypes.data, X.shape[0], sg.ctypes.data, tab.ctypes.data),
          "tq_calibrated_table")
    return tab


def layer_params(seed: int, layer: int, with_qjl: bool = True):
    """(signs int8[128], S float32[128,128] or None) from tq_layer_params."""
    import numpy as np
    s = np.zeros(HEAD_DIM, np.int8)
    S = np.zeros((JL_DIM, HEAD_DIM), np.float32) if with_qjl else None
    check(lib().tq_layer_params(ctypes.c_uint64(seed), layer, HEAD_DIM, JL_DIM, s.ctypes.data,
                                S.ctypes.data if S is not None else None), "tq_layer_params")
    return s, S


def sign_mask(signs):
    import numpy as np
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
    m = np.zeros(4, np.uint32)
    check(lib().tq_sign_mask(s.ctypes.data, s.size, m.ctypes.data), "tq_sign_mask")
    return m


PAGE_PENDING = 1 << 57
RETIER_FROM_PACKED = 1
RETIER_FROM_FP16 = 2


def is_pending(fmt) -> bool:
    """A format (k_bits, v_bits, qjl, pending) with pending set: the page fills
    as fp16 and tq_append_kv packs it into (k_bits, v_bits, qjl) when full."""
    return len(fmt) > 3 and bool(fmt[3])


def page_bytes(fmt) -> int:
    """Bytes of a page slot of this format (a pending page occupies an fp16 slot)."""
    kb, vb, qjl = fmt[:3]
    if is_pending(fmt):
        if lib().tq_page_bytes(int(kb), int(vb), int(bool(qjl))) == 0 or kb == 0:
            raise TQError(f"invalid pending page format {fmt}")
        kb, vb, qjl = 0, 0, False
    n = lib().tq_page_bytes(int(kb), int(vb), int(bool(qjl)))
    if n == 0:
        raise TQError(f"invalid page format {fmt}")
    return int(n)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return DTYPE_F16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TQError(f"unsupported dtype {t.dtype}")


def _stream(device) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ------------------------------------------------------------------- layer
class Layer:
    """Device-side constants of one layer: D, codebook tables, optional S."""

    def __init__(self, signs, device, qjl_s=None, k_codebook: int = LLOYD_MAX,
                 v_codebook: int = LLOYD_MAX, k_table=None, v_table=None):
        """k_table / v_table: a table from calibrated_table (kind FITTED) or
        from polar_table (kind POLAR) in place of the built-in codebook of
        that kind."""
        import numpy as np
        import torch
        self.device = torch.device(device)
        self.signs = np.asarray(signs, dtype=np.int8)
        self.mask = torch.from_numpy(sign_mask(self.signs).view(np.int32).copy()).to(self.device)
        for kind, tab in ((k_codebook, k_table), (v_codebook, v_table)):
            if (kind == FITTED and tab is None) or (tab is not None and kind not in (FITTED, POLAR)):
                raise TQError("a FITTED codebook comes with its table; only FITTED and POLAR take one")
        kt = codebook_table(k_codebook) if k_table is None else np.asarray(k_table, dtype=np.float32)
        vt = codebook_table(v_codebook) if v_table is None else np.asarray(v_table, dtype=np.float32)
        self.k_table = torch.from_numpy(np.ascontiguousarray(kt)).to(self.device)
        self.v_table = torch.from_numpy(np.ascontiguousarray(vt)).to(self.device)
        self.qjl_s = None
        if qjl_s is not None:
            self.qjl_s = torch.from_numpy(np.ascontiguousarray(qjl_s, dtype=np.float32)).to(self.device)
        self.k_codebook, self.v_codebook = k_codebook, v_codebook
        self.struct = tq_layer(HEAD_DIM, k_codebook, v_codebook, JL_DIM, self.mask.data_ptr(),
                               self.k_table.data_ptr(), self.v_table.data_ptr(),
                               self.qjl_s.data_ptr() if self.qjl_s is not None else None)


# ------------------------------------------------------------------- cache
CACHE_COMMON_PAGES = 1
CACHE_OTHER_PAGES = 2
CACHE_WIDE_PAGES = 4


def _format_classes(f) -> int:
    kb, vb, q = f[:3]
    if 1 <= kb <= 4 and 1 <= vb <= 4 and not q:
        bits = CACHE_COMMON_PAGES
    elif kb >= 5 and vb >= 5 and not q:
        bits = CACHE_WIDE_PAGES
    else:
        bits = CACHE_OTHER_PAGES
    if is_pending(f):
        bits |= CACHE_OTHER_PAGES   # fp16 until it is packed
    return bits


def unit_classes(formats):
    """The tq_cache.unit_classes array ([B][H_kv] uint8) of a page table with
    these formats: per (session, KV head), the page classes its pages hold."""
    import numpy as np
    B, H = len(formats), len(formats[0])
    out = np.zeros((B, H), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            bits = 0
            for f in formats[b][h]:
                bits |= _format_classes(f)
            out[b, h] = bits
    return out


def page_classes(formats) -> int:
    """The tq_cache.page_classes bits of a page table with these formats:
    common = 1-4 bit K and V without QJL; wide = 5-8 bit K and V without QJL;
    other = fp16, QJL or mixed widths (a pending page counts as fp16 and as its
    packed format)."""
    bits = 0
    for row in formats:
        for fm in row:
            for f in fm:
                bits |= _format_classes(f)
    return bits


class Cache:
    """Page pool + page table + token counts for B sessions x H_kv heads.

    ``formats[b][h][p]`` is (0, 0, False) for an fp16 page, (k_bits, v_bits,
    qjl, True) for a pending page (see append_kv), or
    (k_bits, v_bits, qjl) for a packed page.  Pages are laid out in the pool
    in (session, head, page) order, followed by ``spare_bytes`` (rounded up
    to 256) of free pool space, e.g. for pages that retier_pages moves.
    """

    def __init__(self, formats, n_tokens: Sequence[int], device, spare_bytes: int = 0):
        import numpy as np
        import torch
        self.device = torch.device(device)
        B = len(formats)
        H = len(formats[0])
        P = max(len(formats[b][h]) for b in range(B) for h in range(H))
        L = lib()
        desc = np.zeros((B, H, P), dtype=np.uint64)
        self.offsets = np.zeros((B, H, P), dtype=np.int64)
        off = 0
        for b in range(B):
            for h in range(H):
                for p, fmt in enumerate(formats[b][h]):
                    kb, vb, q = fmt[:3]
                    n = page_bytes(fmt)
                    d = L.tq_page_descriptor(off, int(kb), int(vb), int(bool(q)))
                    if d == 0:
                        raise TQError(f"cannot describe page {fmt} at {off}")
                    if is_pending(fmt):
                        d |= PAGE_PENDING
                    desc[b, h, p] = d
                    self.offsets[b, h, p] = off
                    off += (n + 255) // 256 * 256
        self.formats = [[list(fm) for fm in row] for row in formats]
        self.n_sessions, self.n_kv_heads, self.max_pages = B, H, P
        self.spare_offset = off     # free pool space past the pages (spare_bytes of it)
        self.pool_bytes = max(off + (int(spare_bytes) + 255) // 256 * 256, 256)
        self.pool = torch.zeros(self.pool_bytes, dtype=torch.uint8, device=self.device)
        self.host_pages = desc
        self.pages = torch.from_numpy(desc.view(np.int64)).to(self.device)
        self.n_tokens = torch.tensor(list(n_tokens), dtype=torch.int32, device=self.device)
        self.page_classes = page_classes(formats)
        self.unit_classes = np.ascontiguousarray(unit_classes(formats))
        self.struct = tq_cache(B, H, P, self.page_classes, self.n_tokens.data_ptr(),
                               self.pages.data_ptr(), self.pool.data_ptr(), self.pool_bytes,
                               self.unit_classes.ctypes.data)

    def set_n_tokens(self, n_tokens: Sequence[int]) -> None:
        self.n_tokens.copy_(self.n_tokens.new_tensor(list(n_tokens)))

    def footprint(self) -> int:
        """Bytes of the pages (tq_cache_bytes over the host page table)."""
        import numpy as np
        flat = np.ascontiguousarray(self.host_pages.reshape(-1))
        return int(lib().tq_cache_bytes(flat.ctypes.data, flat.size))

    def page_view(self, b: int, h: int, p: int):
        """The bytes of one page (a uint8 tensor view of the pool)."""
        off = int(self.offsets[b, h, p])
        return self.pool[off:off + page_bytes(self.formats[b][h][p])]


# ------------------------------------------------------------- device calls
def encode_kv(layer: Layer, cache: Cache, k, v, tok0: int = 0, error_flags=None,
              pages_per_block: int = 0, qjl_workgroups: int = 0) -> None:
    """tq_encode_kv over k, v of shape [B, H_kv, ntok, 128] (fp16 or fp32);
    with a launch shape (pages_per_block, qjl_workgroups), tq_encode_kv_shaped."""
    if k.shape != v.shape or k.dim() != 4 or k.shape[-1] != HEAD_DIM or k.dtype != v.dtype:
        raise TQError(f"k and v must both be [B, H_kv, T, 128] of one dtype, got {tuple(k.shape)}, {tuple(v.shape)}")
    if k.stride() != v.stride() or k.stride(-1) != 1:
        raise TQError("k and v must share strides with a unit innermost stride")
    if k.shape[0] != cache.n_sessions or k.shape[1] != cache.n_kv_heads:
        raise TQError("k/v session or head count does not match the cache")
    inp = tq_kv_input(k.data_ptr(), v.data_ptr(), _dtype_code(k), tok0, k.shape[2], 0,
                      k.stride(0), k.stride(1), k.stride(2),
                      error_flags.data_ptr() if error_flags is not None else None)
    if pages_per_block or qjl_workgroups:
        check(lib().tq_encode_kv_shaped(ctypes.byref(layer.struct), ctypes.byref(cache.struct), ctypes.byref(inp),
                                        pages_per_block, qjl_workgroups, _stream(k.device)), "tq_encode_kv_shaped")
    else:
        check(lib().tq_encode_kv(ctypes.byref(layer.struct), ctypes.byref(cache.struct),
                                 ctypes.byref(inp), _stream(k.device)), "tq_encode_kv")


def workspace_bytes(cache: Cache, n_q_heads: int) -> int:
    return int(lib().tq_decode_workspace_bytes(ctypes.byref(cache.struct), n_q_heads))


def decode_attention(layer: Layer, cache: Cache, q, out=None, workspace=None,
                     softmax_scale: float = 0.0, page_mass=None, qjl_scoring: int = 0,
                     token_mass=None):
    """tq_decode_attention for q [B, H_q, 128]; returns out [B, H_q, 128] float32.
    With ``page_mass`` (float32 [B, H_q, max_pages]), tq_decode_attention_mass
    also fills it with each page's attention mass; with ``token_mass`` (float32
    [B, H_q, 64 max_pages]), tq_decode_attention_token_mass fills it with each
    token's attention weight (one of the two at a time)."""
    import torch
    if q.dim() != 3 or q.shape[0] != cache.n_sessions or q.shape[-1] != HEAD_DIM or q.stride(-1) != 1:
        raise TQError(f"q must be [B, H_q, 128] with unit innermost stride, got {tuple(q.shape)}")
    Hq = q.shape[1]
    if out is None:
        out = torch.empty((q.shape[0], Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = workspace_bytes(cache, Hq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    qs = tq_query(q.data_ptr(), _dtype_code(q), Hq, q.stride(0), q.stride(1), softmax_scale, qjl_scoring)
    if token_mass is not None:
        if page_mass is not None:
            raise TQError("page_mass and token_mass are separate calls")
        if (token_mass.dtype != torch.float32 or not token_mass.is_contiguous()
                or tuple(token_mass.shape) != (cache.n_sessions, Hq, cache.max_pages * PAGE_TOKENS)):
            raise TQError("token_mass must be a contiguous float32 [B, H_q, 64 max_pages] tensor")
        check(lib().tq_decode_attention_token_mass(ctypes.byref(layer.struct), ctypes.byref(cache.struct),
                                                   ctypes.byref(qs), out.data_ptr(), token_mass.data_ptr(),
                                                   workspace.data_ptr(),
                                                   workspace.numel() * workspace.element_size(),
                                                   _stream(q.device)), "tq_decode_attention_token_mass")
        return out
    if page_mass is None:
        check(lib().tq_decode_attention(ctypes.byref(layer.struct), ctypes.byref(cache.struct),
                                        ctypes.byref(qs), out.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(q.device)), "tq_decode_attention")
        return out
    if (page_mass.dtype != torch.float32 or not page_mass.is_contiguous()
            or tuple(page_mass.shape) != (cache.n_sessions, Hq, cache.max_pages)):
        raise TQError(f"page_mass must be a contiguous float32 [B, H_q, max_pages] tensor")
    check(lib().tq_decode_attention_mass(ctypes.byref(layer.struct), ctypes.byref(cache.struct),
                                         ctypes.byref(qs), out.data_ptr(), page_mass.data_ptr(),
                                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         _stream(q.device)), "tq_decode_attention_mass")
    return out


def decode_attention_noalloc(layer: Layer, cache: Cache, q, out, softmax_scale: float = 0.0,
                             qjl_scoring: int = 0):
    """tq_decode_attention_noalloc: decode attention into a caller's ``out``
    [B, H_q, 128] float32 with the library's built-in device scratch in place
    of a workspace; allocates nothing.  Calls that overlap on one GPU race."""
    import torch
    if q.dim() != 3 or q.shape[0] != cache.n_sessions or q.shape[-1] != HEAD_DIM or q.stride(-1) != 1:
        raise TQError(f"q must be [B, H_q, 128] with unit innermost stride, got {tuple(q.shape)}")
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (q.shape[0], q.shape[1], HEAD_DIM):
        raise TQError("out must be a contiguous float32 [B, H_q, 128] tensor")
    qs = tq_query(q.data_ptr(), _dtype_code(q), q.shape[1], q.stride(0), q.stride(1), softmax_scale, qjl_scoring)
    check(lib().tq_decode_attention_noalloc(ctypes.byref(layer.struct), ctypes.byref(cache.struct),
                                            ctypes.byref(qs), out.data_ptr(), _stream(q.device)),
          "tq_decode_attention_noalloc")
    return out


def append_kv(layer: Layer, cache: Cache, k, v, error_flags=None) -> None:
    """tq_append_kv: one new token per session, k and v of shape [B, H_kv, 128]
    (fp16 or fp32); advances cache.n_tokens on the device."""
    if k.shape != v.shape or k.dim() != 3 or k.shape[-1] != HEAD_DIM or k.dtype != v.dtype:
        raise TQError(f"k and v must both be [B, H_kv, 128] of one dtype, got {tuple(k.shape)}, {tuple(v.shape)}")
    if k.stride() != v.stride() or k.stride(-1) != 1:
        raise TQError("k and v must share strides with a unit innermost stride")
    if k.shape[0] != cache.n_sessions or k.shape[1] != cache.n_kv_heads:
        raise TQError("k/v session or head count does not match the cache")
    inp = tq_token_input(k.data_ptr(), v.data_ptr(), _dtype_code(k), 0, k.stride(0), k.stride(1),
                         error_flags.data_ptr() if error_flags is not None else None)
    check(lib().tq_append_kv(ctypes.byref(layer.struct), ctypes.byref(cache.struct), ctypes.byref(inp),
                             _stream(k.device)), "tq_append_kv")


def retier_pages(layer: Layer, cache: Cache, pages, new_formats, new_offsets=None,
                 error_flags=None) -> None:
    """tq_retier_pages: page (b, h, p) of ``pages`` takes the packed format
    (k_bits, v_bits, qjl) of ``new_formats``, in its own slot or at the pool
    byte offset of ``new_offsets`` (a slot clear of every other page).  Updates
    the cache's record of formats, offsets and its page-class bits."""
    import numpy as np
    import torch
    pages = [tuple(int(x) for x in p) for p in pages]
    if len(pages) != len(new_formats):
        raise TQError("one new format per listed page")
    if len(set(pages)) != len(pages):
        raise TQError("a page is listed twice")
    if new_offsets is None:
        new_offsets = [int(cache.offsets[p]) for p in pages]
    if len(new_offsets) != len(pages):
        raise TQError("one offset per listed page")
    L = lib()
    H, P = cache.n_kv_heads, cache.max_pages
    idx = np.zeros(len(pages), dtype=np.int64)
    desc = np.zeros(len(pages), dtype=np.uint64)
    for i, ((b, h, p), fmt, off) in enumerate(zip(pages, new_formats, new_offsets)):
        if not (0 <= b < cache.n_sessions and 0 <= h < H and 0 <= p < len(cache.formats[b][h])):
            raise TQError(f"page {(b, h, p)} is not in the cache")
        kb, vb, q = fmt[:3]
        d = L.tq_page_descriptor(int(off), int(kb), int(vb), int(bool(q)))
        if d == 0 or kb == 0 or is_pending(fmt):
            raise TQError(f"invalid target format {fmt}")
        idx[i] = (b * H + h) * P + p
        desc[i] = d
    if not pages:
        return
    idx_t = torch.from_numpy(idx).to(cache.device)
    desc_t = torch.from_numpy(desc.view(np.int64)).to(cache.device)
    # the source kinds present, from the record of formats
    sources = 0
    for b, h, p in pages:
        sources |= RETIER_FROM_FP16 if cache.formats[b][h][p][0] == 0 else RETIER_FROM_PACKED
    check(L.tq_retier_pages(ctypes.byref(layer.struct), ctypes.byref(cache.struct), idx_t.data_ptr(),
                            desc_t.data_ptr(), len(pages), sources,
                            error_flags.data_ptr() if error_flags is not None else None,
                            _stream(cache.device)), "tq_retier_pages")
    for (b, h, p), fmt, d, off in zip(pages, new_formats, desc, new_offsets):
        cache.formats[b][h][p] = tuple(fmt[:3])
        cache.host_pages[b, h, p] = d
        cache.offsets[b, h, p] = int(off)
    cache.page_classes = page_classes(cache.formats)
    cache.struct.page_classes = cache.page_classes
    cache.unit_classes[...] = unit_classes(cache.formats)


def dequantize(layer: Layer, cache: Cache, which: int, tok0: int, ntok: int, add_qjl: bool = True,
               out=None):
    """tq_dequantize: [B, H_kv, ntok, 128] float32 reconstruction (keys 0, values 1)."""
    import torch
    if out is None:
        out = torch.empty((cache.n_sessions, cache.n_kv_heads, ntok, HEAD_DIM), dtype=torch.float32,
                          device=cache.device)
    check(lib().tq_dequantize(ctypes.byref(layer.struct), ctypes.byref(cache.struct), which,
                              int(add_qjl), tok0, ntok, out.data_ptr(), _stream(cache.device)),
          "tq_dequantize")
    return out
