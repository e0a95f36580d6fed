"""ctypes binding of libtq (include/tq.h): the same entry points, argument marshalling only.

Every computation runs in the library (host C++ for the codec table, HIP kernels for the
device work).  PyTorch is used for device memory and the current stream.  Importing this
module loads the built library and raises if it is absent -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libtq.so not found at {LIB_PATH}: build it first "
        "(python -c 'import __graft_entry__ as g; g.build()' or python vector_quantization_rope_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_ECAPACITY, TQ_ENOSPACE, TQ_EDEVICE = range(6)
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2

EXPORTS = [
    "tq_version", "tq_status_str", "tq_make_codebook", "tq_make_codebook_f64", "tq_codec_bytes",
    "tq_codec_build", "tq_cache_bytes", "tq_cache_init", "tq_quantize_kv",
    "tq_decode_workspace_bytes", "tq_decode_splits", "tq_decode_attend",
    "tq_decode_workspace_bytes_splits", "tq_decode_attend_splits",
    "tq_search_workspace_bytes", "tq_search_topk", "tq_quantize_kv_profiled",
    "tq_decode_attend_profiled", "tq_decode_window_workspace_bytes", "tq_decode_attend_window",
    "tq_decode_step", "tq_nsn_means_workspace_bytes", "tq_nsn_set_means", "tq_make_polar_grid",
    "tq_decode_attend_noalloc",
]

NOALLOC_SCRATCH_BYTES = 16 << 20   # TQ_NOALLOC_SCRATCH_BYTES


class CodecDesc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits_k", ctypes.c_int32), ("bits_v", ctypes.c_int32),
                ("m", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("d", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("bits_k", ctypes.c_int32),
                ("bits_v", ctypes.c_int32), ("m", ctypes.c_int32), ("nsn", ctypes.c_int32),
                ("polar", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
_CD = ctypes.POINTER(CodecDesc)
_KD = ctypes.POINTER(CacheDesc)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_version = _sig("tq_version", ctypes.c_char_p, [])
_status_str = _sig("tq_status_str", ctypes.c_char_p, [ctypes.c_int])
_make_codebook = _sig("tq_make_codebook", ctypes.c_int, [_I, _I, _P, _P])
_make_codebook_f64 = _sig("tq_make_codebook_f64", ctypes.c_int, [_I, _I, _P, _P])
_codec_bytes = _sig("tq_codec_bytes", _S, [_CD])
_codec_build = _sig("tq_codec_build", ctypes.c_int, [_CD, _P, _S])
_cache_bytes = _sig("tq_cache_bytes", _S, [_KD])
_cache_init = _sig("tq_cache_init", ctypes.c_int, [_KD, _P, _P])
_quantize_kv = _sig("tq_quantize_kv", ctypes.c_int, [_KD, _P, _P, _P, _P, ctypes.c_int, _I, _I, _F, _P])
_decode_ws = _sig("tq_decode_workspace_bytes", _S, [_KD, _I, _I])
_decode_splits = _sig("tq_decode_splits", _I, [_KD, _I, _I])
_decode_ws_splits = _sig("tq_decode_workspace_bytes_splits", _S, [_KD, _I, _I])
_decode_attend_splits = _sig("tq_decode_attend_splits", ctypes.c_int,
                             [_KD, _P, _P, _I, _P, ctypes.c_int, _I, _I, _F, _F, _P, _P, _I, _P, _S, _P])
_decode_attend = _sig("tq_decode_attend", ctypes.c_int,
                      [_KD, _P, _P, _I, _P, ctypes.c_int, _I, _I, _F, _F, _P, _P, _P, _S, _P])
_quantize_kv_prof = _sig("tq_quantize_kv_profiled", ctypes.c_int,
                         [_KD, _P, _P, _P, _P, ctypes.c_int, _I, _I, _F, _P, _P, _P])
_decode_attend_prof = _sig("tq_decode_attend_profiled", ctypes.c_int,
                           [_KD, _P, _P, _I, _P, ctypes.c_int, _I, _I, _F, _F, _P, _P, _I, _P, _S, _P, _P, _P])
_decode_attend_noalloc = _sig("tq_decode_attend_noalloc", ctypes.c_int,
                              [_KD, _P, _P, _I, _P, ctypes.c_int, _I, _I, _F, _F, _P, _P, _P])
_decode_win_ws = _sig("tq_decode_window_workspace_bytes", _S, [_KD, _I, _I])
_decode_attend_win = _sig("tq_decode_attend_window", ctypes.c_int,
                          [_KD, _P, _P, _I, _P, _P, ctypes.c_int, _I, _I, _P, ctypes.c_int, _I, _I, _F, _F,
                           _P, _P, _P, _S, _P])
_IP = ctypes.POINTER(ctypes.c_int32)
_decode_step = _sig("tq_decode_step", ctypes.c_int,
                    [_KD, _P, _P, _IP, _P, _P, ctypes.c_int, _IP, _I, _P, _P, _P, ctypes.c_int, _I, _I, _F, _F,
                     _P, _P, _P, _S, _P])
_polar_grid = _sig("tq_make_polar_grid", ctypes.c_int, [_I, _P, _P])
_nsn_ws = _sig("tq_nsn_means_workspace_bytes", _S, [_KD, _I])
_nsn_set = _sig("tq_nsn_set_means", ctypes.c_int, [_KD, _P, _P, _P, _P, ctypes.c_int, _I, _I, _F, _P, _S, _P])
_search_ws = _sig("tq_search_workspace_bytes", _S, [_KD, _I, _I, _I])
_search_topk = _sig("tq_search_topk", ctypes.c_int,
                    [_KD, _P, _P, _I, _P, _I, _I, _P, _P, _P, _S, _P])


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


def version() -> str:
    return _lib_version().decode()


def status_str(s: int) -> str:
    return _status_str(int(s)).decode()


def _check(st: int, where: str):
    if st != TQ_OK:
        raise TQError(st, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _require(t, name: str, *, shape=None, numel=None, dtypes=None, where: str):
    """Host-side checks of a tensor argument before its pointer crosses the C ABI (a raw
    integer pointer is passed through unchecked).  A strided view would make the kernels
    read the wrong rows, and a short or mistyped output would take writes past its end."""
    if t is None or isinstance(t, int):
        return
    if not t.is_contiguous():
        raise ValueError(f"{where}: {name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{where}: {name} has {t.numel()} elements, needs at least {numel}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected one of {dtypes}")


def _float_types():
    import torch
    return (torch.float32, torch.bfloat16, torch.float16)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}[t.dtype]


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ host-only calls
def make_codebook(d: int, bits: int):
    c = np.zeros(1 << bits, dtype=np.float32)
    t = np.zeros(max(1, (1 << bits) - 1), dtype=np.float32)
    _check(_make_codebook(d, bits, c.ctypes.data, t.ctypes.data), "tq_make_codebook")
    return c, t


def make_codebook_f64(d: int, bits: int):
    c = np.zeros(1 << bits, dtype=np.float64)
    t = np.zeros(max(1, (1 << bits) - 1), dtype=np.float64)
    _check(_make_codebook_f64(d, bits, c.ctypes.data, t.ctypes.data), "tq_make_codebook_f64")
    return c, t


def codec_bytes(desc: CodecDesc) -> int:
    return _codec_bytes(ctypes.byref(desc))


def codec_build(desc: CodecDesc) -> np.ndarray:
    n = codec_bytes(desc)
    if n == 0:
        raise TQError(TQ_EUNSUPPORTED, "tq_codec_bytes")
    buf = np.zeros(n, dtype=np.uint8)
    _check(_codec_build(ctypes.byref(desc), buf.ctypes.data, n), "tq_codec_build")
    return buf


def cache_bytes(desc: CacheDesc) -> int:
    return _cache_bytes(ctypes.byref(desc))


# ------------------------------------------------------------------ device calls
def cache_init(desc: CacheDesc, cache, stream=None):
    _check(_cache_init(ctypes.byref(desc), _ptr(cache), _stream(stream)), "tq_cache_init")


def quantize_kv(desc: CacheDesc, codec_dev, cache, k, v, start_pos: int, rope_base: float,
                n_new: int | None = None, stream=None, dtype: int | None = None, events=None):
    """events: optional (start, stop) hipEvent_t handles recorded around the kernel."""
    if n_new is None:
        n_new = 0 if k is None else int(k.shape[-2])
    if k is not None and not isinstance(k, int):
        want = (desc.batch, desc.kv_heads, int(n_new), desc.d)
        _require(k, "k", shape=want, dtypes=_float_types(), where="quantize_kv")
        if desc.bits_v > 0:
            if v is None:
                raise ValueError("quantize_kv: v is required when the cache has value codes")
            _require(v, "v", shape=want, dtypes=(k.dtype,), where="quantize_kv")
    code = dtype if dtype is not None else (_dtype_code(k) if k is not None else TQ_F32)
    ev0, ev1 = events if events else (None, None)
    _check(_quantize_kv_prof(ctypes.byref(desc), _ptr(codec_dev), _ptr(cache), _ptr(k), _ptr(v), code,
                             int(start_pos), int(n_new), float(rope_base), ev0, ev1, _stream(stream)),
           "tq_quantize_kv")


def decode_workspace_bytes(desc: CacheDesc, q_heads: int, length: int, splits: int = 0) -> int:
    if splits:
        return _decode_ws_splits(ctypes.byref(desc), q_heads, splits)
    return _decode_ws(ctypes.byref(desc), q_heads, length)


def decode_splits(desc: CacheDesc, q_heads: int, length: int) -> int:
    return _decode_splits(ctypes.byref(desc), q_heads, length)


def decode_attend(desc: CacheDesc, codec_dev, cache, length: int, q, q_pos: int, rope_base: float,
                  out, scores=None, ws=None, scale: float = 0.0, splits: int = 0, stream=None,
                  ws_bytes: int | None = None, events=None):
    """events: optional (start, stop) hipEvent_t handles recorded around the split-K kernel."""
    q_heads = int(q.shape[1])
    import torch
    _require(q, "q", shape=(desc.batch, q_heads, desc.d), dtypes=_float_types(), where="decode_attend")
    _require(out, "out", numel=desc.batch * q_heads * desc.d, dtypes=(torch.float32,), where="decode_attend")
    _require(scores, "scores", numel=desc.batch * q_heads * int(length), dtypes=(torch.float32,),
             where="decode_attend")
    _require(ws, "ws", where="decode_attend")
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    ev0, ev1 = events if events else (None, None)
    _check(_decode_attend_prof(ctypes.byref(desc), _ptr(codec_dev), _ptr(cache), int(length),
                               _ptr(q), _dtype_code(q), q_heads, int(q_pos), float(rope_base),
                               float(scale), _ptr(out), _ptr(scores), int(splits), _ptr(ws),
                               int(ws_bytes), ev0, ev1, _stream(stream)),
           "tq_decode_attend")


def decode_attend_noalloc(desc: CacheDesc, codec_dev, cache, length: int, q, q_pos: int, rope_base: float,
                          out, scores=None, scale: float = 0.0, stream=None):
    """tq_decode_attend_noalloc: decode attention with the library's own device scratch (no
    workspace argument, no allocation); calls that overlap on one GPU race."""
    import torch
    q_heads = int(q.shape[1])
    _require(q, "q", shape=(desc.batch, q_heads, desc.d), dtypes=_float_types(), where="decode_attend_noalloc")
    _require(out, "out", numel=desc.batch * q_heads * desc.d, dtypes=(torch.float32,),
             where="decode_attend_noalloc")
    _require(scores, "scores", numel=desc.batch * q_heads * int(length), dtypes=(torch.float32,),
             where="decode_attend_noalloc")
    _check(_decode_attend_noalloc(ctypes.byref(desc), _ptr(codec_dev), _ptr(cache), int(length), _ptr(q),
                                  _dtype_code(q), q_heads, int(q_pos), float(rope_base), float(scale), _ptr(out),
                                  _ptr(scores), _stream(stream)),
           "tq_decode_attend_noalloc")


def decode_window_workspace_bytes(desc: CacheDesc, q_heads: int, length: int) -> int:
    return _decode_win_ws(ctypes.byref(desc), q_heads, length)


def decode_attend_window(desc: CacheDesc, codec_dev, cache, length: int, win_k, win_v, win_len: int, q,
                         q_pos: int, rope_base: float, out, scores=None, ws=None, scale: float = 0.0,
                         stream=None, ws_bytes: int | None = None):
    """win_k, win_v: [batch, kv_heads, cap, d] raw keys and values of positions length ...
    length + win_len - 1 (contiguous, one dtype); scores, if given, rows of length + win_len."""
    q_heads = int(q.shape[1])
    if win_k is None or win_v is None:
        raise ValueError("decode_attend_window: window tensors required (win_len may be 0)")
    want = (desc.batch, desc.kv_heads, int(win_k.shape[2]), desc.d)
    for t in (win_k, win_v):
        if t.dim() != 4 or tuple(t.shape) != want or not t.is_contiguous() or t.dtype != win_k.dtype:
            raise ValueError(f"decode_attend_window: window tensors must be contiguous {want} of one dtype")
    if not 0 <= win_len <= int(win_k.shape[2]):
        raise ValueError("decode_attend_window: win_len outside [0, cap]")
    if scores is not None and scores.numel() < desc.batch * q_heads * (length + win_len):
        raise ValueError("decode_attend_window: scores smaller than batch x q_heads x (length + win_len)")
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_decode_attend_win(ctypes.byref(desc), _ptr(codec_dev), _ptr(cache), int(length), _ptr(win_k),
                              _ptr(win_v), _dtype_code(win_k), int(win_len), int(win_k.shape[2]), _ptr(q),
                              _dtype_code(q), q_heads, int(q_pos), float(rope_base), float(scale), _ptr(out),
                              _ptr(scores), _ptr(ws), int(ws_bytes), _stream(stream)),
           "tq_decode_attend_window")


def decode_step(desc: CacheDesc, codec_dev, cache, length: int, win_k, win_v, win_len: int, new_k, new_v, q,
                q_pos: int, rope_base: float, out, scores=None, ws=None, scale: float = 0.0, stream=None,
                ws_bytes: int | None = None):
    """One generation step: flush a full window into the packed cache, append new_k, new_v
    ([batch, kv_heads, d], the window's dtype) to the window, attend.  Returns the new
    (length, win_len)."""
    q_heads = int(q.shape[1])
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    cap = int(win_k.shape[2])
    want = (desc.batch, desc.kv_heads, cap, desc.d)
    for t in (win_k, win_v):
        if t.dim() != 4 or tuple(t.shape) != want or not t.is_contiguous() or t.dtype != win_k.dtype:
            raise ValueError(f"decode_step: window tensors must be contiguous {want} of one dtype")
    for t in (new_k, new_v):
        if t.numel() != desc.batch * desc.kv_heads * desc.d or not t.is_contiguous() or t.dtype != win_k.dtype:
            raise ValueError("decode_step: new_k, new_v must be contiguous [batch, kv_heads, d] of the window dtype")
    n_after = (length + cap + 1) if win_len == cap else (length + win_len + 1)
    if scores is not None and scores.numel() < desc.batch * q_heads * n_after:
        raise ValueError("decode_step: scores smaller than batch x q_heads x tokens after the step")
    L, Wn = ctypes.c_int32(length), ctypes.c_int32(win_len)
    _check(_decode_step(ctypes.byref(desc), _ptr(codec_dev), _ptr(cache), ctypes.byref(L), _ptr(win_k), _ptr(win_v),
                        _dtype_code(win_k), ctypes.byref(Wn), cap, _ptr(new_k), _ptr(new_v), _ptr(q), _dtype_code(q),
                        q_heads, int(q_pos), float(rope_base), float(scale), _ptr(out), _ptr(scores), _ptr(ws),
                        int(ws_bytes), _stream(stream)),
           "tq_decode_step")
    return int(L.value), int(Wn.value)


def make_polar_grid(level: int):
    """fp64 (centroids, boundaries) of a PolarQuant angle level (host)."""
    K = 16 if level == 1 else 4
    c = np.zeros(K, dtype=np.float64)
    t = np.zeros(K - 1, dtype=np.float64)
    _check(_polar_grid(int(level), c.ctypes.data, t.ctypes.data), "tq_make_polar_grid")
    return c, t


def nsn_means_workspace_bytes(desc: CacheDesc, n: int) -> int:
    return _nsn_ws(ctypes.byref(desc), n)


def nsn_set_means(desc: CacheDesc, codec_dev, cache, k, v, start_pos: int, rope_base: float, ws=None,
                  stream=None, ws_bytes: int | None = None):
    """NSN channel means of every unit over the tokens k, v ([batch, kv_heads, n, d])."""
    n = int(k.shape[-2])
    want = (desc.batch, desc.kv_heads, n, desc.d)
    for t in (k, v):
        if t.dim() != 4 or tuple(t.shape) != want or not t.is_contiguous() or t.dtype != k.dtype:
            raise ValueError(f"nsn_set_means: k, v must be contiguous {want} of one dtype")
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_nsn_set(ctypes.byref(desc), _ptr(codec_dev), _ptr(cache), _ptr(k), _ptr(v), _dtype_code(k),
                    int(start_pos), n, float(rope_base), _ptr(ws), int(ws_bytes), _stream(stream)),
           "tq_nsn_set_means")


def search_workspace_bytes(desc: CacheDesc, n_db: int, nq: int, k: int) -> int:
    return _search_ws(ctypes.byref(desc), n_db, nq, k)


def search_topk(desc: CacheDesc, codec_dev, db_cache, n_db: int, queries, k: int, idx_out,
                score_out, ws, stream=None, ws_bytes: int | None = None):
    import torch
    nq = int(queries.shape[0])
    _require(queries, "queries", shape=(nq, desc.d), dtypes=(torch.float32,), where="search_topk")
    _require(idx_out, "idx_out", numel=nq * int(k), dtypes=(torch.int32,), where="search_topk")
    _require(score_out, "score_out", numel=nq * int(k), dtypes=(torch.float32,), where="search_topk")
    _require(ws, "ws", where="search_topk")
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_search_topk(ctypes.byref(desc), _ptr(codec_dev), _ptr(db_cache), int(n_db), _ptr(queries),
                        int(queries.shape[0]), int(k), _ptr(idx_out), _ptr(score_out), _ptr(ws),
                        int(ws_bytes), _stream(stream)),
           "tq_search_topk")


# ------------------------------------------------------------------ conveniences (memory only)
class Codec:
    """Codec table built on the host by the library and copied once to the device."""

    def __init__(self, d: int, bits_k: int, bits_v: int, m: int, seed: int = 0, device="cuda"):
        import torch
        self.desc = CodecDesc(d, bits_k, bits_v, m, seed)
        self.host = codec_build(self.desc)
        self.dev = torch.from_numpy(self.host).to(device)


class PackedCache:
    """A packed cache buffer (torch uint8 tensor) plus its descriptor."""

    def __init__(self, batch, kv_heads, d, capacity, bits_k, bits_v, m, device="cuda", stream=None, nsn=0,
                 polar=0):
        import torch
        self.desc = CacheDesc(batch, kv_heads, d, capacity, bits_k, bits_v, m, nsn, polar)
        n = cache_bytes(self.desc)
        if n == 0:
            raise TQError(TQ_EUNSUPPORTED, "tq_cache_bytes")
        self.buf = torch.zeros(n, dtype=torch.uint8, device=device)
        cache_init(self.desc, self.buf, stream)
