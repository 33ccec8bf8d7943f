"""ctypes binding of the C ABI in include/ska.h (libska.so).

Argument marshalling only: every step of encode and decode runs in the HIP
kernels of libska.so.  PyTorch supplies device memory and the stream.  There
is no fallback: if libska.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libska.so")

SKA_OK, SKA_ERR_INVALID, SKA_ERR_UNSUPPORTED, SKA_ERR_HIP, SKA_ERR_NOMEM = range(5)
RADIUS_UNIFORM, RADIUS_LOG = 0, 1
Q_CODED, Q_EXACT = 0, 1
QDIR_F16, QDIR_F32 = 0, 1
PAGE = 16
DEVERR_SLOT, DEVERR_PAGE, DEVERR_TIER = 1, 2, 4

SYMBOLS = ("ska_encode_keys", "ska_decode_attention", "ska_decode_attention_noalloc", "ska_append_decode_attention",
           "ska_dense_decode_attention",
           "ska_decompress_keys", "ska_rdr_plan", "ska_get_radius_range", "ska_device_errors",
           "ska_profile_begin", "ska_profile_read", "ska_free", "ska_status_string")


class SkaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int),
        ("page_size", ctypes.c_int),
        ("num_pages", ctypes.c_int64),
        ("radius_mode", ctypes.c_int),
        ("radius_bits", ctypes.c_int),
        ("tier_mask", ctypes.c_uint32),
        ("query_mode", ctypes.c_int),
        ("kcode", ctypes.c_void_p),
        ("page_off", ctypes.c_void_p),
        ("rcode", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_bits", ctypes.c_void_p),
        ("head_tiers", ctypes.c_int),
        ("query_precision", ctypes.c_int),
        ("max_batch", ctypes.c_int),
        ("max_heads_q", ctypes.c_int),
        ("max_pages", ctypes.c_int),
        ("max_splits", ctypes.c_int),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libska.so is not built (python -m long_context_decode_ada_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, i, i64, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.ska_encode_keys.restype = i
        L.ska_encode_keys.argtypes = [ctypes.POINTER(P), ctypes.POINTER(PoolDesc), P, P, P, i64, P, P]
        L.ska_decode_attention.restype = i
        L.ska_decode_attention.argtypes = [P, P, i, i, P, i, P, f, i, P, P, P]
        L.ska_decode_attention_noalloc.restype = i
        L.ska_decode_attention_noalloc.argtypes = [P, P, i, i, P, i, P, f, i, P, P]
        L.ska_append_decode_attention.restype = i
        L.ska_append_decode_attention.argtypes = [P, P, P, P, i, i, P, i, P, f, i, P, P, P]
        L.ska_dense_decode_attention.restype = i
        L.ska_dense_decode_attention.argtypes = [P, P, P, i, i, P, i, P, f, i, P, P, P]
        L.ska_decompress_keys.restype = i
        L.ska_decompress_keys.argtypes = [P, P, i, i, P, P, P]
        L.ska_rdr_plan.restype = i
        L.ska_rdr_plan.argtypes = [ctypes.POINTER(RdrParams), P, P, P, P, P, i, i, P, P, P, P, i, P, P, P, P]
        L.ska_get_radius_range.restype = i
        L.ska_get_radius_range.argtypes = [P, P]
        L.ska_device_errors.restype = i
        L.ska_device_errors.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
        L.ska_profile_begin.restype = i
        L.ska_profile_begin.argtypes = [P, i]
        L.ska_profile_read.restype = i
        L.ska_profile_read.argtypes = [P, P, i, ctypes.POINTER(ctypes.c_int)]
        L.ska_free.restype = None
        L.ska_free.argtypes = [P]
        L.ska_status_string.restype = ctypes.c_char_p
        L.ska_status_string.argtypes = [i]
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().ska_status_string(int(s)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_BF16_BITS = (torch.int16, torch.uint16, torch.bfloat16) if hasattr(torch, "uint16") else (torch.int16, torch.bfloat16)


def _dev(name: str, t: Optional[torch.Tensor], dtypes, shape=None, optional: bool = False):
    """The C ABI takes raw device pointers, so a tensor of the wrong dtype,
    device, layout or shape would be read as garbage: refuse it here."""
    if t is None:
        if optional:
            return
        raise ValueError("%s: a tensor is required" % name)
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if not t.is_cuda:
        raise ValueError("%s: must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, " or ".join(str(d) for d in dtypes)))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(s: int, what: str):
    if s != SKA_OK:
        raise SkaError(s, what)


class DevicePools:
    """Caller-owned device pools in the library's layout (torch tensors), with
    the maxima of the decode calls the cache built on them will serve (they
    size its workspace, allocated once when the cache is created)."""

    def __init__(self, *, d: int, hkv: int, num_pages: int, tier_mask: int, radius_mode: int,
                 page_bits: torch.Tensor, kcode_bytes: int, page_off: Optional[torch.Tensor] = None,
                 query_mode: int = Q_CODED, device="cuda", poison: bool = True, head_tiers: bool = False,
                 query_precision: int = QDIR_F16, max_batch: int = 1, max_heads_q: int = 0, max_pages: int = 1,
                 max_splits: int = 0):
        self.d, self.hkv, self.num_pages = d, hkv, num_pages
        self.head_tiers = bool(head_tiers)
        self.tier_mask, self.radius_mode, self.query_mode = tier_mask, radius_mode, query_mode
        self.query_precision = query_precision
        self.max_batch, self.max_pages, self.max_splits = max_batch, max_pages, max_splits
        self.max_heads_q = max_heads_q or 4 * hkv
        self.page_bits = page_bits.to(device=device, dtype=torch.uint8).contiguous()
        self.page_off = None if page_off is None else page_off.to(device=device, dtype=torch.int64).contiguous()
        fill = 0xFF if poison else 0
        self.kcode = torch.full((kcode_bytes,), fill, dtype=torch.uint8, device=device)
        self.rcode = torch.full((num_pages * hkv * PAGE,), fill, dtype=torch.uint8, device=device)
        # bf16 NaN poison (0x7FC0) or zero, stored as raw 16-bit patterns
        self.v = torch.full((num_pages * hkv * d * PAGE,), 0x7FC0 if poison else 0, dtype=torch.int16, device=device)

    @classmethod
    def for_workload(cls, w, device="cuda", poison=True, query_mode=Q_CODED, query_precision=QDIR_F16,
                     max_batch=None, max_heads_q=None, max_pages=None, max_splits=64):
        """Pools for workload w; decode calls up to w's batch, query heads
        and block-table width (or the given maxima), and explicit split
        counts up to max_splits."""
        off = None if w.page_off is None else torch.from_numpy(w.page_off.view(np.int64))
        return cls(d=w.d, hkv=w.hkv, num_pages=w.num_pages, tier_mask=w.tier_mask, radius_mode=w.radius_mode,
                   page_bits=torch.from_numpy(w.page_bits), kcode_bytes=w.kcode_bytes, page_off=off,
                   query_mode=query_mode, device=device, poison=poison, head_tiers=w.head_tiers,
                   query_precision=query_precision, max_batch=max_batch or w.B, max_heads_q=max_heads_q or w.hq,
                   max_pages=max_pages or w.max_pages, max_splits=max_splits)

    def desc(self) -> PoolDesc:
        return PoolDesc(self.d, self.hkv, PAGE, self.num_pages, self.radius_mode, 8, self.tier_mask,
                        self.query_mode, self.kcode.data_ptr(),
                        None if self.page_off is None else self.page_off.data_ptr(),
                        self.rcode.data_ptr(), self.v.data_ptr(), self.page_bits.data_ptr(),
                        int(self.head_tiers), int(self.query_precision), int(self.max_batch),
                        int(self.max_heads_q), int(self.max_pages), int(self.max_splits))

    def to_host(self) -> dict:
        return {"kcode": self.kcode.cpu().numpy(), "rcode": self.rcode.cpu().numpy(),
                "v": self.v.cpu().numpy().view(np.uint16)}


class Cache:
    """Owns one ska_cache handle (freed with ska_free)."""

    def __init__(self, pools: DevicePools):
        self.pools = pools
        self.handle = ctypes.c_void_p(None)

    def free(self):
        if self.handle.value:
            lib().ska_free(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def encode_keys(cache: Cache, keys: torch.Tensor, values: Optional[torch.Tensor], slot: torch.Tensor,
                radius_range: Optional[np.ndarray] = None, stream=None) -> Cache:
    """ska_encode_keys: keys fp32 [n][hkv][d], values bf16 bits (int16/uint16/bf16) [n][hkv][d] or
    None, slot int64 [n], radius_range host [hkv][2] or None."""
    n = int(keys.shape[0]) if keys is not None else 0
    P = cache.pools
    if n > 0:
        _dev("keys", keys, torch.float32, (n, P.hkv, P.d))
        _dev("values", values, _BF16_BITS, (n, P.hkv, P.d), optional=True)
        _dev("slot", slot, torch.int64, (n,))
    desc = cache.pools.desc()
    rr = None
    if radius_range is not None:
        rr = np.ascontiguousarray(radius_range, np.float64)
    s = lib().ska_encode_keys(ctypes.byref(cache.handle), ctypes.byref(desc), _ptr(keys), _ptr(values),
                              _ptr(slot), n, None if rr is None else rr.ctypes.data_as(ctypes.c_void_p),
                              _stream(stream))
    _check(s, "ska_encode_keys")
    return cache


def _decode_checks(cache, q, block_table, seq_lens, out, logits):
    P = cache.pools
    if q.dim() != 3 or q.shape[2] != P.d:
        raise ValueError("q: shape %s, expected [B][Hq][%d]" % (tuple(q.shape), P.d))
    B, hq, d = q.shape
    _dev("q", q, torch.float32)
    _dev("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table: shape %s, expected [%d][max_pages]" % (tuple(block_table.shape), B))
    _dev("seq_lens", seq_lens, torch.int32, (B,))
    _dev("out", out, torch.float32, (B, hq, d), optional=True)
    _dev("logits", logits, torch.float32, (B, hq, block_table.shape[1] * PAGE), optional=True)


def decode_attention(cache: Cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                     scale: float = 0.0, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                     logits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ska_decode_attention: q fp32 [B][hq][d], block_table int32 [B][max_pages], seq_lens int32 [B];
    returns out fp32 [B][hq][d].  logits (fp32 [B][hq][max_pages*16]) is filled if given."""
    B, hq, d = q.shape
    _decode_checks(cache, q, block_table, seq_lens, out, logits)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    s = lib().ska_decode_attention(cache.handle, _ptr(q), B, hq, _ptr(block_table), int(block_table.shape[1]),
                                   _ptr(seq_lens), float(scale), int(num_splits), _ptr(out), _ptr(logits),
                                   _stream(stream))
    _check(s, "ska_decode_attention")
    return out


def prepared_decode(cache: Cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                    out: torch.Tensor, scale: float = 0.0, num_splits: int = 0, stream=None,
                    k_dense: Optional[torch.Tensor] = None):
    """decode_attention (or, given k_dense, dense_decode_attention) with its
    arguments checked and marshalled once: returns a callable that enqueues
    the same call each time it is called, for a decode loop over fixed
    buffers (it holds references to the tensors)."""
    B, hq, d = q.shape
    _decode_checks(cache, q, block_table, seq_lens, out, None)
    tail = (B, hq, _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), float(scale), int(num_splits),
            _ptr(out), None, _stream(stream))
    if k_dense is None:
        name, fn, args = "ska_decode_attention", lib().ska_decode_attention, (cache.handle, _ptr(q)) + tail
    else:
        P = cache.pools
        _dev("k_dense", k_dense, _BF16_BITS, (P.num_pages, P.hkv, PAGE, P.d))
        name, fn = "ska_dense_decode_attention", lib().ska_dense_decode_attention
        args = (cache.handle, _ptr(k_dense), _ptr(q)) + tail
    keep = (cache, q, block_table, seq_lens, out, k_dense)

    def call():
        s = fn(*args)
        if s != SKA_OK:
            raise SkaError(s, name)
        return keep[4]
    return call


def decode_attention_noalloc(cache: Cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                             scale: float = 0.0, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """ska_decode_attention_noalloc: decode_attention with the split workspace in the library's static
    device array (nothing allocated by the library; `out` must be given by a caller that cannot allocate)."""
    B, hq, d = q.shape
    _decode_checks(cache, q, block_table, seq_lens, out, None)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    s = lib().ska_decode_attention_noalloc(cache.handle, _ptr(q), B, hq, _ptr(block_table),
                                           int(block_table.shape[1]), _ptr(seq_lens), float(scale), int(num_splits),
                                           _ptr(out), _stream(stream))
    _check(s, "ska_decode_attention_noalloc")
    return out


def append_decode_attention(cache: Cache, new_keys: torch.Tensor, new_values: torch.Tensor, q: torch.Tensor,
                            block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float = 0.0,
                            num_splits: int = 0, out: Optional[torch.Tensor] = None,
                            logits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ska_append_decode_attention: new_keys fp32 [B][hkv][d] and new_values bf16 bits [B][hkv][d] (int16
    view) are stored at position seq_lens[s]-1 of each sequence (seq_lens include them), then the decode
    as decode_attention."""
    B, hq, d = q.shape
    _decode_checks(cache, q, block_table, seq_lens, out, logits)
    _dev("new_keys", new_keys, torch.float32, (B, cache.pools.hkv, cache.pools.d))
    _dev("new_values", new_values, _BF16_BITS, (B, cache.pools.hkv, cache.pools.d))
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    s = lib().ska_append_decode_attention(cache.handle, _ptr(new_keys), _ptr(new_values), _ptr(q), B, hq,
                                          _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                          float(scale), int(num_splits), _ptr(out), _ptr(logits), _stream(stream))
    _check(s, "ska_append_decode_attention")
    return out


def dense_decode_attention(cache: Cache, k_dense: torch.Tensor, q: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, scale: float = 0.0, num_splits: int = 0,
                           out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """ska_dense_decode_attention: keys bf16 bits k_dense [num_pages][hkv][16][d] (int16/uint16 view),
    the cache's values; otherwise as decode_attention."""
    B, hq, d = q.shape
    _decode_checks(cache, q, block_table, seq_lens, out, logits)
    P = cache.pools
    _dev("k_dense", k_dense, _BF16_BITS, (P.num_pages, P.hkv, PAGE, P.d))
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    s = lib().ska_dense_decode_attention(cache.handle, _ptr(k_dense), _ptr(q), B, hq, _ptr(block_table),
                                         int(block_table.shape[1]), _ptr(seq_lens), float(scale), int(num_splits),
                                         _ptr(out), _ptr(logits), _stream(stream))
    _check(s, "ska_dense_decode_attention")
    return out


def decompress_keys(cache: Cache, block_table: torch.Tensor, seq_lens: torch.Tensor, k_dense: torch.Tensor,
                    stream=None) -> torch.Tensor:
    """ska_decompress_keys: writes bf16 r~ u(c) of the resident pages into k_dense [num_pages][hkv][16][d]."""
    P = cache.pools
    B = int(block_table.shape[0])
    _dev("block_table", block_table, torch.int32)
    _dev("seq_lens", seq_lens, torch.int32, (B,))
    _dev("k_dense", k_dense, _BF16_BITS, (P.num_pages, P.hkv, PAGE, P.d))
    s = lib().ska_decompress_keys(cache.handle, _ptr(block_table), int(block_table.shape[0]),
                                  int(block_table.shape[1]), _ptr(seq_lens), _ptr(k_dense), _stream(stream))
    _check(s, "ska_decompress_keys")
    return k_dense


class RdrParams(ctypes.Structure):
    _fields_ = [("ntiers", ctypes.c_int), ("tiers", ctypes.c_int * 8), ("eps", ctypes.c_double * 8),
                ("bytes", ctypes.c_int64 * 8), ("sigma", ctypes.c_double)]


def rdr_plan(utility: torch.Tensor, key_norm: torch.Tensor, protect: torch.Tensor, num_states: torch.Tensor,
             budget: torch.Tensor, tiers, eps, bytes_per_tier, sigma: float, stream=None) -> dict:
    """ska_rdr_plan on device tensors utility/key_norm fp32 [B][T], protect uint8 [B][T], num_states int32 [B],
    budget int64 [B].  Returns dict of device tensors tier (uint8), page, slot (int32) [B][T],
    page_tier (uint8) [B][P], npages (int32), lambda (float64), status (int32) [B]."""
    B, T = utility.shape
    _dev("utility", utility, torch.float32, (B, T))
    _dev("key_norm", key_norm, torch.float32, (B, T))
    _dev("protect", protect, torch.uint8, (B, T))
    _dev("num_states", num_states, torch.int32, (B,))
    _dev("budget", budget, torch.int64, (B,))
    p = RdrParams()
    p.ntiers = len(tiers)
    for k in range(len(tiers)):
        p.tiers[k], p.eps[k], p.bytes[k] = int(tiers[k]), float(eps[k]), int(bytes_per_tier[k])
    p.sigma = float(sigma)
    dev = utility.device
    P_out = (T + 15) // 16 + len(tiers)
    o = {"tier": torch.zeros((B, T), dtype=torch.uint8, device=dev),
         "page": torch.zeros((B, T), dtype=torch.int32, device=dev),
         "slot": torch.zeros((B, T), dtype=torch.int32, device=dev),
         "page_tier": torch.zeros((B, P_out), dtype=torch.uint8, device=dev),
         "npages": torch.zeros(B, dtype=torch.int32, device=dev),
         "lambda": torch.zeros(B, dtype=torch.float64, device=dev),
         "status": torch.zeros(B, dtype=torch.int32, device=dev)}
    s = lib().ska_rdr_plan(ctypes.byref(p), _ptr(utility), _ptr(key_norm), _ptr(protect), _ptr(num_states),
                           _ptr(budget), B, T, _ptr(o["tier"]), _ptr(o["page"]), _ptr(o["slot"]),
                           _ptr(o["page_tier"]), P_out, _ptr(o["npages"]), _ptr(o["lambda"]), _ptr(o["status"]),
                           _stream(stream))
    _check(s, "ska_rdr_plan")
    return o


def radius_range(cache: Cache) -> np.ndarray:
    r = np.zeros((cache.pools.hkv, 2), np.float64)
    _check(lib().ska_get_radius_range(cache.handle, r.ctypes.data_as(ctypes.c_void_p)), "ska_get_radius_range")
    return r


def device_errors(cache: Cache, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().ska_device_errors(cache.handle, _stream(stream), ctypes.byref(v)), "ska_device_errors")
    return int(v.value)


def profile_begin(cache: Cache, max_calls: int):
    _check(lib().ska_profile_begin(cache.handle, int(max_calls)), "ska_profile_begin")


def profile_read(cache: Cache, max_calls: int) -> np.ndarray:
    """[calls] decode-kernel milliseconds (query prep, paged decode, split merge)."""
    ms = np.zeros(max(1, max_calls), np.float32)
    n = ctypes.c_int(0)
    _check(lib().ska_profile_read(cache.handle, ms.ctypes.data_as(ctypes.c_void_p), int(max_calls),
                                  ctypes.byref(n)), "ska_profile_read")
    return ms[: n.value]


def free(cache: Cache):
    cache.free()
