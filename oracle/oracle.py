"""ctypes wrapper around the plain fp64 CPU oracle (``ska_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg.  The product path never imports this module,
and this module imports nothing from the product package.

Method source: the technical summary in the page "SPHERICAL KV: Angle-Domain
Attention and Rate-Distortion Retention for Efficient Long-Context Inference"
(gist.science, arXiv 2605.18856), section 2.1 (ADA: spherical parametrisation,
quantised radius, packed angle codes, logit estimator computed from codes) and
sections 2.2-2.3 (tier-homogeneous pages in a paged store).  Each function of
the C file names the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ska_oracle.c")
LIB = os.path.join(HERE, "libska_oracle.so")

UNIFORM, LOG = 0, 1
Q_CODED, Q_EXACT = 0, 1
PAGE = 16

CFLAGS = ["-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-builtin",
          "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, fp64, no contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i, d, i64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
        L.ora_polar_code.restype = i
        L.ora_polar_code.argtypes = [d, d, i]
        L.ora_azimuth_code.restype = i
        L.ora_azimuth_code.argtypes = [d, d, i]
        L.ora_angle_thresholds.argtypes = [i, P, P]
        L.ora_angles.argtypes = [P, i, P, P]
        L.ora_unit_from_angles.argtypes = [P, i, P]
        L.ora_key_codes.restype = d
        L.ora_key_codes.argtypes = [P, i, i, P]
        L.ora_direction.argtypes = [P, i, i, P]
        L.ora_radius_tables.argtypes = [i, d, d, P, P]
        L.ora_radius_code.restype = i
        L.ora_radius_code.argtypes = [d, P]
        L.ora_calibrate.argtypes = [P, i64, i, i, P]
        L.ora_kb.restype = i
        L.ora_kb.argtypes = [i, i]
        L.ora_pack.restype = i
        L.ora_pack.argtypes = [P, i, i, P]
        L.ora_unpack.argtypes = [P, i, i, P]
        L.ora_encode.restype = i
        L.ora_encode.argtypes = [i, i, i, P, P, P, i, i, P, P, P, P, P, P, i64]
        L.ora_decode.restype = i
        L.ora_decode.argtypes = [i, i, i, P, P, P, i, i, P, P, P, P, i, i, P, i, P, d, i,
                                 P, P, P, i, i]
        L.ora_decoded_keys.restype = i
        L.ora_decoded_keys.argtypes = [i, i, i, P, P, P, i, i, P, P, P, i, P]
        L.ora_dense_decode.restype = i
        L.ora_dense_decode.argtypes = [i, i, P, P, P, i, i, P, i, P, d, P, P, i]
        L.ora_rdr_plan.restype = i
        L.ora_rdr_plan.argtypes = [i, P, P, P, i, P, P, P, i64, d, P, P, P, P, P, P]
        L.ora_max_threads.restype = i
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# --- scalar / vector pieces (closed-form pins use these) --------------------

def polar_code(x: float, S: float, b: int) -> int:
    return lib().ora_polar_code(float(x), float(S), int(b))


def azimuth_code(x: float, y: float, b: int) -> int:
    return lib().ora_azimuth_code(float(x), float(y), int(b))


def angle_thresholds(b: int):
    n = 1 << b
    c2 = np.zeros(n, np.float64)
    s2 = np.zeros(n, np.float64)
    lib().ora_angle_thresholds(b, _p(c2), _p(s2))
    return c2, s2


def angles(x):
    x = _c(x, np.float32)
    d = x.shape[-1]
    phi = np.zeros(d - 1, np.float64)
    T0 = np.zeros(1, np.float64)
    lib().ora_angles(_p(x), d, _p(phi), _p(T0))
    return phi, float(T0[0])


def unit_from_angles(phi, d: int):
    phi = _c(phi, np.float64)
    u = np.zeros(d, np.float64)
    lib().ora_unit_from_angles(_p(phi), d, _p(u))
    return u


def key_codes(x, b: int):
    """Angle codes (d-1 ints) and |x|^2 of one fp32 vector."""
    x = _c(x, np.float32)
    d = x.shape[-1]
    codes = np.zeros(d - 1, np.int32)
    T0 = lib().ora_key_codes(_p(x), d, b, _p(codes))
    return codes, T0


def direction(codes, d: int, b: int):
    codes = _c(codes, np.int32)
    u = np.zeros(d, np.float64)
    lib().ora_direction(_p(codes), d, b, _p(u))
    return u


def radius_tables(mode: int, rlo: float, rhi: float):
    level = np.zeros(256, np.float64)
    tau2 = np.zeros(255, np.float64)
    lib().ora_radius_tables(mode, float(rlo), float(rhi), _p(level), _p(tau2))
    return level, tau2


def radius_code(S: float, tau2) -> int:
    tau2 = _c(tau2, np.float64)
    return lib().ora_radius_code(float(S), _p(tau2))


def calibrate(keys):
    """keys [n][hkv][d] fp32 -> range [hkv][2] = (R_lo, R_hi)."""
    keys = _c(keys, np.float32)
    n, hkv, d = keys.shape
    rng = np.zeros((hkv, 2), np.float64)
    lib().ora_calibrate(_p(keys), n, hkv, d, _p(rng))
    return rng


def kb(d: int, b: int) -> int:
    return lib().ora_kb(d, b)


def pack(codes, d: int, b: int):
    codes = _c(codes, np.int32)
    rec = np.zeros(kb(d, b), np.uint8)
    if lib().ora_pack(_p(codes), d, b, _p(rec)):
        raise ValueError("layout does not fit")
    return rec


def unpack(rec, d: int, b: int):
    rec = _c(rec, np.uint8)
    codes = np.zeros(d - 1, np.int32)
    lib().ora_unpack(_p(rec), d, b, _p(codes))
    return codes


# --- pools ------------------------------------------------------------------

def encode(pools: dict, keys, values, slot, radius_mode: int, rng) -> None:
    """Encode keys [n][hkv][d] (and values) into host pools in place.

    pools: dict with d, hkv, page_bits (u8[num_pages]), page_off (u64 or None),
    bstride (int), kcode (u8), rcode (u8[num_pages*hkv*16]), v (u16), and
    optionally head_tiers (true: page_bits and page_off are per (page, KV
    head), [num_pages*hkv], the offset of that head's 16 records)."""
    keys = _c(keys, np.float32)
    values = _c(values, np.uint16)
    slot = _c(slot, np.int64)
    rng = _c(rng, np.float64)
    n = keys.shape[0]
    r = lib().ora_encode(pools["d"], pools["hkv"], radius_mode, _p(rng),
                         _p(pools["page_bits"]), _p(pools.get("page_off")), pools["bstride"],
                         int(bool(pools.get("head_tiers", False))),
                         _p(pools["kcode"]), _p(pools["rcode"]), _p(pools["v"]),
                         _p(keys), _p(values), _p(slot), n)
    if r:
        raise ValueError("ora_encode: bad argument")


def decode(pools: dict, radius_mode: int, rng, q, block_table, seq_lens, scale: float = 0.0,
           query_mode: int = Q_CODED, pairs=None, want_logits: bool = False, nthreads: int = 0):
    """ADA decode by the plain definition.  Returns out [B][hq][d] (fp32) and,
    if asked, logits [B][hq][max_pages*16] (fp32, natural units, NaN where not
    computed)."""
    q = _c(q, np.float32)
    B, hq, d = q.shape
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    rng = _c(rng, np.float64)
    max_pages = block_table.shape[1]
    out = np.full((B, hq, d), np.nan, np.float32)
    logits = np.full((B, hq, max_pages * PAGE), np.nan, np.float32) if want_logits else None
    pr = None if pairs is None else np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
    npairs = 0 if pr is None else pr.shape[0]
    r = lib().ora_decode(pools["d"], pools["hkv"], radius_mode, _p(rng),
                         _p(pools["page_bits"]), _p(pools.get("page_off")), pools["bstride"],
                         int(bool(pools.get("head_tiers", False))),
                         _p(pools["kcode"]), _p(pools["rcode"]), _p(pools["v"]),
                         _p(q), B, hq, _p(block_table), max_pages, _p(seq_lens), float(scale),
                         query_mode, _p(out), _p(logits), _p(pr), npairs, int(nthreads))
    if r:
        raise ValueError("ora_decode: bad argument")
    return (out, logits) if want_logits else out


def decoded_keys(pools: dict, radius_mode: int, rng, phys):
    """The dense keys k~ = r~ * u(codes) the stored records stand for, for the
    physical pages `phys`: [len(phys)][hkv][16][d] binary64."""
    phys = _c(phys, np.int32)
    rng = _c(rng, np.float64)
    d, hkv = pools["d"], pools["hkv"]
    out = np.zeros((phys.shape[0], hkv, PAGE, d), np.float64)
    r = lib().ora_decoded_keys(d, hkv, radius_mode, _p(rng), _p(pools["page_bits"]), _p(pools.get("page_off")),
                               pools["bstride"], int(bool(pools.get("head_tiers", False))),
                               _p(pools["kcode"]), _p(pools["rcode"]), _p(phys),
                               phys.shape[0], _p(out))
    if r:
        raise ValueError("ora_decoded_keys: bad page header")
    return out


def dense_decode(k_dense, v, q, block_table, seq_lens, scale: float = 0.0, want_logits: bool = False,
                 nthreads: int = 0):
    """Dense paged attention by the plain definition: keys bf16 bits
    k_dense [num_pages][hkv][16][d], values v bf16 bits [num_pages][hkv][d][16].
    Returns out [B][hq][d] (fp32) and, if asked, logits (natural units)."""
    k_dense = _c(k_dense, np.uint16)
    v = _c(v, np.uint16)
    q = _c(q, np.float32)
    B, hq, d = q.shape
    hkv = k_dense.shape[1]
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    max_pages = block_table.shape[1]
    out = np.full((B, hq, d), np.nan, np.float32)
    logits = np.full((B, hq, max_pages * PAGE), np.nan, np.float32) if want_logits else None
    r = lib().ora_dense_decode(d, hkv, _p(k_dense), _p(v), _p(q), B, hq, _p(block_table), max_pages,
                               _p(seq_lens), float(scale), _p(out), _p(logits), int(nthreads))
    if r:
        raise ValueError("ora_dense_decode: bad argument")
    return (out, logits) if want_logits else out


def rdr_plan(u, knorm, prot, tiers, eps, bytes_per_tier, budget: int, sigma: float):
    """Rate-distortion retention plan for one sequence (see ora_rdr_plan).
    Returns dict: tier [n] (0 = evicted), page [n], slot [n] (-1 evicted),
    page_tier [npages], lambda, status (0 ok, 2 protected states over budget)."""
    u = _c(u, np.float32)
    knorm = _c(knorm, np.float32)
    prot = _c(prot, np.uint8)
    n = u.shape[0]
    tiers = _c(tiers, np.int32)
    eps = _c(eps, np.float64)
    bpt = _c(bytes_per_tier, np.int64)
    tier = np.zeros(n, np.uint8)
    page = np.zeros(n, np.int32)
    slot = np.zeros(n, np.int32)
    pt = np.zeros(max(1, (n + PAGE - 1) // PAGE + len(tiers)), np.uint8)
    npg = ctypes.c_int(0)
    lam = ctypes.c_double(0.0)
    r = lib().ora_rdr_plan(n, _p(u), _p(knorm), _p(prot), len(tiers), _p(tiers), _p(eps), _p(bpt), int(budget),
                           float(sigma), _p(tier), _p(page), _p(slot), _p(pt), ctypes.byref(npg), ctypes.byref(lam))
    if r == 1:
        raise ValueError("ora_rdr_plan: bad argument")
    return {"tier": tier, "page": page, "slot": slot, "page_tier": pt[: npg.value], "lambda": lam.value, "status": r}


def max_threads() -> int:
    return lib().ora_max_threads()
