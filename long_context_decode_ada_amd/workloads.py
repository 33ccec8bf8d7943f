"""Seeded synthetic decode workloads (inputs only).

This module builds the inputs that both the HIP path and the CPU oracle
consume: keys, values, queries, sequence lengths, block tables, page tiers and
page offsets.  It holds none of the method's arithmetic (no angles, no
quantisers, no attention); it only draws random numbers and lays out pages.

Shapes and distributions follow the workloads of the page "SPHERICAL KV:
Angle-Domain Attention and Rate-Distortion Retention for Efficient
Long-Context Inference" (section 4: Llama-3.1-8B-class models, contexts of
8K/32K/128K on a paged, ragged serving substrate, section 2.3).  The models
and datasets of that section are not used: seeded synthetic tensors of the
same shapes stand in for them.

Workloads (sizes at scale 1):
  tiny        B=1, 1/1 heads, d=64, T=256 (16 pages), b=4, uniform radius,
              identity block table, keys/query/values N(0,1)
  gqa_t32k    B=8, 32/8 heads, d=128, T=32768, b=4, log radius, keys
              N(0, diag(s^2)) with s ~ LogNormal(0, 0.5) per (kv head, dim),
              RoPE (theta 5e5) at positions 0..T-1, query N(0,1) with RoPE at
              T, values bf16 N(0,1), physical pages shuffled
  long_t128k  B=1, 32/8, d=128, T=131072, b=3, log radius, as gqa_t32k
  ragged_b64  B=64, 32/8, d=128, lengths floor(LogNormal(ln 8192, 1))
              clipped to [512, 65536], b=4, log radius, shared pool of
              ceil(1.25 * pages) physical pages assigned at random
  mixed_tiers gqa_t32k shapes; logical page 0 (the 4 sink tokens and the
              rest of their page) at b=8; every other page draws b from
              {2,4,6,8} with p={.3,.4,.2,.1}; 1023 of the 2047 non-sink pages
              per sequence are evicted (absent from the block table);
              variable-size pages addressed through page_off

Seeding: one root seed; each workload and role (lengths, pages, tiers,
eviction, channel scales, query) has its own child stream, and keys and
values are drawn in fixed chunks of 8192 tokens, each chunk from its own
seed sequence, so a workload's bytes are the same whatever thread count
draws them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED = 20260609
PAGE = 16
UNIFORM, LOG = 0, 1
ROPE_THETA = 500000.0

NAMES = ("tiny", "gqa_t32k", "long_t128k", "ragged_b64", "mixed_tiers")


def record_bytes(d: int, b: int) -> int:
    """Bytes of one key record in the pool layout (16-byte multiple)."""
    return 16 * (((d - 1) * b + 127) // 128)


@dataclasses.dataclass
class Workload:
    name: str
    d: int
    hq: int
    hkv: int
    B: int
    radius_mode: int
    tier_mask: int
    seq_lens: np.ndarray            # int32 [B] resident tokens
    block_table: np.ndarray         # int32 [B][max_pages]
    num_pages: int
    page_bits: np.ndarray           # uint8 [num_pages] ([num_pages*hkv] with head_tiers): tier in the low
                                    # four bits, empty slots at the page's end in the high four
    page_off: Optional[np.ndarray]  # uint64 [num_pages] ([num_pages*hkv] with head_tiers) or None
    bstride: int                    # tier used for the fixed page stride when page_off is None
    kcode_bytes: int
    keys: np.ndarray                # float32 [n][hkv][d]
    values: np.ndarray              # uint16 (bf16 bits) [n][hkv][d]
    slot: np.ndarray                # int64 [n] = phys*16 + token-in-page
    q: np.ndarray                   # float32 [B][hq][d]
    scale: float = 0.0              # 0 => 1/sqrt(d)
    seed: int = SEED
    head_tiers: bool = False        # tiers per (page, KV head): header and offset of each head's records

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def n_tokens(self) -> int:
        """Resident tokens: positions below each row's length, less the empty
        slots page headers declare."""
        if not np.any(np.asarray(self.page_bits) >> 4):
            return int(self.seq_lens.astype(np.int64).sum())
        tot = 0
        for s in range(self.B):
            n = int(self.seq_lens[s])
            for p in range((n + PAGE - 1) // PAGE):
                phys = int(self.block_table[s, p])
                hdr = int(self.page_bits[phys * self.hkv] if self.head_tiers else self.page_bits[phys])
                tot += min(PAGE - (hdr >> 4), n - p * PAGE)
        return tot

    def bytes_per_step(self) -> int:
        """Algorithmic HBM bytes of one decode step: per resident (token, kv
        head) one record, one radius byte and d bf16 values; per resident
        (page, kv head) one block-table entry and one page header byte
        (plus 8 offset bytes when page_off is used); the query and output."""
        tot = 0
        for s in range(self.B):
            n = int(self.seq_lens[s])
            npg = (n + PAGE - 1) // PAGE
            for p in range(npg):
                phys = int(self.block_table[s, p])
                for g in range(self.hkv):
                    # the header: tier in the low four bits, empty slots in the high four
                    hdr = int(self.page_bits[phys * self.hkv + g] if self.head_tiers else self.page_bits[phys])
                    ntok = min(PAGE - (hdr >> 4), n - p * PAGE)
                    tot += ntok * (record_bytes(self.d, hdr & 15) + 1 + 2 * self.d)
                tot += self.hkv * (4 + 1 + (8 if self.page_off is not None else 0))
        tot += self.B * self.hq * self.d * 4 * 2
        return tot


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _rope(x: np.ndarray, pos: np.ndarray, d: int) -> np.ndarray:
    """Rotate-half RoPE of x [..., n, h, d] at positions pos [n]."""
    half = d // 2
    inv = ROPE_THETA ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    c = np.cos(ang).astype(np.float32)[:, None, :]
    s = np.sin(ang).astype(np.float32)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = x1 * c - x2 * s
    out[..., half:] = x2 * c + x1 * s
    return out


CHUNK = 8192          # tokens per key/value random chunk


def _fill_chunks(idx, n_tok, hkv, d, chan, pos_all, keys, values):
    """Keys and values in fixed chunks of CHUNK tokens, chunk c drawn from
    its own generator (seed sequence (SEED, workload, role, c)), so the
    bytes do not depend on how many threads draw them."""
    def one(c):
        a, b = c * CHUNK, min((c + 1) * CHUNK, n_tok)
        gk = np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=(idx, 100, c)))
        gv = np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=(idx, 101, c)))
        z = gk.standard_normal((b - a, hkv, d), dtype=np.float32)
        keys[a:b] = z if chan is None else _rope(z * chan[None], pos_all[a:b], d)
        values[a:b] = _bf16_bits(gv.standard_normal((b - a, hkv, d), dtype=np.float32))
    nch = (n_tok + CHUNK - 1) // CHUNK
    if nch <= 1:
        for c in range(nch):
            one(c)
        return
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(8, nch)) as ex:
        list(ex.map(one, range(nch)))


def _streams(idx: int, n: int = 10):
    ss = np.random.SeedSequence(SEED).spawn(len(NAMES))[idx]
    return [np.random.default_rng(c) for c in ss.spawn(n)]


def make(name: str, scale: float = 1.0, batch: Optional[int] = None, data: bool = True,
         tiers: Optional[tuple] = None, head_tiers: bool = False, outliers: int = 0) -> Workload:
    """Build one workload.  ``scale`` < 1 shrinks the context (and, for
    ragged_b64, the lengths) for oracle-sized tests; ``batch`` overrides B;
    ``data=False`` builds the page structure only (empty keys/values/query);
    ``tiers`` (mixed_tiers only) replaces the tier set {2,4,6,8} by the given
    widths, drawn with equal probability (the sink page takes the widest);
    ``head_tiers`` (mixed_tiers only) draws the tier per (page, KV head)
    instead of per page (the sink page's heads all take the widest), with a
    header and a record offset per (page, KV head); ``outliers`` (the
    LogNormal-scaled workloads only) multiplies the channel scale of that
    many channels per KV head, chosen at random, by a factor drawn uniformly
    from [20, 50] (keys with a few outlier channels, a wide range of norms).
    Every part draws from its own seeded stream, so the structure does not
    depend on ``data``."""
    if name not in NAMES:
        raise KeyError(name)
    if tiers is not None and name != "mixed_tiers":
        raise ValueError("tiers applies to mixed_tiers only")
    if head_tiers and name != "mixed_tiers":
        raise ValueError("head_tiers applies to mixed_tiers only")
    if outliers and name == "tiny":
        raise ValueError("outliers applies to the LogNormal-scaled workloads only")
    tiers_override = tiers
    idx = NAMES.index(name)
    r_keys, r_vals, r_q, r_len, r_pages, r_tier, r_evict, r_scale, r_out, _ = _streams(idx)

    if name == "tiny":
        d, hq, hkv, B, T = 64, 1, 1, 1, 256
        B = batch or B
        T = max(PAGE, int(T * scale))
        lens = np.full(B, T, np.int32)
        mode, tiers = UNIFORM, {4}
    elif name in ("gqa_t32k", "long_t128k", "mixed_tiers"):
        d, hq, hkv = 128, 32, 8
        B = {"gqa_t32k": 8, "long_t128k": 1, "mixed_tiers": 8}[name]
        T = {"gqa_t32k": 32768, "long_t128k": 131072, "mixed_tiers": 32768}[name]
        B = batch or B
        T = max(2 * PAGE, int(T * scale))
        lens = np.full(B, T, np.int32)
        mode = LOG
        tiers = {"gqa_t32k": {4}, "long_t128k": {3}, "mixed_tiers": {2, 4, 6, 8}}[name]
        if tiers_override is not None:
            tiers = set(tiers_override)
    else:  # ragged_b64
        d, hq, hkv, B = 128, 32, 8, 64
        B = batch or B
        raw = np.floor(r_len.lognormal(np.log(8192.0), 1.0, size=B))
        lens = np.clip(raw, 512, 65536)
        lens = np.maximum(np.floor(lens * scale), 1).astype(np.int32)
        mode, tiers = LOG, {4}

    # ---- logical pages, tiers, eviction (positions of resident tokens) ----
    pos_list, tier_list = [], []
    for s in range(B):
        if name == "mixed_tiers":
            T = int(lens[s])
            npg = (T + PAGE - 1) // PAGE
            shape = (npg, hkv) if head_tiers else npg
            if tiers_override is None:
                tier = r_tier.choice(np.array([2, 4, 6, 8]), size=shape, p=[0.3, 0.4, 0.2, 0.1])
            else:
                tier = r_tier.choice(np.array(sorted(tiers)), size=shape)
            tier[0] = max(tiers)                          # sink page: protected, b_max
            nonsink = np.arange(1, npg)
            evict = r_evict.choice(nonsink, size=len(nonsink) // 2, replace=False)
            keep = np.setdiff1d(np.arange(npg), evict)    # sorted: logical order kept
            pos = np.concatenate([np.arange(p * PAGE, min((p + 1) * PAGE, T)) for p in keep])
            tier_list.append(tier[keep].astype(np.uint8))
            lens[s] = len(pos)
            pos_list.append(pos)
        else:
            n = int(lens[s])
            npg = (n + PAGE - 1) // PAGE
            pos_list.append(np.arange(n))
            tier_list.append(np.full(npg, next(iter(tiers)), np.uint8))
    lens = np.asarray(lens, np.int32)
    npages = [(int(n) + PAGE - 1) // PAGE for n in lens]
    total_pages = int(sum(npages))
    max_pages = max(npages) if npages else 1

    # ---- physical placement ----
    if name == "tiny":
        num_pages = total_pages
        perm = np.arange(num_pages)
    elif name == "ragged_b64":
        num_pages = int(np.ceil(1.25 * total_pages))
        perm = r_pages.permutation(num_pages)[:total_pages]
    else:
        num_pages = total_pages
        perm = r_pages.permutation(num_pages)
    block_table = np.zeros((B, max_pages), np.int32)
    page_bits = np.full((num_pages, hkv) if head_tiers else num_pages, max(tiers), np.uint8)
    k = 0
    for s in range(B):
        block_table[s, : npages[s]] = perm[k: k + npages[s]]
        page_bits[perm[k: k + npages[s]]] = tier_list[s]
        k += npages[s]
    if head_tiers:
        # one header and one record offset per (page, KV head), packed in
        # (page, head) order
        page_bits = page_bits.reshape(-1)
        sizes = PAGE * np.array([record_bytes(d, int(b)) for b in page_bits], np.uint64)
        page_off = np.zeros(num_pages * hkv, np.uint64)
        page_off[1:] = np.cumsum(sizes)[:-1]
        kcode_bytes = int(sizes.sum())
        bstride = max(tiers)
    elif len(tiers) > 1:
        sizes = hkv * PAGE * np.array([record_bytes(d, int(b)) for b in page_bits], np.uint64)
        page_off = np.zeros(num_pages, np.uint64)
        page_off[1:] = np.cumsum(sizes)[:-1]
        kcode_bytes = int(sizes.sum())
        bstride = max(tiers)
    else:
        page_off = None
        bstride = max(tiers)
        kcode_bytes = num_pages * hkv * PAGE * record_bytes(d, bstride)

    # ---- keys, values, query ----
    n_tok = int(lens.astype(np.int64).sum())
    if not data:
        keys = np.zeros((0, hkv, d), np.float32)
        values = np.zeros((0, hkv, d), np.uint16)
        q = np.zeros((B, hq, d), np.float32)
    else:
        plain = name == "tiny"
        chan = None if plain else r_scale.lognormal(0.0, 0.5, size=(hkv, d)).astype(np.float32)
        if outliers:
            for g in range(hkv):
                ch = r_out.choice(d, size=outliers, replace=False)
                chan[g, ch] *= r_out.uniform(20.0, 50.0, size=outliers).astype(np.float32)
        pos_all = np.concatenate(pos_list) if n_tok else np.zeros(0, np.int64)
        keys = np.empty((n_tok, hkv, d), np.float32)
        values = np.empty((n_tok, hkv, d), np.uint16)
        _fill_chunks(idx, n_tok, hkv, d, chan, pos_all, keys, values)
        q = np.empty((B, hq, d), np.float32)
        for s in range(B):
            n = int(lens[s])
            qs = r_q.standard_normal((1, hq, d), dtype=np.float32)
            if plain:
                q[s] = qs[0]
            else:
                qpos = (int(pos_list[s][-1]) + 1) if n else 0
                q[s] = _rope(qs, np.array([qpos]), d)[0]

    slot = np.empty(n_tok, np.int64)
    o = 0
    for s in range(B):
        n = int(lens[s])
        t = np.arange(n)
        slot[o: o + n] = block_table[s, t // PAGE].astype(np.int64) * PAGE + t % PAGE
        o += n

    return Workload(name=name, d=d, hq=hq, hkv=hkv, B=B, radius_mode=mode,
                    tier_mask=sum(1 << b for b in tiers), seq_lens=lens,
                    block_table=block_table, num_pages=num_pages, page_bits=page_bits,
                    page_off=page_off, bstride=bstride, kcode_bytes=kcode_bytes,
                    keys=keys, values=values, slot=slot, q=q, head_tiers=head_tiers)


def host_pools(w: Workload, poison: bool = True) -> dict:
    """Host arrays in the pool layout, filled with poison (0xFF bytes, bf16
    NaN) so that a reader of an unwritten byte is caught."""
    fill8 = 0xFF if poison else 0
    return {
        "d": w.d, "hkv": w.hkv, "bstride": w.bstride,
        "page_bits": w.page_bits, "page_off": w.page_off, "head_tiers": w.head_tiers,
        "kcode": np.full(w.kcode_bytes, fill8, np.uint8),
        "rcode": np.full(w.num_pages * w.hkv * PAGE, fill8, np.uint8),
        "v": np.full(w.num_pages * w.hkv * w.d * PAGE, 0x7FC0 if poison else 0, np.uint16),
    }


def token_keys(w: Workload, s: int) -> slice:
    """Rows of ``keys``/``values``/``slot`` that belong to sequence s."""
    start = int(w.seq_lens[:s].astype(np.int64).sum())
    return slice(start, start + int(w.seq_lens[s]))


# ---- the mixed-tier workload planned by the RDR controller ----------------
#
# Section 2.2 of the page: RDR chooses per state a residency and a tier under
# a byte budget (distortion surrogate: the tier's angular error scaled by the
# query and key magnitudes), keeps protected states (the sinks) at the widest
# tier, and groups the retained states into tier-homogeneous pages.  This
# workload takes the gqa_t32k keys, values and query and lets the controller
# decide the tiers and the evictions that mixed_tiers draws at random.  The
# plan itself is made by the library (ska_rdr_plan) or by the oracle; this
# module only draws the controller's inputs and lays out a given plan.

RDR_TIERS = (2, 4, 6, 8)
# eps(b): RMS over random unit pairs at d = 128 of f_b(c_q, c_k) - <q, k>,
# measured once with the CPU oracle (tests/golden/rdr_eps_d128.txt holds the
# table and the script that wrote it)
RDR_EPS = (2.710757e-01, 5.762753e-02, 1.450992e-02, 3.669538e-03)
# sigma (the query magnitude and softmax scale folded into the surrogate) and
# the budget (a fraction of keeping every state at the widest tier) are
# chosen so that the plan evicts about half of the tokens and keeps the rest
# at a spread of widths (about 26 / 54 / 16 / 4 % at b = 2 / 4 / 6 / 8), the
# regime mixed_tiers draws at random
RDR_SIGMA = 0.02
RDR_BUDGET_FRAC = 0.42
RDR_SINKS = 4             # protected first tokens


@dataclasses.dataclass
class RdrInputs:
    base: Workload            # gqa_t32k-shaped keys, values, query (full pages)
    utility: np.ndarray       # float32 [B][T]
    key_norm: np.ndarray      # float32 [B][T]
    protect: np.ndarray       # uint8 [B][T]
    num_states: np.ndarray    # int32 [B]
    budget: np.ndarray        # int64 [B]
    tiers: tuple
    eps: tuple
    bytes_per_tier: tuple
    sigma: float


def rdr_inputs(scale: float = 1.0, batch: Optional[int] = None) -> RdrInputs:
    """The controller's inputs for every token of a gqa_t32k-shaped batch:
    a seeded utility per token (LogNormal(0, 1.5), five times larger over
    the last 256 tokens, a recent window), its key norm (mean over KV heads),
    the first RDR_SINKS tokens protected, and a byte budget of
    RDR_BUDGET_FRAC of keeping every token at the widest tier."""
    base = make("gqa_t32k", scale, batch=batch)
    B, T = base.B, int(base.seq_lens.max())
    r = np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=(50,)))
    util = r.lognormal(0.0, 1.5, size=(B, T)).astype(np.float32)
    util[:, max(0, T - 256):] *= 5.0
    kn = np.zeros((B, T), np.float32)
    for s in range(B):
        k = base.keys[token_keys(base, s)].astype(np.float64)
        kn[s, : k.shape[0]] = np.sqrt((k * k).sum(axis=2)).mean(axis=1)
    prot = np.zeros((B, T), np.uint8)
    prot[:, :RDR_SINKS] = 1
    per_state = tuple(base.hkv * (record_bytes(base.d, b) + 1 + 2 * base.d) for b in RDR_TIERS)
    budget = (RDR_BUDGET_FRAC * base.seq_lens.astype(np.float64) * per_state[-1]).astype(np.int64)
    return RdrInputs(base=base, utility=util, key_norm=kn, protect=prot, num_states=base.seq_lens.copy(),
                     budget=budget, tiers=RDR_TIERS, eps=RDR_EPS, bytes_per_tier=per_state, sigma=RDR_SIGMA)


def planned_workload(inp: RdrInputs, tier: np.ndarray, page: np.ndarray, slot: np.ndarray,
                     page_hdr: np.ndarray, npages: np.ndarray) -> Workload:
    """Lay out a plan: per sequence s, its npages[s] planned pages (headers
    page_hdr[s], tier and empty slots) become physical pages of one shared,
    shuffled pool, addressed through page_off (their sizes vary with the
    tier), in plan order in row s of the block table; the retained tokens
    (tier[s][i] > 0) go to slot slot[s][i] of planned page page[s][i].  The
    row's length ends at its last page's last token."""
    base = inp.base
    B, hkv, d = base.B, base.hkv, base.d
    npages = np.asarray(npages, np.int64)
    total = int(npages.sum())
    r = np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=(51,)))
    perm = r.permutation(total)
    max_pages = max(1, int(npages.max()))
    bt = np.zeros((B, max_pages), np.int32)
    page_bits = np.zeros(total, np.uint8)
    lens = np.zeros(B, np.int32)
    keys, vals, slots = [], [], []
    k0 = 0
    for s in range(B):
        n_p = int(npages[s])
        phys = perm[k0: k0 + n_p]
        k0 += n_p
        bt[s, :n_p] = phys
        page_bits[phys] = page_hdr[s][:n_p]
        if n_p:
            lens[s] = 16 * (n_p - 1) + PAGE - (int(page_hdr[s][n_p - 1]) >> 4)
        n = int(inp.num_states[s])
        kept = np.nonzero(tier[s][:n])[0]
        rows = token_keys(base, s)
        keys.append(base.keys[rows][kept])
        vals.append(base.values[rows][kept])
        slots.append(phys[page[s][kept]].astype(np.int64) * PAGE + slot[s][kept])
    sizes = hkv * PAGE * np.array([record_bytes(d, int(b) & 15) for b in page_bits], np.uint64)
    page_off = np.zeros(total, np.uint64)
    if total:
        page_off[1:] = np.cumsum(sizes)[:-1]
    return Workload(name="mixed_tiers_rdr", d=d, hq=base.hq, hkv=hkv, B=B, radius_mode=base.radius_mode,
                    tier_mask=sum(1 << b for b in inp.tiers), seq_lens=lens, block_table=bt, num_pages=total,
                    page_bits=page_bits, page_off=page_off, bstride=max(inp.tiers),
                    kcode_bytes=int(sizes.sum()), keys=np.concatenate(keys), values=np.concatenate(vals),
                    slot=np.concatenate(slots), q=base.q)
