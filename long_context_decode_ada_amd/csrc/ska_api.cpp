// ska_api.cpp -- host side of the C ABI declared in include/ska.h:
// argument validation, code and radius tables, the cache handle and its
// workspace, split policy and kernel launches.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary,
// sections 2.1 (spherical codes, logit from codes), 2.2 (tier-homogeneous
// pages) and 2.3 (encode into a paged store; decode consumes the codes).
//
// Host constants that enter integer decisions (angle bin edges, radius
// edges) are computed here in binary64 with the C library's cos, sin, exp,
// log and sqrt, built with -fno-builtin -ffp-contract=off so that each is the
// library call and each product is rounded as written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/ska.h"
#include "ska_internal.h"
#include "ska_rdr.h"

using namespace ska;

struct ska_cache {
    ska_pool_desc pool;
    int device = 0;
    int num_cus = 256;
    int nt = 0;
    int8_t tslot[9];
    int64_t page_stride = 0;
    std::vector<double> range;  // [hkv][2]
    double *d_cos2 = nullptr, *d_sin2 = nullptr, *d_cen = nullptr, *d_tau2 = nullptr;
    float2 *d_lut = nullptr;
    float *d_rlev = nullptr;
    uint32_t *d_err = nullptr;
    // decode workspace, allocated at creation for the pool's declared maxima:
    // split partials (ws_rows rows of (o[d], m, l)) and the per-(sequence,
    // KV head) counters of the in-kernel merge (zero between calls)
    void *d_ws = nullptr;
    size_t ws_rows = 0;
    uint32_t *d_cnt = nullptr;
    size_t cnt_n = 0;
    // the unit order of a batch that runs in several rounds (k_unit_order)
    int2 *d_units = nullptr;
    // stream of the last decode call (calls share the workspace) and the
    // event that orders a call on another stream after it
    mutable hipStream_t last_stream = nullptr;
    hipEvent_t order_ev = nullptr;
    // kernel timing (ska_profile_begin / ska_profile_read)
    std::vector<hipEvent_t> prof_ev;  // 2 per recorded call
    int prof_max = 0;
    mutable int prof_n = 0;
};

namespace {

bool tiers_ok(uint32_t mask) { return mask != 0 && (mask & ~kSupportedTiers) == 0; }

int max_tier(uint32_t mask) {
    int b = 0;
    for (int i = 2; i <= 8; ++i)
        if ((mask >> i) & 1u) b = i;
    return b;
}

ska_status check_pool(const ska_pool_desc *p) {
    if (!p) return SKA_ERR_INVALID;
    if (p->d != 64 && p->d != 128) return (p->d > 0 && p->d % 4 == 0) ? SKA_ERR_UNSUPPORTED : SKA_ERR_INVALID;
    if (p->num_kv_heads < 1 || p->page_size != kPage || p->num_pages < 1) return SKA_ERR_INVALID;
    if (p->radius_mode != SKA_RADIUS_UNIFORM && p->radius_mode != SKA_RADIUS_LOG) return SKA_ERR_INVALID;
    if (p->radius_bits != 8) return SKA_ERR_UNSUPPORTED;
    if (!tiers_ok(p->tier_mask)) return SKA_ERR_INVALID;
    if (p->query_mode != SKA_Q_CODED && p->query_mode != SKA_Q_EXACT) return SKA_ERR_INVALID;
    if (!p->kcode || !p->rcode || !p->v || !p->page_bits) return SKA_ERR_INVALID;
    if (p->head_tiers != 0 && p->head_tiers != 1) return SKA_ERR_INVALID;
    if (p->head_tiers && !p->page_off) return SKA_ERR_INVALID;
    if (p->query_precision != SKA_QDIR_F16 && p->query_precision != SKA_QDIR_F32) return SKA_ERR_INVALID;
    if (p->max_batch < 1 || p->max_heads_q < 1 || p->max_pages < 1 || p->max_splits < 0) return SKA_ERR_INVALID;
    if (p->max_heads_q % p->num_kv_heads != 0) return SKA_ERR_INVALID;
    return SKA_OK;
}

bool same_shape(const ska_pool_desc &a, const ska_pool_desc &b) {
    return a.d == b.d && a.num_kv_heads == b.num_kv_heads && a.page_size == b.page_size &&
           a.num_pages == b.num_pages && a.radius_mode == b.radius_mode && a.radius_bits == b.radius_bits &&
           a.tier_mask == b.tier_mask && a.query_mode == b.query_mode && a.head_tiers == b.head_tiers &&
           a.query_precision == b.query_precision && a.max_batch == b.max_batch &&
           a.max_heads_q == b.max_heads_q && a.max_pages == b.max_pages && a.max_splits == b.max_splits;
}

// Split layout of a decode call (the kernel's split_start/splits_of read it).
// Explicit: num_splits splits of equal size.  Automatic: as if every
// sequence had max_pages pages, with one workgroup per CU (equal splits).
// When the (sequence, KV head) groups alone already fill the CUs, the batch
// runs in several rounds of workgroups, and the work units are sized so that
// the big ones go first and the small ones fill the last round: splits of
// kTailBase, kTailBase, 2 kTailBase, ... pages, doubling up to at most
// kTailBase << kTailMaxDoublings pages (and max_pages), handed out largest
// first; with a batch of at most kCompactMaxBatch (and at most kUnitSortMax
// grid slots) the grid is also compacted: k_unit_order lists the units that
// hold pages in decreasing size and each workgroup takes its slot's entry, so
// no slot is spent on a split past the end of a short sequence.  Measured on
// a ragged batch of 64 (70..3546 pages): four equal splits 442 us; splits of
// 256, 256, 512, 1024, then 2048 pages in split order 387 us, in size order
// 354 us; 384, 384, then 768 each in size order 345 us (a batch of 160 at
// half the lengths: 490 -> 477 us; 512, 512, 1024: 348 and 474 us).
#ifndef SKA_TAIL_BASE
#define SKA_TAIL_BASE 384
#endif
#ifndef SKA_TAIL_DOUBLINGS
#define SKA_TAIL_DOUBLINGS 1
#endif
constexpr int kTailBase = SKA_TAIL_BASE, kTailMaxDoublings = SKA_TAIL_DOUBLINGS;
struct SplitLayout {
    int pps = 0, split_m = 0, nsplit = 0;
    bool rounds = false;
};
SplitLayout split_layout(int num_cus, int batch, int hkv, int max_pages, int num_splits) {
    SplitLayout L;
    int pps;
    if (num_splits > 0) {
        pps = (max_pages + num_splits - 1) / num_splits;
    } else {
        const int64_t total = (int64_t)batch * hkv * max_pages;
        const int64_t target = (int64_t)num_cus * decode_workgroups_per_cu();   // one round of resident workgroups
        pps = (int)std::min<int64_t>((total + target - 1) / target, max_pages);
        if (pps >= max_pages) {
            L.rounds = true;
            pps = std::min(kTailBase, max_pages);
            L.split_m = kTailMaxDoublings;
        }
    }
    pps = ((pps + kWaves - 1) / kWaves) * kWaves;
    if (pps < kWaves) pps = kWaves;
    while (L.split_m > 0 && ((int64_t)pps << L.split_m) > max_pages) --L.split_m;
    // the split index is the grid's z dimension (at most 65535)
    if (L.split_m == 0 && (max_pages + pps - 1) / pps > 65535)
        pps = (((max_pages + 65534) / 65535 + kWaves - 1) / kWaves) * kWaves;
    L.pps = pps;
    const int cap = pps << L.split_m;   // splits of a sequence of max_pages pages (the kernel's layout)
    if (max_pages > cap) {
        L.nsplit = L.split_m + (max_pages + cap - 1) / cap;
    } else {
        int k = 1;
        while (k <= L.split_m + 1 && (pps << (k - 1)) < max_pages) ++k;
        L.nsplit = k;
    }
    return L;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// workspace of `rows` partial rows: [o: rows x d floats | (m, l): rows x 2 floats]
inline size_t ws_off_ml(size_t rows, int d) { return align256(rows * (size_t)d * 4); }
inline size_t ws_bytes(size_t rows, int d) { return ws_off_ml(rows, d) + align256(rows * 2 * 4); }

// Partial rows (sequence, query head, split) that any decode call within the
// pool's maxima can need.  Per query head, a call's batch * nsplit is at most:
// automatic layout, one round: batch * ceil(target / (batch * Hkv)) <=
// target / Hkv + batch (each split is at least total / target pages);
// several rounds: batch * ceil(max_pages / kTailBase) (each split but a
// sequence's last is at least kTailBase pages); explicit: batch * num_splits.
size_t reserve_rows(const ska_pool_desc &p, int num_cus) {
    const int64_t target = (int64_t)num_cus * decode_workgroups_per_cu();
    const int64_t B = p.max_batch, hkv = p.num_kv_heads;
    int64_t per_head = std::max<int64_t>((target + hkv - 1) / hkv + B,
                                         B * std::max<int64_t>(1, (p.max_pages + kTailBase - 1) / kTailBase));
    per_head = std::max<int64_t>(per_head, B * (int64_t)p.max_splits);
    return (size_t)per_head * (size_t)p.max_heads_q;
}

// cos^2, sin^2 of the bin edges j*pi/2^b for b = 1..8 at offset 2^b - 2.
void build_thresholds(std::vector<double> &c2, std::vector<double> &s2) {
    c2.assign(kThrEntries, 0.0);
    s2.assign(kThrEntries, 0.0);
    for (int b = 1; b <= 8; ++b) {
        const int n = 1 << b;
        c2[thr_off(b)] = 1.0;
        s2[thr_off(b)] = 0.0;
        for (int j = 1; j < n; ++j) {
            const double th = std::ldexp((double)j * M_PI, -b);
            const double c = std::cos(th), s = std::sin(th);
            c2[thr_off(b) + j] = c * c;
            s2[thr_off(b) + j] = s * s;
        }
    }
}

// binary64 (cos, sin) of bin centres in the decode table layout.
void build_centres(std::vector<double> &cen) {
    cen.assign(2 * kLutEntries, 0.0);
    const int tiers[5] = {2, 3, 4, 6, 8};
    for (int b : tiers) {
        const int n = 1 << b;
        for (int c = 0; c < n; ++c) {
            const double pp = ((double)c + 0.5) * M_PI / (double)n;
            const double pa = ((double)c + 0.5) * 2.0 * M_PI / (double)n;
            cen[2 * (lut_polar(b) + c) + 0] = std::cos(pp);
            cen[2 * (lut_polar(b) + c) + 1] = std::sin(pp);
            cen[2 * (lut_azimuth(b) + c) + 0] = std::cos(pa);
            cen[2 * (lut_azimuth(b) + c) + 1] = std::sin(pa);
        }
    }
    for (int c = 0; c < 256; ++c) {
        cen[2 * (kLutOnes + c) + 0] = 1.0;
        cen[2 * (kLutOnes + c) + 1] = 1.0;
    }
}

// Radius levels and squared edges of one kv head (8 bits).
void build_radius(int mode, double rlo, double rhi, float *level, double *tau2) {
    if (!(rhi > 0.0)) {
        for (int j = 0; j < 256; ++j) level[j] = 0.f;
        for (int j = 0; j < 255; ++j) tau2[j] = 0.0;
        return;
    }
    if (mode == SKA_RADIUS_UNIFORM) {
        for (int j = 0; j < 256; ++j) level[j] = (float)(((double)j * rhi) / 255.0);
        for (int j = 0; j < 255; ++j) {
            const double e = (((double)j + 0.5) * rhi) / 255.0;
            tau2[j] = e * e;
        }
    } else {
        if (!(rlo > 0.0)) rlo = rhi;
        const double L = std::log(rlo), U = std::log(rhi);
        for (int j = 0; j < 256; ++j) level[j] = (float)std::exp(L + ((double)j * (U - L)) / 255.0);
        for (int j = 0; j < 255; ++j) {
            const double e = std::exp(L + (((double)j + 0.5) * (U - L)) / 255.0);
            tau2[j] = e * e;
        }
    }
}

template <class T>
hipError_t upload(T **dst, const T *src, size_t count) {
    hipError_t e = hipMalloc((void **)dst, count * sizeof(T));
    if (e != hipSuccess) return e;
    return hipMemcpy(*dst, src, count * sizeof(T), hipMemcpyHostToDevice);
}

void prof_clear(ska_cache *c) {
    for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
    c->prof_ev.clear();
    c->prof_max = c->prof_n = 0;
}

void release(ska_cache *c) {
    if (!c) return;
    prof_clear(c);
    (void)hipFree(c->d_cos2);
    (void)hipFree(c->d_sin2);
    (void)hipFree(c->d_cen);
    (void)hipFree(c->d_tau2);
    (void)hipFree(c->d_lut);
    (void)hipFree(c->d_rlev);
    (void)hipFree(c->d_err);
    (void)hipFree(c->d_ws);
    (void)hipFree(c->d_cnt);
    (void)hipFree(c->d_units);
    if (c->order_ev) (void)hipEventDestroy(c->order_ev);
    delete c;
}

ska_status create(ska_cache **out, const ska_pool_desc *pool) {
    ska_cache *c = new (std::nothrow) ska_cache();
    if (!c) return SKA_ERR_NOMEM;
    c->pool = *pool;
    if (hipGetDevice(&c->device) != hipSuccess) { delete c; return SKA_ERR_HIP; }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess && cus > 0)
        c->num_cus = cus;
    c->nt = 0;
    for (int b = 0; b <= 8; ++b) c->tslot[b] = 0;
    for (int b = 2; b <= 8; ++b)
        if ((pool->tier_mask >> b) & 1u) c->tslot[b] = (int8_t)c->nt++;
    c->page_stride = (int64_t)pool->num_kv_heads * kPage * record_bytes(pool->d, max_tier(pool->tier_mask));

    std::vector<double> c2, s2, cen;
    build_thresholds(c2, s2);
    build_centres(cen);
    std::vector<float2> lut(kLutEntries);
    for (int e = 0; e < kLutEntries; ++e) lut[e] = make_float2((float)cen[2 * e], (float)cen[2 * e + 1]);
    hipError_t e = upload(&c->d_cos2, c2.data(), c2.size());
    if (e == hipSuccess) e = upload(&c->d_sin2, s2.data(), s2.size());
    if (e == hipSuccess) e = upload(&c->d_cen, cen.data(), cen.size());
    if (e == hipSuccess) e = upload(&c->d_lut, lut.data(), lut.size());
    uint32_t zero = 0;
    if (e == hipSuccess) e = upload(&c->d_err, &zero, 1);
    // the decode workspace for every call within the declared maxima
    c->ws_rows = reserve_rows(*pool, c->num_cus);
    if (e == hipSuccess) e = hipMalloc(&c->d_ws, ws_bytes(c->ws_rows, pool->d));
    c->cnt_n = (size_t)pool->max_batch * pool->num_kv_heads;
    if (e == hipSuccess) e = hipMalloc((void **)&c->d_cnt, c->cnt_n * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(c->d_cnt, 0, c->cnt_n * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMalloc((void **)&c->d_units, kUnitSortMax * sizeof(int2));
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->order_ev, hipEventDisableTiming);
    if (e != hipSuccess) {
        release(c);
        return e == hipErrorOutOfMemory ? SKA_ERR_NOMEM : SKA_ERR_HIP;
    }
    *out = c;
    return SKA_OK;
}

ska_status set_range(ska_cache *c, const double *range) {
    const int hkv = c->pool.num_kv_heads;
    c->range.assign(range, range + 2 * hkv);
    std::vector<float> lev(256 * (size_t)hkv);
    std::vector<double> tau2(255 * (size_t)hkv);
    for (int g = 0; g < hkv; ++g)
        build_radius(c->pool.radius_mode, range[2 * g], range[2 * g + 1], lev.data() + 256 * g, tau2.data() + 255 * g);
    (void)hipFree(c->d_rlev);
    (void)hipFree(c->d_tau2);
    c->d_rlev = nullptr;
    c->d_tau2 = nullptr;
    hipError_t e = upload(&c->d_rlev, lev.data(), lev.size());
    if (e == hipSuccess) e = upload(&c->d_tau2, tau2.data(), tau2.size());
    return e == hipSuccess ? SKA_OK : (e == hipErrorOutOfMemory ? SKA_ERR_NOMEM : SKA_ERR_HIP);
}

ska_status calibrate(ska_cache *c, const float *keys, int64_t n, hipStream_t s) {
    const int hkv = c->pool.num_kv_heads;
    std::vector<unsigned long long> mm(2 * (size_t)hkv);
    for (int g = 0; g < hkv; ++g) {
        mm[2 * g + 0] = 0ull;                      // max: +0.0
        mm[2 * g + 1] = 0x7FF0000000000000ull;     // min positive: +inf
    }
    unsigned long long *d_mm = nullptr;
    if (hipMalloc((void **)&d_mm, mm.size() * sizeof(mm[0])) != hipSuccess) return SKA_ERR_NOMEM;
    hipError_t e = hipMemcpyAsync(d_mm, mm.data(), mm.size() * sizeof(mm[0]), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_calibrate(keys, n, hkv, c->pool.d, d_mm, s);
    if (e == hipSuccess) e = hipMemcpyAsync(mm.data(), d_mm, mm.size() * sizeof(mm[0]), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)hipFree(d_mm);
    if (e != hipSuccess) return SKA_ERR_HIP;
    std::vector<double> range(2 * (size_t)hkv);
    for (int g = 0; g < hkv; ++g) {
        double smax, smin;
        std::memcpy(&smax, &mm[2 * g + 0], 8);
        std::memcpy(&smin, &mm[2 * g + 1], 8);
        const double rhi = std::sqrt(smax);
        range[2 * g + 0] = std::isinf(smin) ? rhi : std::sqrt(smin);
        range[2 * g + 1] = rhi;
    }
    return set_range(c, range.data());
}

}  // namespace

extern "C" {

const char *ska_status_string(ska_status s) {
    switch (s) {
        case SKA_OK: return "ok";
        case SKA_ERR_INVALID: return "invalid argument";
        case SKA_ERR_UNSUPPORTED: return "unsupported shape or format";
        case SKA_ERR_HIP: return "HIP runtime error";
        case SKA_ERR_NOMEM: return "out of memory";
    }
    return "unknown status";
}

namespace {

// the pool side of the encode arguments (keys, values and slots left empty)
EncodeArgs encode_args(const ska_cache *c) {
    EncodeArgs a{};
    a.d = c->pool.d;
    a.hkv = c->pool.num_kv_heads;
    a.num_pages = c->pool.num_pages;
    a.tier_mask = c->pool.tier_mask;
    a.page_bits = c->pool.page_bits;
    a.page_off = c->pool.page_off;
    a.page_stride = c->page_stride;
    a.head_tiers = c->pool.head_tiers;
    a.kcode = c->pool.kcode;
    a.rcode = c->pool.rcode;
    a.v = c->pool.v;
    a.tau2 = c->d_tau2;
    a.tab = CodeTables{c->d_cos2, c->d_sin2, c->d_cen};
    a.err = c->d_err;
    return a;
}

}  // namespace

ska_status ska_encode_keys(ska_cache **cache, const ska_pool_desc *pool, const float *keys,
                           const uint16_t *values, const int64_t *slot, int64_t n,
                           const double *radius_range, void *stream) {
    if (!cache) return SKA_ERR_INVALID;
    ska_status st = check_pool(pool);
    if (st != SKA_OK) return st;
    if (n < 0 || (n > 0 && (!keys || !slot))) return SKA_ERR_INVALID;
    if (*cache && !same_shape((*cache)->pool, *pool)) return SKA_ERR_INVALID;
    if (!*cache && !radius_range && n == 0) return SKA_ERR_INVALID;  // nothing to calibrate on
    if (radius_range && !*cache) {
        for (int g = 0; g < pool->num_kv_heads; ++g) {
            const double lo = radius_range[2 * g], hi = radius_range[2 * g + 1];
            if (!std::isfinite(lo) || !std::isfinite(hi) || lo < 0.0 || hi < 0.0 || lo > hi) return SKA_ERR_INVALID;
        }
    }
    hipStream_t s = (hipStream_t)stream;
    ska_cache *c = *cache;
    bool created = false;
    if (!c) {
        st = create(&c, pool);
        if (st != SKA_OK) return st;
        created = true;
        st = radius_range ? set_range(c, radius_range) : calibrate(c, keys, n, s);
        if (st != SKA_OK) {
            release(c);
            return st;
        }
    }
    c->pool = *pool;  // same shape; pointers may move
    if (n > 0) {
        EncodeArgs a = encode_args(c);
        a.keys = keys;
        a.values = values;
        a.slot = slot;
        a.n = n;
        if (launch_encode(a, s) != hipSuccess) {
            if (created) release(c);
            return SKA_ERR_HIP;
        }
    }
    *cache = c;
    return SKA_OK;
}

namespace {

// Checks of one decode call and its kernel arguments, the split workspace
// left empty: ADA over the cache's coded pools (k_dense NULL) or, for the
// dense baseline, over bf16 keys k_dense with the cache's values.  Returns
// SKA_OK with *rows = the partial rows (sequence, query head, split) the call
// uses, or an error (nothing to launch; *rows = 0 for an empty batch).
ska_status prepare_decode(const ska_cache *c, const uint16_t *k_dense, const float *q, int batch,
                          int num_q_heads, const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                          float scale, int num_splits, float *out, float *logits_dbg, const float *app_k,
                          const uint16_t *app_v, DecodeArgs &da, int &G, size_t &rows) {
    rows = 0;
    if (!c) return SKA_ERR_INVALID;
    if (batch < 0 || num_q_heads < 1 || max_pages < 1 || num_splits < 0) return SKA_ERR_INVALID;
    if (!std::isfinite(scale) || scale < 0.f) return SKA_ERR_INVALID;
    const int hkv = c->pool.num_kv_heads, d = c->pool.d;
    if (num_q_heads % hkv != 0) return SKA_ERR_INVALID;
    G = num_q_heads / hkv;
    if (G != 1 && G != 2 && G != 4) return SKA_ERR_UNSUPPORTED;
    // within the maxima the cache's workspace was sized for
    if (batch > c->pool.max_batch || num_q_heads > c->pool.max_heads_q || max_pages > c->pool.max_pages ||
        num_splits > c->pool.max_splits)
        return SKA_ERR_INVALID;
    if (batch == 0) return SKA_OK;
    if (!q || !block_table || !seq_lens || !out) return SKA_ERR_INVALID;
    if (batch > 65535 || hkv > 65535) return SKA_ERR_UNSUPPORTED;
    if (scale == 0.f) scale = 1.0f / std::sqrt((float)d);
    const SplitLayout L = split_layout(c->num_cus, batch, hkv, max_pages, num_splits);
    if (L.nsplit > 65535) return SKA_ERR_UNSUPPORTED;
    rows = (size_t)batch * num_q_heads * L.nsplit;

    da = DecodeArgs{};
    da.kcode = c->pool.kcode;
    da.page_off = c->pool.page_off;
    da.rcode = c->pool.rcode;
    da.v = c->pool.v;
    da.page_bits = c->pool.page_bits;
    da.block_table = block_table;
    da.seq_lens = seq_lens;
    da.q = q;
    da.cos2 = c->d_cos2;
    da.sin2 = c->d_sin2;
    da.scale = scale;
    da.query_mode = c->pool.query_mode;
    da.query_f32 = c->pool.query_precision == SKA_QDIR_F32 ? 1 : 0;
    da.lut = c->d_lut;
    da.rlev = c->d_rlev;
    da.logits = logits_dbg;
    da.out = out;
    da.kdense = const_cast<uint16_t *>(k_dense);
    da.dense = k_dense != nullptr;
    da.err = c->d_err;
    da.num_pages = c->pool.num_pages;
    da.page_stride = c->page_stride;
    da.hkv = hkv;
    da.hq = num_q_heads;
    da.max_pages = max_pages;
    da.pps = L.pps;
    da.split_m = L.split_m;
    da.compact = (L.rounds && batch <= kCompactMaxBatch && (int64_t)batch * L.nsplit <= kUnitSortMax) ? 1 : 0;
    da.nsplit = L.nsplit;
    da.tier_mask = c->pool.tier_mask;
    da.nt = c->nt;
    for (int b = 0; b <= 8; ++b) da.tslot[b] = c->tslot[b];
    da.head_tiers = c->pool.head_tiers;
    da.app_k = app_k;
    da.app_v = app_v;
    da.tau2 = c->d_tau2;
    return SKA_OK;
}

// One decode call on the cache's own workspace (allocated at creation).
ska_status decode_impl(const ska_cache *c, const uint16_t *k_dense, const float *q, int batch, int num_q_heads,
                       const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                       float scale, int num_splits, float *out, float *logits_dbg, void *stream,
                       const float *app_k = nullptr, const uint16_t *app_v = nullptr) {
    DecodeArgs da;
    int G = 0;
    size_t rows = 0;
    ska_status st = prepare_decode(c, k_dense, q, batch, num_q_heads, block_table, max_pages, seq_lens, scale,
                                   num_splits, out, logits_dbg, app_k, app_v, da, G, rows);
    if (st != SKA_OK || batch == 0) return st;
    if (rows > c->ws_rows) return SKA_ERR_INVALID;   // (cannot happen within the maxima)
    const int d = c->pool.d;
    char *ws = (char *)c->d_ws;
    da.part_o = (float *)ws;
    da.part_ml = (float *)(ws + ws_off_ml(c->ws_rows, d));
    da.counters = c->d_cnt;
    da.unit_table = da.compact ? c->d_units : nullptr;
    hipStream_t s = (hipStream_t)stream;
    // calls share the workspace: one on another stream waits for the last
    if (s != c->last_stream) {
        if (hipEventRecord(c->order_ev, c->last_stream) != hipSuccess) return SKA_ERR_HIP;
        if (hipStreamWaitEvent(s, c->order_ev, 0) != hipSuccess) return SKA_ERR_HIP;
        c->last_stream = s;
    }
    hipEvent_t *ev = nullptr;
    if (c->prof_n < c->prof_max) ev = const_cast<hipEvent_t *>(&c->prof_ev[2 * (size_t)c->prof_n++]);
    if (ev && hipEventRecord(ev[0], s) != hipSuccess) return SKA_ERR_HIP;
    if (launch_decode(da, d, G, batch, s) != hipSuccess) return SKA_ERR_HIP;
    if (ev && hipEventRecord(ev[1], s) != hipSuccess) return SKA_ERR_HIP;
    return SKA_OK;
}

}  // namespace

// ---- the decode for callers that cannot allocate ----
//
// ska_decode_attention_noalloc keeps its split partials and merge counters in
// this file-scope device array instead of the cache's workspace: one copy per
// GPU, held until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address reaches kernels.
namespace {
constexpr size_t kScratchBytes = (size_t)16 << 20;                  // 16 MiB per GPU
constexpr size_t kScratchCounters = 65536;                          // (sequence, KV head) merge counters
constexpr size_t kScratchCounterBytes = kScratchCounters * sizeof(uint32_t);
constexpr size_t kScratchUnitBytes = kUnitSortMax * sizeof(int2);   // the unit order table
constexpr size_t kScratchPartialBytes = kScratchBytes - kScratchCounterBytes - kScratchUnitBytes;
constexpr int kScratchMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
char *g_scratch[kScratchMaxDevices];   // device address of each GPU's copy (nullptr: not yet set up)

// The device address of `device`'s scratch array; on the first call for that
// device it is looked up (with the device current) and its merge counters
// are cleared on `s` by a fill kernel (every completed call leaves the
// counters it used at zero again).
ska_status scratch_base(int device, hipStream_t s, char **out) {
    if (device < 0 || device >= kScratchMaxDevices) return SKA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[device]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SKA_ERR_HIP;
        if (cur != device && hipSetDevice(device) != hipSuccess) return SKA_ERR_HIP;
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e == hipSuccess && !p) e = hipErrorInvalidSymbol;
        if (e == hipSuccess) e = launch_zero_u32(static_cast<uint32_t *>(p), (int64_t)kScratchCounters, s);
        if (cur != device) (void)hipSetDevice(cur);
        if (e != hipSuccess) return SKA_ERR_HIP;
        g_scratch[device] = static_cast<char *>(p);
    }
    *out = g_scratch[device];
    return SKA_OK;
}
}  // namespace

ska_status ska_decode_attention_noalloc(const ska_cache *c, const float *q, int batch, int num_q_heads,
                                        const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                                        float scale, int num_splits, float *out, void *stream) {
    DecodeArgs da;
    int G = 0;
    size_t rows = 0;
    ska_status st = prepare_decode(c, nullptr, q, batch, num_q_heads, block_table, max_pages, seq_lens, scale,
                                   num_splits, out, nullptr, nullptr, nullptr, da, G, rows);
    if (st != SKA_OK || batch == 0) return st;
    const int d = c->pool.d;
    // beyond the scratch array: rejected before anything is enqueued
    if ((size_t)batch * c->pool.num_kv_heads > kScratchCounters || ws_bytes(rows, d) > kScratchPartialBytes)
        return SKA_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    char *base = nullptr;
    if ((st = scratch_base(c->device, s, &base)) != SKA_OK) return st;
    da.counters = reinterpret_cast<uint32_t *>(base);
    da.unit_table = da.compact ? reinterpret_cast<int2 *>(base + kScratchCounterBytes) : nullptr;
    char *parts = base + kScratchCounterBytes + kScratchUnitBytes;
    da.part_o = reinterpret_cast<float *>(parts);
    da.part_ml = reinterpret_cast<float *>(parts + ws_off_ml(rows, d));
    if (launch_decode(da, d, G, batch, s) != hipSuccess) return SKA_ERR_HIP;
    return SKA_OK;
}

ska_status ska_decode_attention(const ska_cache *c, const float *q, int batch, int num_q_heads,
                                const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                                float scale, int num_splits, float *out, float *logits_dbg, void *stream) {
    return decode_impl(c, nullptr, q, batch, num_q_heads, block_table, max_pages, seq_lens, scale, num_splits,
                       out, logits_dbg, stream);
}

ska_status ska_append_decode_attention(const ska_cache *c, const float *new_keys, const uint16_t *new_values,
                                       const float *q, int batch, int num_q_heads, const int32_t *block_table,
                                       int max_pages, const int32_t *seq_lens, float scale, int num_splits,
                                       float *out, float *logits_dbg, void *stream) {
    if (!c) return SKA_ERR_INVALID;
    if (batch > 0 && (!new_keys || !new_values)) return SKA_ERR_INVALID;
    // (every other argument is checked by the decode before it launches
    // anything, so a rejected call stores nothing)
    return decode_impl(c, nullptr, q, batch, num_q_heads, block_table, max_pages, seq_lens, scale, num_splits,
                       out, logits_dbg, stream, new_keys, new_values);
}

ska_status ska_dense_decode_attention(const ska_cache *c, const uint16_t *k_dense, const float *q, int batch,
                                      int num_q_heads, const int32_t *block_table, int max_pages,
                                      const int32_t *seq_lens, float scale, int num_splits, float *out,
                                      float *logits_dbg, void *stream) {
    if (!k_dense) return SKA_ERR_INVALID;
    return decode_impl(c, k_dense, q, batch, num_q_heads, block_table, max_pages, seq_lens, scale, num_splits,
                       out, logits_dbg, stream);
}

namespace {

// The RDR workspace of the current device: allocated on first use, grown
// (after a device synchronisation, so that no call in flight still uses the
// old one) when a call needs more, kept until the process ends.
struct RdrWorkspace {
    void *p = nullptr;
    size_t n = 0;
};
RdrWorkspace g_rdr_ws[64];

ska_status rdr_workspace(size_t bytes, char **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SKA_ERR_HIP;
    RdrWorkspace &w = g_rdr_ws[dev];
    if (w.n < bytes) {
        if (w.p) {
            if (hipDeviceSynchronize() != hipSuccess) return SKA_ERR_HIP;
            (void)hipFree(w.p);
            w.p = nullptr;
            w.n = 0;
        }
        const size_t want = std::max(bytes, (size_t)1 << 20);
        if (hipMalloc(&w.p, want) != hipSuccess) return SKA_ERR_HIP;
        w.n = want;
    }
    *out = static_cast<char *>(w.p);
    return SKA_OK;
}

}  // namespace

ska_status ska_rdr_plan(const ska_rdr_params *p, const float *utility, const float *key_norm,
                        const uint8_t *protect, const int32_t *num_states, const int64_t *budget, int batch,
                        int max_states, uint8_t *tier_out, int32_t *page_out, int32_t *slot_out,
                        uint8_t *page_tier_out, int max_pages_out, int32_t *npages_out, double *lambda_out,
                        int32_t *status_out, void *stream) {
    if (!p || batch < 0 || max_states < 0) return SKA_ERR_INVALID;
    if (p->ntiers < 1 || p->ntiers > 8 || !(p->sigma >= 0.0) || !std::isfinite(p->sigma)) return SKA_ERR_INVALID;
    for (int k = 0; k < p->ntiers; ++k) {
        const int b = p->tiers[k];
        if (b < 1 || b > 8 || !(p->eps[k] >= 0.0) || !std::isfinite(p->eps[k]) || p->bytes[k] <= 0)
            return SKA_ERR_INVALID;
        if (k > 0 && (b <= p->tiers[k - 1] || p->bytes[k] < p->bytes[k - 1])) return SKA_ERR_INVALID;
    }
    if (max_pages_out < (max_states + 15) / 16 + p->ntiers) return SKA_ERR_INVALID;
    if (batch == 0) return SKA_OK;
    if (batch > 65535) return SKA_ERR_UNSUPPORTED;   // the sequence is the grid's y dimension
    if (!utility || !key_norm || !protect || !num_states || !budget || !tier_out || !page_out || !slot_out ||
        !page_tier_out || !npages_out || !lambda_out || !status_out)
        return SKA_ERR_INVALID;
    RdrArgs a{};
    a.u = utility;
    a.knorm = key_norm;
    a.prot = protect;
    a.nstate = num_states;
    a.budget = budget;
    a.max_states = max_states;
    a.ntiers = p->ntiers;
    for (int k = 0; k < p->ntiers; ++k) {
        a.tiers[k] = p->tiers[k];
        a.eps[k] = p->eps[k];
        a.bytes[k] = p->bytes[k];
    }
    a.sigma = p->sigma;
    a.tier_out = tier_out;
    a.page_out = page_out;
    a.slot_out = slot_out;
    a.page_tier = page_tier_out;
    a.max_pages_out = max_pages_out;
    a.npages = npages_out;
    a.lambda = lambda_out;
    a.status = status_out;
    // workspace (bound, per-round totals and intervals, per-chunk tier
    // counts), kept per device and grown when a call needs more
    hipStream_t s = (hipStream_t)stream;
    a.nchunk = std::max(1, (max_states + rdr_chunk_states() - 1) / rdr_chunk_states());
    const size_t n_hib = (size_t)batch, n_tot = (size_t)batch * 17 * 16, n_iv = (size_t)batch * 17 * 2;
    const size_t n_cnt = (size_t)batch * a.nchunk * 8;
    const size_t off_tot = n_hib * 8, off_iv = off_tot + n_tot * 8, off_cnt = off_iv + n_iv * 8;
    char *ws = nullptr;
    if (rdr_workspace(off_cnt + n_cnt * 4, &ws) != SKA_OK) return SKA_ERR_HIP;
    a.ws_hib = reinterpret_cast<unsigned long long *>(ws);
    a.ws_tot = reinterpret_cast<long long *>(ws + off_tot);
    a.ws_iv = reinterpret_cast<double *>(ws + off_iv);
    a.ws_cnt = reinterpret_cast<int32_t *>(ws + off_cnt);
    if (launch_zero_u32(reinterpret_cast<uint32_t *>(ws), (int64_t)(off_iv / 4), s) != hipSuccess) return SKA_ERR_HIP;
    if (launch_rdr(a, batch, s) != hipSuccess) return SKA_ERR_HIP;
    return SKA_OK;
}

ska_status ska_decompress_keys(const ska_cache *c, const int32_t *block_table, int batch, int max_pages,
                               const int32_t *seq_lens, uint16_t *k_dense, void *stream) {
    if (!c || batch < 0 || max_pages < 1) return SKA_ERR_INVALID;
    if (batch == 0) return SKA_OK;
    if (!block_table || !seq_lens || !k_dense) return SKA_ERR_INVALID;
    if (batch > 65535 || c->pool.num_kv_heads > 65535 || (max_pages + 63) / 64 > 65535) return SKA_ERR_UNSUPPORTED;
    DecodeArgs da{};
    da.kcode = c->pool.kcode;
    da.page_off = c->pool.page_off;
    da.rcode = c->pool.rcode;
    da.page_bits = c->pool.page_bits;
    da.block_table = block_table;
    da.seq_lens = seq_lens;
    da.lut = c->d_lut;
    da.rlev = c->d_rlev;
    da.kdense = k_dense;
    da.err = c->d_err;
    da.num_pages = c->pool.num_pages;
    da.page_stride = c->page_stride;
    da.hkv = c->pool.num_kv_heads;
    da.max_pages = max_pages;
    da.tier_mask = c->pool.tier_mask;
    da.head_tiers = c->pool.head_tiers;
    if (launch_decompress(da, c->pool.d, batch, (hipStream_t)stream) != hipSuccess) return SKA_ERR_HIP;
    return SKA_OK;
}

ska_status ska_profile_begin(ska_cache *c, int max_calls) {
    if (!c || max_calls < 0 || max_calls > (1 << 20)) return SKA_ERR_INVALID;
    prof_clear(c);
    c->prof_ev.assign(2 * (size_t)max_calls, nullptr);
    for (auto &e : c->prof_ev) {
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
            e = nullptr;
            prof_clear(c);
            return SKA_ERR_HIP;
        }
    }
    c->prof_max = max_calls;
    c->prof_n = 0;
    return SKA_OK;
}

ska_status ska_profile_read(ska_cache *c, float *ms_out, int max_calls, int *n_out) {
    if (!c || !n_out || max_calls < 0 || (max_calls > 0 && !ms_out)) return SKA_ERR_INVALID;
    const int n = c->prof_n < max_calls ? c->prof_n : max_calls;
    for (int i = 0; i < n; ++i) {
        hipEvent_t *ev = &c->prof_ev[2 * (size_t)i];
        if (hipEventSynchronize(ev[1]) != hipSuccess) return SKA_ERR_HIP;
        if (hipEventElapsedTime(&ms_out[i], ev[0], ev[1]) != hipSuccess) return SKA_ERR_HIP;
    }
    *n_out = n;
    return SKA_OK;
}

ska_status ska_get_radius_range(const ska_cache *c, double *range_out) {
    if (!c || !range_out) return SKA_ERR_INVALID;
    std::memcpy(range_out, c->range.data(), c->range.size() * sizeof(double));
    return SKA_OK;
}

ska_status ska_device_errors(ska_cache *c, void *stream, uint32_t *flags_out) {
    if (!c || !flags_out) return SKA_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    uint32_t v = 0, zero = 0;
    hipError_t e = hipMemcpyAsync(&v, c->d_err, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(c->d_err, &zero, 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return SKA_ERR_HIP;
    *flags_out = v;
    return SKA_OK;
}

void ska_free(ska_cache *c) { release(c); }

}  // extern "C"
