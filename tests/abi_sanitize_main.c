/*
 * abi_sanitize_main.c -- calls every entry point of include/ska.h with
 * arguments the host checks must reject (and the null-handle forms), for a
 * build of the host library with AddressSanitizer and UndefinedBehavior-
 * Sanitizer on its host code (tests/test_sanitizers.py).  Runs without a GPU:
 * every call here returns before any HIP call, or at the first one (cache
 * creation with no device present).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/ska.h"

static int fails = 0;
#define EXPECT(call, want)                                                                 \
    do {                                                                                   \
        ska_status got_ = (call);                                                          \
        if (got_ != (want)) {                                                              \
            printf("line %d: %s -> %d, expected %d\n", __LINE__, #call, (int)got_, (int)(want)); \
            ++fails;                                                                       \
        }                                                                                  \
    } while (0)

static ska_pool_desc good_desc(void)
{
    static uint8_t dummy[64];
    ska_pool_desc p;
    memset(&p, 0, sizeof p);
    p.d = 128;
    p.num_kv_heads = 8;
    p.page_size = 16;
    p.num_pages = 4;
    p.radius_mode = SKA_RADIUS_LOG;
    p.radius_bits = 8;
    p.tier_mask = 1u << 4;
    p.query_mode = SKA_Q_CODED;
    p.kcode = dummy;
    p.rcode = dummy;
    p.v = (uint16_t *)dummy;
    p.page_bits = dummy;
    p.query_precision = SKA_QDIR_F16;
    p.max_batch = 2;
    p.max_heads_q = 32;
    p.max_pages = 4;
    p.max_splits = 0;
    return p;
}

int main(void)
{
    static float keys[8 * 128];
    static int64_t slot[1];
    ska_cache *c = NULL;
    ska_pool_desc p;
    for (int s = 0; s < 6; ++s)
        if (!ska_status_string((ska_status)s))
            ++fails;
    /* pool descriptors the encode must reject before any HIP call */
    p = good_desc(); p.d = 96;            EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_UNSUPPORTED);
    p = good_desc(); p.d = 3;             EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc(); p.page_size = 32;    EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc(); p.tier_mask = 1u << 5; EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc(); p.query_precision = 7; EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc(); p.max_batch = 0;     EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc(); p.max_heads_q = 12;  EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc(); p.head_tiers = 1;    EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    p = good_desc();
    EXPECT(ska_encode_keys(NULL, &p, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_encode_keys(&c, NULL, keys, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, -1, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_encode_keys(&c, &p, NULL, NULL, slot, 1, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 0, NULL, NULL), SKA_ERR_INVALID);
    double bad_range[16];
    for (int g = 0; g < 8; ++g) { bad_range[2 * g] = 2.0; bad_range[2 * g + 1] = 1.0; }
    EXPECT(ska_encode_keys(&c, &p, keys, NULL, slot, 1, bad_range, NULL), SKA_ERR_INVALID);
    /* a valid descriptor: creation needs a device (SKA_ERR_HIP without one) */
    ska_status st = ska_encode_keys(&c, &p, keys, NULL, slot, 1, NULL, NULL);
    if (st != SKA_ERR_HIP && st != SKA_OK) { printf("create: %d\n", (int)st); ++fails; }
    if (st == SKA_OK) ska_free(c);
    /* decode-side entry points without a cache */
    float q[32 * 128], out[32 * 128];
    int32_t bt[4] = {0, 1, 2, 3}, sl[1] = {16};
    EXPECT(ska_decode_attention(NULL, q, 1, 32, bt, 4, sl, 0.f, 0, out, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_decode_attention_noalloc(NULL, q, 1, 32, bt, 4, sl, 0.f, 0, out, NULL), SKA_ERR_INVALID);
    EXPECT(ska_append_decode_attention(NULL, keys, NULL, q, 1, 32, bt, 4, sl, 0.f, 0, out, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_dense_decode_attention(NULL, NULL, q, 1, 32, bt, 4, sl, 0.f, 0, out, NULL, NULL), SKA_ERR_INVALID);
    EXPECT(ska_decompress_keys(NULL, bt, 1, 4, sl, NULL, NULL), SKA_ERR_INVALID);
    double range[16];
    EXPECT(ska_get_radius_range(NULL, range), SKA_ERR_INVALID);
    uint32_t flags;
    EXPECT(ska_device_errors(NULL, NULL, &flags), SKA_ERR_INVALID);
    EXPECT(ska_profile_begin(NULL, 4), SKA_ERR_INVALID);
    int n;
    float ms[4];
    EXPECT(ska_profile_read(NULL, ms, 4, &n), SKA_ERR_INVALID);
    /* RDR parameter checks */
    ska_rdr_params rp;
    memset(&rp, 0, sizeof rp);
    rp.ntiers = 2; rp.tiers[0] = 4; rp.tiers[1] = 2;     /* not increasing */
    rp.eps[0] = rp.eps[1] = 0.1; rp.bytes[0] = rp.bytes[1] = 100; rp.sigma = 0.1;
    EXPECT(ska_rdr_plan(&rp, NULL, NULL, NULL, NULL, NULL, 1, 16, NULL, NULL, NULL, NULL, 8, NULL, NULL, NULL, NULL),
           SKA_ERR_INVALID);
    rp.tiers[0] = 2; rp.tiers[1] = 4;
    EXPECT(ska_rdr_plan(&rp, NULL, NULL, NULL, NULL, NULL, 1, 16, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL, NULL),
           SKA_ERR_INVALID);   /* max_pages_out too small */
    EXPECT(ska_rdr_plan(&rp, NULL, NULL, NULL, NULL, NULL, 1, 16, NULL, NULL, NULL, NULL, 8, NULL, NULL, NULL, NULL),
           SKA_ERR_INVALID);   /* NULL arrays */
    EXPECT(ska_rdr_plan(NULL, NULL, NULL, NULL, NULL, NULL, 1, 16, NULL, NULL, NULL, NULL, 8, NULL, NULL, NULL, NULL),
           SKA_ERR_INVALID);
    ska_free(NULL);
    printf("host library under sanitizers: %s (%d unexpected results)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
