/*
 * ska.h -- C ABI of the Angle-Domain Attention (ADA) paged-decode library
 * for AMD MI355X (gfx950).
 *
 * Method: the technical summary in the page "SPHERICAL KV: Angle-Domain
 * Attention and Rate-Distortion Retention for Efficient Long-Context
 * Inference" (gist.science summary of arXiv 2605.18856).
 *   section 2.1  keys are split into a radius r = |k| and directional angles
 *                phi = Phi(k/|k|); the cache stores a quantised radius r~ and
 *                packed angle codes c; the decode kernel computes the logit
 *                |q| * r~ * f_b(c_q, c_k) from the codes, f_b a cosine
 *                similarity; no dense key is ever written to HBM.
 *   section 2.2  pages are tier-homogeneous (one bit width b per page) and
 *                read by header-guided streaming.
 *   section 2.3  dense keys are mapped to spherical codes and stored in a
 *                paged (vLLM-style) compressed store that the decode kernel
 *                consumes directly.
 *
 * Format (the pages leave it open; fixed here):
 *   Phi      hyperspherical coordinates: d-2 polar angles in [0, pi] and one
 *            azimuth in [0, 2*pi); suffix sums of squares in binary64,
 *            summed from the last component backwards.
 *   angles   b uniform bins over each angle's range, code = bin index,
 *            decided by binary64 predicates on squared quantities (ties to
 *            the upper bin); decoded at bin centres.
 *   radius   8 bits; uniform levels j*R_hi/255 or log-spaced levels over
 *            [R_lo, R_hi], rounded at the (linear or log) midpoint.
 *   record   KB(b) = 16*ceil((d-1)*b/128) bytes per key, four equal slices;
 *            slice s holds angles [s*d/4, (s+1)*d/4) LSB-first, rest zero.
 *   pools    page_bits[phys] (uint8)        page header: tier b of the page in
 *                                           the low four bits; the number of
 *                                           empty slots at the page's end in
 *                                           the high four (0: 16 tokens), so
 *                                           any page of a row may be partial
 *            kcode + base(phys)             [Hkv][16][KB(b)] records,
 *                                           base = page_off[phys] or
 *                                           phys*Hkv*16*KB(b_max of mask)
 *            rcode[phys][Hkv][16] (uint8)   radius codes
 *            v[phys][Hkv][d][16]  (bf16)    values, dimension-major in a page
 *            A slot is phys*16 + token-in-page.
 *
 * Memory: every pointer argument marked "device" is caller-owned device
 * memory (any allocator; PyTorch in the tests).  The library owns only what
 * it allocates inside a ska_cache (code tables, radius tables, the decode
 * workspace) and frees it in ska_free.  Everything a cache owns is
 * allocated when it is created (the first ska_encode_keys), the decode
 * workspace sized from the maxima the pool descriptor declares; no later
 * call on a cache allocates or frees device memory.
 *
 * Streams: `stream` is a hipStream_t (NULL = the null stream).  All work is
 * enqueued asynchronously on it.  Host synchronisation happens only in the
 * calibrating ska_encode_keys call (it reads the radius range back),
 * ska_device_errors, ska_profile_read, and ska_rdr_plan when its workspace
 * grows (see there).  The decode calls of one cache share its workspace and
 * merge counters, so they run one after another on the device: a decode call
 * on a different stream than the cache's previous decode call is ordered
 * after that call (an event recorded on the previous stream, waited on by
 * the new one; the previous stream must still exist).  Calls on one cache
 * from several host threads at once are not supported.
 *
 * Errors: arguments are checked on the host before any HIP call; a bad one
 * returns SKA_ERR_INVALID (or SKA_ERR_UNSUPPORTED for a legal but unbuilt
 * shape) with nothing enqueued.  Launch failures return SKA_ERR_HIP.  Pages
 * whose id or header is out of range are skipped by the kernels and flagged
 * in a device error word (ska_device_errors).  No C++ exception crosses this
 * ABI.  Calls on one ska_cache are not thread-safe.
 */
#ifndef SKA_H
#define SKA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SKA_OK = 0,
    SKA_ERR_INVALID = 1,
    SKA_ERR_UNSUPPORTED = 2,
    SKA_ERR_HIP = 3,
    SKA_ERR_NOMEM = 4
} ska_status;

enum { SKA_RADIUS_UNIFORM = 0, SKA_RADIUS_LOG = 1 };
enum { SKA_Q_CODED = 0, SKA_Q_EXACT = 1 };
enum { SKA_QDIR_F16 = 0, SKA_QDIR_F32 = 1 };
enum { SKA_PAGE_SIZE = 16 };

/* Device error flags (ska_device_errors). */
enum {
    SKA_DEVERR_SLOT = 1u,     /* encode: slot outside the pool */
    SKA_DEVERR_PAGE = 2u,     /* decode: block-table entry outside the pool */
    SKA_DEVERR_TIER = 4u      /* page_bits value not in tier_mask */
};

typedef struct ska_cache ska_cache; /* opaque, library-owned */

/* Caller-owned device pools (see the format above). */
typedef struct {
    int d;                    /* head dimension: 64 or 128 */
    int num_kv_heads;         /* Hkv >= 1 */
    int page_size;            /* must be 16 */
    int64_t num_pages;        /* physical pages in the pool */
    int radius_mode;          /* SKA_RADIUS_UNIFORM or SKA_RADIUS_LOG */
    int radius_bits;          /* must be 8 */
    uint32_t tier_mask;       /* bit b set => pages of b-bit angles allowed, b in {2,3,4,6,8} */
    int query_mode;           /* SKA_Q_CODED: query angle-coded at each page's tier (f_b of two
                                 codes); SKA_Q_EXACT: exact query direction */
    uint8_t *kcode;           /* device: code records */
    const uint64_t *page_off; /* device [num_pages] byte offsets (multiples of 16) or NULL */
    uint8_t *rcode;           /* device: [num_pages][Hkv][16] */
    uint16_t *v;              /* device: bf16 [num_pages][Hkv][d][16] */
    const uint8_t *page_bits; /* device: [num_pages] */
    int head_tiers;           /* 0: one tier per page (page_bits, page_off as above);
                                 1: one tier per (page, KV head) (section 2.2 allocates per
                                 token, head and layer): page_bits [num_pages][Hkv] holds
                                 the header of each KV head's 16 records and page_off
                                 (required) [num_pages][Hkv] their byte offset */
    int query_precision;      /* precision of the query direction inside f_b (section 2.1's
                                 logit |q| r~ f_b): SKA_QDIR_F16 (default) rounds it to binary16,
                                 which moves a logit by at most 2^-11 (typically ~1e-4 at
                                 d = 128) of its bound scale*|q|*r~; SKA_QDIR_F32 keeps binary32
                                 (for keys with outlier channels, whose large radii turn that
                                 into large output errors; on MI355X about 4 % slower on a
                                 pool of one tier at d = 128 with 4 query heads per KV head,
                                 about 40 % slower on a pool of mixed tiers) */
    /* Maxima of the decode calls on this cache, fixed when it is created:
       they size the decode workspace (split partials and merge counters),
       which is allocated then and never again.  A decode call outside them
       returns SKA_ERR_INVALID. */
    int max_batch;            /* >= 1: sequences per call */
    int max_heads_q;          /* >= 1: query heads per call */
    int max_pages;            /* >= 1: block-table row length */
    int max_splits;           /* >= 0: largest explicit num_splits (0: automatic only) */
} ska_pool_desc;

/* ska_encode_keys -- the write path of section 2.3: map dense keys to
 * spherical codes (section 2.1) and store them, with their values, in the
 * paged pools.
 *   cache   in/out.  *cache == NULL creates a cache for `pool` (tables and
 *           the decode workspace for the pool's declared maxima); otherwise
 *           the pool must have the same shape, precision and maxima fields
 *           as at creation.
 *   keys    device fp32 [n][Hkv][d]
 *   values  device bf16 [n][Hkv][d] or NULL (values not written)
 *   slot    device int64 [n]: phys*16 + token-in-page for each key
 *   radius_range  host [Hkv][2] = (R_lo, R_hi) or NULL.  On creation with
 *           NULL the range is calibrated per KV head over these keys
 *           (R_hi = max |k|, R_lo = min positive |k|); this synchronises.
 *           Ignored when the cache already exists.
 * Each key is encoded at the tier page_bits[slot/16].  Returns SKA_OK. */
ska_status ska_encode_keys(ska_cache **cache, const ska_pool_desc *pool,
                           const float *keys, const uint16_t *values,
                           const int64_t *slot, int64_t n,
                           const double *radius_range, void *stream);

/* ska_decode_attention -- one ADA decode step over a page table (section 2.1
 * logit estimator, section 2.2 header-guided page streaming): for sequence s
 * and query head h (KV head h / (Hq/Hkv)), the logits
 *     l_t = scale * |q| * r~_t * f_b(c_q, c_t)
 * over the resident tokens of row s: position t < seq_lens[s] is page t/16
 * of row s of the block table, slot t%16, and holds a token when that slot
 * is below the page's count (its header); then softmax over them and the
 * value-weighted sum.
 *   q            device fp32 [batch][num_q_heads][d]
 *   block_table  device int32 [batch][max_pages]
 *   seq_lens     device int32 [batch] (0 gives a zero output row)
 *   scale        softmax scale; 0 means 1/sqrt(d)
 *   num_splits   page splits per sequence (split-T).  > 0: that many
 *                equal splits of max_pages pages.  0 (automatic): equal
 *                splits sized for one workgroup per CU when the (sequence,
 *                KV head) groups do not fill the CUs on their own; else
 *                splits of 384, 384, then 768 pages each (capped at
 *                max_pages), handed out in decreasing size.  Results agree
 *                across split counts to rounding.
 *   out          device fp32 [batch][num_q_heads][d]
 *   logits_dbg   device fp32 [batch][num_q_heads][max_pages*16] or NULL;
 *                receives l_t (natural units) at each resident position t
 *                (other positions are left as they are)
 *                (the same kernel as without it, plus the logit stores)
 * Hq/Hkv must be 1, 2 or 4.  batch, num_q_heads, max_pages and an explicit
 * num_splits must lie within the cache's declared maxima (else
 * SKA_ERR_INVALID, nothing enqueued).  Allocates nothing.  Returns SKA_OK. */
ska_status ska_decode_attention(const ska_cache *cache, const float *q, int batch, int num_q_heads,
                                const int32_t *block_table, int max_pages,
                                const int32_t *seq_lens, float scale, int num_splits,
                                float *out, float *logits_dbg, void *stream);

/* ska_decode_attention_noalloc -- for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): ska_decode_attention (without logits_dbg) with its split
 * partials, merge counters and unit order in a static device array of the library
 * (16 MiB per GPU, kept until the process ends) instead of the cache's
 * workspace.  Allocates nothing and frees nothing; the first call on a GPU
 * looks the array up and clears its counters with a small kernel on
 * `stream`.  Rejects with SKA_ERR_INVALID, before enqueueing anything, a
 * call whose partials (batch * num_q_heads * splits rows of (d + 2) floats)
 * exceed 16 MiB - 384 KiB or whose batch * Hkv exceeds 65536, and anything
 * ska_decode_attention rejects.  Every call on one GPU shares that GPU's
 * array: calls that overlap on the device (different streams, not ordered
 * by the caller) race and give wrong results.  Results equal
 * ska_decode_attention's. */
ska_status ska_decode_attention_noalloc(const ska_cache *cache, const float *q, int batch, int num_q_heads,
                                        const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                                        float scale, int num_splits, float *out, void *stream);

/* ska_append_decode_attention -- a decode step that first stores the step's
 * new token (the write path of section 2.3, dense key -> spherical codes ->
 * paged store, run inside the step), then decodes over all tokens including
 * it, exactly as ska_decode_attention.
 *   new_keys    device fp32 [batch][Hkv][d]: the new token's key of each
 *               sequence
 *   new_values  device bf16 [batch][Hkv][d]: its values
 *   seq_lens    device int32 [batch]: lengths including the new token; the
 *               new token of sequence s goes to position seq_lens[s] - 1
 *               (page block_table[s][(seq_lens[s]-1)/16], slot
 *               (seq_lens[s]-1)%16), encoded at that page's tier
 *               (page_bits, and page_off for variable-size pages, must be
 *               set for a new page first).  seq_lens[s] <= 0 appends nothing.
 *   other arguments as ska_decode_attention.
 * One kernel on `stream`: inside the decode, the wave that reads the new
 * token's page for a KV head first stores the token there (codes, radius
 * code, values, as ska_encode_keys would at the cache's radius range).  A
 * position past the row or a block-table entry outside the pool sets
 * SKA_DEVERR_SLOT (nothing is stored for that sequence); a page header
 * outside tier_mask sets SKA_DEVERR_TIER.  Argument errors are those of
 * ska_decode_attention, plus SKA_ERR_INVALID for NULL new_keys/new_values
 * with batch > 0; a rejected call stores nothing.  Returns SKA_OK. */
ska_status ska_append_decode_attention(const ska_cache *cache, const float *new_keys, const uint16_t *new_values,
                                       const float *q, int batch, int num_q_heads,
                                       const int32_t *block_table, int max_pages,
                                       const int32_t *seq_lens, float scale, int num_splits,
                                       float *out, float *logits_dbg, void *stream);

/* ska_dense_decode_attention -- the baseline the codes replace (section 1 of
 * the page: decode streams dense KV pages from HBM): the same decode step as
 * ska_decode_attention over keys stored densely as bf16, with the cache's
 * values, workspace and split policy; the logits are the plain
 *     l_t = scale * sum_e q_e k_t,e
 * (no codes, no radius).  For comparing bytes and time on the same pages.
 *   k_dense  device bf16 [num_pages][Hkv][16][d]: token-major within a page
 *            (the 16 slots of one KV head, d values each), filled by the
 *            caller or by ska_decompress_keys; read, never written
 *   other arguments as ska_decode_attention.
 * Returns SKA_ERR_INVALID for a NULL k_dense; errors as ska_decode_attention. */
ska_status ska_dense_decode_attention(const ska_cache *cache, const uint16_t *k_dense, const float *q, int batch,
                                      int num_q_heads, const int32_t *block_table, int max_pages,
                                      const int32_t *seq_lens, float scale, int num_splits, float *out,
                                      float *logits_dbg, void *stream);

/* ska_decompress_keys -- the "decompress" step of the decompress-then-dot
 * path that section 1 of the page sets against ADA: writes the dense key
 * each stored record stands for, r~ * u(c) (section 2.1), rounded to bf16,
 * for every slot of every resident page (pages 0 .. ceil(seq_lens[s]/16)-1 of
 * each row of the block table) and every KV head, into k_dense (layout as in
 * ska_dense_decode_attention; other pages are left untouched).  Pages whose
 * id or header is out of range are skipped and flagged (ska_device_errors).
 * batch is at most 65535 and max_pages at most 64 * 65535.  Returns SKA_OK. */
ska_status ska_decompress_keys(const ska_cache *cache, const int32_t *block_table, int batch, int max_pages,
                               const int32_t *seq_lens, uint16_t *k_dense, void *stream);

/* Rate-distortion retention parameters (section 2.2 of the page): the tier
 * set B with, per tier, the angular error of f_b (the distortion surrogate:
 * ADA's logit error grows with it, scaled by the query and key magnitudes)
 * and the bytes one retained state occupies. */
typedef struct {
    int ntiers;           /* 1..8 */
    int tiers[8];         /* increasing widths, each in 1..8 */
    double eps[8];        /* angular error of each tier, >= 0 */
    int64_t bytes[8];     /* bytes of one retained state at each tier, > 0, non-decreasing */
    double sigma;         /* >= 0: query magnitude and softmax scale folded into the surrogate */
} ska_rdr_params;

/* ska_rdr_plan -- the RDR controller of section 2.2 of the page: for every
 * state i (token) of each sequence, a residency and a tier under the
 * sequence's byte budget, protected states kept at the widest tier, and the
 * retained states grouped into tier-homogeneous pages for the decode
 * kernel's header-guided streaming.
 * Distortion surrogate (a reading; the page gives no formula): evicting i
 * costs its utility u_i; keeping it at tier k costs
 *     u_i * min(1, sigma * key_norm_i * eps_k).
 * The plan takes, state by state, the option of least D + lambda * bytes
 * (ties: evict, then the narrower tier) for the smallest multiplier lambda
 * reached by 64 bisection steps whose plan fits the budget; by Everett's
 * theorem no plan using no more bytes has a smaller total distortion.
 * Retained states are packed tier by tier (tiers in increasing order),
 * states in index order, 16 per page.  All arrays are device memory.
 *   utility, key_norm  fp32 [batch][max_states];  protect uint8 [batch][max_states]
 *   num_states int32 [batch] (states used in each row);  budget int64 [batch] bytes
 *   tier_out   uint8 [batch][max_states]: 0 = evicted, else the tier's width
 *   page_out, slot_out  int32 [batch][max_states]: page and slot of each
 *              retained state, -1 when evicted
 *   page_tier_out  uint8 [batch][max_pages_out]: the header of each page
 *              (page_bits format: the width in the low four bits; each tier's
 *              last page has its empty slots in the high four), so a row of
 *              the planned pages decodes as one sequence;
 *              max_pages_out >= ceil(max_states/16) + ntiers
 *   npages_out int32 [batch], lambda_out double [batch],
 *   status_out int32 [batch]: 0, or 2 when the protected states alone exceed
 *              the budget (they are kept and every other state is evicted)
 * Decisions are binary64 comparisons made as written (no contraction), so
 * the plan is reproducible bit for bit.  The library keeps a device
 * workspace for this call per device (allocated on first use, about
 * batch * (2.5 KB + 32 B per 512 states), at least 1 MiB; growing it synchronises the
 * device); calls that overlap on one device must not run concurrently.
 * Returns SKA_OK, SKA_ERR_INVALID on a bad parameter or size,
 * SKA_ERR_UNSUPPORTED for batch > 65535, SKA_ERR_HIP if the workspace
 * cannot be allocated. */
ska_status ska_rdr_plan(const ska_rdr_params *params, const float *utility, const float *key_norm,
                        const uint8_t *protect, const int32_t *num_states, const int64_t *budget, int batch,
                        int max_states, uint8_t *tier_out, int32_t *page_out, int32_t *slot_out,
                        uint8_t *page_tier_out, int max_pages_out, int32_t *npages_out, double *lambda_out,
                        int32_t *status_out, void *stream);

/* The radius range in use (host [Hkv][2] = (R_lo, R_hi)). */
ska_status ska_get_radius_range(const ska_cache *cache, double *range_out);

/* OR of the device error flags raised since the last call, then cleared.
 * Synchronises `stream`. */
ska_status ska_device_errors(ska_cache *cache, void *stream, uint32_t *flags_out);

/* Kernel timing, for measuring the decode kernel's achieved HBM throughput
 * on the paged store (sections 1 and 4 of the page weigh the method by HBM
 * traffic per generated token): ska_profile_begin makes the next `max_calls`
 * ska_decode_attention calls on this cache record two HIP events on their
 * stream, around the decode kernel (query preparation, paged decode and split
 * merge); 0 stops recording.  The events skip the system-scope fence, but
 * each pair still adds its markers' dispatch latency to the gap between calls
 * and to the recorded figure (a few microseconds per call on MI355X); for the
 * average of back-to-back calls, time a run of calls between two events
 * instead.  ska_profile_read waits for the recorded
 * events and writes ms_out[i] for call i, *n_out = calls recorded (at most
 * max_calls). */
ska_status ska_profile_begin(ska_cache *cache, int max_calls);
ska_status ska_profile_read(ska_cache *cache, float *ms_out, int max_calls, int *n_out);

/* Release everything the cache owns.  Accepts NULL. */
void ska_free(ska_cache *cache);

const char *ska_status_string(ska_status s);

#ifdef __cplusplus
}
#endif

#endif /* SKA_H */
