/*
 * sanitize_main.c -- drives every entry point of the CPU oracle
 * (ska_oracle.c) on small seeded inputs, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds and runs
 * it; TEST INFRASTRUCTURE ONLY).  It checks nothing numerically: the point
 * is that no access leaves its buffer and no operation is undefined, on
 * pools laid out as the decode reads them (shuffled pages, mixed tiers,
 * page offsets, partial pages, per-(page, KV head) tiers, an empty row).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ora_polar_code(double x, double S, int b);
int ora_azimuth_code(double x, double y, int b);
void ora_angles(const float *x, int d, double *phi, double *T0);
void ora_unit_from_angles(const double *phi, int d, double *u);
double ora_key_codes(const float *x, int d, int b, int32_t *codes);
void ora_direction(const int32_t *codes, int d, int b, double *u);
void ora_radius_tables(int mode, double rlo, double rhi, double *level, double *tau2);
int ora_radius_code(double S, const double *tau2);
void ora_calibrate(const float *keys, int64_t n, int hkv, int d, double *range);
int ora_kb(int d, int b);
int ora_pack(const int32_t *codes, int d, int b, uint8_t *rec);
void ora_unpack(const uint8_t *rec, int d, int b, int32_t *codes);
int ora_encode(int d, int hkv, int radius_mode, const double *range, const uint8_t *page_bits,
               const uint64_t *page_off, int bstride, int head_tiers, uint8_t *kcode, uint8_t *rcode, uint16_t *v,
               const float *keys, const uint16_t *values, const int64_t *slot, int64_t n);
int ora_decode(int d, int hkv, int radius_mode, const double *range, const uint8_t *page_bits,
               const uint64_t *page_off, int bstride, int head_tiers, const uint8_t *kcode, const uint8_t *rcode,
               const uint16_t *v, const float *q, int B, int hq, const int32_t *block_table, int max_pages,
               const int32_t *seq_lens, double scale, int query_mode, float *out, float *logits,
               const int32_t *pairs, int npairs, int nthreads);
int ora_decoded_keys(int d, int hkv, int radius_mode, const double *range, const uint8_t *page_bits,
                     const uint64_t *page_off, int bstride, int head_tiers, const uint8_t *kcode,
                     const uint8_t *rcode, const int32_t *phys, int nphys, double *out);
int ora_dense_decode(int d, int hkv, const uint16_t *k_dense, const uint16_t *v, const float *q, int B, int hq,
                     const int32_t *block_table, int max_pages, const int32_t *seq_lens, double scale, float *out,
                     float *logits, int nthreads);
int ora_rdr_plan(int n, const float *u, const float *knorm, const uint8_t *prot, int ntiers, const int *tiers,
                 const double *eps, const int64_t *bytes, int64_t budget, double sigma, uint8_t *tier_out,
                 int32_t *page_out, int32_t *slot_out, uint8_t *page_tier, int *npages, double *lambda_out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void)   /* xorshift64*, uniform in [0, 1) */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1.0p-53;
}
static float nrand(void)    /* roughly N(0, 1): sum of uniforms */
{
    double s = 0.0;
    for (int i = 0; i < 12; ++i)
        s += urand();
    return (float)(s - 6.0);
}

/* one pool case: B rows over shuffled pages, tiers from `tiers`, optional
 * page offsets, per-head tiers and partial pages */
static int run_case(int d, int hkv, int hq, int B, const int *lens, const int *tiers, int ntiers, int packed,
                    int head_tiers, int partial)
{
    int npg_tot = 0, max_pages = 1;
    for (int s = 0; s < B; ++s) {
        int np = (lens[s] + 15) / 16;
        npg_tot += np;
        if (np > max_pages)
            max_pages = np;
    }
    int num_pages = npg_tot + 2;
    int nh = head_tiers ? hkv : 1;
    uint8_t *hdr = malloc((size_t)num_pages * nh);
    for (int i = 0; i < num_pages * nh; ++i) {
        int b = tiers[(int)(urand() * ntiers)];
        int empty = (partial && urand() < 0.3) ? (int)(urand() * 16) : 0;
        hdr[i] = (uint8_t)(b | (empty << 4));
    }
    uint64_t *off = NULL;
    size_t kbytes;
    int bstride = 0;
    for (int k = 0; k < ntiers; ++k)
        if (tiers[k] > bstride)
            bstride = tiers[k];
    if (packed || head_tiers) {
        off = malloc(sizeof(uint64_t) * (size_t)num_pages * nh);
        size_t acc = 0;
        for (int i = 0; i < num_pages * nh; ++i) {
            off[i] = acc;
            acc += (size_t)(head_tiers ? 1 : hkv) * 16 * ora_kb(d, hdr[i] & 15);
        }
        kbytes = acc;
    } else {
        for (int i = 0; i < num_pages; ++i)
            hdr[i] = (uint8_t)(bstride | (hdr[i] & 0xF0));
        kbytes = (size_t)num_pages * hkv * 16 * ora_kb(d, bstride);
    }
    uint8_t *kcode = malloc(kbytes);
    uint8_t *rcode = malloc((size_t)num_pages * hkv * 16);
    uint16_t *v = malloc(sizeof(uint16_t) * (size_t)num_pages * hkv * d * 16);
    memset(kcode, 0xFF, kbytes);
    memset(rcode, 0xFF, (size_t)num_pages * hkv * 16);
    memset(v, 0, sizeof(uint16_t) * (size_t)num_pages * hkv * d * 16);
    int32_t *bt = calloc((size_t)B * max_pages, sizeof(int32_t));
    int n = 0;
    for (int s = 0; s < B; ++s)
        n += lens[s];
    int64_t *slot = malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    float *keys = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * hkv * d);
    uint16_t *vals = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1) * hkv * d);
    int *perm = malloc(sizeof(int) * (size_t)num_pages);
    for (int i = 0; i < num_pages; ++i)
        perm[i] = i;
    for (int i = num_pages - 1; i > 0; --i) {
        int j = (int)(urand() * (i + 1));
        int t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    int k = 0, o = 0;
    for (int s = 0; s < B; ++s) {
        int np = (lens[s] + 15) / 16;
        for (int p = 0; p < np; ++p)
            bt[(size_t)s * max_pages + p] = perm[k + p];
        for (int t = 0; t < lens[s]; ++t)
            slot[o + t] = (int64_t)perm[k + t / 16] * 16 + t % 16;
        k += np;
        o += lens[s];
    }
    for (size_t i = 0; i < (size_t)n * hkv * d; ++i) {
        keys[i] = nrand();
        vals[i] = (uint16_t)(0x3F80 + (int)(urand() * 256));
    }
    double range[2 * 64];
    ora_calibrate(keys, n, hkv, d, range);
    int bad = ora_encode(d, hkv, 1, range, hdr, off, bstride, head_tiers, kcode, rcode, v, keys, vals, slot, n);
    float *q = malloc(sizeof(float) * (size_t)B * hq * d);
    for (size_t i = 0; i < (size_t)B * hq * d; ++i)
        q[i] = nrand();
    float *out = malloc(sizeof(float) * (size_t)B * hq * d);
    float *lg = malloc(sizeof(float) * (size_t)B * hq * max_pages * 16);
    for (int qm = 0; qm < 2; ++qm)
        bad |= ora_decode(d, hkv, 1, range, hdr, off, bstride, head_tiers, kcode, rcode, v, q, B, hq, bt, max_pages,
                          lens, 0.0, qm, out, lg, NULL, 0, 2);
    int32_t pairs[4] = {0, 0, B - 1, hq - 1};
    bad |= ora_decode(d, hkv, 1, range, hdr, off, bstride, head_tiers, kcode, rcode, v, q, B, hq, bt, max_pages,
                      lens, 0.0, 0, out, NULL, pairs, 2, 1);
    double *dk = malloc(sizeof(double) * 2 * hkv * 16 * d);
    int32_t phys2[2] = {perm[0], perm[num_pages - 1]};
    ora_decoded_keys(d, hkv, 1, range, hdr, off, bstride, head_tiers, kcode, rcode, phys2, 2, dk);
    uint16_t *kd = calloc((size_t)num_pages * hkv * 16 * d, sizeof(uint16_t));
    bad |= ora_dense_decode(d, hkv, kd, v, q, B, hq, bt, max_pages, lens, 0.0, out, lg, 2);
    free(hdr); free(off); free(kcode); free(rcode); free(v); free(bt); free(slot); free(keys); free(vals);
    free(perm); free(q); free(out); free(lg); free(dk); free(kd);
    return bad;
}

int main(void)
{
    int bad = 0;
    /* codes, directions, radius, packing */
    for (int b = 1; b <= 8; ++b) {
        for (int i = 0; i < 200; ++i) {
            bad |= ora_polar_code(nrand(), fabs((double)nrand()), b) < 0;
            bad |= ora_azimuth_code(nrand(), nrand(), b) < 0;
        }
    }
    int ds[3] = {8, 64, 128};
    for (int di = 0; di < 3; ++di) {
        int d = ds[di];
        float x[128];
        double phi[127], u[128], T0;
        int32_t c[127], c2[127];
        uint8_t rec[256];
        for (int i = 0; i < d; ++i)
            x[i] = nrand();
        ora_angles(x, d, phi, &T0);
        ora_unit_from_angles(phi, d, u);
        int bs[5] = {2, 3, 4, 6, 8};
        for (int bi = 0; bi < 5; ++bi) {
            int b = bs[bi];
            ora_key_codes(x, d, b, c);
            ora_direction(c, d, b, u);
            if (ora_pack(c, d, b, rec) == 0) {
                ora_unpack(rec, d, b, c2);
                bad |= memcmp(c, c2, sizeof(int32_t) * (d - 1)) != 0;
            }
        }
    }
    double level[256], tau2[255];
    ora_radius_tables(0, 0.0, 3.0, level, tau2);
    ora_radius_tables(1, 0.5, 3.0, level, tau2);
    bad |= ora_radius_code(4.0, tau2) < 0;
    /* pools */
    int l1[3] = {37, 0, 16}, l2[2] = {200, 33}, l3[1] = {1};
    int t4[1] = {4}, tmix[4] = {2, 4, 6, 8}, t5[5] = {2, 3, 4, 6, 8};
    bad |= run_case(64, 1, 1, 3, l1, t4, 1, 0, 0, 0);
    bad |= run_case(128, 2, 8, 2, l2, tmix, 4, 1, 0, 1);
    bad |= run_case(128, 2, 4, 2, l2, t5, 5, 1, 1, 1);
    bad |= run_case(64, 4, 4, 1, l3, t4, 1, 0, 0, 1);
    /* RDR */
    int n = 700;
    float *uu = malloc(sizeof(float) * n), *kn = malloc(sizeof(float) * n);
    uint8_t *prot = calloc((size_t)n, 1), *tier = malloc((size_t)n), *pt = malloc((size_t)n / 16 + 8);
    int32_t *page = malloc(sizeof(int32_t) * n), *slot = malloc(sizeof(int32_t) * n);
    for (int i = 0; i < n; ++i) {
        uu[i] = (float)(urand() * 3.0);
        kn[i] = (float)(3.0 + 30.0 * urand());
    }
    prot[0] = prot[1] = 1;
    int tiers[4] = {2, 4, 6, 8};
    double eps[4] = {0.27, 0.058, 0.0145, 0.0037};
    int64_t byts[4] = {2312, 2568, 2824, 3080};
    int np = 0;
    double lam = 0.0;
    int st = ora_rdr_plan(n, uu, kn, prot, 4, tiers, eps, byts, (int64_t)(0.4 * n * 3080), 0.02, tier, page, slot,
                          pt, &np, &lam);
    bad |= st == 1;
    st = ora_rdr_plan(0, uu, kn, prot, 4, tiers, eps, byts, 0, 0.02, tier, page, slot, pt, &np, &lam);
    bad |= st == 1;
    free(uu); free(kn); free(prot); free(tier); free(pt); free(page); free(slot);
    printf("oracle under sanitizers: %s\n", bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}
