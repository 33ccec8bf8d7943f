/*
 * ska_oracle.c -- plain, slow fp64 CPU oracle for Angle-Domain Attention (ADA)
 * decode over a paged, tier-homogeneous KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  The product path (the HIP library under
 * long_context_decode_ada_amd/) never calls it, and the two share no source:
 * no headers, tables, helpers or constant generators.
 *
 * Source of the method.  [SKV] below is the technical summary in the page
 * "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion Retention for
 * Efficient Long-Context Inference" (gist.science summary of arXiv 2605.18856;
 * Spanish, French and German versions agree).  Sections cited:
 *   [SKV 1]    problem statement: paged KV, decode streams KV pages from HBM;
 *              the "decompress-then-dot-product" path.
 *   [SKV 2.1]  ADA: spherical parametrisation r = |k|, phi = Phi(k/|k|);
 *              stored quantised radius r~ and packed angle codes c;
 *              logit estimator  l ~= |q| * r~ * f_b(c_q, c_k), f_b a cosine
 *              similarity computed from the codes; no dense key in HBM.
 *   [SKV 2.2]  RDR: per-state tier b in a set B, residency z; tier-homogeneous
 *              pages read by header-guided streaming.
 *   [SKV 2.3]  system integration: dense keys -> spherical codes -> paged,
 *              compressed store consumed directly by the decode kernel.
 *
 * The pages do not define Phi, the quantisers or the byte layout.  The
 * readings taken here (hyperspherical angles, uniform b-bit bins with
 * predicates on squared quantities, 8-bit uniform or log radius, four-slice
 * records) are listed with reasons in the repository's design notes.  This
 * file is the plain definition of each step: no blocking, no fusion.
 *
 * Arithmetic: IEEE binary64, round-to-nearest-even, compiled with
 * -ffp-contract=off and -fno-builtin so that every product and sum is rounded
 * exactly as written.  Each x^2 of a binary32 input is exact in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_UNIFORM 0
#define ORA_LOG 1
#define ORA_Q_CODED 0
#define ORA_Q_EXACT 1
#define ORA_PAGE 16

/* ------------------------------------------------------------------------ */
/* Angle thresholds.  Bin edges theta_j = j*pi/2^b, j = 1..2^b-1.
 * cos2[j] = cos(theta_j)^2, sin2[j] = sin(theta_j)^2, computed with the host
 * libm; theta_j = ldexp(j * pi_double, -b) (the scaling is exact).
 * [SKV 2.1] says only that angles are quantised to b bits; uniform bins over
 * the angle's range is the plain reading. */
void ora_angle_thresholds(int b, double *cos2, double *sin2)
{
    int n = 1 << b;
    cos2[0] = 1.0;
    sin2[0] = 0.0;
    for (int j = 1; j < n; ++j) {
        double th = ldexp((double)j * M_PI, -b);
        double c = cos(th);
        double s = sin(th);
        cos2[j] = c * c;
        sin2[j] = s * s;
    }
}

/* Predicate "phi >= theta_j" for phi = atan2(sqrt(S), x) in [0, pi], decided
 * on squared quantities so that no sqrt/atan2 rounding enters the decision.
 *   theta_j <  pi/2:  x <= 0  or  cos2*S >= sin2*x^2
 *   theta_j == pi/2:  x <= 0
 *   theta_j >  pi/2:  x <  0  and cos2*S <= sin2*x^2                       */
static int ge_theta(double x, double S, int j, int b, const double *cos2, const double *sin2)
{
    int n = 1 << b;
    double x2 = x * x;
    if (2 * j < n)
        return (x <= 0.0) || (cos2[j] * S >= sin2[j] * x2);
    if (2 * j == n)
        return x <= 0.0;
    return (x < 0.0) && (cos2[j] * S <= sin2[j] * x2);
}

/* Polar code of phi = atan2(sqrt(S), x): the number of bin edges at or below
 * phi, i.e. floor(phi * 2^b / pi) clamped to 2^b - 1, ties to the upper bin.
 * A zero 2-vector (x == 0, S == 0) has phi = 0 and code 0.  Counts over every
 * edge (no search).  [SKV 2.1] angle codes c. */
int ora_polar_code_t(double x, double S, int b, const double *cos2, const double *sin2)
{
    if (x == 0.0 && S == 0.0)
        return 0;
    int n = 1 << b, code = 0;
    for (int j = 1; j < n; ++j)
        code += ge_theta(x, S, j, b, cos2, sin2);
    return code;
}

/* Azimuth code of phi = atan2(y, x) mod 2*pi over [0, 2*pi) with 2^b bins:
 * the lower half plane (y < 0, or y == 0 and x < 0) is rotated by pi into the
 * upper one, which is binned like a polar angle at b-1 bits. */
int ora_azimuth_code_t(double x, double y, int b, const double *cos2h, const double *sin2h)
{
    if (x == 0.0 && y == 0.0)
        return 0;
    int h = (y < 0.0) || (y == 0.0 && x < 0.0);
    double xp = h ? -x : x;
    double yp = h ? -y : y;
    return h * (1 << (b - 1)) + ora_polar_code_t(xp, yp * yp, b - 1, cos2h, sin2h);
}

/* Convenience forms that build their own tables (slow; used by tests). */
int ora_polar_code(double x, double S, int b)
{
    double *c2 = malloc(sizeof(double) << b), *s2 = malloc(sizeof(double) << b);
    ora_angle_thresholds(b, c2, s2);
    int r = ora_polar_code_t(x, S, b, c2, s2);
    free(c2);
    free(s2);
    return r;
}

int ora_azimuth_code(double x, double y, int b)
{
    double *c2 = malloc(sizeof(double) << b), *s2 = malloc(sizeof(double) << b);
    ora_angle_thresholds(b - 1, c2, s2);
    int r = ora_azimuth_code_t(x, y, b, c2, s2);
    free(c2);
    free(s2);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Spherical parametrisation [SKV 2.1], hyperspherical coordinates of x in R^d
 * (0-based components x[0..d-1]):
 *   T[i] = sum_{k >= i} x[k]^2, summed backwards: T[d-1] = x[d-1]^2,
 *          T[i] = T[i+1] + x[i]^2  (this order is part of the format);
 *   r = sqrt(T[0]);
 *   polar angles a = 0..d-3:  phi_a = atan2(sqrt(T[a+1]), x[a])  in [0, pi];
 *   azimuth     a = d-2:      phi_a = atan2(x[d-1], x[d-2]) mod 2*pi.
 * Continuous form, used only by the invertibility checks. */
void ora_angles(const float *x, int d, double *phi, double *T0)
{
    double T = (double)x[d - 1] * (double)x[d - 1];
    double az = atan2((double)x[d - 1], (double)x[d - 2]);
    if (az < 0.0)
        az += 2.0 * M_PI;
    phi[d - 2] = az;
    T = T + (double)x[d - 2] * (double)x[d - 2];
    for (int a = d - 3; a >= 0; --a) {
        phi[a] = atan2(sqrt(T), (double)x[a]);
        T = T + (double)x[a] * (double)x[a];
    }
    *T0 = T;
}

/* Unit vector of hyperspherical angles (the inverse of Phi):
 *   u[a] = (prod_{k<a} sin phi_k) * cos phi_a,  a = 0..d-2,
 *   u[d-1] = (prod_{k<d-1} sin phi_k).                                      */
void ora_unit_from_angles(const double *phi, int d, double *u)
{
    double P = 1.0;
    for (int a = 0; a < d - 1; ++a) {
        u[a] = P * cos(phi[a]);
        P = P * sin(phi[a]);
    }
    u[d - 1] = P;
}

/* Threshold tables for tier b and for b-1 (the azimuth's half plane). */
typedef struct {
    int b;
    double *c2, *s2, *c2h, *s2h;
} ora_tables;

static void tables_init(ora_tables *t, int b)
{
    size_t n = (size_t)1 << b;
    t->b = b;
    t->c2 = malloc(sizeof(double) * n);
    t->s2 = malloc(sizeof(double) * n);
    t->c2h = malloc(sizeof(double) * n);
    t->s2h = malloc(sizeof(double) * n);
    ora_angle_thresholds(b, t->c2, t->s2);
    ora_angle_thresholds(b - 1, t->c2h, t->s2h);
}

static void tables_free(ora_tables *t)
{
    free(t->c2);
    free(t->s2);
    free(t->c2h);
    free(t->s2h);
}

/* Angle codes of one vector at b bits [SKV 2.1]: c_a = Q_b(phi_a), exact
 * predicates, same backward sum as ora_angles.  Returns T[0] = |x|^2. */
static double key_codes_t(const float *x, int d, const ora_tables *t, int32_t *codes)
{
    int b = t->b;
    double T = (double)x[d - 1] * (double)x[d - 1];
    codes[d - 2] = ora_azimuth_code_t((double)x[d - 2], (double)x[d - 1], b, t->c2h, t->s2h);
    T = T + (double)x[d - 2] * (double)x[d - 2];
    for (int a = d - 3; a >= 0; --a) {
        codes[a] = ora_polar_code_t((double)x[a], T, b, t->c2, t->s2);
        T = T + (double)x[a] * (double)x[a];
    }
    return T;
}

double ora_key_codes(const float *x, int d, int b, int32_t *codes)
{
    ora_tables t;
    tables_init(&t, b);
    double T = key_codes_t(x, d, &t, codes);
    tables_free(&t);
    return T;
}

/* Bin centres: polar (c + 1/2) * pi / 2^b, azimuth (c + 1/2) * 2*pi / 2^b. */
static double polar_centre(int c, int b) { return ((double)c + 0.5) * M_PI / (double)(1 << b); }
static double azimuth_centre(int c, int b) { return ((double)c + 0.5) * 2.0 * M_PI / (double)(1 << b); }

/* Decoded unit direction u(centres(c)) of a code vector. */
void ora_direction(const int32_t *codes, int d, int b, double *u)
{
    double *phi = malloc(sizeof(double) * (size_t)d);
    for (int a = 0; a < d - 2; ++a)
        phi[a] = polar_centre(codes[a], b);
    phi[d - 2] = azimuth_centre(codes[d - 2], b);
    ora_unit_from_angles(phi, d, u);
    free(phi);
}

/* ------------------------------------------------------------------------ */
/* Radius quantiser, 8 bits [SKV 2.1] "quantised radius r~".
 *   uniform on [0, R_hi]:  level_j = (j*R_hi)/255,  edge_j = ((j+1/2)*R_hi)/255
 *   log on [R_lo, R_hi]:   L = ln R_lo, U = ln R_hi,
 *                          level_j = exp(L + (j*(U-L))/255),
 *                          edge_j  = exp(L + ((j+1/2)*(U-L))/255)
 * tau2[j] = edge_j^2 (j = 0..254); code = #{j : |x|^2 >= tau2[j]}.
 * R_hi <= 0 makes every level and edge 0.  In log mode R_lo <= 0 is read as
 * R_lo = R_hi. */
void ora_radius_tables(int mode, double rlo, double rhi, double *level, double *tau2)
{
    if (!(rhi > 0.0)) {
        for (int j = 0; j < 256; ++j)
            level[j] = 0.0;
        for (int j = 0; j < 255; ++j)
            tau2[j] = 0.0;
        return;
    }
    if (mode == ORA_UNIFORM) {
        for (int j = 0; j < 256; ++j)
            level[j] = ((double)j * rhi) / 255.0;
        for (int j = 0; j < 255; ++j) {
            double e = (((double)j + 0.5) * rhi) / 255.0;
            tau2[j] = e * e;
        }
    } else {
        if (!(rlo > 0.0))
            rlo = rhi;
        double L = log(rlo), U = log(rhi);
        for (int j = 0; j < 256; ++j)
            level[j] = exp(L + ((double)j * (U - L)) / 255.0);
        for (int j = 0; j < 255; ++j) {
            double e = exp(L + (((double)j + 0.5) * (U - L)) / 255.0);
            tau2[j] = e * e;
        }
    }
}

int ora_radius_code(double S, const double *tau2)
{
    int c = 0;
    for (int j = 0; j < 255; ++j)
        c += (S >= tau2[j]);
    return c;
}

/* Radius range per KV head over a set of keys [n][hkv][d]:
 * R_hi = sqrt(max |k|^2), R_lo = sqrt(min positive |k|^2) (R_hi if none). */
void ora_calibrate(const float *keys, int64_t n, int hkv, int d, double *range)
{
    for (int g = 0; g < hkv; ++g) {
        double smax = 0.0, smin = INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            const float *x = keys + ((size_t)i * hkv + g) * d;
            double T = (double)x[d - 1] * (double)x[d - 1];
            for (int a = d - 2; a >= 0; --a)
                T = T + (double)x[a] * (double)x[a];
            if (T > smax)
                smax = T;
            if (T > 0.0 && T < smin)
                smin = T;
        }
        double rhi = sqrt(smax);
        range[2 * g + 0] = (smin < INFINITY) ? sqrt(smin) : rhi;
        range[2 * g + 1] = rhi;
    }
}

/* ------------------------------------------------------------------------ */
/* Record layout (format choice; [SKV 2.1] says only "packed angle codes").
 * A key's record has KB(b) = 16*ceil((d-1)*b/128) bytes split into four equal
 * slices of KB/4 bytes.  Slice s holds the codes of angles
 * a in [s*d/4, min((s+1)*d/4, d-1)), code a at bit (a - s*d/4)*b of the
 * slice, least significant bit first (bit k is bit k%8 of byte k/8).  Every
 * other bit is zero.  Requires d % 4 == 0 and 2*KB >= d*b. */
int ora_kb(int d, int b) { return 16 * (((d - 1) * b + 127) / 128); }

int ora_pack(const int32_t *codes, int d, int b, uint8_t *rec)
{
    int kb = ora_kb(d, b), sb = kb / 4, na = d / 4;
    if (d % 4 != 0 || 8 * sb < na * b)
        return 1;
    memset(rec, 0, (size_t)kb);
    for (int a = 0; a < d - 1; ++a) {
        int s = a / na;
        int bit = (a - s * na) * b;
        for (int k = 0; k < b; ++k) {
            int v = (codes[a] >> k) & 1;
            int pos = bit + k;
            rec[s * sb + pos / 8] |= (uint8_t)(v << (pos % 8));
        }
    }
    return 0;
}

void ora_unpack(const uint8_t *rec, int d, int b, int32_t *codes)
{
    int kb = ora_kb(d, b), sb = kb / 4, na = d / 4;
    for (int a = 0; a < d - 1; ++a) {
        int s = a / na;
        int bit = (a - s * na) * b;
        int c = 0;
        for (int k = 0; k < b; ++k) {
            int pos = bit + k;
            c |= ((rec[s * sb + pos / 8] >> (pos % 8)) & 1) << k;
        }
        codes[a] = c;
    }
}

/* ------------------------------------------------------------------------ */
/* Paged pools (format choice; [SKV 1] paged KV substrate, [SKV 2.2]
 * tier-homogeneous pages with a header, [SKV 2.3] vLLM-style layouts).
 *   page_bits[phys]         : the page header: angle bits b of every key in
 *                             the page in the low four bits; in the high four
 *                             bits the number of empty slots at the end of the
 *                             page (0: all 16 slots hold tokens), so that a
 *                             page may hold fewer than 16 retained tokens
 *                             anywhere in a row ([SKV 2.2]: retained states
 *                             grouped into tier-homogeneous pages)
 *   kcode + base(phys)      : [hkv][16 tokens][KB(b)] records;
 *                             base = page_off[phys] if page_off != NULL,
 *                             else phys * hkv * 16 * KB(bstride)
 *   rcode[phys][hkv][16]    : radius codes
 *   v[phys][hkv][d][16]     : bf16 values, dimension-major inside a page
 * A slot is phys*16 + token-in-page.
 * With head_tiers set, the tier is per (page, KV head) instead ([SKV 2.2]
 * allocates per token, head and layer): page_bits[phys*hkv + g] is the
 * header of KV head g's 16 records in the page, which start at
 * kcode + page_off[phys*hkv + g] (page_off required). */
static size_t page_base(int64_t phys, int hkv, int d, const uint64_t *page_off, int bstride)
{
    if (page_off)
        return (size_t)page_off[phys];
    return (size_t)phys * (size_t)hkv * ORA_PAGE * (size_t)ora_kb(d, bstride);
}

static int header_of(const uint8_t *page_bits, int head_tiers, int64_t phys, int hkv, int g)
{
    return head_tiers ? page_bits[(size_t)phys * hkv + g] : page_bits[phys];
}

/* tier of KV head g's records in page phys */
static int tier_of(const uint8_t *page_bits, int head_tiers, int64_t phys, int hkv, int g)
{
    return header_of(page_bits, head_tiers, phys, hkv, g) & 15;
}

/* slots of page phys (KV head g) that hold tokens: slots 0 .. count-1 */
static int count_of(const uint8_t *page_bits, int head_tiers, int64_t phys, int hkv, int g)
{
    return ORA_PAGE - (header_of(page_bits, head_tiers, phys, hkv, g) >> 4);
}

/* byte offset of the record of (page phys, KV head g, slot), kb bytes each */
static size_t rec_off(int64_t phys, int g, int slot, int kb, int hkv, int d, const uint64_t *page_off,
                      int bstride, int head_tiers)
{
    if (head_tiers)
        return (size_t)page_off[(size_t)phys * hkv + g] + (size_t)slot * kb;
    return page_base(phys, hkv, d, page_off, bstride) + ((size_t)g * ORA_PAGE + slot) * kb;
}

/* Encode keys (and scatter values) into the pools: the step "dense keys ->
 * spherical codes -> compressed store" of [SKV 2.3].  keys [n][hkv][d] fp32,
 * values [n][hkv][d] bf16 bits or NULL, slot[n].  range[hkv][2] = (R_lo, R_hi).
 * Returns 0, or 1 on a bad argument. */
int ora_encode(int d, int hkv, int radius_mode, const double *range,
               const uint8_t *page_bits, const uint64_t *page_off, int bstride, int head_tiers,
               uint8_t *kcode, uint8_t *rcode, uint16_t *v,
               const float *keys, const uint16_t *values, const int64_t *slot, int64_t n)
{
    if (d < 8 || d % 4 != 0 || hkv <= 0 || n < 0 || (head_tiers && !page_off))
        return 1;
    double *level = malloc(sizeof(double) * 256 * (size_t)hkv);
    double *tau2 = malloc(sizeof(double) * 255 * (size_t)hkv);
    for (int g = 0; g < hkv; ++g)
        ora_radius_tables(radius_mode, range[2 * g], range[2 * g + 1], level + 256 * g, tau2 + 255 * g);
    ora_tables *tab = malloc(sizeof(ora_tables) * 9);
    for (int b = 1; b <= 8; ++b)
        tables_init(&tab[b], b);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
    for (int64_t i = 0; i < n; ++i) {
        int64_t phys = slot[i] / ORA_PAGE;
        int s = (int)(slot[i] % ORA_PAGE);
        int32_t codes[1024];
        uint8_t rec[2048];
        for (int g = 0; g < hkv; ++g) {
            int b = tier_of(page_bits, head_tiers, phys, hkv, g);
            if (b < 1 || b > 8) {
                bad = 1;
                continue;
            }
            const float *x = keys + ((size_t)i * hkv + g) * d;
            double S = key_codes_t(x, d, &tab[b], codes);
            if (ora_pack(codes, d, b, rec)) {
                bad = 1;
                continue;
            }
            int kb = ora_kb(d, b);
            size_t off = rec_off(phys, g, s, kb, hkv, d, page_off, bstride, head_tiers);
            memcpy(kcode + off, rec, (size_t)kb);
            rcode[((size_t)phys * hkv + g) * ORA_PAGE + s] = (uint8_t)ora_radius_code(S, tau2 + 255 * g);
            if (values && v)
                for (int e = 0; e < d; ++e)
                    v[(((size_t)phys * hkv + g) * d + e) * ORA_PAGE + s] = values[((size_t)i * hkv + g) * d + e];
        }
    }
    for (int b = 1; b <= 8; ++b)
        tables_free(&tab[b]);
    free(tab);
    free(level);
    free(tau2);
    return bad;
}

/* bf16 bits -> binary64, exact. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* ADA decode, plain definition [SKV 2.1]: for sequence s and query head h
 * (KV head g = h / (hq/hkv)), over the resident tokens t < n = seq_lens[s]
 * (page t/16 of the block table, slot t%16, resident when the slot is below
 * the page's token count from its header):
 *   l_t = scale * |q| * r~_t * <u_q, u_t>
 * with u_t the decoded direction of the key's codes, r~_t its radius level,
 * and u_q the decoded direction of the query's own codes at the page's tier
 * (query_mode ORA_Q_CODED: f_b takes the two codes) or q/|q| (ORA_Q_EXACT);
 * then softmax over the resident tokens and the value-weighted sum.  The keys
 * are reconstructed here in host memory ("decompress-then-dot", [SKV 1]),
 * which is the slow definition that ADA reaches without materialising them.
 * out [B][hq][d] fp32; logits [B][hq][max_pages*16] fp32 or NULL (natural
 * units, at logical positions 16*p + slot of the resident tokens); pairs =
 * list of (s, h) to compute, or NULL for all.  A row with no resident token
 * gets a zero output.  Returns 0, or 1 on a bad argument. */
int ora_decode(int d, int hkv, int radius_mode, const double *range,
               const uint8_t *page_bits, const uint64_t *page_off, int bstride, int head_tiers,
               const uint8_t *kcode, const uint8_t *rcode, const uint16_t *v,
               const float *q, int B, int hq, const int32_t *block_table, int max_pages,
               const int32_t *seq_lens, double scale, int query_mode,
               float *out, float *logits, const int32_t *pairs, int npairs, int nthreads)
{
    if (d < 8 || d % 4 != 0 || hkv <= 0 || hq <= 0 || hq % hkv != 0 || B < 0 || (head_tiers && !page_off))
        return 1;
    if (scale == 0.0)
        scale = 1.0 / sqrt((double)d);
    int grp = hq / hkv;
    int64_t njobs = pairs ? npairs : (int64_t)B * hq;
    double *level = malloc(sizeof(double) * 256 * (size_t)hkv);
    double *tau2 = malloc(sizeof(double) * 255 * (size_t)hkv);
    for (int g = 0; g < hkv; ++g)
        ora_radius_tables(radius_mode, range[2 * g], range[2 * g + 1], level + 256 * g, tau2 + 255 * g);
    ora_tables *tab = malloc(sizeof(ora_tables) * 9);
    for (int b = 1; b <= 8; ++b)
        tables_init(&tab[b], b);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t job = 0; job < njobs; ++job) {
        int s = pairs ? pairs[2 * job] : (int)(job / hq);
        int h = pairs ? pairs[2 * job + 1] : (int)(job % hq);
        int g = h / grp;
        int n = seq_lens[s];
        const float *qv = q + ((size_t)s * hq + h) * d;
        float *o = out + ((size_t)s * hq + h) * d;
        if (n <= 0) {
            for (int e = 0; e < d; ++e)
                o[e] = 0.0f;
            continue;
        }
        /* query norm and, per tier, the query's decoded direction */
        double uq[9][1024];
        int have[9] = {0};
        int32_t qc[1024], kc[1024];
        double qT = (double)qv[d - 1] * (double)qv[d - 1];
        for (int a = d - 2; a >= 0; --a)
            qT = qT + (double)qv[a] * (double)qv[a];
        double qn = sqrt(qT);
        double *l = malloc(sizeof(double) * (size_t)n);
        double *u = malloc(sizeof(double) * (size_t)d);
        char *res = malloc((size_t)n);
        int nres = 0;
        for (int t = 0; t < n; ++t) {
            int64_t phys = block_table[(size_t)s * max_pages + t / ORA_PAGE];
            int slot = t % ORA_PAGE;
            res[t] = slot < count_of(page_bits, head_tiers, phys, hkv, g);
            if (!res[t])
                continue;
            ++nres;
            int b = tier_of(page_bits, head_tiers, phys, hkv, g);
            if (b < 1 || b > 8) {
                bad = 1;
                b = 1;
            }
            if (!have[b]) {
                if (query_mode == ORA_Q_EXACT) {
                    for (int e = 0; e < d; ++e)
                        uq[b][e] = (qn > 0.0) ? (double)qv[e] / qn : 0.0;
                } else {
                    key_codes_t(qv, d, &tab[b], qc);
                    ora_direction(qc, d, b, uq[b]);
                }
                have[b] = 1;
            }
            int kb = ora_kb(d, b);
            const uint8_t *rec = kcode + rec_off(phys, g, slot, kb, hkv, d, page_off, bstride, head_tiers);
            ora_unpack(rec, d, b, kc);
            ora_direction(kc, d, b, u);
            double r = level[256 * g + rcode[((size_t)phys * hkv + g) * ORA_PAGE + slot]];
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += uq[b][e] * u[e];
            l[t] = scale * qn * r * dot;
            if (logits)
                logits[((size_t)s * hq + h) * (size_t)max_pages * ORA_PAGE + t] = (float)l[t];
        }
        if (nres == 0) {
            for (int e = 0; e < d; ++e)
                o[e] = 0.0f;
            free(res);
            free(l);
            free(u);
            continue;
        }
        double m = -INFINITY;
        for (int t = 0; t < n; ++t)
            if (res[t] && l[t] > m)
                m = l[t];
        double den = 0.0;
        double *num = calloc((size_t)d, sizeof(double));
        for (int t = 0; t < n; ++t) {
            if (!res[t])
                continue;
            double w = exp(l[t] - m);
            int64_t phys = block_table[(size_t)s * max_pages + t / ORA_PAGE];
            int slot = t % ORA_PAGE;
            den += w;
            for (int e = 0; e < d; ++e)
                num[e] += w * bf16_to_double(v[(((size_t)phys * hkv + g) * d + e) * ORA_PAGE + slot]);
        }
        for (int e = 0; e < d; ++e)
            o[e] = (float)(num[e] / den);
        free(num);
        free(res);
        free(l);
        free(u);
    }
    for (int b = 1; b <= 8; ++b)
        tables_free(&tab[b]);
    free(tab);
    free(level);
    free(tau2);
    return bad;
}

/* ------------------------------------------------------------------------ */
/* The "decompress" step of decompress-then-dot [SKV 1]: the dense key each
 * stored record stands for, k~ = r~ * u(centres(c)) [SKV 2.1], for the 16
 * slots and every KV head of the given physical pages.  out [n][hkv][16][d]
 * binary64 (page i of phys_list at out + i*hkv*16*d).  Returns 0, or 1 on a
 * bad header. */
int ora_decoded_keys(int d, int hkv, int radius_mode, const double *range,
                     const uint8_t *page_bits, const uint64_t *page_off, int bstride, int head_tiers,
                     const uint8_t *kcode, const uint8_t *rcode,
                     const int32_t *phys_list, int n, double *out)
{
    if (head_tiers && !page_off)
        return 1;
    int bad = 0;
    int32_t codes[1024];
    double u[1024], level[256], tau2[255];
    for (int i = 0; i < n; ++i) {
        int64_t phys = phys_list[i];
        for (int g = 0; g < hkv; ++g) {
            int b = tier_of(page_bits, head_tiers, phys, hkv, g);
            if (b < 1 || b > 8) {
                bad = 1;
                continue;
            }
            int kb = ora_kb(d, b);
            ora_radius_tables(radius_mode, range[2 * g], range[2 * g + 1], level, tau2);
            for (int slot = 0; slot < ORA_PAGE; ++slot) {
                const uint8_t *rec = kcode + rec_off(phys, g, slot, kb, hkv, d, page_off, bstride, head_tiers);
                ora_unpack(rec, d, b, codes);
                ora_direction(codes, d, b, u);
                double r = level[rcode[((size_t)phys * hkv + g) * ORA_PAGE + slot]];
                double *o = out + (((size_t)i * hkv + g) * ORA_PAGE + slot) * d;
                for (int e = 0; e < d; ++e)
                    o[e] = r * u[e];
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Dense paged attention, the baseline ADA replaces [SKV 1]: keys stored as
 * bf16 in pages, k_dense [num_pages][hkv][16][d] (token-major), values as in
 * the ADA pools.  For sequence s and query head h (KV head g = h/(hq/hkv)):
 *   l_t = scale * sum_e q_e k_t,e   over the resident tokens,
 * then softmax and the value-weighted sum; every bf16 input is converted to
 * binary64 exactly.  out [B][hq][d]; logits as in ora_decode or NULL.
 * Returns 0, or 1 on a bad argument. */
int ora_dense_decode(int d, int hkv, const uint16_t *k_dense, const uint16_t *v,
                     const float *q, int B, int hq, const int32_t *block_table, int max_pages,
                     const int32_t *seq_lens, double scale, float *out, float *logits, int nthreads)
{
    if (d < 1 || hkv <= 0 || hq <= 0 || hq % hkv != 0 || B < 0)
        return 1;
    if (scale == 0.0)
        scale = 1.0 / sqrt((double)d);
    int grp = hq / hkv;
    int64_t njobs = (int64_t)B * hq;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t job = 0; job < njobs; ++job) {
        int s = (int)(job / hq), h = (int)(job % hq), g = h / grp;
        int n = seq_lens[s];
        const float *qv = q + ((size_t)s * hq + h) * d;
        float *o = out + ((size_t)s * hq + h) * d;
        if (n <= 0) {
            for (int e = 0; e < d; ++e)
                o[e] = 0.0f;
            continue;
        }
        double *l = malloc(sizeof(double) * (size_t)n);
        for (int t = 0; t < n; ++t) {
            int64_t phys = block_table[(size_t)s * max_pages + t / ORA_PAGE];
            int slot = t % ORA_PAGE;
            const uint16_t *k = k_dense + (((size_t)phys * hkv + g) * ORA_PAGE + slot) * d;
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += (double)qv[e] * bf16_to_double(k[e]);
            l[t] = scale * dot;
            if (logits)
                logits[((size_t)s * hq + h) * (size_t)max_pages * ORA_PAGE + t] = (float)l[t];
        }
        double m = l[0];
        for (int t = 1; t < n; ++t)
            if (l[t] > m)
                m = l[t];
        double den = 0.0;
        double *num = calloc((size_t)d, sizeof(double));
        for (int t = 0; t < n; ++t) {
            double w = exp(l[t] - m);
            int64_t phys = block_table[(size_t)s * max_pages + t / ORA_PAGE];
            int slot = t % ORA_PAGE;
            den += w;
            for (int e = 0; e < d; ++e)
                num[e] += w * bf16_to_double(v[(((size_t)phys * hkv + g) * d + e) * ORA_PAGE + slot]);
        }
        for (int e = 0; e < d; ++e)
            o[e] = (float)(num[e] / den);
        free(num);
        free(l);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Rate-distortion retention (RDR) [SKV 2.2], one sequence: for every state
 * (token) i choose residency z_i and tier b_i under a byte budget.
 * Options: evict (0 bytes, distortion u_i: the state's utility is lost) or
 * keep at tier k (bytes[k] bytes, distortion u_i * min(1, sigma*|k_i|*eps[k]):
 * the logit error of ADA grows with the key's magnitude and the tier's angular
 * error eps[k], sigma folding in the query magnitude and softmax scale).
 * Protected states (prot[i] != 0) are kept at the widest tier.  The choice
 * minimises sum D + lambda * sum bytes for a multiplier lambda found by 64
 * bisection steps (the smallest lambda tried whose plan fits the budget):
 * for each state, the option of least D + lambda*bytes, ties going to the
 * earlier option in the order evict, tiers[0], ..., tiers[ntiers-1].
 * Retained states are then packed into tier-homogeneous pages: tiers in the
 * given (increasing) order, states in index order, 16 per page.
 * Outputs: tier_out[i] (0 = evicted), page_out[i] / slot_out[i] (-1 when
 * evicted), page_tier[p] for p < *npages, *lambda_out.  Returns 0, or 2 when
 * the protected states alone exceed the budget (they are still kept, all
 * others evicted), or 1 on a bad argument.  Arithmetic in binary64. */
static int rdr_choose(double u, double kn, int ntiers, const double *eps, const int64_t *bytes, double sigma,
                      double lambda, int prot)
{
    if (prot)
        return ntiers;                       /* option index ntiers = widest tier */
    int best = 0;                            /* 0: evict, k+1: tier k */
    double bc = u;                           /* + lambda * 0 */
    for (int k = 0; k < ntiers; ++k) {
        double f = sigma * kn * eps[k];
        if (f > 1.0)
            f = 1.0;
        double c = u * f + lambda * (double)bytes[k];
        if (c < bc) {
            bc = c;
            best = k + 1;
        }
    }
    return best;
}

int ora_rdr_plan(int n, const float *u, const float *knorm, const uint8_t *prot, int ntiers, const int *tiers,
                 const double *eps, const int64_t *bytes, int64_t budget, double sigma,
                 uint8_t *tier_out, int32_t *page_out, int32_t *slot_out, uint8_t *page_tier, int *npages,
                 double *lambda_out)
{
    if (n < 0 || ntiers < 1 || ntiers > 8)
        return 1;
    for (int k = 1; k < ntiers; ++k)
        if (tiers[k] <= tiers[k - 1] || bytes[k] < bytes[k - 1])
            return 1;
    /* bytes of a plan at multiplier lambda */
#define RDR_TOTAL(lam, tot)                                                                        \
    do {                                                                                           \
        tot = 0;                                                                                   \
        for (int i_ = 0; i_ < n; ++i_) {                                                           \
            int o_ = rdr_choose(u[i_], knorm[i_], ntiers, eps, bytes, sigma, (lam), prot[i_] != 0); \
            if (o_ > 0)                                                                            \
                tot += bytes[o_ - 1];                                                              \
        }                                                                                          \
    } while (0)
    /* a multiplier at which every unprotected state is evicted: above
     * (u - D_k) / bytes_k for every state and tier */
    double hi = 0.0;
    for (int i = 0; i < n; ++i) {
        if (prot[i])
            continue;
        for (int k = 0; k < ntiers; ++k) {
            double f = sigma * (double)knorm[i] * eps[k];
            if (f > 1.0)
                f = 1.0;
            double gain = (double)u[i] - (double)u[i] * f;
            double r = gain / (double)bytes[k];
            if (r > hi)
                hi = r;
        }
    }
    hi = 2.0 * hi + 1e-300;
    double lo = 0.0, lambda;
    int64_t tot;
    int status = 0;
    RDR_TOTAL(0.0, tot);
    if (tot <= budget) {
        lambda = 0.0;
    } else {
        RDR_TOTAL(hi, tot);
        if (tot > budget)
            status = 2;
        for (int it = 0; it < 64; ++it) {
            double mid = 0.5 * (lo + hi);
            RDR_TOTAL(mid, tot);
            if (tot <= budget)
                hi = mid;
            else
                lo = mid;
        }
        lambda = hi;
    }
#undef RDR_TOTAL
    /* the plan, then tier-homogeneous pages */
    int page = 0;
    for (int i = 0; i < n; ++i) {
        int o = rdr_choose(u[i], knorm[i], ntiers, eps, bytes, sigma, lambda, prot[i] != 0);
        tier_out[i] = (uint8_t)(o > 0 ? tiers[o - 1] : 0);
        page_out[i] = -1;
        slot_out[i] = -1;
    }
    for (int k = 0; k < ntiers; ++k) {
        int cnt = 0;
        for (int i = 0; i < n; ++i) {
            if (tier_out[i] != tiers[k])
                continue;
            page_out[i] = page + cnt / ORA_PAGE;
            slot_out[i] = cnt % ORA_PAGE;
            ++cnt;
        }
        int np = (cnt + ORA_PAGE - 1) / ORA_PAGE;
        for (int p = 0; p < np; ++p) {
            /* the header: the tier, and for the tier's last page its empty slots */
            int empty = (p == np - 1) ? np * ORA_PAGE - cnt : 0;
            page_tier[page + p] = (uint8_t)(tiers[k] | (empty << 4));
        }
        page += np;
    }
    *npages = page;
    *lambda_out = lambda;
    return status;
}

int ora_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
