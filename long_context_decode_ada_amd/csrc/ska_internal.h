// ska_internal.h -- shared between the host library (ska_api.cpp) and the
// HIP kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ska {

constexpr int kPage = 16;
#ifndef SKA_WAVES
#define SKA_WAVES 8
#endif
constexpr int kWaves = SKA_WAVES;       // waves per decode workgroup
constexpr int kThreads = 64 * kWaves;

// A decode workgroup holds two waves on each SIMD of its CU.  Measured on
// MI355X, the wave dispatched first to a SIMD is served memory requests
// ahead of the second and streams pages about 1.3x as fast, so with equal
// page counts the second waves finish last.  The first wave on each SIMD
// therefore takes the larger share of a chunk of n pages: round(n r / (h (1 + r)))
// pages with r the rate ratio and h = kWaves / 2.  The shares depend on n
// only (not on timing), so results are reproducible.
#ifndef SKA_FIRST_WAVE_RATE_PCT
#define SKA_FIRST_WAVE_RATE_PCT 130
#endif
__host__ __device__ constexpr int first_wave_pages(int n) {
    constexpr int h = kWaves / 2, r = SKA_FIRST_WAVE_RATE_PCT;
    const int f = (2 * n * r + h * (100 + r)) / (2 * h * (100 + r));
    return f * h > n ? n / h : f;
}

// Bytes of one key record: 16 * ceil((d-1) * b / 128).
__host__ __device__ constexpr int record_bytes(int d, int b) { return 16 * (((d - 1) * b + 127) / 128); }

// Layout of the decode lookup table (float2 entries, staged into LDS).  Per
// tier: 2^b polar (cos, sin) of bin centres (c + 1/2) pi / 2^b, then 2^b
// azimuth (cos, sin) of (c + 1/2) 2 pi / 2^b.  A final block of 256 (1, 1)
// entries serves the padding slot after the azimuth of the last slice.
__host__ __device__ constexpr int lut_polar(int b) {
    return b == 2 ? 0 : b == 3 ? 8 : b == 4 ? 24 : b == 6 ? 56 : 184;
}
__host__ __device__ constexpr int lut_azimuth(int b) { return lut_polar(b) + (1 << b); }
constexpr int kLutOnes = 696;
constexpr int kLutEntries = 952;

// Encode-side angle threshold tables (binary64): for every b in 1..8, 2^b
// entries of cos^2 and sin^2 of the bin edges j*pi/2^b, at offset
// thr_off(b) = 2^b - 2.
__host__ __device__ constexpr int thr_off(int b) { return (1 << b) - 2; }
constexpr int kThrEntries = 510;

constexpr uint32_t kSupportedTiers = (1u << 2) | (1u << 3) | (1u << 4) | (1u << 6) | (1u << 8);

struct CodeTables {
    const double *cos2;     // [kThrEntries]
    const double *sin2;     // [kThrEntries]
    const double *cen_cs;   // [kLutEntries][2] binary64 cos, sin of bin centres (same layout as the LUT)
};

struct EncodeArgs {
    const float *keys;
    const uint16_t *values;
    const int64_t *slot;
    int64_t n;
    int d, hkv;
    int64_t num_pages;
    uint32_t tier_mask;
    const uint8_t *page_bits;
    const uint64_t *page_off;
    int64_t page_stride;     // bytes per physical page when page_off == NULL
    int head_tiers;          // page_bits/page_off per (page, KV head): [num_pages][hkv]
    uint8_t *kcode;
    uint8_t *rcode;
    uint16_t *v;
    const double *tau2;      // [hkv][255] squared radius edges
    CodeTables tab;
    uint32_t *err;
};


// largest batch whose lengths every decode workgroup reads to find its unit
constexpr int kCompactMaxBatch = 512;
// grid slots (batch x splits) one k_unit_order workgroup orders: its 8-byte
// sort keys fill 128 KiB of LDS; a larger batch is not compacted
constexpr int kUnitSortMax = 16384;

struct DecodeArgs {
    const uint8_t *kcode;
    const uint64_t *page_off;
    const uint8_t *rcode;
    const uint16_t *v;
    const uint8_t *page_bits;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const float *q;          // [B][hq][d]
    const double *cos2;      // [kThrEntries] edge tables (binary64)
    const double *sin2;
    const float2 *lut;       // [kLutEntries]
    const float *rlev;       // [hkv][256] radius levels
    float *part_o;           // [B][hq][nsplit][d]
    float *part_ml;          // [B][hq][nsplit][2]
    float *logits;           // debug [B][hq][max_pages*16] or NULL
    float *out;              // [B][hq][d]
    uint16_t *kdense;        // dense bf16 keys [num_pages][hkv][16][d] (dense decode: read; decompress: written)
    int dense;               // dense decode: keys from kdense, no codes
    uint32_t *counters;      // [B][hkv] finished workgroups per group, zero between calls
    uint32_t *err;
    int64_t num_pages;
    int64_t page_stride;
    int hkv, hq, max_pages;
    int pps;                 // pages of the smallest split (multiple of kWaves)
    int split_m;             // split sizes: pps, pps, 2 pps, ..., pps << split_m, then
                             // pps << split_m each (0: every split has pps pages)
    int nsplit;
    int compact;             // 1: workgroup slots map to the (sequence, split) units in
                             // decreasing size, through unit_table (batch <= kCompactMaxBatch,
                             // batch x nsplit <= kUnitSortMax)
    int2 *unit_table;        // compact: slot -> (sequence << 16 | split, the sequence's
                             // length), written by k_unit_order; -1 past the last unit
    uint32_t tier_mask;
    int nt;
    int8_t tslot[9];         // tier b -> index among the tiers present
    float scale;             // softmax scale
    int query_mode;          // 0: coded query, 1: exact query direction
    int query_f32;           // query direction in f_b: 0 binary16, 1 binary32
    // decode step with append (else NULL): the new token of each sequence,
    // stored at position seq_lens[s] - 1 before that page is read
    const float *app_k;      // [B][hkv][d]
    const uint16_t *app_v;   // [B][hkv][d] bf16
    const double *tau2;      // [hkv][255] squared radius edges
    // page_bits and page_off per (page, KV head), [num_pages][hkv]; the offset
    // is that head's first record (with per-page tiers: the page's, to which
    // the head's 16 records at their tier are added)
    int head_tiers;
};


hipError_t launch_calibrate(const float *keys, int64_t n, int hkv, int d, unsigned long long *minmax,
                            hipStream_t s);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int d, int G, int B, hipStream_t s);
hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_decompress(const DecodeArgs &a, int d, int B, hipStream_t s);
// decode workgroups resident per CU (two waves per SIMD in all)
int decode_workgroups_per_cu();


}  // namespace ska
