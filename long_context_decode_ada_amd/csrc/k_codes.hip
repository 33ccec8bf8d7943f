// k_codes.hip -- spherical encoding on the GPU: radius calibration and key
// encoding into the paged pools.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary,
// section 2.1 (r = |k|, phi = Phi(k/|k|), stored r~ and packed codes c; the
// query's own code c_q enters f_b) and section 2.3 (dense keys -> spherical
// codes -> paged compressed store).  The query's codes are formed inside the
// decode kernel with the same decision functions (ska_codes.h).
//
// Every decision here is an integer that must equal the CPU definition bit
// for bit, so this file is compiled with -ffp-contract=off: each binary64
// product and sum is rounded exactly as written.  The squares of binary32
// inputs are exact in binary64; suffix sums run from the last component
// backwards; angle codes come from comparisons of cos^2 * S against
// sin^2 * x^2 with host-computed binary64 constants, never from atan2, sqrt
// or log.
#include "ska_codes.h"
#include "ska_internal.h"

namespace ska {

// ---------------------------------------------------------------------------
// Radius calibration: per KV head, max |k|^2 and min positive |k|^2 (binary64
// bit patterns of non-negative numbers order like the numbers, so integer
// atomics give the exact, order-independent extremes).
__global__ void k_calibrate(const float *__restrict__ keys, int64_t n, int hkv, int d,
                            unsigned long long *__restrict__ minmax) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n * hkv) return;
    const float *x = keys + i * d;
    double T = (double)x[d - 1] * (double)x[d - 1];
    for (int a = d - 2; a >= 0; --a) T = T + (double)x[a] * (double)x[a];
    const int g = (int)(i % hkv);
    const unsigned long long bits = (unsigned long long)__double_as_longlong(T);
    atomicMax(&minmax[2 * g + 0], bits);
    if (T > 0.0) atomicMin(&minmax[2 * g + 1], bits);
}

hipError_t launch_calibrate(const float *keys, int64_t n, int hkv, int d, unsigned long long *minmax,
                            hipStream_t s) {
    const int64_t tot = n * hkv;
    if (tot == 0) return hipSuccess;
    const int64_t blocks = (tot + 255) / 256;
    hipLaunchKernelGGL(k_calibrate, dim3((unsigned)blocks), dim3(256), 0, s, keys, n, hkv, d, minmax);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Key encoding: one thread per (key, kv head).  Codes go to a per-thread LDS
// row, then the record is packed slice by slice into 32-bit words.
constexpr int kEncThreads = 128;

// Encodes key x (d fp32) of KV head g into pool slot `slot` (phys*16 + s) at
// the tier of its page, with its values vs (d bf16) when given.  cl: a
// 128-byte scratch row.
__device__ void encode_one(const EncodeArgs &A, const float *__restrict__ x, const uint16_t *__restrict__ vs,
                           int g, int64_t slot, uint8_t *cl) {
    const int d = A.d;
    const int64_t phys = slot >> 4;
    const int s = (int)(slot & 15);
    if (slot < 0 || phys >= A.num_pages) {
        atomicOr(A.err, 1u);
        return;
    }
    const int b = A.page_bits[A.head_tiers ? phys * A.hkv + g : phys] & 15;   // (the header's tier bits)
    if (b < 1 || b > 8 || !((A.tier_mask >> b) & 1u)) {
        atomicOr(A.err, 4u);
        return;
    }
    const double *c2 = A.tab.cos2 + thr_off(b), *s2 = A.tab.sin2 + thr_off(b);
    const double *c2h = A.tab.cos2 + thr_off(b - 1), *s2h = A.tab.sin2 + thr_off(b - 1);

    double T = (double)x[d - 1] * (double)x[d - 1];
    cl[d - 2] = (uint8_t)azimuth_code((double)x[d - 2], (double)x[d - 1], b, c2h, s2h);
    T = T + (double)x[d - 2] * (double)x[d - 2];
    for (int a = d - 3; a >= 0; --a) {
        cl[a] = (uint8_t)polar_code((double)x[a], T, b, c2, s2);
        T = T + (double)x[a] * (double)x[a];
    }
    // radius code = #{j : T >= tau2[j]}; tau2 increases with j
    const double *tau2 = A.tau2 + 255 * g;
    int lo = 0, hi = 255;  // answer in [0, 255]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;  // predicate T >= tau2[mid-1]
        if (T >= tau2[mid - 1]) lo = mid; else hi = mid - 1;
    }
    const int rc = lo;

    const int kb = record_bytes(d, b);
    const int sb = kb / 4;          // slice bytes
    const int na = d / 4;           // angles per slice
    uint64_t base;
    if (A.head_tiers) base = A.page_off[phys * A.hkv + g] + (uint64_t)s * kb;
    else base = (A.page_off ? A.page_off[phys] : (uint64_t)phys * (uint64_t)A.page_stride) + ((uint64_t)g * kPage + s) * kb;
    uint32_t *rec = reinterpret_cast<uint32_t *>(A.kcode + base);
    for (int sl = 0; sl < 4; ++sl) {
        uint32_t *w = rec + sl * (sb / 4);
        uint64_t acc = 0;
        int nb = 0, wi = 0;
        const int a1 = min((sl + 1) * na, d - 1);
        for (int a = sl * na; a < a1; ++a) {
            acc |= (uint64_t)cl[a] << nb;
            nb += b;
            if (nb >= 32) {
                w[wi++] = (uint32_t)acc;
                acc >>= 32;
                nb -= 32;
            }
        }
        for (; wi < sb / 4; ++wi) {
            w[wi] = (uint32_t)acc;
            acc >>= 32;
        }
    }
    A.rcode[((uint64_t)phys * A.hkv + g) * kPage + s] = (uint8_t)rc;
    if (vs) {
        uint16_t *vd = A.v + ((uint64_t)phys * A.hkv + g) * (uint64_t)d * kPage + s;
        for (int e = 0; e < d; ++e) vd[(uint64_t)e * kPage] = vs[e];
    }
}

__global__ __launch_bounds__(kEncThreads) void k_encode(EncodeArgs A) {
    __shared__ uint8_t codes_lds[kEncThreads][128];
    const int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
    if (i >= A.n * A.hkv) return;
    const int64_t tok = i / A.hkv;
    const int g = (int)(i % A.hkv);
    encode_one(A, A.keys + i * A.d, A.values ? A.values + i * A.d : nullptr, g, A.slot[tok], codes_lds[threadIdx.x]);
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s) {
    const int64_t tot = a.n * a.hkv;
    if (tot == 0) return hipSuccess;
    const int64_t blocks = (tot + kEncThreads - 1) / kEncThreads;
    hipLaunchKernelGGL(k_encode, dim3((unsigned)blocks), dim3(kEncThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ska
