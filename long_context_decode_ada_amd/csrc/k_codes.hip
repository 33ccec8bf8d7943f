// k_codes.hip -- spherical encoding on the GPU: radius calibration, key
// encoding into the paged pools, and query angle codes for the decode.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary,
// section 2.1 (r = |k|, phi = Phi(k/|k|), stored r~ and packed codes c; the
// query's own code c_q enters f_b) and section 2.3 (dense keys -> spherical
// codes -> paged compressed store).
//
// Every decision here is an integer that must equal the CPU definition bit
// for bit, so this file is compiled with -ffp-contract=off: each binary64
// product and sum is rounded exactly as written.  The squares of binary32
// inputs are exact in binary64; suffix sums run from the last component
// backwards; angle codes come from comparisons of cos^2 * S against
// sin^2 * x^2 with host-computed binary64 constants, never from atan2, sqrt
// or log.
#include "ska_internal.h"

namespace ska {

// "phi >= theta_j" for phi = atan2(sqrt(S), x), theta_j = j*pi/2^b:
//   theta_j < pi/2 : x <= 0 or cos2*S >= sin2*x^2
//   theta_j = pi/2 : x <= 0
//   theta_j > pi/2 : x < 0 and cos2*S <= sin2*x^2
// The predicate is true for j = 1..code and false above, so the code is found
// by bisection.
__device__ __forceinline__ int polar_code(double x, double S, int b, const double *__restrict__ cos2,
                                          const double *__restrict__ sin2) {
    if (x == 0.0 && S == 0.0) return 0;
    const int n = 1 << b;
    const double x2 = x * x;
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        bool p;
        if (2 * mid < n)
            p = (x <= 0.0) || (cos2[mid] * S >= sin2[mid] * x2);
        else if (2 * mid == n)
            p = (x <= 0.0);
        else
            p = (x < 0.0) && (cos2[mid] * S <= sin2[mid] * x2);
        if (p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Azimuth atan2(y, x) mod 2*pi at b bits: the lower half plane is turned by
// pi and binned at b-1 bits like a polar angle.
__device__ __forceinline__ int azimuth_code(double x, double y, int b, const double *__restrict__ cos2h,
                                            const double *__restrict__ sin2h) {
    if (x == 0.0 && y == 0.0) return 0;
    const bool h = (y < 0.0) || (y == 0.0 && x < 0.0);
    const double xp = h ? -x : x;
    const double yp = h ? -y : y;
    return (h ? (1 << (b - 1)) : 0) + polar_code(xp, yp * yp, b - 1, cos2h, sin2h);
}

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

__global__ __launch_bounds__(kEncThreads) void k_encode(EncodeArgs A) {
    __shared__ uint8_t codes_lds[kEncThreads][128];
    const int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
    if (i >= A.n * A.hkv) return;
    const int d = A.d;
    const int64_t tok = i / A.hkv;
    const int g = (int)(i % A.hkv);
    const int64_t slot = A.slot[tok];
    const int64_t phys = slot >> 4;
    const int s = (int)(slot & 15);
    if (slot < 0 || phys >= A.num_pages) {
        atomicOr(A.err, 1u);
        return;
    }
    const int b = A.page_bits[phys];
    if (b < 1 || b > 8 || !((A.tier_mask >> b) & 1u)) {
        atomicOr(A.err, 4u);
        return;
    }
    uint8_t *cl = codes_lds[threadIdx.x];
    const float *x = A.keys + i * d;
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
    const uint64_t base = A.page_off ? A.page_off[phys] : (uint64_t)phys * (uint64_t)A.page_stride;
    uint32_t *rec = reinterpret_cast<uint32_t *>(A.kcode + base + ((uint64_t)g * kPage + s) * kb);
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
    if (A.values) {
        const uint16_t *vs = A.values + i * d;
        uint16_t *vd = A.v + ((uint64_t)phys * A.hkv + g) * (uint64_t)d * kPage + s;
        for (int e = 0; e < d; ++e) vd[(uint64_t)e * kPage] = vs[e];
    }
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s) {
    const int64_t tot = a.n * a.hkv;
    if (tot == 0) return hipSuccess;
    const int64_t blocks = (tot + kEncThreads - 1) / kEncThreads;
    hipLaunchKernelGGL(k_encode, dim3((unsigned)blocks), dim3(kEncThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Query preparation: one workgroup of d threads per (sequence, query head).
// The query's suffix sums are formed by one thread in the same backward order
// as the keys'; thread a then finds the code of angle a at every tier present
// (bisection over LDS copies of the edge tables), and the decoded direction
// u_a = (prod_{k<a} sin c_k) * cos c_a follows from a parallel product scan of
// the bin-centre sines (binary64).  Output, per tier, the unit vector as fp16
// in the decode kernel's register layout
//   uq[((((seq*hkv + kvh)*nt + tier)*4 + slice)*(d/4) + i)*G + h_in_group],
// component a = slice*(d/4) + i, and sq = scale * |q| * log2(e) in fp32.
__global__ __launch_bounds__(128) void k_qprep(QPrepArgs A) {
    __shared__ float xs[128];
    __shared__ double Ts[129];
    __shared__ double thr[4][256];
    __shared__ double cen[4][256];   // polar cos, polar sin, azimuth cos, azimuth sin
    __shared__ double scan[128];
    const int d = A.d;
    const int a = threadIdx.x;
    const int seq = blockIdx.x / A.hq, h = blockIdx.x % A.hq;
    xs[a] = A.q[((int64_t)seq * A.hq + h) * d + a];
    __syncthreads();
    if (a == 0) {
        double T = (double)xs[d - 1] * (double)xs[d - 1];
        Ts[d - 1] = T;
        for (int k = d - 2; k >= 0; --k) {
            T = T + (double)xs[k] * (double)xs[k];
            Ts[k] = T;
        }
    }
    __syncthreads();
    const double qn = sqrt(Ts[0]);
    if (a == 0) A.sq[(int64_t)seq * A.hq + h] = (float)((double)A.scale * qn * 1.4426950408889634);
    const int G = A.G, kvh = h / G, hg = h % G;
    const int slice = a / (d / 4), i = a % (d / 4);
    int ti = 0;
    for (int b = 2; b <= 8; ++b) {
        if (!((A.tier_mask >> b) & 1u)) continue;
        const int n = 1 << b;
        for (int e = a; e < n; e += d) {
            thr[0][e] = A.tab.cos2[thr_off(b) + e];
            thr[1][e] = A.tab.sin2[thr_off(b) + e];
            cen[0][e] = A.tab.cen_cs[2 * (lut_polar(b) + e) + 0];
            cen[1][e] = A.tab.cen_cs[2 * (lut_polar(b) + e) + 1];
            cen[2][e] = A.tab.cen_cs[2 * (lut_azimuth(b) + e) + 0];
            cen[3][e] = A.tab.cen_cs[2 * (lut_azimuth(b) + e) + 1];
        }
        for (int e = a; e < n / 2; e += d) {
            thr[2][e] = A.tab.cos2[thr_off(b - 1) + e];
            thr[3][e] = A.tab.sin2[thr_off(b - 1) + e];
        }
        __syncthreads();
        double u;
        if (A.query_mode == 1) {
            u = qn > 0.0 ? (double)xs[a] / qn : 0.0;
        } else {
            double cs = 1.0, sn = 1.0;
            if (a < d - 2) {
                const int c = polar_code((double)xs[a], Ts[a + 1], b, thr[0], thr[1]);
                cs = cen[0][c];
                sn = cen[1][c];
            } else if (a == d - 2) {
                const int c = azimuth_code((double)xs[d - 2], (double)xs[d - 1], b, thr[2], thr[3]);
                cs = cen[2][c];
                sn = cen[3][c];
            }
            // inclusive product scan of the sines over the components
            scan[a] = sn;
            __syncthreads();
            for (int off = 1; off < d; off <<= 1) {
                const double v = (a >= off) ? scan[a - off] : 1.0;
                __syncthreads();
                scan[a] *= v;
                __syncthreads();
            }
            const double P = (a == 0) ? 1.0 : scan[a - 1];
            u = P * cs;   // the last component has cs = 1: u = prod of all d-1 sines
        }
        const int64_t idx = (((((int64_t)seq * A.hkv + kvh) * A.nt + ti) * 4 + slice) * (d / 4) + i) * G + hg;
        A.uq[idx] = (_Float16)(float)u;
        __syncthreads();   // the tables are refilled for the next tier
        ++ti;
    }
}

hipError_t launch_qprep(const QPrepArgs &a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    hipLaunchKernelGGL(k_qprep, dim3((unsigned)(a.B * a.hq)), dim3(a.d), 0, s, a);
    return hipGetLastError();
}

}  // namespace ska
