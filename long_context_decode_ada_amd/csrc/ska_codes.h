// ska_codes.h -- the exact angle-code decisions shared by the encode kernel
// and the query preparation inside the decode kernel.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary,
// section 2.1: keys (and, inside f_b, the query) are parametrised by
// hyperspherical angles quantised to b bits.  Every decision below is an
// integer that must match the CPU definition bit for bit: suffix sums of
// squares run from the last component backwards in binary64 (each square of
// a binary32 input is exact), and a code is the number of bin edges
// theta_j = j*pi/2^b with "phi >= theta_j", decided on squared quantities
// with host-computed binary64 constants.  Contraction into fused
// multiply-adds is switched off inside these functions, so each product is
// rounded as written whatever the including file's setting.
#pragma once

#include <hip/hip_runtime.h>

namespace ska {

// "phi >= theta_j" for phi = atan2(sqrt(S), x), theta_j = j*pi/2^b:
//   theta_j < pi/2 : x <= 0 or cos2*S >= sin2*x^2
//   theta_j = pi/2 : x <= 0
//   theta_j > pi/2 : x < 0 and cos2*S <= sin2*x^2
// The predicate holds for j = 1..code and fails above, so the code is found
// by bisection.
__device__ __forceinline__ int polar_code(double x, double S, int b, const double *__restrict__ cos2,
                                          const double *__restrict__ sin2) {
#pragma clang fp contract(off)
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
#pragma clang fp contract(off)
    if (x == 0.0 && y == 0.0) return 0;
    const bool h = (y < 0.0) || (y == 0.0 && x < 0.0);
    const double xp = h ? -x : x;
    const double yp = h ? -y : y;
    return (h ? (1 << (b - 1)) : 0) + polar_code(xp, yp * yp, b - 1, cos2h, sin2h);
}

// T <- T + x^2 (binary64; one step of the backward suffix sum).
__device__ __forceinline__ double add_square(double T, float x) {
#pragma clang fp contract(off)
    return T + (double)x * (double)x;
}

}  // namespace ska
