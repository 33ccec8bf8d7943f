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

// The same code found by walking from a starting guess g (any value in
// [0, 2^b - 1]): the predicate holds for j = 1..code and fails above, so the
// walk ends exactly at the code whatever the guess.  With a guess from a
// low-precision angle it takes one or two predicate evaluations.
__device__ __forceinline__ int polar_code_near(double x, double S, int b, const double *__restrict__ cos2,
                                               const double *__restrict__ sin2, int g) {
#pragma clang fp contract(off)
    if (x == 0.0 && S == 0.0) return 0;
    const int n = 1 << b;
    const double x2 = x * x;
    auto pred = [&](int j) {
        if (2 * j < n) return (x <= 0.0) || (cos2[j] * S >= sin2[j] * x2);
        if (2 * j == n) return x <= 0.0;
        return (x < 0.0) && (cos2[j] * S <= sin2[j] * x2);
    };
    g = min(max(g, 0), n - 1);
    while (g > 0 && !pred(g)) --g;
    while (g < n - 1 && pred(g + 1)) ++g;
    return g;
}

// A guess for polar_code_near: floor(atan2(sqrt(S), x) * 2^b / pi) in binary32.
__device__ __forceinline__ int polar_guess(double x, double S, int b) {
    const float phi = atan2f(sqrtf((float)S), (float)x);
    return (int)(phi * (float)(1 << b) * 0.31830988618379067f);
}

// The code from a guess g, confirmed by the two predicates around it: the
// code is g when "phi >= theta_g" holds (or g = 0) and "phi >= theta_{g+1}"
// fails (or g = 2^b - 1).  S may carry a relative error up to rel_err (a sum
// taken in another order than the defining one); a product comparison whose
// two sides differ by less than that error allows could go either way, so
// then, as when the guess is wrong, ok is cleared and the caller must decide
// with the exact S.  With rel_err = 0 the predicates are the defining ones.
__device__ __forceinline__ int polar_code_checked(double x, double S, int b, const double *__restrict__ cos2,
                                                  const double *__restrict__ sin2, int g, double rel_err, bool &ok) {
#pragma clang fp contract(off)
    // straight-line (no branches): both neighbouring edges are read and
    // decided with selects
    const int n = 1 << b;
    const double x2 = x * x;
    g = min(max(g, 0), n - 1);
    const int j1 = max(g, 1), j2 = min(g + 1, n - 1);
    const double a1 = cos2[j1] * S, c1 = sin2[j1] * x2;
    const double a2 = cos2[j2] * S, c2 = sin2[j2] * x2;
    auto decide = [&](int j, double a, double c, bool &sure) {
        const bool low = 2 * j < n, mid = 2 * j == n;
        const bool prod = low ? (a >= c) : (a <= c);
        const bool by_sign = mid || (low && x <= 0.0) || (!low && x >= 0.0);
        sure = by_sign || (fabs(a - c) > 2.0 * rel_err * a);
        return mid ? (x <= 0.0) : (low ? (x <= 0.0 || prod) : (x < 0.0 && prod));
    };
    bool s1, s2;
    const bool p1 = decide(j1, a1, c1, s1), p2 = decide(j2, a2, c2, s2);
    const bool at = (g == 0) || p1;
    const bool above = (g < n - 1) && p2;
    const bool zero = (x == 0.0 && S == 0.0);
    ok = zero || (((g == 0) || s1) && ((g == n - 1) || s2) && at && !above);
    return zero ? 0 : g;
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

// Azimuth code through polar_code_near (same result as azimuth_code).
__device__ __forceinline__ int azimuth_code_near(double x, double y, int b, const double *__restrict__ cos2h,
                                                 const double *__restrict__ sin2h) {
#pragma clang fp contract(off)
    if (x == 0.0 && y == 0.0) return 0;
    const bool h = (y < 0.0) || (y == 0.0 && x < 0.0);
    const double xp = h ? -x : x;
    const double yp = h ? -y : y;
    const double S = yp * yp;
    return (h ? (1 << (b - 1)) : 0) + polar_code_near(xp, S, b - 1, cos2h, sin2h, polar_guess(xp, S, b - 1));
}

}  // namespace ska
