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

// A guess for the code: floor(atan2(sqrt(S), x) * 2^b / pi) from binary32
// arithmetic with the hardware square root and reciprocal and a degree-9 odd
// polynomial for atan on [0, 1] (fitted here, error below 1.2e-5 rad).  Its
// error stays far below one bin (pi / 256 at 8 bits), so the code lies
// within one of it; polar_code_window decides which exactly.
__device__ __forceinline__ int polar_guess(double xd, double Sd, int b) {
    const float x = (float)xd, y = __builtin_amdgcn_sqrtf((float)Sd);
    const float ax = fabsf(x), mx = fmaxf(ax, y), mn = fminf(ax, y);
    const float t = mx > 0.f ? mn * __builtin_amdgcn_rcpf(mx) : 0.f;   // in [0, 1]
    const float s = t * t;
    const float at = t * (0.99986631f + s * (-0.33030480f + s * (0.18015929f + s * (-0.085156336f + s * 0.020845106f))));
    float phi = y > ax ? 1.57079633f - at : at;   // atan2(y, |x|)
    phi = x < 0.f ? 3.14159265f - phi : phi;
    return (int)(phi * (float)(1 << b) * 0.318309886f);
}

// The code from a guess g that is off by at most one, confirmed by the
// predicates "phi >= theta_j" at the four edges j = g-1 .. g+2: the
// predicate holds for j = 1..code and fails above, so with it holding at
// g-1 (or g-1 < 1) and failing at g+2 (or g+2 > 2^b - 1), the code is
// max(g-2, 0) plus the number of edges among g-1 .. g+1 where it holds.  S
// may carry a relative error up to rel_err (a sum taken in another order
// than the defining one); a product comparison whose two sides differ by
// less than that error allows could go either way, so then, as when the
// guess is off by more, ok is cleared and the caller must decide with the
// exact S.  With rel_err = 0 the predicates are the defining ones.
__device__ __forceinline__ int polar_code_window(double x, double S, int b, const double *__restrict__ cos2,
                                                 const double *__restrict__ sin2, int g, double rel_err, bool &ok) {
#pragma clang fp contract(off)
    // Straight-line: the eight table reads of the four edges go out together,
    // then every decision is taken with bitwise operations on the compares
    // (a branch per edge made each edge's reads wait for the previous edge).
    const int n = 1 << b;
    const double x2 = x * x;
    g = min(max(g, 0), n - 1);
    int jc[4];
    double c2[4], s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        jc[i] = min(max(g - 1 + i, 1), n - 1);
        c2[i] = cos2[jc[i]];
        s2[i] = sin2[jc[i]];
    }
    const bool xle0 = x <= 0.0, xlt0 = x < 0.0, xge0 = x >= 0.0;
    int cnt = max(g - 2, 0);
    bool good = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = g - 1 + i;
        const bool inr = (j >= 1) & (j <= n - 1);
        const double a = c2[i] * S, c = s2[i] * x2;
        const bool low = 2 * jc[i] < n, mid = 2 * jc[i] == n;
        const bool prod = (low & (a >= c)) | (!low & (a <= c));
        const bool by_sign = mid | (low & xle0) | (!low & xge0);
        const bool sure = by_sign | (fabs(a - c) > 2.0 * rel_err * a);
        const bool p = (mid & xle0) | (!mid & low & (xle0 | prod)) | (!mid & !low & xlt0 & prod);
        if (i < 3) cnt += (int)(inr & p);
        good = good & (!inr | sure);
        if (i == 0) good = good & (!inr | p);    // holds at g-1
        if (i == 3) good = good & (!inr | !p);   // fails at g+2
    }
    const bool zero = (x == 0.0) & (S == 0.0);
    ok = zero | good;
    return zero ? 0 : cnt;
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
