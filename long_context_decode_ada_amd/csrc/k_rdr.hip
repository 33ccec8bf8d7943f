// k_rdr.hip -- rate-distortion retention (RDR): per sequence, the residency
// and tier of every state under a byte budget, and the packing of the
// retained states into tier-homogeneous pages.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary,
// section 2.2: a discrete rate-distortion allocation choosing for each state
// a residency z and a tier b; a distortion surrogate from ADA's error
// analysis (the logit error grows with the angular error of the tier, scaled
// by the query and key magnitudes); protected states kept at the widest
// tier; retained states grouped into pages of one tier, so that the decode
// kernel streams them guided by the page header.
//
// Reading taken (the pages give no formula): evicting state i costs its
// utility u_i; keeping it at tier k costs u_i * min(1, sigma*|k_i|*eps_k).
// The plan minimises sum D + lambda * sum bytes state by state, lambda found
// by 64 bisection steps as the smallest value tried whose plan fits the
// budget.  Every decision is a binary64 comparison written as in the CPU
// definition and this unit is compiled with -ffp-contract=off, so the plan
// equals the CPU one bit for bit; byte totals are integer sums.
#include "ska_rdr.h"

namespace ska {

constexpr int kRdrThreads = 1024;
constexpr int kRdrWaves = kRdrThreads / 64;

// 0: evict; k + 1: tier k (protected states: the widest tier)
// (the tier loop runs over a fixed 8 with a guard, so that the parameters
// are read at constant indices, once, into scalar registers)
__device__ __forceinline__ int rdr_choose(double u, double kn, const RdrArgs &A, double lambda, bool prot) {
    if (prot) return A.ntiers;
    int best = 0;
    double bc = u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k >= A.ntiers) break;
        double f = A.sigma * kn * A.eps[k];
        if (f > 1.0) f = 1.0;
        const double c = u * f + lambda * (double)A.bytes[k];
        if (c < bc) {
            bc = c;
            best = k + 1;
        }
    }
    return best;
}

template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, Op op, T *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o));
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    T r = red[0];
    for (int w = 1; w < kRdrWaves; ++w) r = op(r, red[w]);
    return r;
}

// exclusive prefix sum over the workgroup, and the total
__device__ __forceinline__ int block_excl_scan(int v, int *red, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < kRdrWaves; ++w) {
        if (w < wave) before += red[w];
        total += red[w];
    }
    return before + x - v;
}

__global__ __launch_bounds__(kRdrThreads) void k_rdr(RdrArgs A) {
    __shared__ double redd[kRdrWaves];
    __shared__ long long redl[kRdrWaves];
    __shared__ int redi[kRdrWaves];
    const int seq = blockIdx.x, tid = threadIdx.x;
    const int n = max(0, min(A.nstate[seq], A.max_states));
    const int64_t base = (int64_t)seq * A.max_states;
    // the passes that only sum or take a maximum stride over the states
    // (adjacent threads, adjacent states); the packing gives each thread a
    // contiguous run, so that runs in thread order are the states in index
    // order
    const int per = (n + kRdrThreads - 1) / kRdrThreads;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    const float *u = A.u + base;
    const float *kn = A.knorm + base;
    const uint8_t *prot = A.prot + base;

    // a multiplier at which every unprotected state is evicted
    double hl = 0.0;
    for (int i = tid; i < n; i += kRdrThreads) {
        if (prot[i]) continue;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k >= A.ntiers) break;
            double f = A.sigma * (double)kn[i] * A.eps[k];
            if (f > 1.0) f = 1.0;
            const double gain = (double)u[i] - (double)u[i] * f;
            const double r = gain / (double)A.bytes[k];
            if (r > hl) hl = r;
        }
    }
    double hi = block_reduce(hl, [](double a, double b) { return a > b ? a : b; }, redd);
    hi = 2.0 * hi + 1e-300;
    auto total = [&](double lam) -> long long {
        long long t = 0;
        // kB states per thread per round: their loads go out together
        constexpr int kB = 8;
        for (int i0s = tid; i0s < n; i0s += kB * kRdrThreads) {
            float uu[kB], kk[kB];
            uint8_t pp[kB];
#pragma unroll
            for (int e = 0; e < kB; ++e) {
                const int i = min(i0s + e * kRdrThreads, n - 1);
                uu[e] = u[i];
                kk[e] = kn[i];
                pp[e] = prot[i];
            }
#pragma unroll
            for (int e = 0; e < kB; ++e) {
                if (i0s + e * kRdrThreads >= n) break;
                const int o = rdr_choose((double)uu[e], (double)kk[e], A, lam, pp[e] != 0);
                if (o > 0) t += A.bytes[o - 1];
            }
        }
        return block_reduce(t, [](long long a, long long b) { return a + b; }, redl);
    };
    const long long budget = A.budget[seq];
    double lambda;
    int status = 0;
    if (total(0.0) <= budget) {
        lambda = 0.0;
    } else {
        if (total(hi) > budget) status = 2;
        double lo = 0.0;
        for (int it = 0; it < 64; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (total(mid) <= budget) hi = mid;
            else lo = mid;
        }
        lambda = hi;
    }

    // the plan, then tier-homogeneous pages: tiers in order, states in
    // index order, 16 per page
    for (int i = tid; i < n; i += kRdrThreads) {
        const int o = rdr_choose((double)u[i], (double)kn[i], A, lambda, prot[i] != 0);
        A.tier_out[base + i] = (uint8_t)(o > 0 ? A.tiers[o - 1] : 0);
        A.page_out[base + i] = -1;
        A.slot_out[base + i] = -1;
    }
    __syncthreads();
    int page = 0;
    for (int k = 0; k < A.ntiers; ++k) {
        const uint8_t tk = (uint8_t)A.tiers[k];
        // (the choices are taken again rather than read back: same inputs,
        // same decisions)
        int c = 0;
        for (int i = i0; i < i1; ++i) c += rdr_choose((double)u[i], (double)kn[i], A, lambda, prot[i] != 0) == k + 1;
        int cnt_k;
        int pos = block_excl_scan(c, redi, cnt_k);
        for (int i = i0; i < i1; ++i) {
            if (rdr_choose((double)u[i], (double)kn[i], A, lambda, prot[i] != 0) != k + 1) continue;
            A.page_out[base + i] = page + pos / 16;
            A.slot_out[base + i] = pos % 16;
            ++pos;
        }
        const int np = (cnt_k + 15) / 16;
        for (int p = tid; p < np; p += kRdrThreads)
            if (page + p < A.max_pages_out) A.page_tier[(int64_t)seq * A.max_pages_out + page + p] = tk;
        page += np;
    }
    if (tid == 0) {
        A.npages[seq] = page;
        A.lambda[seq] = lambda;
        A.status[seq] = status;
    }
}

hipError_t launch_rdr(const RdrArgs &a, int batch, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rdr, dim3((unsigned)batch), dim3(kRdrThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ska
