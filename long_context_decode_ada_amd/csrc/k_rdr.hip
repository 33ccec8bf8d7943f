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

// Many workgroups per sequence: each takes a chunk of kRdrChunk states
// (kRdrPer per thread, the thread's states contiguous), and the byte totals
// of a candidate multiplier are summed over the chunks with integer atomics
// (exact in any order).  The bisection runs four steps per kernel: the 15
// midpoints the next four steps can visit are evaluated together, and the
// next kernel walks them with the totals, so the steps taken are exactly
// those of a one-at-a-time bisection.
constexpr int kRdrThreads = 256;
constexpr int kRdrWaves = kRdrThreads / 64;
constexpr int kRdrPer = 2;
constexpr int kRdrChunk = kRdrThreads * kRdrPer;

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

// this workgroup's states of sequence seq: [i0, i1)
struct Chunk {
    int seq, n, i0, i1;
    int64_t base;
};
__device__ __forceinline__ Chunk chunk_of(const RdrArgs &A) {
    Chunk c;
    c.seq = blockIdx.y;
    c.n = max(0, min(A.nstate[c.seq], A.max_states));
    c.i0 = min(c.n, (int)blockIdx.x * kRdrChunk);
    c.i1 = min(c.n, c.i0 + kRdrChunk);
    c.base = (int64_t)c.seq * A.max_states;
    return c;
}

__device__ __forceinline__ double hi_of(const RdrArgs &A, int seq) {
    return 2.0 * __longlong_as_double((long long)A.ws_hib[seq]) + 1e-300;
}

// the 15 midpoints the next four bisection steps can visit from [lo, hi],
// in heap order (node k's children are 2k+1 (kept half [lo, mid]) and
// 2k+2 (kept half [mid, hi]))
__device__ __forceinline__ void subtree_mids(double lo, double hi, double (&lam)[15]) {
    double nlo[15], nhi[15];
    nlo[0] = lo;
    nhi[0] = hi;
#pragma unroll
    for (int k = 0; k < 15; ++k) {
        lam[k] = 0.5 * (nlo[k] + nhi[k]);
        if (2 * k + 2 < 15) {
            nlo[2 * k + 1] = nlo[k];
            nhi[2 * k + 1] = lam[k];
            nlo[2 * k + 2] = lam[k];
            nhi[2 * k + 2] = nhi[k];
        }
    }
}

// four bisection steps from [lo, hi] with the totals of its 15 midpoints
__device__ __forceinline__ void walk4(double &lo, double &hi, const long long *tot, long long budget) {
    double lam[15];
    subtree_mids(lo, hi, lam);
    int k = 0;
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        double lk = 0.0;
        long long tk = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
            if (j == k) {
                lk = lam[j];
                tk = tot[j];
            }
        }
        if (tk <= budget) hi = lk;
        else lo = lk;
        k = tk <= budget ? 2 * k + 1 : 2 * k + 2;
    }
}

// A multiplier at which every unprotected state is evicted: the largest
// distortion saved per byte, over the chunks (binary64 bit patterns of
// non-negative numbers order like the numbers).
__global__ __launch_bounds__(kRdrThreads) void k_rdr_hi(RdrArgs A) {
    __shared__ double redd[kRdrWaves];
    const Chunk c = chunk_of(A);
    double hl = 0.0;
    for (int i = c.i0 + threadIdx.x; i < c.i1; i += kRdrThreads) {
        if (A.prot[c.base + i]) continue;
        const double u = (double)A.u[c.base + i], kn = (double)A.knorm[c.base + i];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k >= A.ntiers) break;
            double f = A.sigma * kn * A.eps[k];
            if (f > 1.0) f = 1.0;
            const double gain = u - u * f;
            const double r = gain / (double)A.bytes[k];
            if (r > hl) hl = r;
        }
    }
    const double m = block_reduce(hl, [](double x, double y) { return x > y ? x : y; }, redd);
    if (threadIdx.x == 0) atomicMax(&A.ws_hib[c.seq], (unsigned long long)__double_as_longlong(m));
}

// Round r of the multiplier search.  r = 0: the totals at 0 and at the upper
// bound.  r = 1..16: the interval of this round (from the previous round's
// interval and totals), then the totals at its 15 midpoints.  Chunk 0
// records the interval for the next round and for the plan.
__global__ __launch_bounds__(kRdrThreads) void k_rdr_round(RdrArgs A, int r) {
    __shared__ long long redm[kRdrWaves][16];
    const Chunk c = chunk_of(A);
    // this thread's states are requested first: they do not depend on the
    // interval, which takes two dependent reads to find
    const int j0 = c.i0 + threadIdx.x * kRdrPer, j1 = min(c.i1, j0 + kRdrPer);
    float su[kRdrPer], skn[kRdrPer];
    uint8_t spr[kRdrPer];
#pragma unroll
    for (int e = 0; e < kRdrPer; ++e) {
        const int i = min(j0 + e, max(c.n - 1, 0));
        su[e] = c.n ? A.u[c.base + i] : 0.f;
        skn[e] = c.n ? A.knorm[c.base + i] : 0.f;
        spr[e] = c.n ? A.prot[c.base + i] : 0;
    }
    const long long budget = A.budget[c.seq];
    long long *tot = A.ws_tot + (int64_t)c.seq * 17 * 16;
    double *iv = A.ws_iv + (int64_t)c.seq * 17 * 2;
    const double hi0 = hi_of(A, c.seq);
    double lam[15];
    int nl;
    if (r == 0) {
        lam[0] = 0.0;
        lam[1] = hi0;
        nl = 2;
    } else {
        if (tot[0] <= budget) return;   // the plan at multiplier 0 fits: no search
        double lo, hi;
        if (r == 1) {
            lo = 0.0;
            hi = hi0;
        } else {
            lo = iv[2 * (r - 1)];
            hi = iv[2 * (r - 1) + 1];
            walk4(lo, hi, tot + 16 * (r - 1), budget);
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            iv[2 * r] = lo;
            iv[2 * r + 1] = hi;
        }
        subtree_mids(lo, hi, lam);
        nl = 15;
    }
    // the byte totals of this chunk's states at the nl multipliers; per
    // state the distortion of each tier is formed once (as rdr_choose forms
    // it) and its cost compared at every multiplier
    long long top_bytes = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (k == A.ntiers - 1) top_bytes = A.bytes[k];
    long long t[15];
#pragma unroll
    for (int m = 0; m < 15; ++m) t[m] = 0;
#pragma unroll
    for (int e = 0; e < kRdrPer; ++e) {
        if (j0 + e >= j1) break;
        if (spr[e]) {
#pragma unroll
            for (int m = 0; m < 15; ++m)
                if (m < nl) t[m] += top_bytes;
            continue;
        }
        const double ud = (double)su[e], kd = (double)skn[e];
        double dk[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k >= A.ntiers) break;
            double f = A.sigma * kd * A.eps[k];
            if (f > 1.0) f = 1.0;
            dk[k] = ud * f;
        }
        for (int m = 0; m < 15; ++m) {
            if (m >= nl) break;
            long long bb = 0;
            double bc = ud;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (k >= A.ntiers) break;
                const double cst = dk[k] + lam[m] * (double)A.bytes[k];
                if (cst < bc) {
                    bc = cst;
                    bb = A.bytes[k];
                }
            }
            t[m] += bb;
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < 15; ++m) {
        long long v = t[m];
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (lane == m) redm[wave][m] = v;
    }
    __syncthreads();
    if (threadIdx.x < nl) {
        long long v = 0;
        for (int w = 0; w < kRdrWaves; ++w) v += redm[w][threadIdx.x];
        atomicAdd(reinterpret_cast<unsigned long long *>(tot + 16 * r + threadIdx.x), (unsigned long long)v);
    }
}

// the multiplier of the plan: 0 when the plan at 0 fits, else the upper end
// of the interval after the 64 steps
__device__ __forceinline__ double final_lambda(const RdrArgs &A, int seq, long long budget) {
    const long long *tot = A.ws_tot + (int64_t)seq * 17 * 16;
    const double *iv = A.ws_iv + (int64_t)seq * 17 * 2;
    if (tot[0] <= budget) return 0.0;
    double lo = iv[2 * 16], hi = iv[2 * 16 + 1];
    walk4(lo, hi, tot + 16 * 16, budget);
    return hi;
}

// The plan of each state, and per chunk the count of each tier.
__global__ __launch_bounds__(kRdrThreads) void k_rdr_plan(RdrArgs A) {
    __shared__ int redi[kRdrWaves];
    const Chunk c = chunk_of(A);
    const long long budget = A.budget[c.seq];
    const double lambda = final_lambda(A, c.seq, budget);
    const int j0 = c.i0 + threadIdx.x * kRdrPer, j1 = min(c.i1, j0 + kRdrPer);
    int cnt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) cnt[k] = 0;
    for (int i = j0; i < j1; ++i) {
        const int o = rdr_choose((double)A.u[c.base + i], (double)A.knorm[c.base + i], A, lambda, A.prot[c.base + i] != 0);
        int tb = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (o == k + 1) {
                tb = A.tiers[k];
                ++cnt[k];
            }
        }
        A.tier_out[c.base + i] = (uint8_t)tb;
    }
    int *ccnt = A.ws_cnt + ((int64_t)c.seq * A.nchunk + blockIdx.x) * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k >= A.ntiers) break;
        int tot_k;
        block_excl_scan(cnt[k], redi, tot_k);
        if (threadIdx.x == 0) ccnt[k] = tot_k;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const long long *tot = A.ws_tot + (int64_t)c.seq * 17 * 16;
        A.lambda[c.seq] = lambda;
        A.status[c.seq] = (tot[0] > budget && tot[1] > budget) ? 2 : 0;
    }
}

// Tier-homogeneous pages: tiers in order, states in index order, 16 per
// page.  Each chunk starts each tier after the earlier chunks' states of
// that tier; chunk 0 writes the page tiers and the page count.
__global__ __launch_bounds__(kRdrThreads) void k_rdr_pack(RdrArgs A) {
    __shared__ int redi[kRdrWaves];
    const Chunk c = chunk_of(A);
    const int *cnt = A.ws_cnt + (int64_t)c.seq * A.nchunk * 8;
    const int nch = (c.n + kRdrChunk - 1) / kRdrChunk;
    const int j0 = c.i0 + threadIdx.x * kRdrPer, j1 = min(c.i1, j0 + kRdrPer);
    int page = 0;
    for (int k = 0; k < A.ntiers; ++k) {
        // the earlier chunks' count of tier k, and all chunks' (a block
        // reduction over the per-chunk counts)
        int vb = 0, vt = 0;
        for (int ch = threadIdx.x; ch < nch; ch += kRdrThreads) {
            const int v = cnt[ch * 8 + k];
            vt += v;
            if (ch < (int)blockIdx.x) vb += v;
        }
        int total;
        block_excl_scan(vt, redi, total);
        int before;
        block_excl_scan(vb, redi, before);
        const uint8_t tk = (uint8_t)A.tiers[k];
        int mine = 0;
        for (int i = j0; i < j1; ++i) mine += A.tier_out[c.base + i] == tk;
        int blk;
        int pos = before + block_excl_scan(mine, redi, blk);
        for (int i = j0; i < j1; ++i) {
            if (A.tier_out[c.base + i] != tk) continue;
            A.page_out[c.base + i] = page + pos / 16;
            A.slot_out[c.base + i] = pos % 16;
            ++pos;
        }
        const int np = (total + 15) / 16;
        // page headers: the tier, and on the tier's last page its empty slots
        if (blockIdx.x == 0)
            for (int p = threadIdx.x; p < np; p += kRdrThreads)
                if (page + p < A.max_pages_out)
                    A.page_tier[(int64_t)c.seq * A.max_pages_out + page + p] =
                        (uint8_t)(tk | ((p == np - 1 ? np * 16 - total : 0) << 4));
        page += np;
    }
    for (int i = j0; i < j1; ++i) {
        if (A.tier_out[c.base + i] == 0) {
            A.page_out[c.base + i] = -1;
            A.slot_out[c.base + i] = -1;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) A.npages[c.seq] = page;
}

hipError_t launch_rdr(const RdrArgs &a, int batch, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    const dim3 grid((unsigned)a.nchunk, (unsigned)batch);
    hipLaunchKernelGGL(k_rdr_hi, grid, dim3(kRdrThreads), 0, s, a);
    for (int r = 0; r <= 16; ++r) hipLaunchKernelGGL(k_rdr_round, grid, dim3(kRdrThreads), 0, s, a, r);
    hipLaunchKernelGGL(k_rdr_plan, grid, dim3(kRdrThreads), 0, s, a);
    hipLaunchKernelGGL(k_rdr_pack, grid, dim3(kRdrThreads), 0, s, a);
    return hipGetLastError();
}

int rdr_chunk_states() { return kRdrChunk; }

}  // namespace ska
