// k_decode.hip -- launch dispatch of the decode kernels (their templates are
// in k_decode.h, instantiated per (head dimension, group size) in
// k_decode_inst.hip) and the decompress step of the decompress-then-dot
// baseline.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary,
// section 1 (decompress-then-dot re-adds HBM traffic) and section 2.1.
#include "k_decode.h"

namespace ska {

extern template hipError_t launch_dg<128, 4, false>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<128, 4, true>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<128, 2, false>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<128, 2, true>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<128, 1, false>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<128, 1, true>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<64, 4, false>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<64, 4, true>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<64, 2, false>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<64, 2, true>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<64, 1, false>(const DecodeArgs &, int, dim3, hipStream_t);
extern template hipError_t launch_dg<64, 1, true>(const DecodeArgs &, int, dim3, hipStream_t);
// ---- decompress (the first step of decompress-then-dot, the path the codes
// avoid): the dense key r~ * u(centres(c)) of every (token, KV head) of the
// resident pages, rounded to bf16 and written token-major to the dense key
// pool.  One wave per (sequence, page, KV head); lane (t, j) decodes the d/4
// components of slice j of token t as the coded kernels do and stores them
// as 2*(d/4) contiguous bytes. ----
template <int D, int B>
__device__ __forceinline__ void decompress_pack(const uint32_t (&cw)[8], const float2 *__restrict__ lut, float rr,
                                                uint32_t (&pk)[D / 8]) {
    constexpr int NA = D / 4;
    const int j = threadIdx.x & 3;
    const uint32_t az_base = 8u * ((j == 3) ? lut_azimuth(B) : lut_polar(B));
    const uint32_t pad_base = 8u * ((j == 3) ? kLutOnes : lut_polar(B));
    const char *lutb = reinterpret_cast<const char *>(lut);
    CodeAddr<B> ca;
    ca.init(cw);
    float w[NA];
    float P = 1.f;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const uint32_t c8 = ca.at(cw, i);
        uint32_t e8;
        if (i == NA - 2) e8 = az_base + c8;
        else if (i == NA - 1) e8 = pad_base + c8;
        else e8 = 8u * lut_polar(B) + c8;
        const float2 cs = *reinterpret_cast<const float2 *>(lutb + e8);
        w[i] = P * cs.x;
        P = P * cs.y;
    }
    const float sc = rr * slice_prefix(P, j);
    // gfx950 converts a pair of binary32 values to bf16 (round to nearest
    // even) in one instruction
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < NA / 2; ++i) {
        const f32x2 v = {sc * w[2 * i], sc * w[2 * i + 1]};
        pk[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
}

constexpr int kDecompChunk = 64;   // pages per decompress workgroup

// Decompression of the keys to a dense bf16 pool [num_pages][hkv][16][D]:
// one workgroup per (KV head, sequence, chunk of kDecompChunk pages), wave w
// taking pages w, w + kWaves, ... of the chunk.  TB is the tier of a pool of
// one tier at a fixed stride; TB = 0 reads the tier of each page from its
// header (and its offset from the page offsets when the pool has them).
//
// The block-table entries of a wave's pages (and for TB = 0 their headers
// and offsets) are read once, one page per lane, and the radius levels of
// the head sit in LDS, so inside the loop the only global accesses are the
// page loads and the stores.  Every page slot issues the same loads and
// stores whether or not it holds a page: a slot past the chunk, a bad page id
// or a bad header gets an empty descriptor (its loads read zeros, its stores
// are dropped), and errors are gathered in a register and posted once at the
// end.  With the memory operations the same on every path the compiler's
// wait before decoding a page counts exactly that page's loads, not the
// stores of the page before.
//
// The dense block of a (page, head) leaves through LDS so that each store
// covers one contiguous 1 KB run, and the stores are marked non-temporal:
// the dense pool streams out to HBM rather than displacing cached lines.
template <int D, int TB>
__global__ __launch_bounds__(kThreads) void k_decompress(DecodeArgs A) {
    constexpr int kPer = kDecompChunk / kWaves;
    static_assert(kDecompChunk % kWaves == 0 && kPer <= 64, "pages per wave");
    constexpr int kOut = kPage * D * 2;                  // bytes of one (page, head) dense block
    static_assert(kOut == (D / 32) * 64 * 16, "one store per lane and 1 KB run");
    constexpr int kStoreNT = 2;                          // cache policy: non-temporal
    __shared__ float2 lut[kLutEntries];
    __shared__ float rlev[256];
    __shared__ uint4 stage[kWaves][kOut / 16];
    const int kvh = blockIdx.x, seq = blockIdx.y;
    for (int e = threadIdx.x; e < kLutEntries; e += kThreads) lut[e] = A.lut[e];
    for (int e = threadIdx.x; e < 256; e += kThreads) rlev[e] = A.rlev[kvh * 256 + e];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int len = max(0, min(A.seq_lens[seq], A.max_pages * kPage));
    const int npages = (len + kPage - 1) / kPage;
    const int p_end = min(npages, (int)(blockIdx.z + 1) * kDecompChunk);
    const int p0 = blockIdx.z * kDecompChunk + wave;       // this wave: pages p0 + kWaves * i
    const int cnt = p_end > p0 ? (p_end - p0 + kWaves - 1) / kWaves : 0;
    // page ids are int32: a 32-bit unsigned test against the pool size
    // (capped at 2^31) is the range check, and stays on the scalar unit
    const uint32_t npg32 = (uint32_t)min<int64_t>(A.num_pages, 0x80000000LL);
    int btv = -1, hbv = 0;
    uint64_t offv = 0;
    if (lane < cnt) {
        btv = A.block_table[(int64_t)seq * A.max_pages + p0 + kWaves * lane];
        if (TB == 0 && (uint32_t)btv < npg32) {
            const int64_t hix = A.head_tiers ? (int64_t)btv * A.hkv + kvh : (int64_t)btv;
            hbv = A.page_bits[hix] & 15;   // (the tier bits of the header)
            offv = A.page_off ? A.page_off[hix] : (uint64_t)btv * (uint64_t)A.page_stride;
        }
    }
    uint32_t err = 0;
    __syncthreads();
    struct Pg {
        uint32_t cw[8];
        uint32_t rc, hb;
        int ph, b, live;
    };
    auto fetch = [&](int i, Pg &g) {
        const int li = min(i, kPer - 1);
        const int ph = __builtin_amdgcn_readlane(btv, li);
        const bool inr = i < cnt;
        const bool ok = inr && (uint32_t)ph < npg32;
        err |= (inr && !ok) ? 2u : 0u;
        const int phc = ok ? ph : 0;
        int b = TB, KB = record_bytes(D, TB == 0 ? 8 : TB);
        uint64_t off = (uint64_t)phc * (uint64_t)A.page_stride;
        bool live = ok;
        if (TB == 0) {
            b = __builtin_amdgcn_readlane(hbv, li);
            const bool tier_ok = b >= 2 && b <= 8 && ((A.tier_mask >> b) & 1u) && ((kSupportedTiers >> b) & 1u);
            err |= (ok && !tier_ok) ? 4u : 0u;
            live = ok && tier_ok;
            KB = live ? record_bytes(D, b) : 0;
            off = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(offv >> 32), li) << 32) |
                  __builtin_amdgcn_readlane((uint32_t)offv, li);
        }
        // (the bases are read back as scalars: without that the compiler
        // may form a 64-bit sum on the vector unit and then loop over lanes
        // to build the descriptor)
        const uint64_t hoff = (TB == 0 && A.head_tiers) ? 0 : (uint64_t)kvh * kPage * KB;
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(scalar_ptr(A.kcode + off + hoff),
                                                   __builtin_amdgcn_readfirstlane(live ? kPage * KB : 0));
        const __amdgpu_buffer_rsrc_t rr = buf_rsrc(scalar_ptr(A.rcode + ((int64_t)phc * A.hkv + kvh) * kPage),
                                                   __builtin_amdgcn_readfirstlane(live ? kPage : 0));
        const int vo = t * KB + j * (KB / 4);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 16 * k, 0, 0);
            g.cw[4 * k + 0] = x[0]; g.cw[4 * k + 1] = x[1]; g.cw[4 * k + 2] = x[2]; g.cw[4 * k + 3] = x[3];
        }
        g.rc = __builtin_amdgcn_raw_buffer_load_b8(rr, t, 0, 0);
        if (TB != 0) {
            // one tier: the header travels with the page and is checked
            // before the stores
            const __amdgpu_buffer_rsrc_t rh =
                buf_rsrc(scalar_ptr(A.page_bits + phc), __builtin_amdgcn_readfirstlane(ok ? 1 : 0));
            g.hb = __builtin_amdgcn_raw_buffer_load_b8(rh, 0, 0, 0);
        } else {
            g.hb = b;
        }
        g.ph = phc;
        g.b = b;
        g.live = live ? 1 : 0;
    };
    auto emit = [&](const Pg &g) {
        bool st = g.live;
        if (TB != 0) {
            const bool hdr_ok = (__builtin_amdgcn_readfirstlane(g.hb) & 15u) == (uint32_t)TB;
            err |= (g.live && !hdr_ok) ? 4u : 0u;
            st = g.live && hdr_ok;
        }
        const __amdgpu_buffer_rsrc_t rd = buf_rsrc(scalar_ptr(A.kdense + ((int64_t)g.ph * A.hkv + kvh) * (kPage * D)),
                                                   __builtin_amdgcn_readfirstlane(st ? kOut : 0));
        uint32_t pk[D / 8];
        const float rr = rlev[g.rc & 255u];
        if (TB != 0) {
            decompress_pack<D, TB>(g.cw, lut, rr, pk);
        } else {
            switch (g.b) {
                case 2: decompress_pack<D, 2>(g.cw, lut, rr, pk); break;
                case 3: decompress_pack<D, 3>(g.cw, lut, rr, pk); break;
                case 4: decompress_pack<D, 4>(g.cw, lut, rr, pk); break;
                case 6: decompress_pack<D, 6>(g.cw, lut, rr, pk); break;
                default: decompress_pack<D, 8>(g.cw, lut, rr, pk); break;
            }
        }
        // The lane's D/4 values are 16-byte pieces at a 64-byte lane stride
        // (token t, quarter j); stored straight from the lanes every store
        // would scatter 16-byte pieces.  The 16-byte slots of the stage are
        // swizzled (bits 0-1 of the slot index XOR bits 4-5), which spreads
        // both the lane-strided writes and the contiguous reads over
        // distinct LDS banks.
        uint4 *sw = stage[wave];
        auto slot = [](int idx) { return idx ^ ((idx >> 4) & 3); };
#pragma unroll
        for (int k = 0; k < D / 32; ++k)
            sw[slot(t * (D / 8) + j * (D / 32) + k)] = make_uint4(pk[4 * k], pk[4 * k + 1], pk[4 * k + 2], pk[4 * k + 3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
            const uint4 x = sw[slot(k * 64 + lane)];
            const __attribute__((ext_vector_type(4))) uint32_t v4 = {x.x, x.y, x.z, x.w};
            __builtin_amdgcn_raw_buffer_store_b128(v4, rd, (k * 64 + lane) * 16, 0, kStoreNT);
        }
        // (the next page's writes to the stage come after these reads)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // (the scheduling barriers keep each page's loads issued ahead of the
    // wait for the page before)
    Pg b0, b1;
    fetch(0, b0);
    {
        // stores through an empty descriptor (dropped): on entry the queue of
        // memory operations then looks as it does on every later turn of the
        // loop (a page's loads, then D/32 stores), so the wait counts
        // computed for the loop need not cover the stores
        const __amdgpu_buffer_rsrc_t rz = buf_rsrc(A.kdense, 0);
        const __attribute__((ext_vector_type(4))) uint32_t z4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < D / 32; ++k) __builtin_amdgcn_raw_buffer_store_b128(z4, rz, 16 * k, 0, kStoreNT);
    }
    // two buffers used in turn (no register copies, which would wait for
    // the loads in flight and the stores before them)
#pragma unroll 1
    for (int i = 0; i < cnt; i += 2) {
        fetch(i + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        emit(b0);
        fetch(i + 2, b0);
        __builtin_amdgcn_sched_barrier(0);
        emit(b1);
    }
    if (err && lane == 0) atomicOr(A.err, err);
}

hipError_t launch_decompress(const DecodeArgs &a, int d, int B, hipStream_t s) {
    if (B == 0) return hipSuccess;
    const dim3 grid((unsigned)a.hkv, (unsigned)B, (unsigned)((a.max_pages + kDecompChunk - 1) / kDecompChunk));
    int tb = 0;
    if (__builtin_popcount(a.tier_mask) == 1 && !a.page_off) tb = __builtin_ctz(a.tier_mask);
#define SKA_DECOMP(DD)                                                                              \
    switch (tb) {                                                                                   \
        case 2: hipLaunchKernelGGL((k_decompress<DD, 2>), grid, dim3(kThreads), 0, s, a); break;    \
        case 3: hipLaunchKernelGGL((k_decompress<DD, 3>), grid, dim3(kThreads), 0, s, a); break;    \
        case 4: hipLaunchKernelGGL((k_decompress<DD, 4>), grid, dim3(kThreads), 0, s, a); break;    \
        case 6: hipLaunchKernelGGL((k_decompress<DD, 6>), grid, dim3(kThreads), 0, s, a); break;    \
        case 8: hipLaunchKernelGGL((k_decompress<DD, 8>), grid, dim3(kThreads), 0, s, a); break;    \
        default: hipLaunchKernelGGL((k_decompress<DD, 0>), grid, dim3(kThreads), 0, s, a); break;   \
    }
    if (d == 128) {
        SKA_DECOMP(128)
    } else {
        SKA_DECOMP(64)
    }
#undef SKA_DECOMP
    return hipGetLastError();
}

// The order of the units of a batch that runs in several rounds.  The
// workgroup dispatcher starts workgroups strictly in grid order, and on each
// XCD a workgroup waits for a free CU in its own shader engine (consecutive
// slots of an XCD cycle over its engines) while the later ones wait behind
// it; units of very different sizes in consecutive slots therefore left up to
// a quarter of the CUs idle (in-kernel timestamps on a ragged batch of 64).
// Handed out in decreasing size, neighbouring slots hold units of similar
// size and the engines fill and drain together.  One workgroup: the units of
// each sequence (as the decode splits it) get the key (size descending, split
// descending, sequence), unique, so the order is the same on every call;
// slot i of the table receives the unit of the i-th smallest key and its
// sequence's length (-1 past the last unit).  Up to kUnitRankMax units, each
// unit's slot is the number of keys below its own (one pass over the keys in
// LDS, read by every lane of a wave at once); more units are sorted with a
// bitonic network in LDS.  Which workgroup computes a unit does not change
// the unit's result, so the outputs do not depend on the order.
constexpr int kUnitSortThreads = 1024;
constexpr int kUnitRankMax = kUnitSortThreads;
static_assert(kCompactMaxBatch <= kUnitSortThreads, "one thread per sequence");
static_assert(kUnitRankMax % 2 == 0 && kUnitRankMax < kUnitSortMax, "pairs of keys, one key per thread");
__global__ __launch_bounds__(kUnitSortThreads) void k_unit_order(DecodeArgs A, int B, int nslots) {
    __shared__ __attribute__((aligned(16))) uint64_t key[kUnitSortMax];
    __shared__ int wsum[kUnitSortThreads / 64];
    __shared__ int lens[kCompactMaxBatch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int len = 0, np = 0, ns = 0;
    if (tid < B) {
        len = A.seq_lens[tid];
        np = (max(0, min(len, A.max_pages * kPage)) + kPage - 1) / kPage;
        ns = max(1, splits_of(A, np));   // a sequence without pages still has one unit
        lens[tid] = len;
    }
    // exclusive prefix of the unit counts: a scan within each wave, then the
    // waves' totals
    int incl = ns;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        incl += lane >= o ? v : 0;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int total = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kUnitSortThreads / 64; ++w) {
        const int t = wsum[w];
        total += t;
        before += w < wave ? t : 0;
    }
    const int first = before + incl - ns;
    for (int j = 0; j < ns; ++j) {
        const int size = min(np, split_start(A, j + 1)) - split_start(A, j);
        key[first + j] = ((uint64_t)(0xFFFFF - size) << 36) | ((uint64_t)(0xFFFF - j) << 16) | (uint64_t)tid;
    }
    auto unit_of = [&](uint64_t kk) {
        const int sq = (int)(kk & 0xFFFF), sp = 0xFFFF - (int)((kk >> 16) & 0xFFFF);
        return make_int2((sq << 16) | sp, lens[sq]);
    };
    if (total <= kUnitRankMax) {
        if (tid == 0 && (total & 1)) key[total] = ~0ull;   // (pairs: a key above every unit's)
        __syncthreads();
        if (tid < total) {
            const uint64_t k = key[tid];
            const ulonglong2 *kp = reinterpret_cast<const ulonglong2 *>(key);
            int rank = 0;
            for (int v = 0; v < (total + 1) / 2; ++v) {
                const ulonglong2 kk = kp[v];
                rank += (kk.x < k ? 1 : 0) + (kk.y < k ? 1 : 0);
            }
            A.unit_table[rank] = unit_of(k);
        }
        for (int i = total + tid; i < nslots; i += kUnitSortThreads) A.unit_table[i] = make_int2(-1, 0);
        return;
    }
    int P = 1;
    while (P < total) P <<= 1;
    for (int i = total + tid; i < P; i += kUnitSortThreads) key[i] = ~0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += kUnitSortThreads) {
                const int l = i ^ j;
                if (l > i) {
                    const uint64_t a = key[i], b = key[l];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        key[i] = b;
                        key[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < nslots; i += kUnitSortThreads) A.unit_table[i] = i < total ? unit_of(key[i]) : make_int2(-1, 0);
}

hipError_t launch_decode(const DecodeArgs &a, int d, int G, int B, hipStream_t s) {
    if (B == 0) return hipSuccess;
    if (a.compact) {
        hipLaunchKernelGGL(k_unit_order, dim3(1), dim3(kUnitSortThreads), 0, s, a, B, B * a.nsplit);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)a.hkv, (unsigned)B, (unsigned)a.nsplit);
    int tb = 0;
    // single-tier pools at a fixed page stride take the tier-specialised kernel
    if (__builtin_popcount(a.tier_mask) == 1 && !a.page_off) tb = __builtin_ctz(a.tier_mask);
    if (a.dense) tb = kDenseTB;
    const bool qf = a.query_f32 != 0 && !a.dense;
#define SKA_DG(DD, GG)                                                                   \
    return qf ? launch_dg<DD, GG, true>(a, tb, grid, s) : launch_dg<DD, GG, false>(a, tb, grid, s)
    if (d == 128) {
        if (G == 4) SKA_DG(128, 4);
        if (G == 2) SKA_DG(128, 2);
        SKA_DG(128, 1);
    }
    if (G == 4) SKA_DG(64, 4);
    if (G == 2) SKA_DG(64, 2);
    SKA_DG(64, 1);
#undef SKA_DG
}

int decode_workgroups_per_cu() { return 8 / kWaves; }

__global__ void k_zero_u32(uint32_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace ska
