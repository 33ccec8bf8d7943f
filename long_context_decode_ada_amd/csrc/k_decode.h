// k_decode.h -- Angle-Domain Attention decode over the paged code store: the
// kernel templates.  Each (head dimension, group size) family is
// instantiated in its own translation unit (k_decode_inst.hip); k_decode.hip
// holds the launch dispatch and the decompress baseline.
//
// Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
// Retention for Efficient Long-Context Inference", technical summary:
//   section 2.1  logit l = |q| * r~ * f_b(c_q, c_k), f_b the cosine of the two
//                decoded directions, computed from the codes inside the
//                decode loop; no dense key is materialised in HBM;
//   section 2.2  tier-homogeneous pages read by single-pass, header-guided
//                streaming (the header is page_bits[phys]).
// The pages describe no kernel.  This design is for CDNA4 (gfx950, wave64):
//
//  * Work: one workgroup of 8 waves (two per SIMD, one workgroup per CU)
//    per (sequence, kv head, split of pages); each wave walks a contiguous
//    run of the split's pages, one page per step.  The wave dispatched first
//    to a SIMD is served memory ahead of the second, so the first four waves
//    take a larger, fixed share of the split (set on the host).
//  * f_b: a wave holds one page of one kv head: lane (t, j) = (token t of 16,
//    slice j of 4).  Slice j covers components [j*d/4, (j+1)*d/4) of the
//    direction.  In hyperspherical coordinates component a of u is
//    (prod_{k<a} sin phi_k) * cos phi_a, so the lane forms a running product
//    of sines P in registers, starting at 1 for its slice, and accumulates
//    F_h = sum_a uq_h[a] * P_a * cos phi_a for the G query heads of the kv
//    head; (cos, sin) of the bin centres come from an LDS table indexed by
//    the b-bit code.  The four slices are joined by a 4-lane exclusive
//    product scan of the slice sine products (DPP quad permutes):
//    f_h = sum_j C_j F_h,j with C_j = prod_{i<j} S_i.
//  * The query side, the unit vector uq = u(centres(c_q)) per tier, is
//    prepared in each workgroup's prologue (from the G query rows of its kv
//    head) as fp16 pairs and held packed in registers; v_fma_mix_f32
//    multiplies a half by the fp32 w and accumulates in fp32.  Rounding uq to
//    fp16 moves f by at most 2^-11 (Cauchy-Schwarz over two unit vectors).
//    The logit is sq_h * r~ * f with sq_h = scale * |q_h| * log2(e) in fp32,
//    so logits are in log2 units.
//  * Softmax: online, per head, with the running max raised only when a logit
//    exceeds it by more than 8 (a wave ballot); probabilities are bounded by
//    2^8, which fp32 accumulation absorbs.
//  * P.V: for one page the group's product is (G heads x 16 tokens) times
//    (16 tokens x d) -- a dense contraction, run on MFMA
//    v_mfma_f32_16x16x16_bf16.  P is split exactly as P = hi + lo with hi,
//    lo in bf16 (rows 0..G-1 and G..2G-1 of the A operand), so the product
//    keeps 16 mantissa bits of P; V enters as stored (bf16), dimension-major
//    pages giving each lane its 4 consecutive tokens as one 8-byte load.
//  * Page pipeline: the loads of page k+1 are in flight (a second register
//    set) while page k is computed; loads are issued on every path (through
//    empty descriptors past the end), so the compiler's wait counts stay
//    exact and the pipeline never drains.  Single-tier pools read the block
//    table 64 entries at a time into two rotating register slots; pools of
//    mixed tiers order each 64-page chunk by tier (one query reload per tier).
//  * Split-T: each workgroup merges its 8 waves in LDS and writes one
//    (m, l, o[d]) partial per query head with device-coherent stores; the
//    last workgroup of a (sequence, kv head) to finish (a device-scope
//    counter) merges the splits with device-coherent loads.  No cache
//    write-back or invalidation is involved: a device-scope fence, which
//    writes back and invalidates a whole XCD's L2, measured about 6 us per
//    launch on this part.
#pragma once

#include <type_traits>

#include "ska_codes.h"
#include "ska_internal.h"

namespace ska {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994531f;

// Pipeline depth and occupancy: two waves per SIMD, each keeping the loads
// of the next page in flight while it computes one (kBufs register sets).
#ifndef SKA_BUFS
#define SKA_BUFS 2
#endif
#ifndef SKA_WAVES_PER_SIMD
#define SKA_WAVES_PER_SIMD 2
#endif
constexpr int kBufs = SKA_BUFS;
// kernel variant reading dense bf16 keys (the baseline the codes replace)
constexpr int kDenseTB = 16;
constexpr int kWavesPerSimd = SKA_WAVES_PER_SIMD;

// DPP quad permutations (within groups of 4 lanes).
template <int CTRL>
__device__ __forceinline__ float qperm(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadShr1 = 0x90;  // lane j <- lane max(j-1, 0)
constexpr int kQuadShr2 = 0x44;  // lane j <- lane j-2 (j >= 2), j (j < 2)
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// x from the lane DPP control CTRL names, or 1 where there is no such lane
// (or the row is outside ROWS)
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), CTRL, ROWS, 0xF, false));
}

// binary64 lane operations, one 32-bit half at a time
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_or_zero_d(double x) {
    const int64_t v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, ROWS, 0xF, false);
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double bpermute_d(int src_lane, double x) {
    const int64_t v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_ds_bpermute(src_lane * 4, (int)(uint32_t)v);
    const int hi = __builtin_amdgcn_ds_bpermute(src_lane * 4, (int)(v >> 32));
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
    const int64_t v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}
// sum of x over the lanes above this one (binary64; a scan over the
// reversed lanes: row shifts, row broadcasts, one lane shift)
__device__ __forceinline__ double wave_suffix_sum_excl(double x) {
    const int lane = threadIdx.x & 63;
    double v = bpermute_d(63 - lane, x);
    v += dpp_or_zero_d<0x111, 0xF>(v);   // row_shr:1
    v += dpp_or_zero_d<0x112, 0xF>(v);   // row_shr:2
    v += dpp_or_zero_d<0x114, 0xF>(v);   // row_shr:4
    v += dpp_or_zero_d<0x118, 0xF>(v);   // row_shr:8
    v += dpp_or_zero_d<0x142, 0xA>(v);   // row_bcast:15
    v += dpp_or_zero_d<0x143, 0xC>(v);   // row_bcast:31
    v = dpp_or_zero_d<0x138, 0xF>(v);    // wave_shr:1: exclusive
    return bpermute_d(63 - lane, v);
}

template <int CTRL>
__device__ __forceinline__ float rowperm(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Reduce over the 16 token lanes (and, for G < 4, over the slices j that map
// to the same head) of every head.
template <int G, bool MAX>
__device__ __forceinline__ float head_reduce(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if (G == 1) x = op(x, qperm<kQuadXor1>(x));
    if (G <= 2) x = op(x, qperm<kQuadXor2>(x));
    x = op(x, rowperm<kRowRor4>(x));
    x = op(x, rowperm<kRowRor8>(x));
    x = op(x, __shfl_xor(x, 16));
    x = op(x, __shfl_xor(x, 32));
    return x;
}

template <int B>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&cw)[8], int i) {
    const int bit = i * B, w = bit >> 5, o = bit & 31;
    const uint32_t mask = (1u << B) - 1u;
    if (o + B <= 32) return (cw[w] >> o) & mask;
    return __builtin_amdgcn_alignbit(cw[w + 1], cw[w], o) & mask;
}

// 8 * (code i) of a slice: the byte offset of its (cos, sin) entry.  For
// b = 4, 8 and 2 the codes of each word are first spread (two or four masked
// shifts per word) so that every 8*code sits in its own byte or half-word and
// takes one extraction; other widths use a field extract and a shift.
// SPREAD = false: plain field extracts, no spread words (for kernels at the
// register limit, where eight or sixteen more live registers cost more than
// the extracts they save).
template <int B, bool SPREAD = true>
struct CodeAddr {
    uint32_t s[16];
    __device__ __forceinline__ void init(const uint32_t (&cw)[8]) {
        if constexpr (!SPREAD) {
            (void)cw;
            return;
        }
        constexpr int SW = record_bytes(B == 3 ? 128 : 128, B) / 16;
        if constexpr (B == 4) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                s[2 * k + 0] = (cw[k] & 0x0F0F0F0Fu) << 3;     // even codes * 8, one per byte
                s[2 * k + 1] = (cw[k] >> 1) & 0x78787878u;     // odd codes * 8
            }
        } else if constexpr (B == 8) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                s[2 * k + 0] = (cw[k] & 0x00FF00FFu) << 3;     // codes 0, 2 of the word, one per half-word
                s[2 * k + 1] = (cw[k] >> 5) & 0x07F807F8u;     // codes 1, 3
            }
        } else if constexpr (B == 2) {
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int m = 0; m < 4; ++m) s[4 * k + m] = ((cw[k] >> (2 * m)) & 0x03030303u) << 3;
        }
        if constexpr (B == 2 || B == 4 || B == 8) {
            // keep the spread words as computed: folded back into the code
            // words, each extraction would again cost a shift and a mask
            constexpr int NS = (B == 8) ? 16 : 8;
#pragma unroll
            for (int k = 0; k < NS; ++k) asm volatile("" : "+v"(s[k]));
        }
        (void)SW;
    }
    __device__ __forceinline__ uint32_t at(const uint32_t (&cw)[8], int i) const {
        if constexpr (!SPREAD) {
            return code_at<B>(cw, i) << 3;
        } else if constexpr (B == 4) {
            const uint32_t w = s[2 * (i >> 3) + (i & 1)];
            return __builtin_amdgcn_ubfe(w, 8 * ((i & 7) >> 1), 8);
        } else if constexpr (B == 8) {
            const uint32_t w = s[2 * (i >> 2) + (i & 1)];
            return __builtin_amdgcn_ubfe(w, 16 * ((i & 3) >> 1), 16);
        } else if constexpr (B == 2) {
            const uint32_t w = s[4 * (i >> 4) + (i & 3)];
            return __builtin_amdgcn_ubfe(w, 8 * ((i & 15) >> 2), 8);
        } else {
            return code_at<B>(cw, i) << 3;
        }
    }
};

// F + fp16(u half) * w in fp32 (v_fma_mix_f32).  Written as inline asm so
// that the packed query halves stay packed in registers: the compiler would
// otherwise hoist their conversion to fp32 out of the page loop.
__device__ __forceinline__ float fma_mix_lo(uint32_t u, float w, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(u), "v"(w), "v"(acc));
    return r;
}
__device__ __forceinline__ float fma_mix_hi(uint32_t u, float w, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(u), "v"(w), "v"(acc));
    return r;
}

// The query direction's precision in f_b (QF, the pool's query_precision):
// binary16 halves, two per register, multiplied in by v_fma_mix_f32, or
// binary32 words (v_fma_f32).  Rounding the direction to binary16 moves f by
// at most 2^-11 and typically by about 1e-4 at d = 128 (measured against the
// oracle), inside the logit tolerance; but where keys carry a few outlier
// channels (large radii, a sharp softmax) that logit error, scaled by the
// radius, moves the outputs by more than theirs.  binary32 takes the same
// instructions but twice the registers ((d/4 angles) x G heads per lane):
// at G = 4, d = 128 the kernels run at the register limit, so they extract
// the codes without spread words (CodeAddr); single-tier pools then decode
// about 4 % slower than with binary16 (b = 4; 1-2 % at b = 3); the
// header-dispatched kernel reads the query words from LDS instead
// (slice_fb_lds) and runs about 40 % slower.  So binary16 is the default and
// binary32 the precise mode.// 32-bit words of the query direction per lane: (D/4 angles) x G heads
template <int D, int G, bool QF>
constexpr int query_words() { return QF ? D * G / 4 : D * G / 8; }

// F + u * w for element e2 (angle-major, head-minor) of the lane's query words
template <int D, int G, bool QF>
__device__ __forceinline__ float query_fma(const uint32_t (&u)[query_words<D, G, QF>()], int e2, float w,
                                           float acc) {
    if constexpr (QF) return __builtin_fmaf(__uint_as_float(u[e2]), w, acc);
    else return (e2 & 1) ? fma_mix_hi(u[e2 >> 1], w, acc) : fma_mix_lo(u[e2 >> 1], w, acc);
}

// binary32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct WaveState {
    float m;     // running max (log2 units) of this lane's head
    float l;     // this lane's share of the softmax denominator
};

// Per-lane registers of one page: the lane's code slice, the radius byte of
// its token, and its V fragments for the MFMA B operand.
template <int D>
struct PageBuf {
    uint32_t cw[8];
    uint32_t rc;
    uint32_t hb;   // the page header (its angle bit width), single-tier kernels
    uint2 vf[D / 16];
    uint2 kf[D / 16];   // dense keys: the MFMA B operand of Q.K^T
};

// Wave-uniform description of one page.
struct PageDesc {
    int phys, b, p;
    int cnt;        // slots holding tokens (header-dispatched pages; single-tier kernels
                    // read the count from the header loaded with the page)
    uint64_t off;   // byte offset of the physical page's code block
    bool live;      // false: the loads go through empty descriptors and read nothing
};

// A wave-uniform address, read back into scalar registers.
__device__ __forceinline__ const void *scalar_ptr(const void *p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

// Cache policy of the value loads: non-temporal.  Each value is read once
// per call, and with this policy the decode runs about 13 % faster on the
// gqa_t32k batch (125 -> 109 us) and 7 % on long_t128k; marking the key
// codes as well gains nothing more.
constexpr int kValueLoadPolicy = 2;

// Raw buffer descriptor (V#) over `bytes` bytes at a wave-uniform address:
// loads past the end return 0 instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Loads of one page: the page's code block, radius bytes and V block each
// get a descriptor built in scalar registers; the per-lane offsets inside a
// block are the same for every page.
template <int D, int B, bool HDR>
__device__ __forceinline__ void load_page_b(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    constexpr int KB = record_bytes(D, B);
    constexpr int SW = KB / 16;
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int q4 = lane >> 4, n16 = lane & 15;
    const int64_t pk = (int64_t)pd.phys * A.hkv + kvh;
    const int lv = __builtin_amdgcn_readfirstlane(pd.live ? 1 : 0);   // scalar: descriptors stay uniform
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(A.kcode + pd.off + (uint64_t)kvh * kPage * KB, lv * kPage * KB);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(A.v + pk * (int64_t)D * kPage, lv * D * kPage * 2);
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(A.rcode + pk * kPage, lv * kPage);
    const int vo = t * KB + j * (KB / 4);
    if constexpr (SW == 1) {
        r.cw[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, vo, 0, 0);
    } else if constexpr (SW == 2) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rk, vo, 0, 0);
        r.cw[0] = x[0]; r.cw[1] = x[1];
    } else if constexpr (SW == 3) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b96(rk, vo, 0, 0);
        r.cw[0] = x[0]; r.cw[1] = x[1]; r.cw[2] = x[2];
    } else {
#pragma unroll
        for (int k = 0; k < SW / 4; ++k) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 16 * k, 0, 0);
            r.cw[4 * k + 0] = x[0]; r.cw[4 * k + 1] = x[1]; r.cw[4 * k + 2] = x[2]; r.cw[4 * k + 3] = x[3];
        }
        if constexpr (SW % 4 == 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(rk, vo + 16 * (SW / 4), 0, 0);
            r.cw[SW - 2] = x[0]; r.cw[SW - 1] = x[1];
        }
    }
    r.rc = __builtin_amdgcn_raw_buffer_load_b8(rr, t, 0, 0);
    if constexpr (HDR) {
        // the header travels with the page's data, so checking it waits for nothing else
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(A.page_bits + pd.phys, lv);
        r.hb = __builtin_amdgcn_raw_buffer_load_b8(rh, 0, 0, 0);
    }
    const int vv = (n16 * kPage + 4 * q4) * 2;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, vv + k * 16 * kPage * 2, 0, kValueLoadPolicy);
        r.vf[k] = make_uint2(x[0], x[1]);
    }
}

// Loads of one page of any tier (pools of mixed tiers): the same
// instructions whatever the page's width, so that the loads of the next page
// stay in flight across the tier dispatch of the computation.  Each lane
// reads 32 bytes from the start of its slice (KB/4 <= 32 bytes); the buffer
// range check is per dword, so the words past the page's record block read
// as 0 and the rest repeat bytes of the same cache lines.
template <int D>
__device__ __forceinline__ void load_page_any(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int q4 = lane >> 4, n16 = lane & 15;
    const int KB = record_bytes(D, pd.b);
    const int64_t pk = (int64_t)pd.phys * A.hkv + kvh;
    const int lv = __builtin_amdgcn_readfirstlane(pd.live ? 1 : 0);
    // (per-(page, KV head) tiers: pd.off is already this head's records)
    const __amdgpu_buffer_rsrc_t rk =
        buf_rsrc(A.kcode + pd.off + (A.head_tiers ? 0 : (uint64_t)kvh * kPage * KB), lv * kPage * KB);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(A.v + pk * (int64_t)D * kPage, lv * D * kPage * 2);
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(A.rcode + pk * kPage, lv * kPage);
    const int vo = t * KB + j * (KB / 4);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 16 * k, 0, 0);
        r.cw[4 * k + 0] = x[0]; r.cw[4 * k + 1] = x[1]; r.cw[4 * k + 2] = x[2]; r.cw[4 * k + 3] = x[3];
    }
    r.rc = __builtin_amdgcn_raw_buffer_load_b8(rr, t, 0, 0);
    const int vv = (n16 * kPage + 4 * q4) * 2;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, vv + k * 16 * kPage * 2, 0, kValueLoadPolicy);
        r.vf[k] = make_uint2(x[0], x[1]);
    }
}

// Loads of one page of dense bf16 keys and its values.  Keys are token-major
// ([16][d] per (page, KV head)); the lane takes the four dimensions
// 16k + 4(l/16) .. +3 of token l%16 for each k, the B operand of a 16x16x16
// MFMA over (dimension, token).
template <int D>
__device__ __forceinline__ void load_page_dense(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4, n16 = lane & 15;
    const int64_t pk = (int64_t)pd.phys * A.hkv + kvh;
    const int lv = __builtin_amdgcn_readfirstlane(pd.live ? 1 : 0);
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(A.kdense + pk * (int64_t)kPage * D, lv * kPage * D * 2);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(A.v + pk * (int64_t)D * kPage, lv * D * kPage * 2);
    const int ko = (n16 * D + 4 * q4) * 2;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rk, ko + 32 * k, 0, 0);
        r.kf[k] = make_uint2(x[0], x[1]);
    }
    const int vv = (n16 * kPage + 4 * q4) * 2;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, vv + k * 16 * kPage * 2, 0, kValueLoadPolicy);
        r.vf[k] = make_uint2(x[0], x[1]);
    }
}

template <int D, int TB>
__device__ __forceinline__ void load_page(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    if constexpr (TB == kDenseTB) load_page_dense<D>(A, pd, kvh, r);
    else if constexpr (TB != 0) load_page_b<D, TB, true>(A, pd, kvh, r);
    else load_page_any<D>(A, pd, kvh, r);
}

// The product of the sine products P of the slices before this lane's slice
// j within its token's four lanes (exclusive quad scan): C_j = prod_{i<j} P_i.
__device__ __forceinline__ float slice_prefix(float P, int j) {
    float C = qperm<kQuadShr1>(P);
    C = (j == 0) ? 1.f : C;
    const float z = qperm<kQuadShr1>(C);
    C = (j >= 1) ? C * z : C;
    const float z2 = qperm<kQuadShr2>(C);
    C = (j >= 2) ? C * z2 : C;
    return C;
}

// Online softmax of one page's logits lg (log2 units; lane 4t + j holds token
// t for head j % G) and the MFMA update of the G output rows with the page's
// values.  DBG also stores the logits.
template <int D, int G, bool DBG>
__device__ __forceinline__ void softmax_pv(const DecodeArgs &A, float lg, int ntok, int64_t logit_base,
                                           uint2 (&vf)[D / 16], float *__restrict__ pb, WaveState &st,
                                           v4f (&acc)[D / 16]) {
    constexpr int NT = D / 16;
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int q4 = lane >> 4, n16 = lane & 15;
    if constexpr (DBG) {
        if (j < G && t < ntok) A.logits[logit_base + (int64_t)j * A.max_pages * kPage + t] = lg * kLn2;
    }
    if (__builtin_amdgcn_ballot_w64(lg > st.m + 8.f) != 0ull) {
        const float pm = head_reduce<G, true>(lg);
        const float mn = fmaxf(st.m, pm);
        const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
        st.l *= alpha;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = __shfl(alpha, i % G);  // lane h carries head h
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            acc[k].x *= sc[0]; acc[k].y *= sc[1]; acc[k].z *= sc[2]; acc[k].w *= sc[3];
        }
        st.m = mn;
    }
    const float pe = __builtin_amdgcn_exp2f(lg - st.m);
    st.l += (j < G) ? pe : 0.f;   // for G < 4 several lanes carry the same head: count it once

    // ---- P (G x 16) to the MFMA A layout, split hi + lo in bf16 ----
    if (j < G) pb[j * 16 + t] = pe;
    v4s af = {0, 0, 0, 0};
    if (n16 < 2 * G) {
        const float4 pv = *reinterpret_cast<const float4 *>(pb + (n16 % G) * 16 + 4 * q4);
        const bool lo = n16 >= G;
        const float pr[4] = {pv.x, pv.y, pv.z, pv.w};
        short sh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t bits = __float_as_uint(pr[i]);
            const float hi = __uint_as_float(bits & 0xFFFF0000u);
            const float x = lo ? (pr[i] - hi) : pr[i];
            sh[i] = (short)(__float_as_uint(x) >> 16);
        }
        af = v4s{sh[0], sh[1], sh[2], sh[3]};
    }
    if (ntok < kPage) {
        // zero the values of tokens past the end (the page tail may hold anything)
        const int base = 4 * q4;
        const uint32_t m0 = (base + 0 < ntok ? 0x0000FFFFu : 0u) | (base + 1 < ntok ? 0xFFFF0000u : 0u);
        const uint32_t m1 = (base + 2 < ntok ? 0x0000FFFFu : 0u) | (base + 3 < ntok ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int k = 0; k < NT; ++k) { vf[k].x &= m0; vf[k].y &= m1; }
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        v4s bfr;
        __builtin_memcpy(&bfr, &vf[k], 8);
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, bfr, acc[k], 0, 0, 0);
    }
}


// The lane's share of f_b on its slice of a page of tier B: the running
// sine product P over the slice's angles and, per head h, the sum F[h] of
// u_q,h[a] * (product of the slice's sines before a) * cos of angle a.
template <int D, int G, int B, bool QF>
__device__ __forceinline__ void slice_fb(const PageBuf<D> &r, const uint32_t (&u)[query_words<D, G, QF>()],
                                         const float2 *__restrict__ lut, float (&F)[G], float &P) {
    constexpr int NA = D / 4;
    const int j = threadIdx.x & 3;
    const uint32_t az_base = 8u * ((j == 3) ? lut_azimuth(B) : lut_polar(B));
    const uint32_t pad_base = 8u * ((j == 3) ? kLutOnes : lut_polar(B));
    const char *lutb = reinterpret_cast<const char *>(lut);
    // binary32 words of four heads at d = 128 fill the register file: no spread words there
    CodeAddr<B, !(QF && G * D >= 512)> ca;
    ca.init(r.cw);
#pragma unroll
    for (int h = 0; h < G; ++h) F[h] = 0.f;
    P = 1.f;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const uint32_t c8 = ca.at(r.cw, i);
        uint32_t e8;
        if (i == NA - 2) e8 = az_base + c8;
        else if (i == NA - 1) e8 = pad_base + c8;
        else e8 = 8u * lut_polar(B) + c8;
        const float2 cs = *reinterpret_cast<const float2 *>(lutb + e8);
        const float w = P * cs.x;
        P = P * cs.y;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int e2 = i * G + h;   // element (angle i, head h) of the packed halves
            F[h] = query_fma<D, G, QF>(u, e2, w, F[h]);
        }
    }
}

// The header-dispatched kernel with the binary32 direction at G = 4,
// d = 128: its registers cannot hold the 128 query words besides everything
// else (the compiler spilled inside the page loop and the kernel ran at half
// speed), so the slice loop reads each angle's four heads from the
// workgroup's LDS copy (one 16-byte read per angle; uqs = the lane's slice
// of the tier's block, [angle][head]) instead.
template <int D, int B>
__device__ __forceinline__ void slice_fb_lds(const PageBuf<D> &r, const float *__restrict__ uqs,
                                             const float2 *__restrict__ lut, float (&F)[4], float &P) {
    constexpr int NA = D / 4;
    const int j = threadIdx.x & 3;
    const uint32_t az_base = 8u * ((j == 3) ? lut_azimuth(B) : lut_polar(B));
    const uint32_t pad_base = 8u * ((j == 3) ? kLutOnes : lut_polar(B));
    const char *lutb = reinterpret_cast<const char *>(lut);
    CodeAddr<B, false> ca;
    ca.init(r.cw);
#pragma unroll
    for (int h = 0; h < 4; ++h) F[h] = 0.f;
    P = 1.f;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const uint32_t c8 = ca.at(r.cw, i);
        uint32_t e8;
        if (i == NA - 2) e8 = az_base + c8;
        else if (i == NA - 1) e8 = pad_base + c8;
        else e8 = 8u * lut_polar(B) + c8;
        const float2 cs = *reinterpret_cast<const float2 *>(lutb + e8);
        const float4 uv = *reinterpret_cast<const float4 *>(uqs + 4 * i);
        const float w = P * cs.x;
        P = P * cs.y;
        F[0] = __builtin_fmaf(uv.x, w, F[0]);
        F[1] = __builtin_fmaf(uv.y, w, F[1]);
        F[2] = __builtin_fmaf(uv.z, w, F[2]);
        F[3] = __builtin_fmaf(uv.w, w, F[3]);
    }
}
// (whether a kernel takes that path)
template <int D, int G, int TB, bool QF>
constexpr bool query_in_lds() { return TB == 0 && QF && G == 4 && D == 128; }

// The rest of a coded page, the same for every tier: the four slices joined
// into f_b, the logits, online softmax and the MFMA P.V update.  DBG also
// stores the logits (a separate kernel variant, so that the store does not
// enter the memory-wait accounting of the production loop).
template <int D, int G, bool DBG>
__device__ __forceinline__ void finish_page(const DecodeArgs &A, PageBuf<D> &r, int ntok, int64_t logit_base,
                                            const float (&F)[G], float P, float sq, const float *__restrict__ rlev,
                                            float *__restrict__ pb, WaveState &st, v4f (&acc)[D / 16]) {
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;

    // ---- join the four slices: C_j = prod_{i<j} S_i ----
    const float C = slice_prefix(P, j);
    float f;
    if constexpr (G == 4) {
        const float X0 = C * F[0], X1 = C * F[1], X2 = C * F[2], X3 = C * F[3];
        const bool odd = j & 1;
        const float s0 = odd ? X0 : X1, k0 = odd ? X1 : X0;
        const float s1 = odd ? X2 : X3, k1 = odd ? X3 : X2;
        const float Y0 = k0 + qperm<kQuadXor1>(s0);
        const float Y1 = k1 + qperm<kQuadXor1>(s1);
        const bool hi2 = j & 2;
        const float s2 = hi2 ? Y0 : Y1, k2 = hi2 ? Y1 : Y0;
        f = k2 + qperm<kQuadXor2>(s2);
    } else if constexpr (G == 2) {
        const float X0 = C * F[0], X1 = C * F[1];
        const bool odd = j & 1;
        const float s0 = odd ? X0 : X1, k0 = odd ? X1 : X0;
        const float Y = k0 + qperm<kQuadXor1>(s0);
        f = Y + qperm<kQuadXor2>(Y);
    } else {
        const float X = C * F[0];
        const float Y = X + qperm<kQuadXor1>(X);
        f = Y + qperm<kQuadXor2>(Y);
    }

    // ---- logits (log2 units), online softmax and P.V ----
    const float lg = (t < ntok) ? sq * rlev[r.rc] * f : -INFINITY;
    softmax_pv<D, G, DBG>(A, lg, ntok, logit_base, r.vf, pb, st, acc);
}

// Dense keys: the page's logits S = Q.K^T on MFMA (query rows, the G heads
// padded to 16, as the A operand, split exactly into bf16 hi + lo halves:
// qd[4k], qd[4k+1] hold the hi pairs of dimensions 16k + 4(l/16) .. +3 of
// head l%16, qd[4k+2], qd[4k+3] the lo pairs), then the same softmax and
// P.V as the coded kernels.
template <int D, int G, bool DBG>
__device__ __forceinline__ void compute_page_dense(const DecodeArgs &A, PageBuf<D> &r, int ntok, int64_t logit_base,
                                                   const uint32_t (&qd)[D / 4], float sq, float *__restrict__ pb,
                                                   WaveState &st, v4f (&acc)[D / 16]) {
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    v4f s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        v4s bk, ah, al;
        __builtin_memcpy(&bk, &r.kf[k], 8);
        __builtin_memcpy(&ah, &qd[4 * k], 8);
        __builtin_memcpy(&al, &qd[4 * k + 2], 8);
        s4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bk, s4, 0, 0, 0);
        s4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bk, s4, 0, 0, 0);
    }
    // S[h][token n] sits in lane n (h < 4), element h; lane 4t + j takes head
    // j % G of token t
    const int src = t * 4;
    const float e0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(s4.x)));
    const float e1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(s4.y)));
    const float e2 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(s4.z)));
    const float e3 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(s4.w)));
    const int hj = j % G;
    const float f = hj == 0 ? e0 : hj == 1 ? e1 : hj == 2 ? e2 : e3;
    const float lg = (t < ntok) ? sq * f : -INFINITY;
    softmax_pv<D, G, DBG>(A, lg, ntok, logit_base, r.vf, pb, st, acc);
}

template <int D, int G, int TB, bool DBG, bool QF>
__device__ __forceinline__ void compute_page(const DecodeArgs &A, const PageDesc &pd, PageBuf<D> &r, int len,
                                             int64_t head0, const uint32_t (&u)[query_words<D, G, QF>()],
                                             const uint32_t (&qd)[D / 4], float sq,
                                             const float2 *__restrict__ lut, const float *__restrict__ rlev,
                                             float *__restrict__ pb, WaveState &st, v4f (&acc)[D / 16],
                                             const float *__restrict__ uq_all = nullptr) {
    // tokens of the page: its first slots, up to the row's length and (coded
    // pools) the header's count (the high four bits count empty slots)
    int ntok = min(kPage, len - pd.p * kPage);
    const int64_t lbase = head0 * A.max_pages * kPage + (int64_t)pd.p * kPage;
    if constexpr (TB == kDenseTB) {
        compute_page_dense<D, G, DBG>(A, r, ntok, lbase, qd, sq, pb, st, acc);
    } else if constexpr (TB != 0) {
        // a page whose header disagrees with the kernel's tier is flagged and skipped
        const uint32_t hb = __builtin_amdgcn_readfirstlane(r.hb);
        if ((hb & 15u) != (uint32_t)TB) {
            if ((threadIdx.x & 63) == 0) atomicOr(A.err, 4u);
            return;
        }
        ntok = min(ntok, kPage - (int)(hb >> 4));
        float F[G], P;
        slice_fb<D, G, TB, QF>(r, u, lut, F, P);
        finish_page<D, G, DBG>(A, r, ntok, lbase, F, P, sq, rlev, pb, st, acc);
    } else {
        // only the slice part depends on the tier: the join, the softmax and
        // the P.V product exist once, after the dispatch
        ntok = min(ntok, pd.cnt);
        float F[G], P;
        if constexpr (query_in_lds<D, G, TB, QF>()) {
            // the tier's block of the LDS copy: slot among the tiers present, the lane's slice
            const int slot = __builtin_popcount(A.tier_mask & ((1u << pd.b) - 1u));
            const float *uqs = uq_all + ((slot * 4 + (int)(threadIdx.x & 3)) * (D / 4)) * G;
            switch (pd.b) {
                case 2: slice_fb_lds<D, 2>(r, uqs, lut, F, P); break;
                case 3: slice_fb_lds<D, 3>(r, uqs, lut, F, P); break;
                case 4: slice_fb_lds<D, 4>(r, uqs, lut, F, P); break;
                case 6: slice_fb_lds<D, 6>(r, uqs, lut, F, P); break;
                default: slice_fb_lds<D, 8>(r, uqs, lut, F, P); break;
            }
        } else {
            switch (pd.b) {
                case 2: slice_fb<D, G, 2, QF>(r, u, lut, F, P); break;
                case 3: slice_fb<D, G, 3, QF>(r, u, lut, F, P); break;
                case 4: slice_fb<D, G, 4, QF>(r, u, lut, F, P); break;
                case 6: slice_fb<D, G, 6, QF>(r, u, lut, F, P); break;
                default: slice_fb<D, G, 8, QF>(r, u, lut, F, P); break;
            }
        }
        finish_page<D, G, DBG>(A, r, ntok, lbase, F, P, sq, rlev, pb, st, acc);
    }
}

// The lane's packed query halves for one tier, from global memory (single
// tier, once per workgroup) or from the workgroup's LDS copy (mixed tiers).
template <int D, int G, bool QF>
__device__ __forceinline__ void load_query(const uint4 *src, uint32_t (&u)[query_words<D, G, QF>()]) {
    constexpr int NW = query_words<D, G, QF>();
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
        const uint4 x = src[i];
        u[4 * i + 0] = x.x; u[4 * i + 1] = x.y; u[4 * i + 2] = x.z; u[4 * i + 3] = x.w;
    }
}

// The decode step with append: the wave whose page run holds position
// len - 1 (the new token) first stores the token there for its KV head --
// angle codes at the page's tier, record, radius code, values, exactly as
// the encoder writes them (the write path of section 2.3 of the page) -- and
// only then reads that page, so the decode sees it like any stored token.
// The suffix sums of squares run in one lane from the last component
// backwards (the defining order); the lanes then decide the codes against
// the edge tables already in LDS, pack the record's 32-bit words and store
// the values.  Nothing else in the call reads this (page, KV head), so a
// workgroup-scope fence orders the stores before the wave's own page loads.
// S: D doubles of LDS scratch, cl: D bytes of LDS scratch (this wave's).
template <int D, int TB>
__device__ __forceinline__ void append_token(const DecodeArgs &A, int seq, int kvh, int len_in, int ph,
                                             const float *xk, const double *tau2, const double *c2s,
                                             const double *s2s, double *S, uint8_t *cl) {
    const int lane = threadIdx.x & 63;
    constexpr int PL = D / 64;
    if (len_in > A.max_pages * kPage) {   // past the block-table row: nothing stored
        if (lane == 0) atomicOr(A.err, 1u);
        return;
    }
    if (ph < 0 || (int64_t)ph >= A.num_pages) {
        if (lane == 0) atomicOr(A.err, 1u);
        return;
    }
    const int pos = len_in - 1, s = pos % kPage;
    // (the header is read now and checked before the stores; with a single
    // tier the codes need not wait for it)
    const int64_t hix = A.head_tiers ? (int64_t)ph * A.hkv + kvh : (int64_t)ph;
    const int hb = A.page_bits[hix] & 15;   // (the tier bits of the header)
    const int b = TB != 0 ? TB : hb;
    if (TB == 0 && !(b >= 2 && b <= 8 && ((A.tier_mask >> b) & 1u))) {
        if (lane == 0) atomicOr(A.err, 4u);
        return;
    }
    const uint64_t off = (TB == 0 && A.page_off) ? A.page_off[hix] : (uint64_t)ph * (uint64_t)A.page_stride;
    if (lane == 0) {
        double T = add_square(0.0, xk[D - 1]);
        T = add_square(T, xk[D - 2]);
#pragma unroll
        for (int a = D - 3; a >= 0; --a) {
            S[a] = T;
            T = add_square(T, xk[a]);
        }
        S[D - 1] = T;   // |k|^2 (S[D-1] itself is not a suffix sum any code uses)
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int r = 0; r < PL; ++r) {
        const int a = lane * PL + r;
        if (a < D - 2) cl[a] = (uint8_t)polar_code((double)xk[a], S[a], b, c2s + thr_off(b), s2s + thr_off(b));
        else if (a == D - 2)
            cl[a] = (uint8_t)azimuth_code((double)xk[D - 2], (double)xk[D - 1], b, c2s + thr_off(b - 1),
                                          s2s + thr_off(b - 1));
    }
    const double Tall = S[D - 1];
    // radius code = #{j : |k|^2 >= tau2[j]} (tau2 increases with j)
    int rc = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int j = lane + 64 * k;
        rc += __popcll(__builtin_amdgcn_ballot_w64(j < 255 && Tall >= tau2[min(j, 254)]));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (TB != 0 && hb != TB) {
        if (lane == 0) atomicOr(A.err, 4u);
        return;
    }
    // the record: slice sl holds the codes of angles [sl*na, min((sl+1)*na,
    // D-1)) as one bit string, b bits each, least significant first; word wi
    // of a slice is bits [32 wi, 32 wi + 32) of that string
    const int kb = record_bytes(D, b), wps = kb / 16;
    constexpr int na = D / 4;
    uint32_t *rec = reinterpret_cast<uint32_t *>(
        const_cast<uint8_t *>(A.kcode) + off + (A.head_tiers ? (uint64_t)s * kb : ((uint64_t)kvh * kPage + s) * kb));
    for (int wq = lane; wq < 4 * wps; wq += 64) {
        const int sl = wq / wps, bit0 = 32 * (wq % wps);
        const int a0 = sl * na, a1 = min((sl + 1) * na, D - 1);
        uint32_t word = 0;
        for (int k = bit0 / b; a0 + k < a1 && k * b < bit0 + 32; ++k) {
            const int sh = k * b - bit0;
            const uint32_t c = cl[a0 + k];
            word |= sh >= 0 ? (c << sh) : (c >> -sh);
        }
        rec[wq] = word;
    }
    if (lane == 0) const_cast<uint8_t *>(A.rcode)[((int64_t)ph * A.hkv + kvh) * kPage + s] = (uint8_t)rc;
    const uint16_t *vs = A.app_v + ((int64_t)seq * A.hkv + kvh) * D;
    uint16_t *vd = const_cast<uint16_t *>(A.v) + ((int64_t)ph * A.hkv + kvh) * (int64_t)D * kPage + s;
    for (int e = lane; e < D; e += 64) vd[(int64_t)e * kPage] = vs[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// TB: the angle bit width of every page when the pool has a single tier, or 0
// (pages of mixed tiers, dispatched per page on the header).  APP: the decode
// step with append (append_token).
// The split layout of a sequence's pages: split j starts at page
// split_start(j).  With b = pps and m = split_m the sizes are b, b, 2b, 4b,
// ..., b 2^m, then b 2^m each; m = 0 gives splits of b pages throughout.
__device__ __forceinline__ int split_start(const DecodeArgs &A, int j) {
    const int m = A.split_m;
    if (j <= m + 1) return j == 0 ? 0 : A.pps << (j - 1);
    return (j - m) * (A.pps << m);
}
// number of splits that hold pages of a sequence of n pages
__device__ __forceinline__ int splits_of(const DecodeArgs &A, int n) {
    if (n <= 0) return 0;
    const int m = A.split_m, cap = A.pps << m;
    if (n > cap) return m + (n + cap - 1) / cap;
    int k = 1;
    while (k <= m + 1 && (A.pps << (k - 1)) < n) ++k;
    return k;
}

template <int D, int G, int TB, bool DBG, bool APP, bool QF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void k_decode(DecodeArgs A) {
    constexpr int NA = D / 4;
    constexpr int NT = D / 16;
    // The split is the slowest grid dimension, taken in reverse: the
    // dispatcher hands out the last split of every group first, so in a
    // batch of one round the longest sequences start first.  In a batch of
    // several rounds the splits grow with their index (split_start) and the
    // grid is compacted, so the largest units go first and the smallest
    // fill the last round.
    const int kvh = blockIdx.x;
    int seq = blockIdx.y, split = (int)gridDim.z - 1 - (int)blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    int len_known = 0;
    if (A.compact) {
        // Compacted grid: this workgroup's unit, in decreasing size (written
        // by k_unit_order), and its sequence's length.  A sequence with no
        // page still has one unit (it writes its zero rows).
        const int2 ent = A.unit_table[blockIdx.z * gridDim.y + blockIdx.y];
        if (ent.x < 0) return;   // a slot past the last unit
        seq = ent.x >> 16;
        split = ent.x & 0xFFFF;
        len_known = ent.y;
    }
    seq = __builtin_amdgcn_readfirstlane(seq);
    split = __builtin_amdgcn_readfirstlane(split);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps per-wave values scalar
    const int q4 = lane >> 4, n16 = lane & 15;
    const int64_t head0 = (int64_t)seq * A.hq + (int64_t)kvh * G;
    // The prologue is a short dependent chain; at raised priority it is not
    // starved by the page loops of the other workgroup sharing the CU.
    __builtin_amdgcn_s_setprio(2);

    __shared__ float2 lut[kLutEntries];
    __shared__ float rlev[256];
    __shared__ __attribute__((aligned(16))) float pbuf[kWaves][G * 16];
    __shared__ float mo[kWaves][2 * G][D];
    __shared__ float mml[kWaves][G][2];
    // query preparation: the G query rows, their suffix sums, the edge tables
    // of the tiers present, and the resulting packed unit directions
    __shared__ float qs[G][D];
    __shared__ double qT[kWaves][D];
    __shared__ double c2s[kThrEntries], s2s[kThrEntries];
    typedef std::conditional_t<QF, float, _Float16> query_t;
    __shared__ __attribute__((aligned(16))) query_t uq_lds[(TB == 0 ? 5 : 1) * D * G];
    __shared__ float sq_lds[G];
    // append: the new token's key for this KV head and the head's radius edges
    __shared__ float akey[APP ? D : 1];
    __shared__ double atau2[APP ? 256 : 1];

    // ---- prologue.  Every global read it needs is issued at once: the
    // sequence length, the block-table entries of this wave's run (taken as
    // if the split were full, which it is except for the last split of a
    // sequence) and the tables; then the loads of the waves' first pages go
    // out around the query preparation (see there), which runs under their
    // latency. ----
    const int64_t bt_row = (int64_t)seq * A.max_pages;
    // block-table entries of a chunk: one clamped, unconditional load per lane
    auto bt_raw = [&](int c0) { return A.block_table[bt_row + min(c0 + lane, A.max_pages - 1)]; };
    // this wave's run of a split of n pages: the first wave on each SIMD
    // (waves 0..kWaves/2-1) takes first_wave_pages(n) of them, the second
    // waves share the rest
    constexpr int kHalf = kWaves / 2;
    auto wave_run = [&](int n, int &wofs, int &wcnt) {   // (selects, no branch)
        const int fpw = first_wave_pages(n);
        const int rest = n - kHalf * fpw;
        const int per = (rest + kHalf - 1) / kHalf;
        const bool first = wave < kHalf;
        wofs = first ? wave * fpw : kHalf * fpw + (wave - kHalf) * per;
        wcnt = first ? fpw : max(0, min(per, rest - (wave - kHalf) * per));
    };
    const int p0 = split_start(A, split);
    const int psz = split_start(A, split + 1) - p0;
    int wofs, wcnt;
    wave_run(psz, wofs, wcnt);
    int ph_raw = bt_raw(p0 + wofs);
    int ph1_raw = TB != 0 ? bt_raw(p0 + wofs + 64) : 0;
    static_assert(kBufs >= 2, "at least one page in flight");
    // Tables and query rows to LDS: all loads first (clamped indices, no
    // branches), then the stores, so the staging costs one memory round trip.
    constexpr int kNL = (kLutEntries + kThreads - 1) / kThreads;
    constexpr int kNT = (kThrEntries + kThreads - 1) / kThreads;
    constexpr int kNQ = (G * D + kThreads - 1) / kThreads;
    float2 st_lut[kNL];
    double st_c2[kNT], st_s2[kNT];
    float st_q[kNQ];
#pragma unroll
    for (int i = 0; i < kNL; ++i) st_lut[i] = A.lut[min(tid + i * kThreads, kLutEntries - 1)];
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
        const int e = min(tid + i * kThreads, kThrEntries - 1);
        st_c2[i] = A.cos2[e];
        st_s2[i] = A.sin2[e];
    }
#pragma unroll
    for (int i = 0; i < kNQ; ++i) st_q[i] = A.q[head0 * D + min(tid + i * kThreads, G * D - 1)];
    const float st_r = A.rlev[kvh * 256 + (tid & 255)];
    float st_k = 0.f;
    double st_t = 0.0;
    if constexpr (APP) {
        st_k = A.app_k[((int64_t)seq * A.hkv + kvh) * D + min(tid, D - 1)];
        st_t = A.tau2[255 * kvh + min(tid, 254)];
    }
    int len = A.compact ? len_known : A.seq_lens[seq];
    __builtin_amdgcn_sched_barrier(0);   // (every load above is issued before the wait for len)

    const int len_in = len;   // (append: a length past the row is an error, not clamped)
    len = max(0, min(len, A.max_pages * kPage));
    const int npages = (len + kPage - 1) / kPage;
    if (p0 >= npages) {   // whole workgroup, before any barrier
        // the loads above are consumed here too, so that they stay ahead of
        // this branch (issued with the length load, not after it)
        auto keep = [](auto x) { asm volatile("" ::"v"(x)); };
        keep(ph_raw);
        keep(ph1_raw);
#pragma unroll
        for (int i = 0; i < kNL; ++i) keep(st_lut[i]);
#pragma unroll
        for (int i = 0; i < kNT; ++i) {
            keep(st_c2[i]);
            keep(st_s2[i]);
        }
#pragma unroll
        for (int i = 0; i < kNQ; ++i) keep(st_q[i]);
        keep(st_r);
        if constexpr (APP) {
            keep(st_k);
            keep(st_t);
        }
        // a sequence with no resident token: its output rows are 0
        if (npages == 0 && split == 0)
            for (int e = threadIdx.x; e < G * D; e += kThreads) A.out[head0 * D + e] = 0.f;
        return;
    }
    const int p1 = min(p0 + psz, npages);
    if (p1 - p0 != psz) {   // the last split of its sequence: the wave's run moves
        wave_run(p1 - p0, wofs, wcnt);
        ph_raw = bt_raw(p0 + wofs);
        if constexpr (TB != 0) ph1_raw = bt_raw(p0 + wofs + 64);
    }
    const int wp0 = min(p0 + wofs, p1);
    const int wp1 = min(wp0 + wcnt, p1);
    const int ph_first = (wp0 + lane < wp1) ? ph_raw : -1;
    // (the stores use the same clamped indices: a thread past the end writes
    // the last element's own value again, so every load is consumed on every
    // path and the compiler's wait counts stay exact)
#pragma unroll
    for (int i = 0; i < kNL; ++i) lut[min(tid + i * kThreads, kLutEntries - 1)] = st_lut[i];
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
        const int e = min(tid + i * kThreads, kThrEntries - 1);
        c2s[e] = st_c2[i];
        s2s[e] = st_s2[i];
    }
#pragma unroll
    for (int i = 0; i < kNQ; ++i) {
        const int e = min(tid + i * kThreads, G * D - 1);
        qs[e / D][e % D] = st_q[i];
    }
    rlev[tid & 255] = st_r;
    if constexpr (APP) {
        akey[min(tid, D - 1)] = st_k;
        atau2[min(tid, 255)] = st_t;
    }

    // The wave's page list, 64 pages at a time, one page per lane: valid
    // pages first (ordered by tier when tiers are mixed, so that the query
    // registers change at most once per tier).  With a single tier the
    // addresses follow from the block table alone; each page header is then
    // read with the page's data and checked before the page is used.
    int e_pg = 0, e_phys = -1, e_bits = 0, nvalid = 0;
    uint32_t e_lo = 0, e_hi = 0;
    // (mixed tiers) the header and the record offset of the lane's page (of
    // this KV head's records with per-head tiers), read at a clamped (valid)
    // id; the page list checks them
    auto page_meta = [&](int c0, int ph, int &hdr, uint64_t &off) {
        const bool ok = lane < min(64, wp1 - c0) && ph >= 0 && (int64_t)ph < A.num_pages;
        const int phc = ok ? ph : 0;
        const int64_t hix = A.head_tiers ? (int64_t)phc * A.hkv + kvh : (int64_t)phc;
        hdr = (int)A.page_bits[hix];
        off = A.page_off ? A.page_off[hix] : (uint64_t)phc * (uint64_t)A.page_stride;
    };
    auto page_list = [&](int c0, int ph, int hdr, uint64_t off) {
        const int cn = min(64, wp1 - c0);
        e_pg = c0 + lane;
        e_phys = -1;
        e_bits = 0;
        e_lo = e_hi = 0;
        int key = 15;
        const bool inr = lane < cn;
        const bool ok = inr && ph >= 0 && (int64_t)ph < A.num_pages;
        if (inr && !ok) atomicOr(A.err, 2u);
        if constexpr (TB != 0) {
            e_phys = ok ? ph : -1;
            key = ok ? TB : 15;
        } else {
            const int bb = hdr & 15;   // tier bits; the high four count empty slots
            const bool okb = ok && bb >= 2 && bb <= 8 && ((A.tier_mask >> bb) & 1u);
            if (ok && !okb) atomicOr(A.err, 4u);
            e_phys = okb ? ph : -1;
            e_bits = okb ? hdr : 0;
            key = okb ? bb : 15;
            e_lo = okb ? (uint32_t)off : 0u;
            e_hi = okb ? (uint32_t)(off >> 32) : 0u;
        }
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int rank = 0;
        nvalid = 0;
        constexpr int kKeys[6] = {2, 3, 4, 6, 8, 15};
#pragma unroll
        for (int vi = 0; vi < 6; ++vi) {
            const int v = kKeys[vi];
            if (TB != 0 && v != TB && v != 15) continue;
            const uint64_t bal = __builtin_amdgcn_ballot_w64(key == v);
            if (v < key) rank += __popcll(bal);
            else if (v == key) rank += __popcll(bal & lt);
            if (v != 15) nvalid += __popcll(bal);
        }
        e_pg = __builtin_amdgcn_ds_permute(rank * 4, e_pg);
        e_phys = __builtin_amdgcn_ds_permute(rank * 4, e_phys);
        if constexpr (TB == 0) {
            e_bits = __builtin_amdgcn_ds_permute(rank * 4, e_bits);
            e_lo = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)e_lo);
            e_hi = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)e_hi);
        }
    };
    auto desc = [&](int k) {
        PageDesc pd;
        pd.phys = __builtin_amdgcn_readlane(e_phys, k);
        const int hdr = TB != 0 ? TB : __builtin_amdgcn_readlane(e_bits, k);
        pd.b = hdr & 15;
        pd.cnt = kPage - (hdr >> 4);
        pd.p = __builtin_amdgcn_readlane(e_pg, k);
        pd.live = true;
        if constexpr (TB != 0) {
            pd.off = (uint64_t)(uint32_t)pd.phys * (uint64_t)A.page_stride;
        } else {
            pd.off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)e_hi, k) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane((int)e_lo, k);
        }
        return pd;
    };
    // kBufs register sets: the loads of pages k+1 .. k+kBufs-1 are in flight
    // while page k is computed.  Loads are issued unconditionally (past the
    // end through empty descriptors that read nothing) so that the wait
    // before each compute only covers the loads of the page being computed.
    PageBuf<D> R[kBufs];
    PageDesc dd[kBufs];
    auto issue_chunk = [&]() {
        // issued even when the chunk has no valid page (then through empty
        // descriptors that read nothing), so every path issues the same loads
#pragma unroll
        for (int i = 0; i < kBufs; ++i) {
            dd[i] = desc(max(0, min(i, nvalid - 1)));
            dd[i].live = i < nvalid;
            load_page<D, TB>(A, dd[i], kvh, R[i]);
        }
    };
    // (pools of mixed tiers request the first chunk's headers and offsets
    // before the query preparation, and list and request its pages after
    // it: two page buffers held across the preparation would spill)
    int m_hdr = 0;
    uint64_t m_off = 0;
    // Single tier: the wave walks its pages in order, reading the block
    // table 64 entries (one per lane) at a time into two rotating register
    // slots, the next slot always requested a chunk ahead; the page loads
    // run kBufs pages ahead of the computation without a break at chunk
    // boundaries.  Pages whose id is out of range are flagged and skipped.
    const int nw = wp1 - wp0;
    int e_ph0 = ph_first, e_ph1 = 0;
    // descriptor of page k of the run, its id read from slot S (the caller
    // knows which slot holds k's chunk; reading only that slot keeps the
    // other one free to be refilled while its loads are in flight)
    auto rdesc = [&](int k, auto slot) {
        constexpr int S = decltype(slot)::value;
        PageDesc pd;
        const int kc = max(0, min(k, nw - 1));
        const int ph = __builtin_amdgcn_readlane(S ? e_ph1 : e_ph0, kc & 63);
        const bool ok = ph >= 0 && (int64_t)ph < A.num_pages;
        pd.live = ok && k < nw;
        pd.phys = ok ? ph : 0;
        pd.b = TB != 0 ? TB : 8;
        pd.cnt = kPage;   // (single tier: the count comes with the page's header)
        pd.p = wp0 + kc;
        pd.off = (uint64_t)(uint32_t)pd.phys * (uint64_t)A.page_stride;
        if (!ok && k < nw && lane == 0) atomicOr(A.err, 2u);
        return pd;
    };
    if constexpr (TB != 0) {
        e_ph1 = ph1_raw;
#pragma unroll
        for (int i = 0; i < kBufs; ++i) dd[i] = rdesc(i, std::integral_constant<int, 0>{});
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    if constexpr (TB == 0) page_meta(wp0, ph_first, m_hdr, m_off);

    // The loads of the wave's first pages.  At the start of the kernel every
    // wave of the chip requests its first pages at once, and a wave's requests
    // wait for room in the memory queue (about 2 us here).  The waves that
    // prepare a query row therefore request theirs after the preparation,
    // which then runs while the other waves' loads wait and stream.  (With
    // mixed tiers every wave's first chunk is listed and requested in the
    // page loop, after the preparation.)
    // (mixed tiers: the kWaves/G waves of a head share its tiers, each taking
    // every (kWaves/G)-th tier present; a wave left without one loads early)
    constexpr int kWpH = kWaves / G;   // waves per head
    static_assert(kWaves % G == 0, "heads divide the waves");
    const int ntiers = TB != 0 ? 1 : __builtin_popcount(A.tier_mask & 0x1FCu);
    const bool prep_wave = TB != kDenseTB && (TB == 0 ? wave / G < ntiers : wave < G);
    auto first_loads = [&]() {
        if constexpr (TB != 0) {
#pragma unroll
            for (int i = 0; i < kBufs; ++i) load_page<D, TB>(A, dd[i], kvh, R[i]);
        }
    };

    bool loaded = false;
    if constexpr (APP) {
        // the wave whose run holds the new token's page stores the token; a
        // wave that prepares no query requests its first pages first, so
        // that they are in flight during the store, and requests them again
        // after it if the new page is among them
        const int pnew = (len - 1) / kPage;
        if (pnew >= wp0 && pnew < wp1) {
            if (!prep_wave) {
                first_loads();
                loaded = true;
            }
            // the page's id: among this wave's staged block-table entries
            // (one per lane from p0 + wofs) when it is within the first 64
            const int rel = pnew - (p0 + wofs);
            const int ph_new = rel < 64 ? __builtin_amdgcn_readlane(ph_raw, rel) : A.block_table[bt_row + pnew];
            append_token<D, TB>(A, seq, kvh, len_in, ph_new, akey, atau2, c2s, s2s, qT[wave],
                                reinterpret_cast<uint8_t *>(mo[wave][0]));
            if (loaded && pnew - wp0 < kBufs) first_loads();
        }
    }

    // Query prep, section 2.1's c_q: per tier, the angle codes of each query
    // row and the decoded direction u_a = (prod_{k<a} sin c_k) * cos c_a
    // (D/64 components per lane): with a single tier one wave per head
    // (waves 0..G-1), with mixed tiers the head's waves share its tiers.  The
    // suffix sums of squares the codes compare against are taken by a wave
    // scan (fast, but in another order than the keys' backward sum); a code
    // is accepted only when its decisions hold with a margin covering that
    // reordering.  Any decision inside the margin sends the wave to the exact
    // backward sum and the plain search, so the codes always equal the
    // defining ones.  The bins of every tier are uniform and nest: each edge
    // j*pi/2^b is the edge (j*2^(m-b))*pi/2^m of the widest tier m, with the
    // same binary64 table values, so a code at b is the code at m shifted
    // right by m - b (the azimuth's half-plane offset shifts with it).  The
    // codes are decided once, at the widest tier present.
    if (prep_wave) {
        const int h = wave % G, part = wave / G;
        constexpr int PL = D / 64;   // components per lane: a = lane * PL + r
        float xr[PL];
#pragma unroll
        for (int r = 0; r < PL; ++r) xr[r] = qs[h][lane * PL + r];
        double loc = 0.0;
#pragma unroll
        for (int r = PL - 1; r >= 0; --r) loc = add_square(loc, xr[r]);
        const double above = wave_suffix_sum_excl(loc);
        double Sr[PL];   // S of component a = sum of x_k^2 over k > a
        double t = above;
#pragma unroll
        for (int r = PL - 1; r >= 0; --r) {
            Sr[r] = t;
            t = add_square(t, xr[r]);
        }
        const double T0 = readlane_d(t, 0);   // |q|^2
        const double qn = sqrt(T0);
        if (lane == 0 && part == 0) sq_lds[h] = (float)((double)A.scale * qn * 1.4426950408889634);
        const double xa = (double)qs[h][D - 2], ya = (double)qs[h][D - 1];   // the azimuth pair
        const bool hp = (ya < 0.0) || (ya == 0.0 && xa < 0.0);
        const double xpa = hp ? -xa : xa, ypa = hp ? -ya : ya;
        // the exact query direction (query mode 1), the same for every tier
        float ux[PL];
#pragma unroll
        for (int r = 0; r < PL; ++r) ux[r] = 0.f;
        const bool exact_q = A.query_mode == 1;
        if (__builtin_expect(exact_q, 0)) {
#pragma unroll
            for (int r = 0; r < PL; ++r) ux[r] = qn > 0.0 ? (float)((double)xr[r] / qn) : 0.f;
        }
        // the codes at the widest tier present (polar; for the azimuth the
        // code within its half plane)
        const int bm = TB != 0 ? TB : 31 - __builtin_clz(A.tier_mask & 0x1FCu);
        int code_m[PL];
#pragma unroll
        for (int r = 0; r < PL; ++r) code_m[r] = 0;
        if (!exact_q) {
            bool ok = true;
#pragma unroll
            for (int r = 0; r < PL; ++r) {
                const int a = lane * PL + r;
                const bool az = a == D - 2;
                const double x = az ? xpa : (double)xr[r];
                const double S = az ? ypa * ypa : Sr[r];
                const int bb = az ? bm - 1 : bm;
                bool okr;
                code_m[r] = polar_code_window(x, S, bb, c2s + thr_off(bb), s2s + thr_off(bb), polar_guess(x, S, bb),
                                              az ? 0.0 : 5e-14, okr);
                ok = ok && (a >= D - 1 || okr);
            }
            if (__builtin_amdgcn_ballot_w64(!ok) != 0) {
                // rare: the exact backward suffix sums (one lane), then the plain search
                if (lane == 0) {
                    double T = 0.0;
                    for (int a2 = D - 1; a2 >= 0; --a2) {
                        qT[wave][a2] = T;   // sum over k > a2
                        T = add_square(T, qs[h][a2]);
                    }
                }
#pragma unroll
                for (int r = 0; r < PL; ++r) {
                    const int a = lane * PL + r;
                    if (a < D - 2) {
                        const double x = (double)xr[r], S = qT[wave][a];
                        code_m[r] = polar_code_near(x, S, bm, c2s + thr_off(bm), s2s + thr_off(bm), code_m[r]);
                    } else if (a == D - 2) {
                        code_m[r] = polar_code_near(xpa, ypa * ypa, bm - 1, c2s + thr_off(bm - 1), s2s + thr_off(bm - 1),
                                                    code_m[r]);
                    }
                }
            }
        }
        int ti = 0;
        // the tiers present: only the kernel's own when the pool has one
        for (int b = (TB != 0 ? TB : 2); b <= (TB != 0 ? TB : 8); ++b) {
            if (TB == 0 && !((A.tier_mask >> b) & 1u)) continue;
            if (TB == 0 && ti % kWpH != part) {   // another wave of this head takes it
                ++ti;
                continue;
            }
            float uv[PL];
            if (exact_q) {
#pragma unroll
                for (int r = 0; r < PL; ++r) uv[r] = ux[r];
            } else {
                float cs[PL], sn[PL];
#pragma unroll
                for (int r = 0; r < PL; ++r) {
                    const int a = lane * PL + r;
                    const int code = code_m[r] >> (bm - b);
                    cs[r] = 1.f;
                    sn[r] = 1.f;
                    if (a < D - 1) {
                        const int e = (a == D - 2) ? lut_azimuth(b) + (hp ? (1 << (b - 1)) : 0) + code
                                                   : lut_polar(b) + code;
                        const float2 v = lut[e];
                        cs[r] = v.x;
                        sn[r] = v.y;
                    }
                }
                float tot = 1.f;
#pragma unroll
                for (int r = 0; r < PL; ++r) tot *= sn[r];
                // exclusive product scan of the lanes' sine products (DPP:
                // row shifts, then the row broadcasts of lanes 15 and 31)
                float incl = tot;
                incl *= dpp_or_one<0x111, 0xF>(incl);   // row_shr:1
                incl *= dpp_or_one<0x112, 0xF>(incl);   // row_shr:2
                incl *= dpp_or_one<0x114, 0xF>(incl);   // row_shr:4
                incl *= dpp_or_one<0x118, 0xF>(incl);   // row_shr:8
                incl *= dpp_or_one<0x142, 0xA>(incl);   // row_bcast:15
                incl *= dpp_or_one<0x143, 0xC>(incl);   // row_bcast:31
                float P = dpp_or_one<0x138, 0xF>(incl);  // wave_shr:1 (lane 0 gets 1)
#pragma unroll
                for (int r = 0; r < PL; ++r) {
                    uv[r] = P * cs[r];   // the last component has cs = 1: the product of all d-1 sines
                    P *= sn[r];
                }
            }
#pragma unroll
            for (int r = 0; r < PL; ++r) {
                const int a = lane * PL + r;
                const int sl = a / (D / 4), i = a % (D / 4);
                uq_lds[((ti * 4 + sl) * (D / 4) + i) * G + h] = (query_t)uv[r];
            }
            ++ti;
        }
        first_loads();
    } else if (!loaded) {
        first_loads();
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    WaveState st{-INFINITY, 0.f};
    v4f acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t u[query_words<D, G, QF>()];
    uint32_t qd[D / 4];   // dense keys: the query rows as MFMA A operands (bf16 hi, lo)
    int cur_b = -1;
    const int jq = lane & 3;
    const uint32_t *uqw = reinterpret_cast<const uint32_t *>(uq_lds);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) qd[i] = 0u;
    if constexpr (TB == kDenseTB) {
#pragma unroll
        for (int i = 0; i < query_words<D, G, QF>(); ++i) u[i] = 0u;
        // lane l: head l%16 (rows past G stay 0), dimensions 16k + 4(l/16) .. +3
        const int hq_row = lane & 15;
        if (hq_row < G) {
#pragma unroll
            for (int k = 0; k < D / 16; ++k) {
                uint32_t hi2[2], lo2[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    uint32_t hb[2], lb[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const float x = qs[hq_row][16 * k + 4 * (lane >> 4) + 2 * m + e];
                        hb[e] = bf16_rne(x);
                        lb[e] = bf16_rne(x - __uint_as_float(hb[e] << 16));
                    }
                    hi2[m] = hb[0] | (hb[1] << 16);
                    lo2[m] = lb[0] | (lb[1] << 16);
                }
                qd[4 * k + 0] = hi2[0];
                qd[4 * k + 1] = hi2[1];
                qd[4 * k + 2] = lo2[0];
                qd[4 * k + 3] = lo2[1];
            }
        }
        cur_b = TB;
    } else if constexpr (TB != 0) {
        load_query<D, G, QF>(reinterpret_cast<const uint4 *>(uqw + jq * query_words<D, G, QF>()), u);
        cur_b = TB;
    } else {
#pragma unroll
        for (int i = 0; i < query_words<D, G, QF>(); ++i) u[i] = 0u;
    }
    // this lane's head in the softmax: j % G (dense keys: the plain scale)
    const float sq = TB == kDenseTB ? A.scale * 1.4426950408889634f : sq_lds[(lane & 3) % G];
    float *pb = pbuf[wave];

    auto ensure_query = [&](int b) {
        if constexpr (TB == 0) {
            if (b != cur_b) {
                // the tier's slot among the tiers present, in increasing width
                const int slot = __builtin_popcount(A.tier_mask & ((1u << b) - 1u));
                load_query<D, G, QF>(reinterpret_cast<const uint4 *>(uqw + (slot * 4 + jq) * query_words<D, G, QF>()), u);
                cur_b = b;
            }
        }
    };
    if constexpr (TB != 0) {
        static_assert(64 % kBufs == 0, "pipeline depth divides the chunk");
        // Pages [kc, kc + 64) take their ids from slot 0 and [kc + 64, kc + 128)
        // from slot 1.  Within a half, the loads issued while its last kBufs
        // pages are computed belong to the next chunk (the other slot); at
        // that point this half's slot is refilled with the chunk after next.
        auto step = [&](int k, auto cur, auto nxt, bool refill, int refill_c0) {
            constexpr int SC = decltype(cur)::value;
#pragma unroll
            for (int i = 0; i < kBufs; ++i) {
                if (dd[i].live) compute_page<D, G, TB, DBG, QF>(A, dd[i], R[i], len, head0, u, qd, sq, lut, rlev, pb, st, acc);
                if (refill && i == 0) {
                    if (SC == 0) e_ph0 = bt_raw(refill_c0);
                    else e_ph1 = bt_raw(refill_c0);
                }
                dd[i] = rdesc(k + i + kBufs, nxt);
                load_page<D, TB>(A, dd[i], kvh, R[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        for (int kc = 0; kc < nw; kc += 128) {
            // first half: slot 0
            int k = kc;
            for (; k + kBufs < kc + 64 && k < nw; k += kBufs) step(k, S0{}, S0{}, false, 0);
            if (k < nw) step(k, S0{}, S1{}, true, wp0 + kc + 128);
            k = kc + 64;
            if (k >= nw) break;
            // second half: slot 1
            for (; k + kBufs < kc + 128 && k < nw; k += kBufs) step(k, S1{}, S1{}, false, 0);
            if (k < nw) step(k, S1{}, S0{}, true, wp0 + kc + 192);
        }
    }
    int ph_next = -1;   // the next chunk's block-table entries, requested a chunk ahead
    for (int c0 = wp0; TB == 0 && c0 < wp1; c0 += 64) {
        if (c0 != wp0) page_meta(c0, ph_next, m_hdr, m_off);   // (the first chunk's: before the preparation)
        page_list(c0, c0 == wp0 ? ph_first : ph_next, m_hdr, m_off);
        issue_chunk();
        ph_next = bt_raw(c0 + 64);
        ph_next = (c0 + 64 + lane < wp1) ? ph_next : -1;   // (all -1 past the wave's run)
        if (nvalid == 0) continue;
        const int last = nvalid - 1;
        for (int k = 0; k < nvalid; k += kBufs) {
#pragma unroll
            for (int i = 0; i < kBufs; ++i) {
                if (k + i < nvalid) {
                    if constexpr (!query_in_lds<D, G, TB, QF>()) ensure_query(dd[i].b);
                    compute_page<D, G, TB, DBG, QF>(A, dd[i], R[i], len, head0, u, qd, sq, lut, rlev, pb, st, acc,
                                                    reinterpret_cast<const float *>(uq_lds));
                }
                dd[i] = desc(min(k + i + kBufs, last));
                dd[i].live = k + i + kBufs < nvalid;   // (past the chunk: empty descriptors, no reads)
                load_page<D, TB>(A, dd[i], kvh, R[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- merge the eight waves of this workgroup ----
    const float lsum = head_reduce<G, false>(st.l);
    if (lane < G) {
        mml[wave][lane][0] = st.m;
        mml[wave][lane][1] = lsum;
    }
    // rows 0..2G-1 of the accumulators (P hi and lo): lanes of the first
    // 2G/4 lane groups hold them (all four of a group's rows when 2G is a
    // multiple of 4), so one condition covers every store
    if (4 * q4 < 2 * G) {
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const float a4[4] = {acc[k].x, acc[k].y, acc[k].z, acc[k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 4 * q4 + i;
                if ((2 * G) % 4 == 0 || rr < 2 * G) mo[wave][rr][16 * k + n16] = a4[i];
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, e = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mml[w][h][0]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = exp2f(mml[w][h][0] - M);
                L += sc * mml[w][h][1];
                O += sc * (mo[w][h][e] + mo[w][G + h][e]);
            }
        }
        // device-coherent stores (written through to memory): the merging
        // workgroup, on any XCD, reads them with device-coherent loads
        const int64_t pi = (head0 + h) * A.nsplit + split;
        __hip_atomic_store(&A.part_o[pi * D + e], O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (e == 0) {
            __hip_atomic_store(&A.part_ml[2 * pi + 0], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&A.part_ml[2 * pi + 1], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- merge of the splits by the last workgroup of this (sequence, KV
    // head) to finish.  The partials above are device-coherent stores; once
    // every wave has seen its stores complete (vmcnt(0): with device-scope
    // stores that means visible to every XCD), one thread raises the group's
    // counter.  The workgroup that raises it last reads the partials with
    // device-coherent loads, merges them and clears
    // the counter for the next call.  No cache write-back or invalidation is
    // needed, since no plain store or load takes part. ----
    __shared__ int s_last;
    const int ns_g = splits_of(A, npages);   // workgroups that work on this group
    const int group = seq * A.hkv + kvh;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&A.counters[group], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev + 1 == (unsigned)ns_g);
    }
    __syncthreads();
    if (!s_last) return;
    auto ld = [](float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    // Up to kMergeFast splits: one round of loads and no barrier.  A wave's
    // 64 elements belong to one head (D is a multiple of 64): lane i requests
    // split i's (m, l) pair (one 8-byte load) while every lane requests its
    // element's partial of each split; the wave reduces the maxima and the
    // weighted sums across lanes and reads each split's weight from its lane.
    // The merge runs while the rest of the chip still streams pages, so each
    // round trip is long.  The partial loads are unconditional: N, the split
    // count rounded up to a power of two (at least 4), are issued, with
    // indices past the last split clamped to it.  (Fewer in the mixed-tier
    // kernel, whose register file is full.)
    constexpr int kMergeFast = (TB == 0 && QF) ? 8 : 32;   // (the binary32-direction mixed-tier kernel: fewer registers)
    static_assert(D % 64 == 0, "a wave's merge elements share one head");
    auto merge_fast = [&](auto n_c) {
        constexpr int N = decltype(n_c)::value;
        for (int idx = tid; idx < G * D; idx += kThreads) {
            const int h = idx / D, e = idx % D;
            const int64_t row = head0 + h;
            float *po = A.part_o + row * A.nsplit * D + e;
            const uint64_t *pml = reinterpret_cast<const uint64_t *>(A.part_ml + row * A.nsplit * 2);
            const bool has = lane < ns_g;
            const uint64_t mlv = __hip_atomic_load(pml + min(lane, ns_g - 1), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            float pv[N];
#pragma unroll
            for (int i = 0; i < N; ++i) pv[i] = ld(po + (int64_t)min(i, ns_g - 1) * D);
            const float m = has ? __uint_as_float((uint32_t)mlv) : -INFINITY;
            float M = m;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
            const float w = (m != -INFINITY) ? exp2f(m - M) : 0.f;
            float L = has ? w * __uint_as_float((uint32_t)(mlv >> 32)) : 0.f;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
            float O = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) O += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i)) * pv[i];
            A.out[row * D + e] = (M != -INFINITY && L > 0.f) ? O / L : 0.f;
        }
        if (tid == 0) __hip_atomic_store(&A.counters[group], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (ns_g <= 4) return merge_fast(std::integral_constant<int, 4>{});
    if (ns_g <= 8) return merge_fast(std::integral_constant<int, 8>{});
    if (kMergeFast >= 16 && ns_g <= 16) return merge_fast(std::integral_constant<int, (kMergeFast >= 16 ? 16 : 8)>{});
    if (kMergeFast >= 32 && ns_g <= 32) return merge_fast(std::integral_constant<int, (kMergeFast >= 32 ? 32 : 8)>{});
    constexpr int kMergeMax = 256;   // splits whose weights one LDS pass holds
    if (ns_g <= kMergeMax) {
        // Each split's weight, once per head (one wave per head, in the LDS
        // of the in-workgroup merge, which is done): w_s = 2^(m_s - M) with M
        // the largest partial max, and L = sum_s w_s l_s.  Each output
        // element then needs only its own partials: O = sum_s w_s o_s.
        static_assert(G * kMergeMax + G <= kWaves * 2 * G * D, "merge weights fit the merge LDS");
        float *W = &mo[0][0][0];          // [G][kMergeMax]
        float *Lh = W + G * kMergeMax;    // [G]; 0 for a group without tokens
        if (wave < G) {
            float *ml = A.part_ml + (head0 + wave) * A.nsplit * 2;
            constexpr int kPer = kMergeMax / 64;
            float pm[kPer], pl[kPer];
            float M = -INFINITY;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int sp = lane + 64 * i;
                pm[i] = sp < ns_g ? ld(ml + 2 * sp) : -INFINITY;
                pl[i] = sp < ns_g ? ld(ml + 2 * sp + 1) : 0.f;
                M = fmaxf(M, pm[i]);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
            float L = 0.f;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const float w = (pm[i] != -INFINITY) ? exp2f(pm[i] - M) : 0.f;
                W[wave * kMergeMax + lane + 64 * i] = w;
                L += w * pl[i];
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
            if (lane == 0) Lh[wave] = (M != -INFINITY) ? L : 0.f;
        }
        __syncthreads();
        for (int idx = tid; idx < G * D; idx += kThreads) {
            const int h = idx / D, e = idx % D;
            const int64_t row = head0 + h;
            float *po = A.part_o + row * A.nsplit * D + e;
            constexpr int kMB = 16;   // partials requested at once
            float O = 0.f;
            for (int sp0 = 0; sp0 < ns_g; sp0 += kMB) {
                float pv[kMB];
#pragma unroll
                for (int i = 0; i < kMB; ++i) pv[i] = sp0 + i < ns_g ? ld(po + (int64_t)(sp0 + i) * D) : 0.f;
#pragma unroll
                for (int i = 0; i < kMB; ++i)
                    if (sp0 + i < ns_g) O += W[h * kMergeMax + sp0 + i] * pv[i];
            }
            const float L = Lh[h];
            A.out[row * D + e] = L > 0.f ? O / L : 0.f;
        }
        if (tid == 0) __hip_atomic_store(&A.counters[group], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, e = idx % D;
        const int64_t row = head0 + h;
        float *ml = A.part_ml + row * A.nsplit * 2;
        float *po = A.part_o + row * A.nsplit * D + e;
        // up to kMB splits' partials are requested at once, then folded into
        // the running (M, L, O) in split order
        constexpr int kMB = 16;
        float M = -INFINITY, O = 0.f, L = 0.f;
        for (int sp0 = 0; sp0 < ns_g; sp0 += kMB) {
            float pm[kMB], pl[kMB], pv[kMB];
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
                pm[i] = -INFINITY;
                pl[i] = pv[i] = 0.f;
                if (sp0 + i < ns_g) {
                    const int sp = sp0 + i;
                    pm[i] = ld(ml + 2 * sp);
                    pl[i] = ld(ml + 2 * sp + 1);
                    pv[i] = ld(po + (int64_t)sp * D);
                }
            }
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
                const float Mn = fmaxf(M, pm[i]);
                if (sp0 + i < ns_g && Mn != -INFINITY) {
                    const float a = exp2f(M - Mn), c = exp2f(pm[i] - Mn);
                    L = L * a + pl[i] * c;
                    O = O * a + pv[i] * c;
                    M = Mn;
                }
            }
        }
        A.out[row * D + e] = (M != -INFINITY) ? O / L : 0.f;
    }
    if (tid == 0) __hip_atomic_store(&A.counters[group], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Launch of one (D, G) family.  tb: the angle bit width of a single-tier pool
// at a fixed page stride (the tier-specialised kernel), 0 for pools read
// through their page headers (mixed tiers, page offsets), kDenseTB for the
// dense-key baseline.  DBG variants also store the logits; they are the same
// kernels as the production ones apart from that store, so a logits request
// runs the kernel that produces `out` in production.  APP variants store the
// step's new token first.
template <int D, int G, bool DBG, bool APP, bool QF>
void launch_tier(const DecodeArgs &a, int tb, dim3 grid, hipStream_t s) {
    switch (tb) {
        case 2: hipLaunchKernelGGL((k_decode<D, G, 2, DBG, APP, QF>), grid, dim3(kThreads), 0, s, a); break;
        case 3: hipLaunchKernelGGL((k_decode<D, G, 3, DBG, APP, QF>), grid, dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_decode<D, G, 4, DBG, APP, QF>), grid, dim3(kThreads), 0, s, a); break;
        case 6: hipLaunchKernelGGL((k_decode<D, G, 6, DBG, APP, QF>), grid, dim3(kThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_decode<D, G, 8, DBG, APP, QF>), grid, dim3(kThreads), 0, s, a); break;
        case kDenseTB:   // (no query direction: one variant)
            if constexpr (!APP && !QF)
                hipLaunchKernelGGL((k_decode<D, G, kDenseTB, DBG, false, false>), grid, dim3(kThreads), 0, s, a);
            break;
        default: hipLaunchKernelGGL((k_decode<D, G, 0, DBG, APP, QF>), grid, dim3(kThreads), 0, s, a); break;
    }
}

// One (D, G, query precision) family; instantiated in its own translation
// unit (k_decode_inst.hip).
template <int D, int G, bool QF>
hipError_t launch_dg(const DecodeArgs &a, int tb, dim3 grid, hipStream_t s) {
    const bool app = a.app_k != nullptr;   // (never with dense keys)
    if (a.logits) {
        if (app) launch_tier<D, G, true, true, QF>(a, tb, grid, s);
        else launch_tier<D, G, true, false, QF>(a, tb, grid, s);
    } else {
        if (app) launch_tier<D, G, false, true, QF>(a, tb, grid, s);
        else launch_tier<D, G, false, false, QF>(a, tb, grid, s);
    }
    return hipGetLastError();
}

}  // namespace ska
