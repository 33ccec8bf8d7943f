// k_decode.hip -- Angle-Domain Attention decode over the paged code store.
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
//  * Work: one workgroup of 4 waves per (sequence, kv head, split of pages);
//    each wave walks a contiguous run of pages, one page per iteration.
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
//    head: exact codes, then a product scan) as fp16 pairs and held packed in
//    registers; v_fma_mix_f32 multiplies a half by the fp32 w and accumulates
//    in fp32.  Rounding uq to fp16 moves f by at most 2^-11 (Cauchy-Schwarz
//    over two unit vectors).  The logit is sq_h * r~ * f with
//    sq_h = scale * |q_h| * log2(e) in fp32, so logits are in log2 units.
//  * Softmax: online, per head, with the running max raised only when a logit
//    exceeds it by more than 8 (a wave ballot); probabilities are bounded by
//    2^8, which fp32 accumulation absorbs.
//  * P.V: for one page the group's product is (G heads x 16 tokens) times
//    (16 tokens x d) -- a dense contraction, run on MFMA
//    v_mfma_f32_16x16x16_bf16.  P is split exactly as P = hi + lo with hi,
//    lo in bf16 (rows 0..G-1 and G..2G-1 of the A operand), so the product
//    keeps 16 mantissa bits of P; V enters as stored (bf16), dimension-major
//    pages giving each lane its 4 consecutive tokens as one 8-byte load.
//  * Split-T: each workgroup merges its 4 waves in LDS and writes one
//    (m, l, o[d]) partial per query head; a second kernel (k_merge) combines
//    the splits.  (Combining them in the last workgroup to finish, behind a
//    device-scope fence, costs far more on this 8-XCD part: the fence writes
//    back and invalidates the L2 of every workgroup's XCD.)
//  * Page pipeline: each wave orders its next 64 pages (valid first, by tier)
//    in registers, then keeps the loads of page k+1 in flight (a second
//    register set) while page k is computed.
#include "ska_codes.h"
#include "ska_internal.h"

namespace ska {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994531f;

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
template <int B>
struct CodeAddr {
    uint32_t s[16];
    __device__ __forceinline__ void init(const uint32_t (&cw)[8]) {
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
        if constexpr (B == 4) {
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
    uint2 vf[D / 16];
};

// Wave-uniform description of one page.
struct PageDesc {
    int phys, b, p;
    uint64_t off;   // byte offset of the physical page's code block
};

// Raw buffer descriptor (V#) over `bytes` bytes at a wave-uniform address:
// loads past the end return 0 instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Loads of one page: the page's code block, radius bytes and V block each
// get a descriptor built in scalar registers; the per-lane offsets inside a
// block are the same for every page.
template <int D, int B>
__device__ __forceinline__ void load_page_b(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    constexpr int KB = record_bytes(D, B);
    constexpr int SW = KB / 16;
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int q4 = lane >> 4, n16 = lane & 15;
    const int64_t pk = (int64_t)pd.phys * A.hkv + kvh;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(A.kcode + pd.off + (uint64_t)kvh * kPage * KB, kPage * KB);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(A.v + pk * (int64_t)D * kPage, D * kPage * 2);
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(A.rcode + pk * kPage, kPage);
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
    const int vv = (n16 * kPage + 4 * q4) * 2;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, vv + k * 16 * kPage * 2, 0, 0);
        r.vf[k] = make_uint2(x[0], x[1]);
    }
}

template <int D, int TB>
__device__ __forceinline__ void load_page(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    if constexpr (TB != 0) {
        load_page_b<D, TB>(A, pd, kvh, r);
    } else {
        switch (pd.b) {
            case 2: load_page_b<D, 2>(A, pd, kvh, r); break;
            case 3: load_page_b<D, 3>(A, pd, kvh, r); break;
            case 4: load_page_b<D, 4>(A, pd, kvh, r); break;
            case 6: load_page_b<D, 6>(A, pd, kvh, r); break;
            default: load_page_b<D, 8>(A, pd, kvh, r); break;
        }
    }
}

// f_b, logits, online softmax and the MFMA P.V update of one page.  DBG also
// stores the logits (a separate kernel variant, so that the store does not
// enter the memory-wait accounting of the production loop).
template <int D, int G, int B, bool DBG>
__device__ __forceinline__ void compute_page_b(const DecodeArgs &A, PageBuf<D> &r, int ntok, int64_t logit_base,
                                               const uint32_t (&u)[D * G / 8], float sq, const float2 *__restrict__ lut,
                                               const float *__restrict__ rlev, float *__restrict__ pb,
                                               WaveState &st, v4f (&acc)[D / 16]) {
    constexpr int NA = D / 4;
    constexpr int NT = D / 16;
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int q4 = lane >> 4, n16 = lane & 15;

    // ---- f_b on the lane's slice ----
    const uint32_t az_base = 8u * ((j == 3) ? lut_azimuth(B) : lut_polar(B));
    const uint32_t pad_base = 8u * ((j == 3) ? kLutOnes : lut_polar(B));
    const char *lutb = reinterpret_cast<const char *>(lut);
    CodeAddr<B> ca;
    ca.init(r.cw);
    float F[G];
#pragma unroll
    for (int h = 0; h < G; ++h) F[h] = 0.f;
    float P = 1.f;
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
            F[h] = (e2 & 1) ? fma_mix_hi(u[e2 >> 1], w, F[h]) : fma_mix_lo(u[e2 >> 1], w, F[h]);
        }
    }

    // ---- join the four slices: C_j = prod_{i<j} S_i ----
    float C = qperm<kQuadShr1>(P);
    C = (j == 0) ? 1.f : C;
    {
        const float z = qperm<kQuadShr1>(C);
        C = (j >= 1) ? C * z : C;
        const float z2 = qperm<kQuadShr2>(C);
        C = (j >= 2) ? C * z2 : C;
    }
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

    // ---- logits (log2 units) and online softmax ----
    const float lg = (t < ntok) ? sq * rlev[r.rc] * f : -INFINITY;
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
        for (int k = 0; k < NT; ++k) { r.vf[k].x &= m0; r.vf[k].y &= m1; }
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        v4s bfr;
        __builtin_memcpy(&bfr, &r.vf[k], 8);
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, bfr, acc[k], 0, 0, 0);
    }
}

template <int D, int G, int TB, bool DBG>
__device__ __forceinline__ void compute_page(const DecodeArgs &A, const PageDesc &pd, PageBuf<D> &r, int len,
                                             int64_t head0, const uint32_t (&u)[D * G / 8], float sq,
                                             const float2 *__restrict__ lut, const float *__restrict__ rlev,
                                             float *__restrict__ pb, WaveState &st, v4f (&acc)[D / 16]) {
    const int ntok = min(kPage, len - pd.p * kPage);
    const int64_t lbase = head0 * A.max_pages * kPage + (int64_t)pd.p * kPage;
    if constexpr (TB != 0) {
        compute_page_b<D, G, TB, DBG>(A, r, ntok, lbase, u, sq, lut, rlev, pb, st, acc);
    } else {
        switch (pd.b) {
            case 2: compute_page_b<D, G, 2, DBG>(A, r, ntok, lbase, u, sq, lut, rlev, pb, st, acc); break;
            case 3: compute_page_b<D, G, 3, DBG>(A, r, ntok, lbase, u, sq, lut, rlev, pb, st, acc); break;
            case 4: compute_page_b<D, G, 4, DBG>(A, r, ntok, lbase, u, sq, lut, rlev, pb, st, acc); break;
            case 6: compute_page_b<D, G, 6, DBG>(A, r, ntok, lbase, u, sq, lut, rlev, pb, st, acc); break;
            default: compute_page_b<D, G, 8, DBG>(A, r, ntok, lbase, u, sq, lut, rlev, pb, st, acc); break;
        }
    }
}

// The lane's packed query halves for one tier, from global memory (single
// tier, once per workgroup) or from the workgroup's LDS copy (mixed tiers).
template <int D, int G>
__device__ __forceinline__ void load_query(const uint4 *src, uint32_t (&u)[D * G / 8]) {
    constexpr int NW = D * G / 8;   // packed words per lane: (d/4) angles x G heads / 2
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
        const uint4 x = src[i];
        u[4 * i + 0] = x.x; u[4 * i + 1] = x.y; u[4 * i + 2] = x.z; u[4 * i + 3] = x.w;
    }
}

// TB: the angle bit width of every page when the pool has a single tier, or 0
// (pages of mixed tiers, dispatched per page on the header).
template <int D, int G, int TB, bool DBG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_decode(DecodeArgs A) {
    constexpr int NA = D / 4;
    constexpr int NT = D / 16;
    const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q4 = lane >> 4, n16 = lane & 15;
    const int64_t head0 = (int64_t)seq * A.hq + (int64_t)kvh * G;

    int len = A.seq_lens[seq];
    len = max(0, min(len, A.max_pages * kPage));
    const int npages = (len + kPage - 1) / kPage;
    const int p0 = split * A.pps;
    if (p0 >= npages) return;  // whole workgroup, before any barrier
    const int p1 = min(p0 + A.pps, npages);

    __shared__ float2 lut[kLutEntries];
    __shared__ float rlev[256];
    __shared__ __attribute__((aligned(16))) float pbuf[kWaves][G * 16];
    __shared__ float mo[kWaves][2 * G][D];
    __shared__ float mml[kWaves][G][2];
    // query preparation: the G query rows, their suffix sums, the edge tables
    // of the tiers present, and the resulting packed unit directions
    __shared__ float qs[G][D];
    __shared__ double qT[G][D];
    __shared__ double c2s[kThrEntries], s2s[kThrEntries];
    __shared__ __attribute__((aligned(16))) _Float16 uq_lds[(TB == 0 ? 5 : 1) * D * G];
    __shared__ float sq_lds[G];

    if constexpr (TB != 0) {
        // only this tier's tables and the (1, 1) padding entries it can index
        for (int e = tid; e < 2 << TB; e += kThreads) lut[lut_polar(TB) + e] = A.lut[lut_polar(TB) + e];
        for (int e = tid; e < 1 << TB; e += kThreads) lut[kLutOnes + e] = A.lut[kLutOnes + e];
    } else {
        for (int e = tid; e < kLutEntries; e += kThreads) lut[e] = A.lut[e];
    }
    rlev[tid] = A.rlev[kvh * 256 + tid];
    for (int e = tid; e < G * D; e += kThreads) qs[e / D][e % D] = A.q[head0 * D + e];
    // this wave's first block-table entries, requested before the query prep
    const int64_t bt_row = (int64_t)seq * A.max_pages;
    const int ppw = A.pps / kWaves;
    const int wp0 = p0 + wave * ppw;
    const int wp1 = min(wp0 + ppw, p1);
    const int ph_first = (wp0 + lane < wp1) ? A.block_table[bt_row + wp0 + lane] : -1;
    for (int b = 2; b <= 8; ++b) {
        if (!((A.tier_mask >> b) & 1u)) continue;
        for (int e = tid; e < (1 << b); e += kThreads) {
            c2s[thr_off(b) + e] = A.cos2[thr_off(b) + e];
            s2s[thr_off(b) + e] = A.sin2[thr_off(b) + e];
        }
        for (int e = tid; e < (1 << (b - 1)); e += kThreads) {
            c2s[thr_off(b - 1) + e] = A.cos2[thr_off(b - 1) + e];
            s2s[thr_off(b - 1) + e] = A.sin2[thr_off(b - 1) + e];
        }
    }
    __syncthreads();
    // Query prep, section 2.1's c_q: suffix sums of each query row in the
    // keys' backward order (one thread per head), then per tier the angle
    // codes (bisection over the edge tables) and the decoded direction
    // u_a = (prod_{k<a} sin c_k) * cos c_a as a product scan across a wave
    // (one wave per head; fp32 is ample for a value stored as fp16).
    if (tid < G) {
        float x[D];   // the row in registers: the LDS reads leave the serial add chain
#pragma unroll
        for (int a = 0; a < D; ++a) x[a] = qs[tid][a];
        double T = add_square(0.0, x[D - 1]);
        qT[tid][D - 1] = T;
#pragma unroll
        for (int a = D - 2; a >= 0; --a) {
            T = add_square(T, x[a]);
            qT[tid][a] = T;
        }
        sq_lds[tid] = (float)((double)A.scale * sqrt(T) * 1.4426950408889634);
    }
    __syncthreads();
    if (wave < G) {
        const int h = wave;
        constexpr int PL = D / 64;   // components per lane
        const double qn = sqrt(qT[h][0]);
        int ti = 0;
        for (int b = 2; b <= 8; ++b) {
            if (!((A.tier_mask >> b) & 1u)) continue;
            float uv[PL];
            if (A.query_mode == 1) {
#pragma unroll
                for (int r = 0; r < PL; ++r) {
                    const int a = lane * PL + r;
                    uv[r] = qn > 0.0 ? (float)((double)qs[h][a] / qn) : 0.f;
                }
            } else {
                float cs[PL], sn[PL];
#pragma unroll
                for (int r = 0; r < PL; ++r) {
                    const int a = lane * PL + r;
                    cs[r] = 1.f;
                    sn[r] = 1.f;
                    if (a < D - 2) {
                        const int c = polar_code((double)qs[h][a], qT[h][a + 1], b, c2s + thr_off(b), s2s + thr_off(b));
                        const float2 e = lut[lut_polar(b) + c];
                        cs[r] = e.x;
                        sn[r] = e.y;
                    } else if (a == D - 2) {
                        const int c = azimuth_code((double)qs[h][D - 2], (double)qs[h][D - 1], b,
                                                   c2s + thr_off(b - 1), s2s + thr_off(b - 1));
                        const float2 e = lut[lut_azimuth(b) + c];
                        cs[r] = e.x;
                        sn[r] = e.y;
                    }
                }
                float tot = 1.f;
#pragma unroll
                for (int r = 0; r < PL; ++r) tot *= sn[r];
                float incl = tot;   // inclusive product scan of the lanes' sine products
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float v = __shfl_up(incl, off);
                    if (lane >= off) incl *= v;
                }
                float P = __shfl_up(incl, 1);
                if (lane == 0) P = 1.f;
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
                uq_lds[((ti * 4 + sl) * (D / 4) + i) * G + h] = (_Float16)uv[r];
            }
            ++ti;
        }
    }
    __syncthreads();
    WaveState st{-INFINITY, 0.f};
    v4f acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t u[D * G / 8];
    int cur_b = -1;
    const int jq = lane & 3;
    const uint32_t *uqw = reinterpret_cast<const uint32_t *>(uq_lds);
    if constexpr (TB != 0) {
        load_query<D, G>(reinterpret_cast<const uint4 *>(uqw + jq * (D * G / 8)), u);
        cur_b = TB;
    } else {
#pragma unroll
        for (int i = 0; i < D * G / 8; ++i) u[i] = 0u;
    }
    // this lane's head in the softmax: j % G
    const float sq = sq_lds[(lane & 3) % G];

    float *pb = pbuf[wave];

    for (int c0 = wp0; c0 < wp1; c0 += 64) {
        const int cn = min(64, wp1 - c0);
        // this chunk's page list, one page per lane, valid pages first
        // (ordered by tier when tiers are mixed, so that the query registers
        // change at most once per tier)
        int e_pg = c0 + lane, e_phys = -1, e_bits = 0;
        uint32_t e_lo = 0, e_hi = 0;
        if (lane < cn) {
            const int ph = (c0 == wp0) ? ph_first : A.block_table[bt_row + c0 + lane];
            const bool ok = ph >= 0 && (int64_t)ph < A.num_pages;
            const int bb = ok ? (int)A.page_bits[ph] : 0;
            const bool okb = ok && bb >= 2 && bb <= 8 && ((A.tier_mask >> bb) & 1u);
            if (!ok) atomicOr(A.err, 2u);
            else if (!okb) atomicOr(A.err, 4u);
            if (okb) {
                e_phys = ph;
                e_bits = bb;
                const uint64_t off = A.page_off ? A.page_off[ph] : (uint64_t)ph * (uint64_t)A.page_stride;
                e_lo = (uint32_t)off;
                e_hi = (uint32_t)(off >> 32);
            }
        }
        const int key = (e_phys >= 0) ? e_bits : 15;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int rank = 0, nvalid = 0;
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
        e_bits = __builtin_amdgcn_ds_permute(rank * 4, e_bits);
        e_lo = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)e_lo);
        e_hi = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)e_hi);
        if (nvalid == 0) continue;

        auto desc = [&](int k) {
            PageDesc pd;
            pd.phys = __builtin_amdgcn_readlane(e_phys, k);
            pd.b = TB != 0 ? TB : __builtin_amdgcn_readlane(e_bits, k);
            pd.p = __builtin_amdgcn_readlane(e_pg, k);
            pd.off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)e_hi, k) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane((int)e_lo, k);
            return pd;
        };
        auto ensure_query = [&](int b) {
            if constexpr (TB == 0) {
                if (b != cur_b) {
                    load_query<D, G>(reinterpret_cast<const uint4 *>(uqw + (A.tslot[b] * 4 + jq) * (D * G / 8)), u);
                    cur_b = b;
                }
            }
        };
        // two register sets: the loads of page k+1 are in flight while page k
        // is computed.  The loads are issued unconditionally (past the end
        // they repeat the last page) so that the wait before each compute
        // only covers the loads of the page being computed.
        PageBuf<D> R0, R1;
        const int last = nvalid - 1;
        PageDesc d0 = desc(0);
        load_page<D, TB>(A, d0, kvh, R0);
        for (int k = 0; k < nvalid; k += 2) {
            const PageDesc d1 = desc(min(k + 1, last));
            load_page<D, TB>(A, d1, kvh, R1);
            __builtin_amdgcn_sched_barrier(0);   // issue these loads before waiting on page k
            ensure_query(d0.b);
            compute_page<D, G, TB, DBG>(A, d0, R0, len, head0, u, sq, lut, rlev, pb, st, acc);
            d0 = desc(min(k + 2, last));
            load_page<D, TB>(A, d0, kvh, R0);
            __builtin_amdgcn_sched_barrier(0);
            if (k + 1 < nvalid) {
                ensure_query(d1.b);
                compute_page<D, G, TB, DBG>(A, d1, R1, len, head0, u, sq, lut, rlev, pb, st, acc);
            }
        }
    }

    // ---- merge the four waves of this workgroup ----
    const float lsum = head_reduce<G, false>(st.l);
    if (lane < G) {
        mml[wave][lane][0] = st.m;
        mml[wave][lane][1] = lsum;
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const float a4[4] = {acc[k].x, acc[k].y, acc[k].z, acc[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 4 * q4 + i;
            if (rr < 2 * G) mo[wave][rr][16 * k + n16] = a4[i];
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
        const int64_t pi = (head0 + h) * A.nsplit + split;
        A.part_o[pi * D + e] = O;
        if (e == 0) {
            A.part_ml[2 * pi + 0] = M;
            A.part_ml[2 * pi + 1] = L;
        }
    }

}

// Split merge: one workgroup of d threads per (sequence, query head):
// M = max_s m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.  The
// (m, l) pairs are read by one thread each and combined in LDS; every o_s
// read of a thread is independent of the others.  A sequence with no
// resident token gets 0.
template <int D>
__global__ __launch_bounds__(D) void k_merge(MergeArgs A) {
    __shared__ float sm[D], sl[D];
    __shared__ float red[D / 64];
    const int row = blockIdx.x;
    const int seq = row / A.hq;
    const int e = threadIdx.x;
    int len = A.seq_lens[seq];
    len = max(0, min(len, A.max_pages * kPage));
    const int npages = (len + kPage - 1) / kPage;
    const int ns = (npages + A.pps - 1) / A.pps;
    const float *ml = A.part_ml + (int64_t)row * A.nsplit * 2;
    const float *po = A.part_o + (int64_t)row * A.nsplit * D + e;
    float O = 0.f, L = 0.f, M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += D) {   // D splits per round (one round in practice)
        const int n = min(D, ns - s0);
        float m = -INFINITY;
        if (e < n) {
            m = ml[2 * (s0 + e)];
            sm[e] = m;
            sl[e] = ml[2 * (s0 + e) + 1];
        }
        float v = m;
        for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
        if ((e & 63) == 0) red[e >> 6] = v;
        __syncthreads();
        float Mr = red[0];
#pragma unroll
        for (int w = 1; w < D / 64; ++w) Mr = fmaxf(Mr, red[w]);
        const float Mn = fmaxf(M, Mr);
        if (Mn != -INFINITY) {
            const float r = exp2f(M - Mn);
            O *= r;
            L *= r;
#pragma unroll 8
            for (int s = 0; s < n; ++s) {
                const float sc = exp2f(sm[s] - Mn);
                L += sc * sl[s];
                O += sc * po[(int64_t)(s0 + s) * D];
            }
        }
        M = Mn;
        __syncthreads();
    }
    A.out[(int64_t)row * D + e] = (M != -INFINITY) ? O / L : 0.f;
}

template <int D, int G>
static void launch_dg(const DecodeArgs &a, int tb, dim3 grid, hipStream_t s) {
    if (a.logits) {  // debug variant: stores the logits; generic tier dispatch
        hipLaunchKernelGGL((k_decode<D, G, 0, true>), grid, dim3(kThreads), 0, s, a);
        return;
    }
    switch (tb) {
        case 2: hipLaunchKernelGGL((k_decode<D, G, 2, false>), grid, dim3(kThreads), 0, s, a); break;
        case 3: hipLaunchKernelGGL((k_decode<D, G, 3, false>), grid, dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_decode<D, G, 4, false>), grid, dim3(kThreads), 0, s, a); break;
        case 6: hipLaunchKernelGGL((k_decode<D, G, 6, false>), grid, dim3(kThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_decode<D, G, 8, false>), grid, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((k_decode<D, G, 0, false>), grid, dim3(kThreads), 0, s, a); break;
    }
}

hipError_t launch_decode(const DecodeArgs &a, int d, int G, int B, hipStream_t s) {
    if (B == 0) return hipSuccess;
    const dim3 grid((unsigned)a.nsplit, (unsigned)a.hkv, (unsigned)B);
    int tb = 0;
    if (__builtin_popcount(a.tier_mask) == 1) tb = __builtin_ctz(a.tier_mask);
    if (d == 128) {
        if (G == 4) launch_dg<128, 4>(a, tb, grid, s);
        else if (G == 2) launch_dg<128, 2>(a, tb, grid, s);
        else launch_dg<128, 1>(a, tb, grid, s);
    } else {
        if (G == 4) launch_dg<64, 4>(a, tb, grid, s);
        else if (G == 2) launch_dg<64, 2>(a, tb, grid, s);
        else launch_dg<64, 1>(a, tb, grid, s);
    }
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, int B, hipStream_t s) {
    if (B == 0) return hipSuccess;
    const dim3 grid((unsigned)(B * a.hq));
    if (a.d == 128) hipLaunchKernelGGL(k_merge<128>, grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL(k_merge<64>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace ska
