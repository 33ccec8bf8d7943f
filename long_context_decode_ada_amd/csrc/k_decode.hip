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
//    prepared once per step (k_qprep) as fp16 pairs and held packed in
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

// Load the lane's slice of a record: SW dwords at byte address p (4-aligned).
template <int SW>
__device__ __forceinline__ void load_slice(const uint8_t *p, uint32_t (&cw)[8]) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    if constexpr (SW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < SW / 4; ++k) {
            const uint4 x = *reinterpret_cast<const uint4 *>(q + 4 * k);
            cw[4 * k + 0] = x.x; cw[4 * k + 1] = x.y; cw[4 * k + 2] = x.z; cw[4 * k + 3] = x.w;
        }
    } else if constexpr (SW % 2 == 0) {
#pragma unroll
        for (int k = 0; k < SW / 2; ++k) {
            const uint2 x = *reinterpret_cast<const uint2 *>(q + 2 * k);
            cw[2 * k + 0] = x.x; cw[2 * k + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < SW; ++k) cw[k] = q[k];
    }
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

template <int D, int B>
__device__ __forceinline__ void load_page_b(const DecodeArgs &A, const PageDesc &pd, int kvh, PageBuf<D> &r) {
    constexpr int KB = record_bytes(D, B);
    constexpr int SW = KB / 16;
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, j = lane & 3;
    const int q4 = lane >> 4, n16 = lane & 15;
    const uint8_t *blk = A.kcode + pd.off + (uint64_t)kvh * kPage * KB;
    load_slice<SW>(blk + t * KB + j * (KB / 4), r.cw);
    const int64_t pk = (int64_t)pd.phys * A.hkv + kvh;
    r.rc = A.rcode[pk * kPage + t];
    const uint16_t *vblk = A.v + pk * (int64_t)D * kPage;
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
        r.vf[k] = *reinterpret_cast<const uint2 *>(vblk + (16 * k + n16) * kPage + 4 * q4);
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
    const int az_base = (j == 3) ? lut_azimuth(B) : lut_polar(B);
    const int pad_base = (j == 3) ? kLutOnes : lut_polar(B);
    float F[G];
#pragma unroll
    for (int h = 0; h < G; ++h) F[h] = 0.f;
    float P = 1.f;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const uint32_t c = code_at<B>(r.cw, i);
        int e;
        if (i == NA - 2) e = az_base + (int)c;
        else if (i == NA - 1) e = pad_base + (int)c;
        else e = lut_polar(B) + (int)c;
        const float2 cs = lut[e];
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
        const float alpha = exp2f(st.m - mn);
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
    const float pe = exp2f(lg - st.m);
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
    // query halves of every tier present (mixed-tier pools only)
    __shared__ __attribute__((aligned(16))) uint32_t uq_lds[TB == 0 ? 5 * D * G / 2 : 4];

    if constexpr (TB != 0) {
        // only this tier's tables and the (1, 1) padding entries it can index
        for (int e = tid; e < 2 << TB; e += kThreads) lut[lut_polar(TB) + e] = A.lut[lut_polar(TB) + e];
        for (int e = tid; e < 1 << TB; e += kThreads) lut[kLutOnes + e] = A.lut[kLutOnes + e];
    } else {
        for (int e = tid; e < kLutEntries; e += kThreads) lut[e] = A.lut[e];
    }
    rlev[tid] = A.rlev[kvh * 256 + tid];
    const uint32_t *uq_glb = reinterpret_cast<const uint32_t *>(A.uq + ((int64_t)seq * A.hkv + kvh) * A.nt * D * G);
    if constexpr (TB == 0)
        for (int e = tid; e < A.nt * D * G / 2; e += kThreads) uq_lds[e] = uq_glb[e];
    __syncthreads();

    const int ppw = A.pps / kWaves;
    const int wp0 = p0 + wave * ppw;
    const int wp1 = min(wp0 + ppw, p1);

    WaveState st{-INFINITY, 0.f};
    v4f acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t u[D * G / 8];
    int cur_b = -1;
    const int jq = lane & 3;
    if constexpr (TB != 0) {
        load_query<D, G>(reinterpret_cast<const uint4 *>(uq_glb + (A.tslot[TB] * 4 + jq) * (D * G / 8)), u);
        cur_b = TB;
    } else {
#pragma unroll
        for (int i = 0; i < D * G / 8; ++i) u[i] = 0u;
    }
    // this lane's head in the softmax: j % G
    const float sq = A.sq[head0 + ((lane & 3) % G)];

    const int64_t bt_row = (int64_t)seq * A.max_pages;
    float *pb = pbuf[wave];

    for (int c0 = wp0; c0 < wp1; c0 += 64) {
        const int cn = min(64, wp1 - c0);
        // this chunk's page list, one page per lane, valid pages first
        // (ordered by tier when tiers are mixed, so that the query registers
        // change at most once per tier)
        int e_pg = c0 + lane, e_phys = -1, e_bits = 0;
        uint32_t e_lo = 0, e_hi = 0;
        if (lane < cn) {
            const int ph = A.block_table[bt_row + c0 + lane];
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
                    load_query<D, G>(reinterpret_cast<const uint4 *>(uq_lds + (A.tslot[b] * 4 + jq) * (D * G / 8)), u);
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
// (m, l) pairs are wave-uniform (scalar loads); the o_s loads of a thread
// are independent and unrolled.  A sequence with no resident token gets 0.
template <int D>
__global__ __launch_bounds__(D) void k_merge(MergeArgs A) {
    const int row = blockIdx.x;
    const int seq = row / A.hq;
    const int e = threadIdx.x;
    int len = A.seq_lens[seq];
    len = max(0, min(len, A.max_pages * kPage));
    const int npages = (len + kPage - 1) / kPage;
    const int ns = (npages + A.pps - 1) / A.pps;
    const float *ml = A.part_ml + (int64_t)row * A.nsplit * 2;
    const float *po = A.part_o + (int64_t)row * A.nsplit * D + e;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
        for (int s = 0; s < ns; ++s) {
            const float sc = exp2f(ml[2 * s] - M);
            L += sc * ml[2 * s + 1];
            O += sc * po[(int64_t)s * D];
        }
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
