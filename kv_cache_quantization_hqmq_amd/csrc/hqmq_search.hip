// HQMQ encode search for fp16 inputs on the gfx950 f16 matrix cores.
//
// Method (arXiv 2605.27646; the abstract as shown on paperdance.org and
// thelatestinai.com; gist.science/nl "Technische Samenvatting",
// Methodologie 1-3): each 4-element chunk x takes the codeword q_p * q_s
// (q_p one of the 24 units of 2T, q_s one of the slice's S secondary
// codewords) of largest inner product; by linearity in q_p the best of the 24
// for a given s scores max(|t|_inf, |t|_1 / 2) with t_m = <x, e_m q_s>.
//
// v_mfma_f32_32x32x8_f16 computes 32 rows (8 secondary codewords x 4 basis
// units e_m) against 32 chunks with K = 8: k = 0..3 multiply the chunk's four
// fp16 components by the hi parts of the rows e_m q_s, k = 4..7 by the lo
// parts.  Every product is exact in fp32 and D accumulates in fp32, so t is
// the fp32 transform of the exact codebook value.  Lane l supplies A row
// l % 32, k block l / 32, and B column l % 32 (the raw 8-byte chunk, the same
// for both k blocks); D VGPR 4 a + r of lane l is row 8 a + 4 (l / 32) + r,
// column l % 32.  Row 8 a + 4 h + r of tile t holds m = r of
// s = h H + 4 t + a, H = 4 x (tiles): lanes 0..31 score the first H secondary
// codewords and lanes 32..63 the rest, so every candidate of the upper lanes
// has the larger index.
//
// The scoring epilogue is VALU work, the kernel's bound.  This file is built
// with IEEE mode off and fp32 denormals flushed so that the halving in
// |t|_1 / 2 rides on the add that forms the sum (the VOP3 output modifier
// div:2, which the hardware applies only in that mode): one instruction per
// score fewer.  Both settings leave every value unchanged here: inputs are
// finite binary16 values and the codebook sits on the double-binary16 grid,
// so every nonzero product, transform component, score and squared norm the
// kernel forms is a multiple of 2^-48 and far above the fp32 denormal range,
// and without NaNs the IEEE-mode differences (signalling-NaN quieting, NaN
// operands of min / max) cannot arise.  Functions that are not inlined across
// a mode difference (the device library's) are not called.
#include <hip/hip_runtime.h>

#include "hqmq_device.h"
#include "hqmq_encode.h"

namespace hqmq {
namespace {

// (a + b) / 2 as one v_add_f32 with the div:2 output modifier.  The halving is
// exact for the normal values it sees, so the result is fl(a + b) / 2.
__device__ __forceinline__ float half_sum(float a, float b) {
    float r;
    asm("v_add_f32_e64 %0, %1, %2 div:2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// v_sqrt_f32(a) / 2 with the halving as the div:2 output modifier.
__device__ __forceinline__ float sqrt_half(float a) {
    float r;
    asm("v_sqrt_f32_e64 %0, %1 div:2" : "=v"(r) : "v"(a));
    return r;
}

// l - |t| as one v_sub_f32 with the abs source modifier (kept from being
// folded back into a compare of |t|, which would need |t| in a register).
__device__ __forceinline__ float abs_gap(float l, float t) {
    float r;
    asm("v_sub_f32_e64 %0, %1, |%2|" : "=v"(r) : "v"(l), "v"(t));
    return r;
}

// Index of the first zero among gaps g0, g1, g2 (3 when none is zero), for
// gaps that are +0 or at least 2^-48: as bit patterns they order like their
// values, so the keys g0, g1 | 1 and med3(g2, 2, 3) are 0, 1 and 2 for a zero
// gap and above 3 otherwise, and their minimum is the index (one bitwise op,
// v_med3_u32 and v_min3_u32 instead of three compares and three selects).
__device__ __forceinline__ uint32_t first_zero_gap(float g0, float g1, float g2) {
    uint32_t k2;
    asm("v_med3_u32 %0, %1, 2, 3" : "=v"(k2) : "v"(__float_as_uint(g2)));
    return min(min(__float_as_uint(g0), __float_as_uint(g1) | 1u), k2);
}

// Score of the best 2T element for one s from t = (<x, e_m q_s>)_m:
// max(|t|_inf, |t|_1 / 2) (a unit +-e_m scores +-t_m, a half-unit
// (s0..s3)/2 scores sum s_m t_m / 2, largest with s_m = sign t_m).
__device__ __forceinline__ float best_primary(float t0, float t1, float t2, float t3) {
    const float e0 = fabsf(t0), e1 = fabsf(t1), e2 = fabsf(t2), e3 = fabsf(t3);
    const float m3 = fmaxf(fmaxf(e0, e1), e2);
    return fmaxf(fmaxf(m3, e3), half_sum(e0 + e1, e2 + e3));
}

// Index p of the best 2T element for secondary codeword qs: t = (<x, e_m q_s>)_m
// in fp32; a unit +-e_m (p = 2 m + sign) wins when |t|_inf >= |t|_1 / 2
// (lowest m, + before -), otherwise the half-unit with s_m = sign t_m
// (p = 8 + sum of (t_m < 0) 2^m; 0 counts as +).  Each component's fma chain
// starts from +0, so an exact zero comes out +0 (a -0 sum needs every addend
// to be -0) and its sign bit is the half-unit's sign.  Branch-free.
__device__ __forceinline__ uint32_t primary_index(const float *qs, float x0, float x1, float x2, float x3) {
    const float q0 = qs[0], q1 = qs[1], q2 = qs[2], q3 = qs[3];
    const float t0 = __builtin_fmaf(q3, x3, __builtin_fmaf(q2, x2, __builtin_fmaf(q1, x1, __builtin_fmaf(q0, x0, 0.0f))));
    const float t1 = __builtin_fmaf(q2, x3, __builtin_fmaf(-q3, x2, __builtin_fmaf(q0, x1, __builtin_fmaf(-q1, x0, 0.0f))));
    const float t2 = __builtin_fmaf(-q1, x3, __builtin_fmaf(q0, x2, __builtin_fmaf(q3, x1, __builtin_fmaf(-q2, x0, 0.0f))));
    const float t3 = __builtin_fmaf(q0, x3, __builtin_fmaf(q1, x2, __builtin_fmaf(-q2, x1, __builtin_fmaf(-q3, x0, 0.0f))));
    const float e0 = fabsf(t0), e1 = fabsf(t1), e2 = fabsf(t2), e3 = fabsf(t3);
    // first argmax of |t_m|: the first m reaching the largest, from the gaps
    // linf - |t_m| (zero exactly when equal: every t_m is a multiple of
    // 2^-48, so a nonzero difference is far above the denormal range)
    const float linf = fmaxf(fmaxf(e0, e1), fmaxf(e2, e3));
    const uint32_t m = first_zero_gap(abs_gap(linf, t0), abs_gap(linf, t1), abs_gap(linf, t2));
    // sign bits: v_perm selectors 9 and 11 give 0xFF or 0x00 from the sign of
    // the low and the high source word, one byte per value; masking byte m
    // to 2^m and summing the bytes (v_sad_u8 against zero) gives the nibble
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x0c0c0b09u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t3), __float_as_uint(t2), 0x0b090c0cu);
    const uint32_t nib = __builtin_amdgcn_sad_u8((lo | hi) & 0x08040201u, 0u, 0u);
    const uint32_t unit = 2u * m + __builtin_amdgcn_ubfe(nib, m, 1u);
    return linf >= half_sum(e0 + e1, e2 + e3) ? unit : 8u + nib;
}

template <int NT8, bool MED>
__global__ __launch_bounds__(kEncThreads) void encode_search_h_kernel(EncArgs a) {
    constexpr int kQ = NT8 > 0 ? 32 * NT8 : 4 * kMaxS;
    __shared__ __attribute__((aligned(16))) float sq[kQ];
    __shared__ uint32_t sword[4][64];   // the group's packed index words, per wave
    __shared__ uint32_t shist[MED ? 2048 : 1];
    __shared__ uint32_t sh[kEncThreads / 64 + 3];

    const TileCoords tc = tile_coords(a);
    const int64_t slice = tc.slice;
    const int64_t c_begin = tc.c_begin;
    const int64_t c_end = tc.c_end;
    const int NT = NT8 > 0 ? NT8 : (a.S + 7) / 8;
    {
        const float *q = a.cb + slice * a.S * 4;
        const int nq = 32 * NT;
        for (int i = thread_id(); i < nq; i += kEncThreads) sq[i] = i < 4 * a.S ? double_f16(q[i]) : 0.0f;
        if constexpr (MED)
            for (int i = thread_id(); i < 2048; i += kEncThreads) shist[i] = 0;
    }
    __syncthreads();

    const int lane = thread_id() & 63;
    // wave-uniform (a scalar register), so the loop and the block-relative
    // offsets below are scalar work
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(thread_id() >> 6));
    const int col = lane & 31;
    // A: K block (0 = hi parts, 1 = lo parts); D: row half (0 = the first H
    // secondary codewords, 1 = the rest)
    const int hh = lane >> 5;
    const int m_row = col & 3;
    const int half_q = 4 * NT;               // H
    // the A row's s relative to 4 t
    const int s_row = ((col >> 2) & 1) * half_q + (col >> 3);

    // A operand of tile t: row (s = s_row + 4 t, m = m_row), k = 0..3 of the
    // hi (hh = 0) or lo (hh = 1) part of (e_m q_s)[k] = sign(m, k) q_s[m ^ k]
    auto a_operand = [&](int t) {
        const float *qs = &sq[4 * (s_row + 4 * t)];
        f16x4 r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float v = qs[m_row ^ k];
            const _Float16 hi = static_cast<_Float16>(v);
            const _Float16 part = hh ? static_cast<_Float16>(v - static_cast<float>(hi)) : hi;
            r[k] = ((kNegMask >> (4 * m_row + k)) & 1u) ? -part : part;
        }
        return r;
    };
    f16x4 A[NT8 > 0 ? NT8 : 1];
    if constexpr (NT8 > 0) {
#pragma unroll
        for (int t = 0; t < NT8; ++t) A[t] = a_operand(t);
    }

    const f32x16 zero = {};
    const int wpg = (64 >> a.log2_cpt) * a.words;
    // buffer resources over the wave's current 64 chunks onward (rebuilt per
    // step from uniform values, so scalar work): the block's chunks
    // [c_begin, c_end) start on a token row and number at most 8192, so
    // offsets are 32-bit and the resources' sizes do the range checks (loads
    // past the end read 0, stores there are dropped)
    const uint32_t n =
        __builtin_amdgcn_readfirstlane(c_end > c_begin ? static_cast<uint32_t>(c_end - c_begin) : 0u);
    const uint32_t tok_lim = (n + static_cast<uint32_t>(a.cpt) - 1u) >> a.log2_cpt;   // token rows of the block
    const uint2 *xb = uniform(static_cast<const uint2 *>(a.x) + slice * a.n_slice + c_begin);
    uint16_t *hb = uniform(a.hnorm + slice * a.n_slice + c_begin);
    uint32_t *wb = uniform(a.idx + (slice * a.tokens + (c_begin >> a.log2_cpt)) * a.words);

    // x of the wave's steps (64 chunks from o0): B operands chunk o0 + 32 b + col
    // of both column blocks, and the lane's own chunk o0 + lane (a third load,
    // cheaper than selecting it).  Each step's loads are issued one step ahead;
    // a step at or past the end has an empty resource, so its loads read 0
    // without touching memory.
    struct XStep {
        u32x2 b[2];
        u32x2 own;
    };
    auto load_x = [&](uint32_t o) {
        const bool in = o < n;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(static_cast<const void *>(xb + (in ? o : 0u))), 0,
            static_cast<int>(in ? (n - o) * 8u : 0u), kBufWord3);
        XStep xs;
#pragma unroll
        for (int b = 0; b < 2; ++b)
            xs.b[b] = __builtin_amdgcn_raw_buffer_load_b64(rs, static_cast<int>((32u * b + col) * 8u), 0, 0);
        xs.own = __builtin_amdgcn_raw_buffer_load_b64(rs, lane * 8, 0, 0);
        return xs;
    };
    XStep next = load_x(64u * wave);
    for (uint32_t o0 = 64u * wave; o0 < n; o0 += 64u * 4u) {
        const uint32_t r0 = o0 >> a.log2_cpt;   // the step's first token row
        const __amdgpu_buffer_rsrc_t hrs =
            __builtin_amdgcn_make_buffer_rsrc(hb + o0, 0, static_cast<int>((n - o0) * 2u), kBufWord3);
        const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
            wb + r0 * static_cast<uint32_t>(a.words), 0,
            static_cast<int>((tok_lim - r0) * static_cast<uint32_t>(a.words) * 4u), kBufWord3);
        const XStep cur = next;
        next = load_x(o0 + 64u * 4u);
        uint2 xr[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) xr[b] = make_uint2(cur.b[b][0], cur.b[b][1]);
        const u32x2 own = cur.own;
        float bsc[2];      // best score and its s, per column block
        uint32_t bsi[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const f16x4 bv = __builtin_bit_cast(f16x4, xr[b]);
            // Running best over the MFMA tiles t: the best of a tile's four
            // scores (s = hh H + 4 t + g, g = 0..3) replaces the running one
            // when strictly larger, with the tile and its first three scores;
            // which g it was is resolved once at the end (first g reaching
            // it), so the result is the sequential strict argmax in s order.
            // The first tile sets the running best unconditionally.
            float best = 0.0f;
            uint32_t bt4 = 0;   // 4 t of the running best's tile
            float bs0 = 0.0f, bs1 = 0.0f, bs2 = 0.0f;
            auto tile = [&](int t, const f32x16 &d) {
                float sc[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) sc[g] = best_primary(d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3]);
                const float m = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                if (t == 0 || m > best) {
                    best = m;
                    bt4 = 4u * t;
                    bs0 = sc[0];
                    bs1 = sc[1];
                    bs2 = sc[2];
                }
            };
            if constexpr (NT8 > 0) {
#pragma unroll
                for (int t = 0; t < NT8; ++t) tile(t, __builtin_amdgcn_mfma_f32_32x32x8f16(A[t], bv, zero, 0, 0, 0));
            } else {
                tile(0, __builtin_amdgcn_mfma_f32_32x32x8f16(a_operand(0), bv, zero, 0, 0, 0));
                for (int t = 1; t < NT; ++t)
                    tile(t, __builtin_amdgcn_mfma_f32_32x32x8f16(a_operand(t), bv, zero, 0, 0, 0));
            }
            // first g reaching the best: the gaps best - bs_g are >= 0, zero
            // only when equal (multiples of 2^-48), and g = 3 when none is
            const uint32_t g = first_zero_gap(best - bs0, best - bs1, best - bs2);
            bsc[b] = best;
            // (disjoint bit fields when H is a power of two: one v_or3)
            constexpr bool kPow2 = NT8 > 0 && (NT8 & (NT8 - 1)) == 0;
            const uint32_t hoff = static_cast<uint32_t>(hh * half_q);
            bsi[b] = kPow2 ? (bt4 | g | hoff) : bt4 + g + hoff;
        }

        // lane l < 32 holds the first half's best of chunks l and l + 32, lane
        // l + 32 the second half's of the same chunks; swapping the upper half
        // of block 0 with the lower half of block 1 leaves every lane l with
        // both halves' of chunk o0 + l (v_permlane32_swap)
        uint32_t s_best;
        {
            const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(bsc[0]), __float_as_uint(bsc[1]), false, false);
            const auto pi = __builtin_amdgcn_permlane32_swap(bsi[0], bsi[1], false, false);
            const float s0 = __uint_as_float(ps[0]), s1 = __uint_as_float(ps[1]);
            const uint32_t i0 = pi[0], i1 = pi[1];
            // i1 > i0 always: the first half wins ties
            const bool take1 = s1 > s0;
            // 4 bt + g + hh H < 8 NT <= kMaxS: inside the codebook copy sq
            s_best = take1 ? i1 : i0;
            __builtin_assume(s_best < static_cast<uint32_t>(kMaxS));
        }
        const f16x4 xh = __builtin_bit_cast(f16x4, own);
        float v0 = static_cast<float>(xh[0]);
        float v1 = static_cast<float>(xh[1]);
        float v2 = static_cast<float>(xh[2]);
        float v3 = static_cast<float>(xh[3]);
        // one conversion each, then plain fp32 arithmetic (the compiler would
        // otherwise fold conversions into mixed-precision fmas, which issue at
        // half the rate of fp32 fmas here)
        asm("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));

        // declared fp32 squared norm and its binary16 half-norm code
        float s2 = v0 * v0;
        s2 = __builtin_fmaf(v1, v1, s2);
        s2 = __builtin_fmaf(v2, v2, s2);
        s2 = __builtin_fmaf(v3, v3, s2);
        const uint16_t hn = half_norm_code(s2, sqrt_half(s2));

        // A zero chunk (s2 = 0; any chunk past the range loads as one) comes
        // out as code 0 with no test: all its scores are 0, so s = 0 wins the
        // ties, and its transform is +0 throughout, so the primary is the
        // first unit.
        const uint32_t pidx = primary_index(&sq[4 * s_best], v0, v1, v2, v3);
        const uint32_t code = 24u * s_best + pidx;
        __builtin_amdgcn_raw_buffer_store_b16(hn, hrs, lane * 2, 0, 0);
        // every lane counts; a lane past the range holds a zero chunk (code
        // 0) and is taken back out of bin 0 after the loop
        if constexpr (MED) atomicAdd(&shist[hn >> 4], 1u);
        // pack the group's codes into its token rows' words: every code is
        // ORed into the one or two words it spans, then lane w < wpg stores
        // word w (codes past the range are 0 and leave their words as they are)
        if (lane < wpg) sword[wave][lane] = 0u;
        wave_sync();
        {
            const int bit = (lane & (a.cpt - 1)) * a.bits;
            uint32_t *wr = &sword[wave][(lane >> a.log2_cpt) * a.words + (bit >> 5)];
            const int sft = bit & 31;
            atomicOr(wr, code << sft);
            if (sft + a.bits > 32) atomicOr(wr + 1, code >> (32 - sft));
        }
        wave_sync();
        if (lane < wpg) {
            // word lane % words of token row r0 + lane / words
            __builtin_amdgcn_raw_buffer_store_b32(sword[wave][lane], wrs, lane * 4, 0, 0);
        }
        wave_sync();
    }
    if constexpr (MED) {
        // the block's last step counted (64 - n % 64) % 64 lanes past the range
        if (thread_id() == 0 && (n & 63u) != 0u) atomicSub(&shist[0], 64u - (n & 63u));
        med3_after_tile(a, tc, shist, sh);
    }
}


}  // namespace

hipError_t launch_search_h(const EncArgs &a, int64_t blocks, int nt8, bool med, int blocks_per_cu,
                           hipStream_t st) {
    const void *k = nullptr;
#define HQMQ_ENC_H(NT8)                                                                         \
    k = med ? reinterpret_cast<const void *>(&encode_search_h_kernel<NT8, true>)                 \
            : reinterpret_cast<const void *>(&encode_search_h_kernel<NT8, false>)
    if (nt8 == 1) HQMQ_ENC_H(1);
    else if (nt8 == 4) HQMQ_ENC_H(4);
    else HQMQ_ENC_H(0);
#undef HQMQ_ENC_H
    // an occupancy cap: the block's LDS (static + reserved) is sized so that
    // blocks_per_cu fit in a CU's 160 KB and one more does not (allocation in
    // 512-byte granules)
    size_t lds = 0;
    if (blocks_per_cu > 0) {
        hipFuncAttributes fa;
        const hipError_t e = hipFuncGetAttributes(&fa, k);
        if (e != hipSuccess) return e;
        constexpr size_t kLdsPerCu = 160 * 1024;
        const size_t per_block = (kLdsPerCu / static_cast<size_t>(blocks_per_cu + 1) + 1 + 511) / 512 * 512;
        lds = per_block > fa.sharedSizeBytes ? per_block - fa.sharedSizeBytes : 0;
    }
    EncArgs args = a;
    void *argv[] = {&args};
    const hipError_t e = hipLaunchKernel(k, dim3(static_cast<unsigned>(blocks)), dim3(kEncThreads), argv, lds, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace hqmq
