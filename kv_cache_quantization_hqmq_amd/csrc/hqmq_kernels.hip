// HQMQ encode / Med3x / decode kernels for AMD Instinct MI355X (gfx950).
//
// Method (arXiv 2605.27646; the abstract as shown on paperdance.org and
// thelatestinai.com; gist.science/nl "Technische Samenvatting",
// Methodologie 1-3): every 4-element chunk x of a K or V head vector is a
// quaternion; its norm is kept and its direction goes to the codeword
// q_p * q_s (q_p in 2T, q_s in the slice's S-entry codebook) of largest inner
// product; a per-batch Med3x step keeps chunks with r > C r_med in fp16.
//
// Encode search.  By linearity in q_p, <x, q_p q_s> = sum_m a_pm t_m(s) with
// t_m(s) = <x, e_m q_s> (e = 1, i, j, k), which is the conj(q_p) identity of
// the isometry argument (abstract) applied to the four basis units.  The best
// of the 24 primaries for a given s is max(|t|_inf, |t|_1 / 2): a unit +-e_m
// scores +-t_m, a half-unit (s0..s3)/2 scores sum s_m t_m / 2 (signs chosen
// to match t).  So the work per (chunk, s) is one 4x4 orthogonal transform
// (16 FMA) plus a short max/abs epilogue.  The transforms of 16 chunks against
// 4 secondary codewords are one v_mfma_f32_16x16x4f32: A = the 16 rows
// e_m q_s (4 s x 4 m) of the slice, B = 16 chunks x 4 components, and lane l
// of D holds the four t_m of s = 4 tile + l / 16 for chunk l % 16, so the
// epilogue runs in-lane.  The matrix core does the 16 FMA / (chunk, s), the
// VALU the epilogue, concurrently.
//
// Parity contract: hnorm and the Med3x outlier set are bit-exact with the
// declared fp32 arithmetic; codes are exact except where two codewords'
// scores differ by less than fp32 rounding (near ties).
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "hqmq_device.h"
#include "hqmq_encode.h"
#include "hqmq_launch.h"

namespace hqmq {
namespace {

constexpr int kFlagThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kDecThreads = 256;   // each thread decodes 4 chunks per step
constexpr int kDecUnroll = 8;      // steps whose loads a thread issues together
constexpr int kTableMaxS = 64;     // decode keeps the 24 S codewords in LDS up to here

// Score of the best 2T element for one s from t = (<x, e_m q_s>)_m:
// max(|t|_inf, |t|_1 / 2) (a unit +-e_m scores +-t_m; a half-unit
// (s0..s3)/2 scores sum s_m t_m / 2, largest with s_m = sign t_m).
__device__ __forceinline__ float best_primary(f32x4 d) {
    const float e0 = fabsf(d[0]), e1 = fabsf(d[1]), e2 = fabsf(d[2]), e3 = fabsf(d[3]);
    const float m3 = fmaxf(fmaxf(e0, e1), e2);
    const float h = ((e0 + e1) + (e2 + e3)) * 0.5f;
    return fmaxf(fmaxf(m3, e3), h);
}

// Index p of the best 2T element for secondary codeword qs: t = (<x, e_m q_s>)_m
// in fp32; a unit +-e_m (p = 2 m + sign) wins when |t|_inf >= |t|_1 / 2
// (lowest m, + before -), otherwise the half-unit with s_m = sign t_m
// (p = 8 + sum of (t_m < 0) 2^m; 0 counts as +).  Branch-free: the sign
// nibble comes from the top bits of t_m + 0 (which turns -0 into +0).
__device__ __forceinline__ int primary_index(const float *qs, float x0, float x1, float x2, float x3) {
    const float q0 = qs[0], q1 = qs[1], q2 = qs[2], q3 = qs[3];
    const float t0 = __builtin_fmaf(q3, x3, __builtin_fmaf(q2, x2, __builtin_fmaf(q1, x1, q0 * x0)));
    const float t1 = __builtin_fmaf(q2, x3, __builtin_fmaf(-q3, x2, __builtin_fmaf(q0, x1, -q1 * x0)));
    const float t2 = __builtin_fmaf(-q1, x3, __builtin_fmaf(q0, x2, __builtin_fmaf(q3, x1, -q2 * x0)));
    const float t3 = __builtin_fmaf(q0, x3, __builtin_fmaf(q1, x2, __builtin_fmaf(-q2, x1, -q3 * x0)));
    const float e0 = fabsf(t0), e1 = fabsf(t1), e2 = fabsf(t2), e3 = fabsf(t3);
    const float linf = fmaxf(fmaxf(fmaxf(e0, e1), e2), e3);
    const float l1 = (e0 + e1) + (e2 + e3);
    const uint32_t m = e0 == linf ? 0u : (e1 == linf ? 1u : (e2 == linf ? 2u : 3u));
    // top bytes of the four signed values side by side, then their sign bits
    // moved to bits 28..31 by one multiply (no two partial products overlap)
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t1 + 0.0f), __float_as_uint(t0 + 0.0f), 0x0c0c0703u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t3 + 0.0f), __float_as_uint(t2 + 0.0f), 0x07030c0cu);
    const uint32_t nib = (((lo | hi) & 0x80808080u) * 0x00204081u) >> 28;
    const uint32_t unit = 2u * m + ((nib >> m) & 1u);
    return static_cast<int>(linf + linf >= l1 ? unit : 8u + nib);
}

// Strict order of (score, s) candidates: higher score, then lower s.
__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// --------------------------------------------------------------------------
// Encode search kernel.
// --------------------------------------------------------------------------
// NT_REG > 0: S <= 4 NT_REG and the A operands live in registers.
// NT_REG == 0: any S <= kMaxS, A read from the LDS copy of the codebook.
template <int NT_REG, bool F32IN, bool MED>
__global__ __launch_bounds__(kEncThreads) void encode_search_kernel(EncArgs a) {
    constexpr int kQ = NT_REG > 0 ? 16 * NT_REG : 4 * kMaxS;
    __shared__ __attribute__((aligned(16))) float sq[kQ];
    __shared__ __attribute__((aligned(16))) float sx[4][64 * 4];
    __shared__ uint32_t sword[4][64];   // the group's packed index words, per wave
    __shared__ uint32_t shist[MED ? 2048 : 1];
    __shared__ uint32_t sh[kEncThreads / 64 + 3];

    const TileCoords tc = tile_coords(a);
    const int64_t slice = tc.slice;
    const int64_t c_begin = tc.c_begin;
    const int64_t c_end = tc.c_end;
    const int NT = NT_REG > 0 ? NT_REG : a.NT;

    {
        const float *q = a.cb + slice * a.S * 4;
        const int nq = 16 * NT;
        for (int i = threadIdx.x; i < nq; i += kEncThreads) sq[i] = i < 4 * a.S ? double_f16(q[i]) : 0.0f;
        if constexpr (MED)
            for (int i = threadIdx.x; i < 2048; i += kEncThreads) shist[i] = 0;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;          // MFMA k (B row / A column) and D row block
    const int row = lane & 15;          // MFMA A row i = 4 s_local + m, B/D column
    const int m_row = row & 3;
    const int s_loc = row >> 2;
    const bool neg = (kNegMask >> (4 * m_row + grp)) & 1u;
    const int a_off = 4 * s_loc + (m_row ^ grp);

    float A[NT_REG > 0 ? NT_REG : 1];
    if constexpr (NT_REG > 0) {
#pragma unroll
        for (int t = 0; t < NT_REG; ++t) {
            const float v = sq[16 * t + a_off];
            A[t] = neg ? -v : v;
        }
    }

    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // packing: lane w < wpg stores word ww of token row tt of the group
    const int wpg = (64 >> a.log2_cpt) * a.words;
    const int p_tt = lane / a.words;
    const int p_ww = lane - p_tt * a.words;
    uint32_t *idx_slice = a.idx + slice * a.tokens * a.words;

    for (int64_t g0 = c_begin + 64 * wave; g0 < c_end; g0 += 64 * 4) {
        const int64_t c = g0 + lane;
        const bool valid = c < c_end;
        const int64_t gc = slice * a.n_slice + c;

        float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f, v3 = 0.0f;
        if (valid) {
            if constexpr (F32IN) {
                const float4 f = static_cast<const float4 *>(a.x)[gc];
                v0 = f.x; v1 = f.y; v2 = f.z; v3 = f.w;
            } else {
                const uint2 r = static_cast<const uint2 *>(a.x)[gc];
                v0 = f16_bits_to_f32(static_cast<uint16_t>(r.x));
                v1 = f16_bits_to_f32(static_cast<uint16_t>(r.x >> 16));
                v2 = f16_bits_to_f32(static_cast<uint16_t>(r.y));
                v3 = f16_bits_to_f32(static_cast<uint16_t>(r.y >> 16));
            }
        }

        // declared fp32 squared norm and its binary16 half-norm code
        float s2 = v0 * v0;
        s2 = __builtin_fmaf(v1, v1, s2);
        s2 = __builtin_fmaf(v2, v2, s2);
        s2 = __builtin_fmaf(v3, v3, s2);
        const uint16_t hn = half_norm_code(s2);

        // fp32 inputs: exact power-of-two normalisation for the search (the
        // argmax is scale-invariant; keeps every product far from the
        // denormal range).  fp16 inputs are at least 2^-24 and need none.
        float x0 = v0, x1 = v1, x2 = v2, x3 = v3;
        if constexpr (F32IN) {
            const float mx = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
            const int ex = mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) : 0;
            x0 = __builtin_ldexpf(v0, -ex);
            x1 = __builtin_ldexpf(v1, -ex);
            x2 = __builtin_ldexpf(v2, -ex);
            x3 = __builtin_ldexpf(v3, -ex);
        }
        *reinterpret_cast<float4 *>(&sx[wave][4 * lane]) = make_float4(x0, x1, x2, x3);
        wave_sync();

        float bsc[4];
        int bsi[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float bv = sx[wave][4 * (16 * b + row) + grp];
            float best = -1.0f;
            int bt = 0;
            if constexpr (NT_REG > 0) {
#pragma unroll
                for (int t = 0; t < NT_REG; ++t) {
                    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(A[t], bv, zero, 0, 0, 0);
                    const float sc = best_primary(d);
                    if (sc > best) { best = sc; bt = t; }
                }
            } else {
                for (int t = 0; t < NT; ++t) {
                    const float v = sq[16 * t + a_off];
                    const float at = neg ? -v : v;
                    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(at, bv, zero, 0, 0, 0);
                    const float sc = best_primary(d);
                    if (sc > best) { best = sc; bt = t; }
                }
            }
            bsc[b] = best;
            bsi[b] = 4 * bt + grp;
        }

        // Transposed reduction over the 4 lane groups: afterwards lane l holds
        // the best (score, s) of chunk g0 + l over all S.
        float m1s[2];
        int m1i[2];
        const bool h1 = (lane >> 5) & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float ss = h1 ? bsc[j] : bsc[2 + j];
            const int si = h1 ? bsi[j] : bsi[2 + j];
            float ks = h1 ? bsc[2 + j] : bsc[j];
            int ki = h1 ? bsi[2 + j] : bsi[j];
            const float rs = __shfl_xor(ss, 32);
            const int ri = __shfl_xor(si, 32);
            if (better(rs, ri, ks, ki)) { ks = rs; ki = ri; }
            m1s[j] = ks;
            m1i[j] = ki;
        }
        const bool h0 = (lane >> 4) & 1;
        int s_best;
        {
            const float ss = h0 ? m1s[0] : m1s[1];
            const int si = h0 ? m1i[0] : m1i[1];
            float ks = h0 ? m1s[1] : m1s[0];
            int ki = h0 ? m1i[1] : m1i[0];
            const float rs = __shfl_xor(ss, 16);
            const int ri = __shfl_xor(si, 16);
            if (better(rs, ri, ks, ki)) { ks = rs; ki = ri; }
            s_best = min(ki, 4 * NT - 1);
        }

        const uint32_t code = s2 > 0.0f ? static_cast<uint32_t>(24 * s_best + primary_index(&sq[4 * s_best], x0, x1, x2, x3)) : 0u;

        if (valid) {
            a.hnorm[gc] = hn;
            if constexpr (MED) atomicAdd(&shist[hn >> 4], 1u);
        }
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
            const int64_t tok = (g0 >> a.log2_cpt) + p_tt;
            if ((tok << a.log2_cpt) < c_end) idx_slice[tok * a.words + p_ww] = sword[wave][lane];
        }
        wave_sync();
    }
    if constexpr (MED) med3_after_tile(a, tc, shist, sh);
}

// --------------------------------------------------------------------------
// Block-wide exclusive scan (all threads of the block must call it).
// --------------------------------------------------------------------------
template <typename T, int NTHREADS>
__device__ __forceinline__ T block_exclusive_scan(T v, T *total, T *sh) {
    constexpr int kWaves = NTHREADS / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    T incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const T o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        T run = 0;
        for (int w = 0; w < kWaves; ++w) {
            const T t = sh[w];
            sh[w] = run;
            run += t;
        }
        sh[kWaves] = run;
    }
    __syncthreads();
    const T res = sh[wave] + incl - v;
    *total = sh[kWaves];
    __syncthreads();
    return res;
}

// --------------------------------------------------------------------------
// Med3x.  The batch's median is the exact lower median of its fp32 squared
// norms s2 (rank floor((n-1)/2)); outliers are the chunks with
// s2 > fl(fl(C*C) * median) (r > C r_med, strict).
//
// The stored half-norm code h(s2) = fp16_rn(sqrt_rn(s2) / 2) is monotone in
// s2, so ranks by s2 refine ranks by h: h_a < h_b implies s2_a < s2_b.  The
// search kernel histograms h >> 4 per batch; the select kernel finds the
// median's code h_med and its rank among the chunks with that code, then the
// exact s2 median among those few chunks (s2 recomputed from x with the same
// declared fp32 operations); a chunk is an outlier if h > h(thr), or if
// h == h(thr) and its exact s2 > thr.
// --------------------------------------------------------------------------

constexpr int kSelThreads = 512;
constexpr int kCandCap = 4096;

struct SelArgs {
    const void *x;
    uint16_t *hnorm;        // read; the single-pass select also sets outlier flags
    const uint32_t *hist;   // [nbatch][2048] counts of h >> 4
    uint32_t *counts;       // [nbatch]
    uint32_t *mask;         // [nbatch][mask_words]
    int64_t mask_words;
    int64_t n_slice;
    int64_t batch_chunks;
    int64_t bps;
    float C;
    int32_t f32;
    // packed norm format, single-pass select: the select packs its batch's
    // final codes into the record's norm words (nullptr: a separate pass does)
    uint32_t *pwords;       // [slices][tokens][words]
    int64_t tokens;
    int32_t log2_cpt, bits, words;
};

// Declared fp32 squared norm of chunk gc (the search kernel's operations).
__device__ __forceinline__ float chunk_s2(const SelArgs &a, int64_t gc) {
    float v0, v1, v2, v3;
    if (a.f32) {
        const float4 f = static_cast<const float4 *>(a.x)[gc];
        v0 = f.x; v1 = f.y; v2 = f.z; v3 = f.w;
    } else {
        const uint2 r = static_cast<const uint2 *>(a.x)[gc];
        v0 = f16_bits_to_f32(static_cast<uint16_t>(r.x));
        v1 = f16_bits_to_f32(static_cast<uint16_t>(r.x >> 16));
        v2 = f16_bits_to_f32(static_cast<uint16_t>(r.y));
        v3 = f16_bits_to_f32(static_cast<uint16_t>(r.y >> 16));
    }
    float s2 = v0 * v0;
    s2 = __builtin_fmaf(v1, v1, s2);
    s2 = __builtin_fmaf(v2, v2, s2);
    s2 = __builtin_fmaf(v3, v3, s2);
    return s2;
}

// Digit of rank k in hist[0 .. nbins) (nbins a multiple of the block size or
// smaller than it): found[0] = digit, found[1] = rank within it.  All
// threads of the block must call it.
__device__ void select_digit(const uint32_t *hist, int nbins, uint32_t k, uint32_t *found, uint32_t *sh) {
    const int per = nbins >= kSelThreads ? nbins / kSelThreads : 1;
    const int first = threadIdx.x * per;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j)
        if (first + j < nbins) local += hist[first + j];
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<uint32_t, kSelThreads>(local, &tot, sh);
    if (k >= ex && k < ex + local) {
        uint32_t cum = ex;
        for (int j = 0; j < per; ++j) {
            const uint32_t h = hist[first + j];
            if (k < cum + h) {
                found[0] = static_cast<uint32_t>(first + j);
                found[1] = k - cum;
                break;
            }
            cum += h;
        }
    }
    __syncthreads();
}

// The k-th smallest (0-based) of the fp32 values s2 of the chunks of the
// batch whose code equals hsel, by three radix digits of the bit pattern.
// Values come from vals[0 .. m) in LDS when vals != nullptr, otherwise they
// are recomputed from x in passes over the batch.
__device__ float kth_s2(const SelArgs &a, const uint16_t *codes, int64_t gbase, int64_t n, uint32_t hsel,
                        const float *vals, uint32_t m, uint32_t k, uint32_t *hist, uint32_t *found,
                        uint32_t *sh) {
    const int shifts[3] = {20, 9, 0};
    const int widths[3] = {11, 11, 9};
    uint32_t prefix = 0;
    for (int d = 0; d < 3; ++d) {
        const int shift = shifts[d], width = widths[d], above = shift + width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = threadIdx.x; i < (1 << width); i += kSelThreads) hist[i] = 0;
        __syncthreads();
        if (vals) {
            for (uint32_t i = threadIdx.x; i < m; i += kSelThreads) {
                const uint32_t key = __float_as_uint(vals[i]);
                if ((key >> above) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
        } else {
            for (int64_t i = threadIdx.x; i < n; i += kSelThreads) {
                // (a flag set by the single-pass select is not part of the code)
                if ((codes[i] & 0x7FFFu) != hsel) continue;
                const uint32_t key = __float_as_uint(chunk_s2(a, gbase + i));
                if ((key >> above) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        select_digit(hist, 1 << width, k, found, sh);
        prefix = (prefix << width) | found[0];
        k = found[1];
        __syncthreads();
    }
    return __uint_as_float(prefix);
}

__global__ __launch_bounds__(kSelThreads) void med3_select_kernel(SelArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t cand[kCandCap];
    __shared__ float candv[kCandCap];
    __shared__ uint32_t sh[kSelThreads / 64 + 4];
    uint32_t *found = sh + kSelThreads / 64 + 1;

    const int64_t bid = blockIdx.x;
    const int64_t slice = bid / a.bps;
    const int64_t lo = (bid - slice * a.bps) * a.batch_chunks;
    const int64_t n = min(a.batch_chunks, a.n_slice - lo);
    const int64_t gbase = slice * a.n_slice + lo;
    const uint16_t *codes = a.hnorm + gbase;
    const uint32_t k = static_cast<uint32_t>((n - 1) / 2);

    // code bits 14..4 (bit 15 is 0 before outliers are flagged)
    const uint32_t *gh = a.hist + bid * 2048;
    for (int i = threadIdx.x; i < 2048; i += kSelThreads) hist[i] = gh[i];
    __syncthreads();
    select_digit(hist, 2048, k, found, sh);
    const uint32_t d1 = found[0];
    const uint32_t k1 = found[1];
    const uint32_t m1 = hist[d1];
    __syncthreads();

    // code bits 3..0 among the chunks of digit d1; their positions are kept
    // in LDS when they fit
    const bool keep = m1 <= static_cast<uint32_t>(kCandCap);
    if (threadIdx.x < 16) hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) sh[kSelThreads / 64 + 3] = 0;
    __syncthreads();
    {
        // 4 codes per 8-byte load (a batch starts at a multiple of 4 chunks)
        const uint2 *c4 = reinterpret_cast<const uint2 *>(codes);
        const int64_t n4 = n >> 2;
        constexpr int U = 8;
        for (int64_t i0 = threadIdx.x; i0 < n4; i0 += static_cast<int64_t>(kSelThreads) * U) {
            uint2 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + static_cast<int64_t>(u) * kSelThreads;
                v[u] = i < n4 ? c4[i] : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + static_cast<int64_t>(u) * kSelThreads;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = e < 2 ? v[u].x : v[u].y;
                    const uint32_t c = (w >> (16 * (e & 1))) & 0xFFFFu;
                    if ((c >> 4) != d1 || i >= n4) continue;
                    atomicAdd(&hist[c & 15u], 1u);
                    if (keep) {
                        const uint32_t slot = atomicAdd(&sh[kSelThreads / 64 + 3], 1u);
                        if (slot < static_cast<uint32_t>(kCandCap)) cand[slot] = static_cast<uint32_t>(4 * i + e);
                    }
                }
            }
        }
        for (int64_t i = 4 * n4 + threadIdx.x; i < n; i += kSelThreads) {
            const uint32_t c = codes[i];
            if ((c >> 4) != d1) continue;
            atomicAdd(&hist[c & 15u], 1u);
            if (keep) {
                const uint32_t slot = atomicAdd(&sh[kSelThreads / 64 + 3], 1u);
                if (slot < static_cast<uint32_t>(kCandCap)) cand[slot] = static_cast<uint32_t>(i);
            }
        }
    }
    __syncthreads();
    select_digit(hist, 16, k1, found, sh);
    const uint32_t hmed = (d1 << 4) | found[0];
    const uint32_t k2 = found[1];
    __syncthreads();

    // exact s2 of the chunks with code hmed, then the k2-th smallest
    float med;
    if (keep) {
        if (threadIdx.x == 0) sh[kSelThreads / 64 + 3] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < m1; i += kSelThreads) {
            const uint32_t off = min(cand[i], static_cast<uint32_t>(n - 1));
            if ((codes[off] & 0x7FFFu) == hmed) {
                const uint32_t slot = atomicAdd(&sh[kSelThreads / 64 + 3], 1u);
                if (slot < static_cast<uint32_t>(kCandCap)) candv[slot] = chunk_s2(a, gbase + off);
            }
        }
        __syncthreads();
        const uint32_t m2 = min(sh[kSelThreads / 64 + 3], static_cast<uint32_t>(kCandCap));
        __syncthreads();
        med = kth_s2(a, codes, gbase, n, hmed, candv, m2, k2, hist, found, sh);
    } else {
        med = kth_s2(a, codes, gbase, n, hmed, nullptr, 0, k2, hist, found, sh);
    }
    const float cc = a.C * a.C;
    const float thr = cc * med;
    const uint32_t hthr = half_norm_code(thr);

    // outlier bitmask: wave w ballots 64 consecutive chunks at a time, eight
    // groups per iteration in flight
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t *mrow = a.mask + bid * a.mask_words;
    uint32_t cnt = 0;
    constexpr int U = 8;
    constexpr int kWv = kSelThreads / 64;
    for (int64_t g0 = 64 * wave; g0 < n; g0 += 64 * kWv * U) {
        uint32_t cv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = g0 + 64 * kWv * u + lane;
            cv[u] = i < n ? codes[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t gb = g0 + 64 * kWv * u;
            const int64_t i = gb + lane;
            bool f = i < n && cv[u] > hthr;
            if (i < n && cv[u] == hthr) f = chunk_s2(a, gbase + i) > thr;
            const uint64_t m = __ballot(f);
            if (gb < n && lane < 2) mrow[(gb >> 5) + lane] = static_cast<uint32_t>(m >> (32 * lane));
            cnt += lane == 0 ? static_cast<uint32_t>(__popcll(m)) : 0u;
        }
    }
    uint32_t tot;
    block_exclusive_scan<uint32_t, kSelThreads>(cnt, &tot, sh);
    if (threadIdx.x == 0) a.counts[bid] = tot;
}

// Single-pass select for batches of at most kSel1MaxChunks chunks.  The
// median's top bin d1 (from the search kernel's histogram) bounds the median
// s2 to [4 v(16 d1 - 1)^2, 4 v(16 d1 + 16)^2] (v the binary16 value of a
// code: the half-norm of any s2 with a code in the bin lies strictly between
// the neighbouring codes' values), hence the threshold code to [hlo, hhi]
// (the code is monotone in s2).  One read of the batch's codes then (1)
// refines the median as before (low 4 bits, candidate positions), (2) flags
// every code above hhi as an outlier (bitmask bit, bit 15 in hnorm) and
// (3) keeps the positions of codes in [hlo, hhi]; once the exact threshold
// is known those are decided exactly (s2 recomputed where the code equals
// the threshold's).  Bits are ORed into the batch's bitmask, which the
// encode call zeroes together with the histograms.  The decisions are the two-pass kernel's.  If the
// undecided list overflows, one more pass decides the codes in [hlo, hhi].
// A batch is a whole number of token rows (n a multiple of 4).
constexpr int kSel1MaxChunks = 131072;
constexpr int kCand1Cap = 3000;
constexpr int kUnc1Cap = 2048;
// listed loads whose 8 bytes the single-pass select keeps in LDS, per wave:
// 12 KB of their own (with the other arrays 52.7 KB, 3 blocks per CU, which
// the kernel's 74 VGPRs allow anyway) plus the histogram's bins 16..2047
constexpr uint32_t kValPerWave = 192;
constexpr uint32_t kHistVal = (2048 - 16) / 2 / (kSelThreads / 64);

__global__ __launch_bounds__(kSelThreads) void med3_select1_kernel(SelArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t cand[kCand1Cap];
    __shared__ float candv[kCand1Cap];
    __shared__ uint32_t unc[kUnc1Cap];
    __shared__ uint2 lval[kSelThreads / 64 * kValPerWave];
    __shared__ uint32_t sh[kSelThreads / 64 + 6];
    uint32_t *found = sh + kSelThreads / 64 + 1;
    uint32_t *ncand = sh + kSelThreads / 64 + 3;
    uint32_t *nunc = sh + kSelThreads / 64 + 4;
    uint32_t *nout = sh + kSelThreads / 64 + 5;

    const int64_t bid = blockIdx.x;
    const int64_t slice = bid / a.bps;
    const int64_t lo = (bid - slice * a.bps) * a.batch_chunks;
    const int n = static_cast<int>(min(a.batch_chunks, a.n_slice - lo));
    const int64_t gbase = slice * a.n_slice + lo;
    uint16_t *codes = a.hnorm + gbase;
    const uint32_t k = static_cast<uint32_t>((n - 1) / 2);

    const uint32_t *gh = a.hist + bid * 2048;
    for (int i = threadIdx.x; i < 2048; i += kSelThreads) hist[i] = gh[i];
    __syncthreads();
    select_digit(hist, 2048, k, found, sh);
    const uint32_t d1 = found[0];
    const uint32_t k1 = found[1];
    const uint32_t m1 = hist[d1];
    __syncthreads();

    // threshold code bounds from the median's bin
    const float cc = a.C * a.C;
    const uint32_t cl = d1 << 4, ch = cl | 15u;
    const float vlo = cl > 0 ? f16_bits_to_f32(static_cast<uint16_t>(cl - 1)) : 0.0f;
    const float vhi = f16_bits_to_f32(static_cast<uint16_t>(ch + 1 < 0x7C00u ? ch + 1 : 0x7BFFu));
    const uint32_t hlo = half_norm_code(cc * (4.0f * vlo * vlo));
    const uint32_t hhi = ch + 1 < 0x7C00u ? half_norm_code(cc * (4.0f * vhi * vhi)) : 0x7FFFu;

    const bool keep = m1 <= static_cast<uint32_t>(kCand1Cap);
    if (threadIdx.x < 16) hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) { *ncand = 0; *nunc = 0; *nout = 0; }
    __syncthreads();

    // the one pass over the batch's codes, 4 codes per 8-byte load (a batch
    // is a whole number of token rows, so n is a multiple of 4), eight loads
    // per thread in flight, without per-code branches:
    //  - definite outliers (code > hhi) are flagged with packed 16-bit
    //    arithmetic; the 8 lanes holding one bitmask word (32 chunks) combine
    //    their nibbles by DPP and, when any is set, store the word (the mask
    //    is zeroed before the search and no other thread writes it here);
    //    a lane holding a flagged code writes its 8 bytes back with the
    //    flags set (not the whole line: on K, with its outliers in a few
    //    channels, 38% fewer bytes written);
    //  - loads holding a code of the median's bin or an undecided code (in
    //    [hlo, hhi]), about 1% of them, are listed per wave in LDS (no
    //    atomics: the wave's count is uniform) and visited in a second step.
    uint32_t *mrow = a.mask + bid * a.mask_words;
    uint32_t cnt = 0;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    constexpr int kWaves = kSelThreads / 64;
    constexpr uint32_t kEntPerWave = kCand1Cap / kWaves;
    // the lists use candv, which is free until the median step below; the
    // values of a wave's first kValPerWave listed loads are kept in lval, the
    // next kHistVal in the histogram's bins 16.. (unused from here until the
    // second step has read them), and later ones are re-read from memory
    uint32_t *ent = reinterpret_cast<uint32_t *>(candv);
    uint2 *hval = reinterpret_cast<uint2 *>(hist + 16);
    uint32_t went = 0;
    uint2 *c4 = reinterpret_cast<uint2 *>(codes);
    const int n4 = n >> 2;
    {
        const u16x2 v_hhi = {static_cast<uint16_t>(hhi), static_cast<uint16_t>(hhi)};
        const u16x2 v_7fff = {0x7FFFu, 0x7FFFu};
        const u16x2 v_cl = {static_cast<uint16_t>(cl), static_cast<uint16_t>(cl)};
        const u16x2 v_hlo = {static_cast<uint16_t>(hlo), static_cast<uint16_t>(hlo)};
        const uint32_t band_w = hhi - hlo;   // hlo <= hhi: vlo < vhi
        const uint32_t wshift = 4u * static_cast<uint32_t>(lane & 7);
        constexpr int U = 8;
        for (int i0 = threadIdx.x; i0 - lane < n4; i0 += kSelThreads * U) {
            // loads issued unconditionally (lanes past the batch read its
            // last word and then hold zeros); the empty asm consumes each
            // word where it is first used, so that the loads stay
            // unconditional and each u waits for its own load only
            uint2 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = i0 + kSelThreads * u;
                v[u] = c4[q < n4 ? q : n4 - 1];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = i0 + kSelThreads * u;
                const bool valid = q < n4;
                {
                    uint32_t vx = v[u].x, vy = v[u].y;
                    asm volatile("" : "+v"(vx), "+v"(vy));
                    v[u] = valid ? make_uint2(vx, vy) : make_uint2(0u, 0u);
                }
                const u16x2 wx = __builtin_bit_cast(u16x2, v[u].x);
                const u16x2 wy = __builtin_bit_cast(u16x2, v[u].y);
                // bit 15 of each halfword set iff its code exceeds hhi
                const uint32_t fx = __builtin_bit_cast(uint32_t, __builtin_elementwise_add_sat(
                                        __builtin_elementwise_sub_sat(wx, v_hhi), v_7fff)) & 0x80008000u;
                const uint32_t fy = __builtin_bit_cast(uint32_t, __builtin_elementwise_add_sat(
                                        __builtin_elementwise_sub_sat(wy, v_hhi), v_7fff)) & 0x80008000u;
                const uint32_t t = (fx >> 15) | (fy >> 13);       // codes 0, 2 at bits 0, 2; 1, 3 at 16, 18
                const uint32_t nib = (t | (t >> 15)) & 15u;
                // q & 7 == lane & 7: lanes 8 j .. 8 j + 7 hold the word's 8 nibbles
                uint32_t wv = nib << wshift;
                wv |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(wv), 0xB1, 0xF, 0xF, false));
                wv |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(wv), 0x4E, 0xF, 0xF, false));
                wv |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(wv), 0x141, 0xF, 0xF, false));
                // a group's lanes past the batch's end (n4 need not be a
                // multiple of 8) hold no codes: they write nothing; lane 8 j
                // is valid whenever any lane of its group is
                if (wv != 0u) {
                    if ((lane & 7) == 0) mrow[q >> 3] = wv;
                    if (valid) {
                        cnt += static_cast<uint32_t>(__popc(nib));
                        if (nib) c4[q] = make_uint2(v[u].x | fx, v[u].y | fy);
                    }
                }
                // median's bin: (c - cl) mod 2^16 < 16; undecided: (c - hlo) mod 2^16 <= hhi - hlo
                const u16x2 tm = __builtin_elementwise_min(wx - v_cl, wy - v_cl);
                const u16x2 tb = __builtin_elementwise_min(wx - v_hlo, wy - v_hlo);
                const bool listed = valid && (min(static_cast<uint32_t>(tm.x), static_cast<uint32_t>(tm.y)) < 16u ||
                                              min(static_cast<uint32_t>(tb.x), static_cast<uint32_t>(tb.y)) <= band_w);
                const uint64_t bal = __ballot(listed);
                if (bal != 0u) {
                    const uint32_t slot = went + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                                           __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
                    if (listed && slot < kEntPerWave) {
                        ent[wave * kEntPerWave + slot] = static_cast<uint32_t>(q);
                        if (slot < kValPerWave) lval[wave * kValPerWave + slot] = v[u];
                        else if (slot < kValPerWave + kHistVal) hval[wave * kHistVal + (slot - kValPerWave)] = v[u];
                    }
                    went += static_cast<uint32_t>(__popcll(bal));
                }
            }
        }
    }
    if (lane == 0) unc[kUnc1Cap - kWaves + wave] = went;   // the lists' lengths, read below
    __syncthreads();
    uint32_t wcnt[kWaves];
    bool overflow = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        wcnt[w] = unc[kUnc1Cap - kWaves + w];
        overflow |= wcnt[w] > kEntPerWave;
    }
    __syncthreads();

    // second step: the codes of the listed loads (or, if a list overflowed,
    // of the whole batch): the median bin's sub-histogram and candidates,
    // and the undecided codes
    auto visit = [&](int i, uint32_t c) {
        // a code re-read from memory may carry the flag the pass above set
        // (with C < 1 even a code of the median's bin exceeds hhi): the
        // median and the undecided band are about the code without it
        c &= 0x7FFFu;
        // positions (< 2^17) keep their code's low bits beside them, so the
        // later phases read no code back from HBM
        if ((c >> 4) == d1) {
            atomicAdd(&hist[c & 15u], 1u);
            if (keep) {
                const uint32_t slot = atomicAdd(ncand, 1u);
                if (slot < static_cast<uint32_t>(kCand1Cap))
                    cand[slot] = (static_cast<uint32_t>(i) << 4) | (c & 15u);
            }
        }
        // (both when the median's bin starts at 0: then hlo = 0; a code above
        // hhi is a definite outlier, flagged and counted by the pass)
        if (c >= hlo && c <= hhi) {
            const uint32_t slot = atomicAdd(nunc, 1u);
            if (slot < static_cast<uint32_t>(kUnc1Cap - kWaves))
                unc[slot] = (static_cast<uint32_t>(i) << 15) | (c - hlo);
        }
    };
    if (!overflow) {
        uint32_t total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += wcnt[w];
        for (uint32_t j0 = threadIdx.x; j0 < total; j0 += 4 * kSelThreads) {
            int qs[4];
            uint2 vs[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t j = j0 + r * kSelThreads, w = 0;
                while (w + 1 < kWaves && j >= wcnt[w]) j -= wcnt[w++];
                qs[r] = j0 + r * kSelThreads < total ? static_cast<int>(ent[w * kEntPerWave + j]) : -1;
                vs[r] = make_uint2(0u, 0u);
                if (qs[r] >= 0) {
                    if (j < kValPerWave) vs[r] = lval[w * kValPerWave + j];
                    else if (j < kValPerWave + kHistVal) vs[r] = hval[w * kHistVal + (j - kValPerWave)];
                    else vs[r] = c4[qs[r]];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (qs[r] < 0) continue;
                visit(4 * qs[r], vs[r].x & 0xFFFFu);
                visit(4 * qs[r] + 1, vs[r].x >> 16);
                visit(4 * qs[r] + 2, vs[r].y & 0xFFFFu);
                visit(4 * qs[r] + 3, vs[r].y >> 16);
            }
        }
    } else {
        for (int i = threadIdx.x; i < n; i += kSelThreads) visit(i, codes[i]);
    }
    __syncthreads();
    select_digit(hist, 16, k1, found, sh);
    const uint32_t hmed = (d1 << 4) | found[0];
    const uint32_t k2 = found[1];
    __syncthreads();

    // exact median among the chunks with code hmed (their positions and
    // unflagged low code bits are in cand)
    float med;
    if (keep) {
        if (threadIdx.x == 0) *ncand = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < m1; i += kSelThreads) {
            const uint32_t off = min(cand[i] >> 4, static_cast<uint32_t>(n - 1));
            if ((cand[i] & 15u) == (hmed & 15u)) {
                const uint32_t slot = atomicAdd(ncand, 1u);
                if (slot < static_cast<uint32_t>(kCand1Cap)) candv[slot] = chunk_s2(a, gbase + off);
            }
        }
        __syncthreads();
        const uint32_t m2 = min(*ncand, static_cast<uint32_t>(kCand1Cap));
        __syncthreads();
        if (m2 <= 256) {
            // few values: the k2-th smallest directly, by counting for each
            // value those below it and those not above it
            float *res = reinterpret_cast<float *>(found);
            if (threadIdx.x == 0) *res = candv[0];
            __syncthreads();
            if (threadIdx.x < m2) {
                const float v = candv[threadIdx.x];
                uint32_t below = 0, upto = 0;
                for (uint32_t j = 0; j < m2; ++j) {
                    const float w = candv[j];
                    below += w < v ? 1u : 0u;
                    upto += w <= v ? 1u : 0u;
                }
                if (below <= k2 && k2 < upto) *res = v;
            }
            __syncthreads();
            med = *res;
            __syncthreads();
        } else {
            med = kth_s2(a, codes, gbase, n, hmed, candv, m2, k2, hist, found, sh);
        }
    } else {
        med = kth_s2(a, codes, gbase, n, hmed, nullptr, 0, k2, hist, found, sh);
    }
    const float thr = cc * med;
    const uint32_t hthr = half_norm_code(thr);

    // the undecided codes in [hlo, hhi]
    auto decide = [&](int i, uint32_t c) {
        if (c > hthr || (c == hthr && chunk_s2(a, gbase + i) > thr)) {
            atomicOr(&mrow[i >> 5], 1u << (i & 31));
            codes[i] = static_cast<uint16_t>(c | 0x8000u);
            atomicAdd(nout, 1u);
        }
    };
    const uint32_t nu = *nunc;
    if (nu <= static_cast<uint32_t>(kUnc1Cap - kSelThreads / 64)) {
        for (uint32_t j = threadIdx.x; j < nu; j += kSelThreads) {
            const int i = static_cast<int>(unc[j] >> 15);
            decide(i, hlo + (unc[j] & 0x7FFFu));
        }
    } else {
        for (int i = threadIdx.x; i < n; i += kSelThreads) {
            const uint32_t c = codes[i];
            if (c >= hlo && c <= hhi) decide(i, c);
        }
    }
    uint32_t tot;
    block_exclusive_scan<uint32_t, kSelThreads>(cnt, &tot, sh);
    if (threadIdx.x == 0) a.counts[bid] = tot + *nout;

    // packed norm format: the batch's codes are final now (flags included),
    // so pack them into the record's norm words here, in rounds of up to
    // 3 x 2048 chunks (whole token rows; as many as the LDS word buffer
    // holds, at least two: 2048 chunks take at most 2048 * 15 / 32 + 512
    // words) with the words ORed together in LDS; a thread's loads of a round
    // are issued together, before the round's first barrier
    if (a.pwords != nullptr) {
        __syncthreads();   // every decision has been written to codes[]
        uint32_t *sw = cand;
        const int cpt = 1 << a.log2_cpt;
        const int W = a.words;
        uint32_t *out = a.pwords + (slice * a.tokens + (lo >> a.log2_cpt)) * W;
        constexpr int kSub = 4 * kSelThreads;   // chunks per sub-round, one load per thread
        const int nsub = min(3, kCand1Cap / ((kSub >> a.log2_cpt) * W));
        const int round = nsub * kSub;
        for (int r0 = 0; r0 < n; r0 += round) {
            const int rows = min(round, n - r0) >> a.log2_cpt;
            for (int i = threadIdx.x; i < rows * W; i += kSelThreads) sw[i] = 0u;
            uint2 u[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int c = r0 + kSub * j + 4 * static_cast<int>(threadIdx.x);
                u[j] = j < nsub && c < n ? *reinterpret_cast<const uint2 *>(codes + c) : make_uint2(0u, 0u);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int c = r0 + kSub * j + 4 * static_cast<int>(threadIdx.x);
                if (j < nsub && c < n) {   // n and c are multiples of 4
                    const uint32_t h[4] = {u[j].x & 0xFFFFu, u[j].x >> 16, u[j].y & 0xFFFFu, u[j].y >> 16};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int lc = c - r0 + e;
                        const uint32_t code = compact_norm_code(h[e], a.bits);
                        const int bit = (lc & (cpt - 1)) * a.bits;
                        uint32_t *wr = &sw[(lc >> a.log2_cpt) * W + (bit >> 5)];
                        const int sft = bit & 31;
                        atomicOr(wr, code << sft);
                        if (sft + a.bits > 32) atomicOr(wr + 1, code >> (32 - sft));
                    }
                }
            }
            __syncthreads();
            uint32_t *dst = out + (r0 >> a.log2_cpt) * W;
            for (int i = threadIdx.x; i < rows * W; i += kSelThreads) dst[i] = sw[i];
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(kScanThreads) void med3_scan_kernel(int64_t nb, const uint32_t *counts,
                                                                 uint64_t *offsets, uint64_t capacity,
                                                                 uint64_t *status) {
    __shared__ uint64_t sh[kScanThreads / 64 + 1];
    uint64_t carry = 0;
    for (int64_t base = 0; base < nb; base += kScanThreads) {
        const int64_t i = base + threadIdx.x;
        const uint64_t v = i < nb ? counts[i] : 0;
        uint64_t tot;
        const uint64_t ex = block_exclusive_scan<uint64_t, kScanThreads>(v, &tot, sh);
        if (i < nb) offsets[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) {
        offsets[nb] = carry;
        if (status) {
            status[0] = carry;
            status[1] = carry > capacity ? 1u : 0u;
        }
    }
}

struct GatherArgs {
    const void *x;
    const uint32_t *mask;
    const uint64_t *offsets;
    uint16_t *hnorm;
    uint32_t *out_pos;
    uint16_t *out_val;
    uint64_t capacity;
    int64_t n_slice;
    int64_t batch_chunks;
    int64_t bps;
    int64_t mask_words;
    int32_t f32;
    int32_t set_flags;   // 0 when the select kernel has already flagged hnorm
};

// Ordered outlier write: one block per batch walks the batch's bitmask, 256
// words (8192 chunks) per round with the next round's words already in
// flight; a block-wide scan of the words' popcounts places each outlier's
// chunk offset in an LDS list in position order.  The list is written out
// when the next round might not fit and at the end: every thread then loads
// the inputs of four entries before storing any, so a batch's side-list
// writes wait on a few rounds of loads rather than one per outlier.
constexpr int kGatherList = 32 * kFlagThreads;   // one round's worth of entries

__global__ __launch_bounds__(kFlagThreads) void med3_gather_kernel(GatherArgs a) {
    __shared__ uint32_t sh[kFlagThreads / 64 + 1];
    __shared__ uint32_t list[kGatherList];
    const int64_t bid = blockIdx.x;
    const int64_t slice = bid / a.bps;
    const int64_t lo = (bid - slice * a.bps) * a.batch_chunks;
    const int64_t n = min(a.batch_chunks, a.n_slice - lo);
    const int64_t nw = (n + 31) >> 5;
    const int64_t bbase = slice * a.n_slice + lo;   // the batch's first chunk
    const uint32_t *mrow = a.mask + bid * a.mask_words;
    uint64_t running = a.offsets[bid];
    uint32_t fill = 0;   // list entries not yet written (uniform)

    auto flush = [&]() {
        constexpr int U = 4;
        for (uint32_t i0 = threadIdx.x; i0 < fill; i0 += kFlagThreads * U) {
            uint32_t cs[U];
            uint2 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + kFlagThreads * u;
                cs[u] = i < fill ? list[i] : 0u;
                v[u] = make_uint2(0u, 0u);
                if (i < fill) {
                    if (a.f32) {
                        const float4 xf = static_cast<const float4 *>(a.x)[bbase + cs[u]];
                        v[u].x = static_cast<uint32_t>(f32_to_f16_bits(xf.x)) |
                                 (static_cast<uint32_t>(f32_to_f16_bits(xf.y)) << 16);
                        v[u].y = static_cast<uint32_t>(f32_to_f16_bits(xf.z)) |
                                 (static_cast<uint32_t>(f32_to_f16_bits(xf.w)) << 16);
                    } else {
                        v[u] = static_cast<const uint2 *>(a.x)[bbase + cs[u]];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + kFlagThreads * u;
                if (i >= fill) continue;
                const uint64_t pos = running + i;
                if (pos < a.capacity) {
                    a.out_pos[pos] = static_cast<uint32_t>(lo + cs[u]);
                    reinterpret_cast<uint2 *>(a.out_val)[pos] = v[u];
                }
                if (a.set_flags) a.hnorm[bbase + cs[u]] = static_cast<uint16_t>(a.hnorm[bbase + cs[u]] | 0x8000u);
            }
        }
        running += fill;
        fill = 0;
        __syncthreads();   // the list is refilled next
    };

    uint32_t next = threadIdx.x < nw ? mrow[threadIdx.x] : 0u;
    for (int64_t w0 = 0; w0 < nw; w0 += kFlagThreads) {
        const int64_t w = w0 + threadIdx.x;
        uint32_t word = next;
        next = w + kFlagThreads < nw ? mrow[w + kFlagThreads] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan<uint32_t, kFlagThreads>(static_cast<uint32_t>(__popc(word)), &tot, sh);
        if (fill + tot > static_cast<uint32_t>(kGatherList)) flush();
        uint32_t p = fill + ex;
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1u;
            list[p++] = static_cast<uint32_t>(32 * w + b);
        }
        fill += tot;
        __syncthreads();
    }
    if (fill > 0) flush();
}

__global__ void fill_u32_kernel(uint32_t *p, int64_t n, uint32_t v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void fill_u64_kernel(uint64_t *p, int64_t n, uint64_t v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// --------------------------------------------------------------------------
// Packed norm format: the compact codes of a binary16 half-norm plane, packed
// per token row like the index codes.  Each thread converts 4 chunks (one
// 8-byte load); a block covers 1024 chunks, i.e. whole token rows, ORs the
// codes into its rows' words in LDS and stores them.
// --------------------------------------------------------------------------
constexpr int kPackThreads = 256;
constexpr int kPackChunks = 4 * kPackThreads;

__global__ __launch_bounds__(kPackThreads) void pack_norms_kernel(const uint16_t *h16, uint32_t *words, int64_t total,
                                                                  int32_t log2_cpt, int32_t bits, int32_t W) {
    __shared__ uint32_t sw[kPackChunks];   // rows * W <= 1024 * 15 / 32 + 256
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kPackChunks;
    const int rows = kPackChunks >> log2_cpt;
    const int nw = rows * W;
    for (int i = threadIdx.x; i < nw; i += kPackThreads) sw[i] = 0u;
    __syncthreads();
    const int64_t c = c0 + 4 * threadIdx.x;
    if (c < total) {   // total and c are multiples of 4
        const uint2 u = *reinterpret_cast<const uint2 *>(h16 + c);
        const uint32_t h[4] = {u.x & 0xFFFFu, u.x >> 16, u.y & 0xFFFFu, u.y >> 16};
        const int cmask = (1 << log2_cpt) - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int lc = 4 * threadIdx.x + j;
            const uint32_t code = compact_norm_code(h[j], bits);
            const int bit = (lc & cmask) * bits;
            uint32_t *wr = &sw[(lc >> log2_cpt) * W + (bit >> 5)];
            const int sft = bit & 31;
            atomicOr(wr, code << sft);
            if (sft + bits > 32) atomicOr(wr + 1, code >> (32 - sft));
        }
    }
    __syncthreads();
    const int64_t row0 = c0 >> log2_cpt;
    const int64_t valid = min(static_cast<int64_t>(rows), (total >> log2_cpt) - row0) * W;
    uint32_t *dst = words + row0 * W;
    for (int i = threadIdx.x; i < valid; i += kPackThreads) dst[i] = sw[i];
}

// --------------------------------------------------------------------------
// Exact-rate records: whole-bit codes and binary16 half-norms (flags set)
// turned into groups of 4 token rows.  A block takes kPackExChunks chunks
// (whole groups) of one slice, in three steps without atomics:
//  1. every thread forms the index and norm codes of two runs of 4
//     consecutive chunks (the loads of both runs issued before either is
//     used: an 8-byte half-norm load and the code words per run) into LDS;
//  2. one thread per low-bit word ORs the (at most 11) codes it holds, and
//     one thread per 13-bit digit field sums its 8 digits;
//  3. the digit words are gathered from up to four fields each, and every
//     word of the block's groups is stored once.
// --------------------------------------------------------------------------
constexpr int kPackExThreads = 256;
constexpr int kPackExChunks = 2048;   // 4 rows x cpt chunks divides it for every head_dim
constexpr int kPackExRuns = kPackExChunks / (4 * kPackExThreads);   // 4-chunk runs per thread
// a block's low-bit words (8 ceil(cpt m / 32) per group) and digit fields
// (8 ceil(cpt / 8) per group), at most over head_dim 16..256 and m <= 13
constexpr int kPackExLowWords = 2048;
constexpr int kPackExFields = 1024;

struct PackExArgs {
    const uint32_t *idx;    // [slices][tokens][words] whole-bit codes
    const uint16_t *h16;    // [slices][tokens][cpt]
    uint32_t *out;          // [slices][gps][gw]
    int64_t tokens, gps, blocks_per_slice;
    int32_t log2_cpt, log2_fh, bits, words, m, wl, fh, gw;
    uint32_t gw_magic;      // ceil(2^24 / gw): w / gw for the block's word indices
    uint32_t wl_magic;      // ceil(2^20 / wl): w / wl for the block's low-bit words
    uint32_t m_recip;       // ceil(2^16 / m): b / m for bit offsets b < 2^11
    uint32_t nmax;
    float step;
};

__global__ __launch_bounds__(kPackExThreads) void pack_exact_kernel(PackExArgs a) {
    __shared__ uint16_t codes[2 * kPackExChunks];   // [plane][chunk of the block]
    __shared__ uint32_t lows[kPackExLowWords];
    __shared__ uint32_t fields[kPackExFields];
    const int64_t slice = blockIdx.x / a.blocks_per_slice;
    const int64_t gb = blockIdx.x - slice * a.blocks_per_slice;
    const int cpt = 1 << a.log2_cpt;
    const int gpb = kPackExChunks >> (a.log2_cpt + 2);   // groups per block
    const int64_t g0 = gb * gpb;
    const int64_t t0 = g0 * kExactRows;
    const int lw = 8 * a.wl;                   // low-bit words per group
    const int log2_nfg = 3 + a.log2_fh;        // digit fields per group: 8 fh
    uint16_t *kc = codes, *nc = codes + kPackExChunks;

    // step 1
    {
        const uint32_t kmask = (1u << a.bits) - 1u;
        uint2 hv[kPackExRuns];
        uint32_t cw[kPackExRuns][3];
        int bit0[kPackExRuns];
        bool ok[kPackExRuns];
#pragma unroll
        for (int u = 0; u < kPackExRuns; ++u) {
            const int i = 4 * (threadIdx.x + u * kPackExThreads);   // first chunk of the run
            const int lr = i >> a.log2_cpt, c = i & (cpt - 1);
            const int64_t t = t0 + lr;
            ok[u] = t < a.tokens;                                    // rows past the end pack as zeros
            const int64_t tr = ok[u] ? t : a.tokens - 1;
            const int64_t rowi = slice * a.tokens + tr;
            hv[u] = *reinterpret_cast<const uint2 *>(a.h16 + rowi * cpt + c);
            const uint32_t *row = a.idx + rowi * a.words;
            bit0[u] = c * a.bits;
            const int w = bit0[u] >> 5;
#pragma unroll
            for (int k = 0; k < 3; ++k) cw[u][k] = row[min(w + k, a.words - 1)];
        }
#pragma unroll
        for (int u = 0; u < kPackExRuns; ++u) {
            const int i = 4 * (threadIdx.x + u * kPackExThreads);
            const uint32_t h[4] = {hv[u].x & 0xFFFFu, hv[u].x >> 16, hv[u].y & 0xFFFFu, hv[u].y >> 16};
            const uint32_t sh = static_cast<uint32_t>(bit0[u] & 31);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // code j starts at bit q of the 3 loaded words and ends inside
                // them (sh + 4 b <= 96): its two-word window by alignbit
                const uint32_t q = sh + static_cast<uint32_t>(j * a.bits);
                const uint32_t wj = q >> 5;
                const uint32_t lo = wj == 0u ? cw[u][0] : (wj == 1u ? cw[u][1] : cw[u][2]);
                const uint32_t hi = wj == 0u ? cw[u][1] : cw[u][2];
                const uint32_t k = __builtin_amdgcn_alignbit(hi, lo, q & 31u) & kmask;
                kc[i + j] = static_cast<uint16_t>(ok[u] ? k : 0u);
                nc[i + j] = static_cast<uint16_t>(ok[u] ? exact_norm_code(h[j], a.m, a.nmax, a.step) : 0u);
            }
        }
    }
    __syncthreads();

    // step 2: low-bit words (w = (stream s, word wi), s = (group, plane, row))
    const uint32_t lmask = (1u << a.m) - 1u;
    for (int w = threadIdx.x; w < gpb * lw; w += kPackExThreads) {
        const int s = static_cast<int>(__umul24(static_cast<uint32_t>(w), a.wl_magic) >> 20);
        const int wi = w - s * a.wl;
        const int gi = s >> 3, pl = (s >> 2) & 1, r = s & 3;
        const uint16_t *src = (pl ? nc : kc) + ((gi * kExactRows + r) << a.log2_cpt);
        const int b0 = 32 * wi;
        const int c_lo = static_cast<int>(__umul24(static_cast<uint32_t>(b0), a.m_recip) >> 16);
        const int c_hi = min(cpt - 1, static_cast<int>(__umul24(static_cast<uint32_t>(b0 + 31), a.m_recip) >> 16));
        uint32_t v = 0u;
        for (int c = c_lo; c <= c_hi; ++c) {
            const int sft = c * a.m - b0;   // -(m - 1) .. 31
            const uint32_t low = src[c] & lmask;
            v |= sft >= 0 ? (low << sft) : (low >> -sft);
        }
        lows[w] = v;
    }
    // digit fields: field f of a group is (row f / 2fh, plane (f / fh) % 2, f % fh)
    for (int f = threadIdx.x; f < (gpb << log2_nfg); f += kPackExThreads) {
        const int gi = f >> log2_nfg, ff = f & ((1 << log2_nfg) - 1);
        const int r = ff >> (a.log2_fh + 1), pl = (ff >> a.log2_fh) & 1, fi = ff & (a.fh - 1);
        const uint16_t *src = (pl ? nc : kc) + ((gi * kExactRows + r) << a.log2_cpt);
        uint32_t val = 0u;
#pragma unroll
        for (int q = kDigitsPerField - 1; q >= 0; --q) {
            const int c = fi * kDigitsPerField + q;
            val = 3u * val + (c < cpt ? static_cast<uint32_t>(src[c]) >> a.m : 0u);
        }
        fields[f] = val;
    }
    __syncthreads();

    // step 3: every word of the block's groups
    const int nfg = 1 << log2_nfg;
    const int groups = static_cast<int>(min(static_cast<int64_t>(gpb), a.gps - g0));
    uint32_t *dst = a.out + (slice * a.gps + g0) * a.gw;
    for (int w = threadIdx.x; w < groups * a.gw; w += kPackExThreads) {
        const int gi = static_cast<int>(__umul24(static_cast<uint32_t>(w), a.gw_magic) >> 24);
        const int ww = w - gi * a.gw;
        uint32_t v;
        if (ww < lw) {
            v = lows[gi * lw + ww];
        } else {
            const int b0 = 32 * (ww - lw);
            const int f_hi = min(nfg - 1, (b0 + 31) / kFieldBits);
            v = 0u;
            for (int f = b0 / kFieldBits; f <= f_hi; ++f) {
                const uint32_t val = fields[gi * nfg + f];
                const int sft = f * kFieldBits - b0;   // -12 .. 31
                v |= sft >= 0 ? (val << sft) : (val >> -sft);
            }
        }
        dst[w] = v;
    }
}

// Exact-rate packing specialised for 32 chunks per row (head_dim 128) and a
// fixed m (S = 8: m = 6, S = 32: m = 8).  A block packs 32 groups (128 token
// rows) whose records are contiguous.  Its work items are (plane, row, digit
// field): 8 codes each, whole-bit index codes (m + 2 bits) or binary16
// half-norms turned into norm codes.  Consecutive threads take consecutive
// items, so the loads are contiguous, and every thread takes two items of
// each plane.  An item puts its 8 m-bit low parts into the group's low-bit
// words and its digit field value (digit i weighing 3^i) into LDS; the 13
// digit words per group are assembled there and the block's records are
// written out word by word (coalesced stores).
template <int M>
__global__ __launch_bounds__(kPackExThreads) void pack_exact32_kernel(PackExArgs a) {
    constexpr int CPT = 32, B = M + 2, WL = M, FH = 4, NFG = 8 * FH, LW = 8 * WL;
    constexpr int GW = LW + (kExactRows * 2 * FH * kFieldBits + 31) / 32;
    constexpr int GPB = 32;                       // groups per block
    constexpr int ROWS = GPB * kExactRows;        // token rows per block
    constexpr int ITEMS = 2 * ROWS * FH;          // (plane, row, field)
    static_assert(ITEMS % kPackExThreads == 0, "whole items per thread");
    __shared__ uint32_t fields[GPB * NFG];
    __shared__ uint32_t stage[GPB * GW];
    const int64_t slice = blockIdx.x / a.blocks_per_slice;
    const int64_t g0 = (blockIdx.x - slice * a.blocks_per_slice) * GPB;
    const int64_t t0 = g0 * kExactRows;   // the block's first token row
    // low-bit words are ORed together from the items (with m = 6 an item's
    // 48 bits share words with its neighbours')
    for (int i = threadIdx.x; i < GPB * LW; i += kPackExThreads) stage[(i / LW) * GW + i % LW] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS / kPackExThreads; ++j) {
        const int item = threadIdx.x + j * kPackExThreads;
        const int pl = item / (ROWS * FH);
        const int rb = (item % (ROWS * FH)) / FH, f = item % FH;   // row in the block, field
        const int gi = rb / kExactRows, r = rb % kExactRows;
        const int64_t t = t0 + rb;
        uint32_t code[kDigitsPerField];
        if (t < a.tokens) {
            const int64_t rowi = slice * a.tokens + t;
            if (pl == 0) {
                constexpr int NWI = (8 * B + 31) / 32 + 1;
                const int b0 = 8 * f * B, w0 = b0 >> 5, sh = b0 & 31;
                const uint32_t *src = a.idx + rowi * B + w0;
                uint32_t w[NWI];
#pragma unroll
                for (int k = 0; k < NWI; ++k) w[k] = w0 + k < B ? src[k] : 0u;
#pragma unroll
                for (int c = 0; c < kDigitsPerField; ++c) {
                    constexpr uint32_t kmask = (1u << B) - 1u;
                    const int p = sh + c * B, k = p >> 5, sft = p & 31;
                    code[c] = __builtin_amdgcn_alignbit(w[k + 1], w[k], sft) & kmask;
                }
            } else {
                const uint4 v = reinterpret_cast<const uint4 *>(a.h16 + rowi * CPT)[f];
                const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < kDigitsPerField; ++e)
                    code[e] = exact_norm_code((h[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, M, a.nmax, a.step);
            }
        } else {
#pragma unroll
            for (int c = 0; c < kDigitsPerField; ++c) code[c] = 0u;
        }
        // low parts: 8 M bits at bit 8 f M of the (plane, row) low-bit words
        {
            constexpr uint32_t lmask = (1u << M) - 1u;
            uint32_t lo0 = 0u, lo1 = 0u;   // the 8 M <= 64 bits from the item's first bit
#pragma unroll
            for (int c = 0; c < kDigitsPerField; ++c) {
                const uint32_t low = code[c] & lmask;
                const int p = c * M;
                if (p < 32) {
                    lo0 |= low << p;
                    if (p + M > 32) lo1 |= low >> (32 - p);
                } else {
                    lo1 |= low << (p - 32);
                }
            }
            uint32_t *lw = stage + gi * GW + (pl * kExactRows + r) * WL;
            const int b0 = 8 * f * M, k = b0 >> 5, sh = b0 & 31;
            if constexpr ((8 * M) % 32 == 0) {
                lw[k] = lo0;            // whole words (m = 8)
                lw[k + 1] = lo1;
            } else {
                atomicOr(&lw[k], lo0 << sh);
                if (sh > 0) atomicOr(&lw[k + 1], (lo0 >> (32 - sh)) | (lo1 << sh));
                else atomicOr(&lw[k + 1], lo1);
                if (sh + 8 * M > 64) atomicOr(&lw[k + 2], lo1 >> (32 - sh));
            }
        }
        // the digit field's value
        uint32_t val = 0u;
#pragma unroll
        for (int q = kDigitsPerField - 1; q >= 0; --q) val = 3u * val + (code[q] >> M);
        fields[gi * NFG + r * 2 * FH + pl * FH + f] = val;
    }
    __syncthreads();
    constexpr int DW = GW - LW;   // digit words per group
    for (int w = threadIdx.x; w < GPB * DW; w += kPackExThreads) {
        const int gj = w / DW, ww = w - gj * DW;
        const int b0 = 32 * ww;
        const int f_hi = min(NFG - 1, (b0 + 31) / kFieldBits);
        uint32_t v = 0u;
        for (int f = b0 / kFieldBits; f <= f_hi; ++f) {
            const uint32_t val = fields[gj * NFG + f];
            const int sft = f * kFieldBits - b0;
            v |= sft >= 0 ? (val << sft) : (val >> -sft);
        }
        stage[gj * GW + LW + ww] = v;
    }
    __syncthreads();
    // the block's groups that exist, contiguous in the record
    const int64_t ng = min(static_cast<int64_t>(GPB), a.gps - g0);
    uint32_t *dst = a.out + (slice * a.gps + g0) * GW;
    for (int i = threadIdx.x; i < ng * GW; i += kPackExThreads) dst[i] = stage[i];
}

// --------------------------------------------------------------------------
// Decode kernel: one block per contiguous chunk range of one slice.
// --------------------------------------------------------------------------
struct DecArgs {
    const uint32_t *idx;
    const void *hnorm;   // binary16 half-norms, or (NPACK) packed compact codes
    const uint64_t *offsets;
    const uint32_t *out_pos;
    const uint16_t *out_val;
    uint64_t capacity;
    const float *cb;
    void *y;
    int64_t n_slice;
    int64_t tokens;
    int64_t wg_per_slice;
    int64_t wg_chunks;
    int64_t batch_chunks;
    int64_t bps;
    int32_t S;
    int32_t cpt;
    int32_t log2_cpt;
    int32_t bits;
    int32_t words;
    // exact-rate records (NF == 2): idx holds [slices][gps][gw] group words
    int64_t gps;
    int32_t m, wl, fh, gw;
    float step;
};

template <bool F32OUT>
__device__ __forceinline__ void store_chunk(void *y, int64_t gc, f32x4 v) {
    if constexpr (F32OUT) {
        reinterpret_cast<float4 *>(y)[gc] = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        uint2 o;
        o.x = static_cast<uint32_t>(f32_to_f16_bits(v[0])) | (static_cast<uint32_t>(f32_to_f16_bits(v[1])) << 16);
        o.y = static_cast<uint32_t>(f32_to_f16_bits(v[2])) | (static_cast<uint32_t>(f32_to_f16_bits(v[3])) << 16);
        reinterpret_cast<uint2 *>(y)[gc] = o;
    }
}

// Codes and half-norms of the 2 chunks c, c+1 of one token row.
struct DecPair {
    uint32_t w0, w1;   // the row words holding the 2 codes (exact: their low bits)
    uint32_t sh;       // bit offset of the first code in w0
    uint32_t h;        // 2 binary16 half-norm codes
    uint32_t n0, n1;   // NF 1: the norm row words at the index words' places; NF 2: the norm low bits
    uint32_t dk0, dk1, dn0, dn1;   // NF 2: words holding the index and norm digit fields
    uint32_t dsh;      // NF 2: bit offsets of the two fields (index | norm << 8)
};

// Norm formats of the decode and attention kernels: binary16 half-norms,
// packed compact codes, exact-rate groups.
constexpr int kNormF16 = 0, kNormPacked = 1, kNormExact = 2;

// Ternary digits i0 and i0 + 1 of a 13-bit digit field v, i0 = 2 sel in
// {0, 2, 4, 6}: v / 3^i0 by a 24-bit multiply and shift (exact for v < 2^13),
// then two base-3 digits of the quotient.
__device__ __forceinline__ void digit_pair(uint32_t v, uint32_t sel, uint32_t *d0, uint32_t *d1) {
    const uint32_t mul = sel == 1u ? 116509u : (sel == 2u ? 207127u : 23015u);
    const uint32_t sft = sel == 1u ? 20u : 24u;
    const uint32_t q = sel == 0u ? v : (__umul24(v, mul) >> sft);
    const uint32_t q3 = div3_small(q);
    *d0 = q - 3u * q3;
    *d1 = q3 - 3u * div3_small(q3);
}

// (5 waves per SIMD where the registers allow it: the decode is bound by
// memory latency and bandwidth, so it wants many waves in flight)
//
// EM > 0 (exact-rate records, head_dim 128, m = EM in {6, 8}): a wave step
// of 128 chunks is one whole group of 4 token rows (8 EM + 13 words), so the
// wave loads the group with one or two coalesced loads per lane (lane l
// holds words l and 64 + l) and every lane takes the words its two chunks
// need from the others by ds_bpermute, in place of eight loads of its own.
template <bool F32OUT, bool TABLE, int NF, int EM = 0>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(NF == 1 ? 4 : 5)))
void decode_kernel(DecArgs a) {
    constexpr bool NPACK = NF == kNormPacked;
    constexpr bool EXACT = NF == kNormExact;
    constexpr bool GROUPED = EXACT && EM > 0;
    static_assert(!GROUPED || EM == 6 || EM == 8, "grouped exact-rate decode: m = 6 or 8");
    // words per group: 4 rows x 2 planes x EM words of low bits, 32 digit
    // fields of 13 bits; EM = 8: low bits in words 0..63, digits 64..76;
    // EM = 6: everything in words 0..60
    constexpr int kGW = 8 * EM + (4 * 2 * 4 * kFieldBits + 31) / 32;
    // steps whose loads a thread issues together (an exact-rate step holds
    // twice the record words, so half as many keep the register count;
    // grouped steps hold at most two words)
    constexpr int kUnroll = EXACT && !GROUPED ? kDecUnroll / 2 : kDecUnroll;
    extern __shared__ f32x4 tab[];   // TABLE: the 24 S codewords; else the S q_s
    const int64_t slice = blockIdx.x / a.wg_per_slice;
    const int64_t r0 = (blockIdx.x - slice * a.wg_per_slice) * a.wg_chunks;
    const int64_t r1 = min(r0 + a.wg_chunks, a.n_slice);
    const int64_t sbase = slice * a.n_slice;
    const float *q = a.cb + slice * a.S * 4;
    const int ncw = 24 * a.S;

    if constexpr (TABLE) {
        for (int k = threadIdx.x; k < ncw; k += kDecThreads) {
            const int s = k / 24;
            const float qe[4] = {double_f16(q[4 * s]), double_f16(q[4 * s + 1]),
                                 double_f16(q[4 * s + 2]), double_f16(q[4 * s + 3])};
            tab[k] = codeword_f32(qe, k - 24 * s);
        }
    } else {
        for (int s = threadIdx.x; s < a.S; s += kDecThreads) {
            f32x4 v = {double_f16(q[4 * s]), double_f16(q[4 * s + 1]), double_f16(q[4 * s + 2]),
                       double_f16(q[4 * s + 3])};
            tab[s] = v;
        }
    }
    __syncthreads();

    const uint32_t *idx_s = EXACT ? a.idx + slice * a.gps * a.gw : a.idx + slice * a.tokens * a.words;
    // half-norm code pairs (u32 per 2 chunks), or the packed norm rows
    const uint32_t *hn_s = NPACK ? static_cast<const uint32_t *>(a.hnorm) + slice * a.tokens * a.words
                                 : static_cast<const uint32_t *>(a.hnorm) + (sbase >> 1);
    const int cmask = a.cpt - 1;
    const uint32_t kmask = (1u << a.bits) - 1u;
    const int last_word = a.words - 1;

    // Each wave decodes a contiguous quarter of the block's range, 2 chunks
    // per lane per step, so one 16-byte store per lane writes 1 KB of
    // contiguous fp16 output.  Outlier chunks (bit 15 of the half-norm code)
    // take their side-list values in the same pass: the side list is sorted
    // by position, so a wave finds the first entry at or after its range
    // once and then ranks its flagged chunks step by step with a ballot.
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t wlen = (r1 - r0 + 4 * 128 - 1) / (4 * 128) * 128;   // multiple of a wave step
    const int64_t w0 = min(r0 + wave * wlen, r1);
    const int64_t w1 = min(w0 + wlen, r1);
    const uint2 *sval = reinterpret_cast<const uint2 *>(a.out_val);

    // first side-list entry with position >= w0: one probe of 64 entries
    // around the index interpolated from w0's place in its batches (enough
    // when the outliers are spread evenly), then 64-way search rounds
    uint64_t e_next = 0, e_end = 0;
    if (a.bps > 0 && w0 < w1) {
        const int64_t bl = w0 / a.batch_chunks;
        const int64_t bh = (w1 - 1) / a.batch_chunks;
        uint64_t lo = a.offsets[slice * a.bps + bl];
        uint64_t hi = a.offsets[slice * a.bps + bh + 1];
        hi = hi < a.capacity ? hi : a.capacity;
        lo = lo < hi ? lo : hi;
        e_end = hi;
        if (hi - lo > 64) {
            const int64_t p0 = bl * a.batch_chunks;
            const int64_t p1 = min((bh + 1) * a.batch_chunks, a.n_slice);
            const double f = static_cast<double>(w0 - p0) / static_cast<double>(p1 - p0);
            const uint64_t guess = lo + static_cast<uint64_t>(f * static_cast<double>(hi - lo));
            const uint64_t g0 = min(max(guess, lo + 32) - 32, hi - 64);
            const bool below = static_cast<int64_t>(a.out_pos[g0 + lane]) < w0;
            const int cnt = __popcll(__ballot(below));
            if (cnt == 0) hi = g0;                       // the answer is at or before g0
            else if (cnt == 64) lo = g0 + 64;            // after the window
            else lo = hi = g0 + static_cast<uint64_t>(cnt);
        }
        while (hi > lo) {
            const uint64_t len = hi - lo;
            const uint64_t step = (len + 63) / 64;
            const uint64_t i = lo + static_cast<uint64_t>(lane) * step;
            const bool below = i < hi && static_cast<int64_t>(a.out_pos[i]) < w0;
            const int cnt = __popcll(__ballot(below));
            if (cnt == 0) break;
            const uint64_t nlo = lo + static_cast<uint64_t>(cnt - 1) * step + 1;
            const uint64_t nhi = lo + static_cast<uint64_t>(cnt) * step;
            hi = nhi < hi ? nhi : hi;
            lo = nlo;
        }
        e_next = lo;
    }

    auto load = [&](int64_t c) {
        DecPair d;
        if constexpr (EXACT) {
            // row r of group row / 4: the low bits of chunks cc, cc + 1 in both
            // planes, and the 13-bit index and norm digit fields holding
            // their digits (each read as a 2-word window)
            const int64_t row = c >> a.log2_cpt;
            const int cc = static_cast<int>(c & cmask);
            const int r = static_cast<int>(row & 3);
            const uint32_t *gp = idx_s + (row >> 2) * a.gw;
            const int ob = cc * a.m, w = ob >> 5;
            const int w1 = min(w + 1, a.wl - 1);
            d.w0 = gp[r * a.wl + w];
            d.w1 = gp[r * a.wl + w1];
            d.n0 = gp[(4 + r) * a.wl + w];
            d.n1 = gp[(4 + r) * a.wl + w1];
            d.sh = static_cast<uint32_t>(ob & 31);
            const int dbase = 8 * a.wl, dlast = a.gw - 1;
            const int fk = kFieldBits * (2 * a.fh * r + (cc >> 3));
            const int fn = fk + kFieldBits * a.fh;
            d.dk0 = gp[dbase + (fk >> 5)];
            d.dk1 = gp[min(dbase + (fk >> 5) + 1, dlast)];
            d.dn0 = gp[dbase + (fn >> 5)];
            d.dn1 = gp[min(dbase + (fn >> 5) + 1, dlast)];
            d.dsh = static_cast<uint32_t>(fk & 31) | (static_cast<uint32_t>(fn & 31) << 8) |
                    (static_cast<uint32_t>((cc >> 1) & 3) << 16);
            d.h = 0u;
            return d;
        }
        const int64_t row = c >> a.log2_cpt;
        const int o = static_cast<int>(c & cmask) * a.bits;
        const int w = o >> 5;
        const uint32_t *rp = idx_s + row * a.words;
        d.w0 = rp[w];
        d.w1 = rp[min(w + 1, last_word)];
        d.sh = static_cast<uint32_t>(o & 31);
        if constexpr (NPACK) {
            const uint32_t *np = hn_s + row * a.words;
            d.n0 = np[w];
            d.n1 = np[min(w + 1, last_word)];
            d.h = 0u;
        } else {
            d.h = hn_s[c >> 1];
            d.n0 = d.n1 = 0u;
        }
        return d;
    };
    constexpr int kWaveStep = 128;   // chunks per wave step
    // grouped exact-rate records: the group of wave step base (a multiple of
    // 128, as every wave's range starts and ends on a group), words l and
    // 64 + l.  The loads are unconditional (steps past the range read its
    // last group, lanes past the group's words its last word; the permutes
    // read neither), so that each step waits for its own loads only.
    auto load_group = [&](int64_t sbase_) {
        const uint32_t *gp = idx_s + ((sbase_ < w1 ? sbase_ : w1 - kWaveStep) >> 7) * kGW;
        return make_uint2(gp[lane < kGW ? lane : kGW - 1], gp[64 + lane < kGW ? 64 + lane : kGW - 1]);
    };
    // the lane's DecPair from the wave's group words (every lane runs it:
    // the permutes read all lanes); row r = lane / 16, chunks 2 (lane % 16)
    // and the next
    auto from_group = [&](uint2 g) {
        const int r = lane >> 4, q = lane & 15;
        auto perm = [](uint32_t v, int src) {
            return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(v)));
        };
        DecPair d;
        const int ob = 2 * q * EM, w = r * EM + (ob >> 5);
        d.w0 = perm(g.x, w);
        d.n0 = perm(g.x, 4 * EM + w);
        if constexpr (EM == 8) {
            d.w1 = d.n1 = 0u;   // 16 bits at bit 0 or 16 of one word
        } else {
            d.w1 = perm(g.x, w + 1);   // (w + 1 stays inside the row when used)
            d.n1 = perm(g.x, 4 * EM + w + 1);
        }
        d.sh = static_cast<uint32_t>(ob & 31);
        const int fk = kFieldBits * (8 * r + (q >> 2));
        const int fn = fk + kFieldBits * 4;
        const uint32_t dg = EM == 8 ? g.y : g.x;
        constexpr int kDig = EM == 8 ? 0 : 8 * EM;   // first digit word's lane in dg
        d.dk0 = perm(dg, kDig + (fk >> 5));
        d.dk1 = perm(dg, kDig + (fk >> 5) + 1);
        d.dn0 = perm(dg, kDig + (fn >> 5));
        d.dn1 = perm(dg, kDig + (fn >> 5) + 1);
        d.dsh = static_cast<uint32_t>(fk & 31) | (static_cast<uint32_t>(fn & 31) << 8) |
                (static_cast<uint32_t>(q & 3) << 16);
        d.h = 0u;
        return d;
    };
    // exact-rate records: full codes 2^m d + l of the two chunks as indices
    // in w0 / w1 (read below with a zero shift), the norm codes as half-norm
    // records
    const int em = GROUPED ? EM : a.m;
    auto finish_exact = [&](DecPair &p) {
        const uint32_t lmask = (1u << em) - 1u;
        const uint32_t flag = (3u << em) - 1u;
        const uint32_t sel = (p.dsh >> 16) & 3u;
        const uint32_t vk = static_cast<uint32_t>(((static_cast<uint64_t>(p.dk1) << 32) | p.dk0) >> (p.dsh & 31u)) & 0x1FFFu;
        const uint32_t vn = static_cast<uint32_t>(((static_cast<uint64_t>(p.dn1) << 32) | p.dn0) >> ((p.dsh >> 8) & 31u)) & 0x1FFFu;
        uint32_t ka, kb, na, nb;
        digit_pair(vk, sel, &ka, &kb);
        digit_pair(vn, sel, &na, &nb);
        const uint32_t lk = static_cast<uint32_t>(((static_cast<uint64_t>(p.w1) << 32) | p.w0) >> p.sh);
        const uint32_t ln = static_cast<uint32_t>(((static_cast<uint64_t>(p.n1) << 32) | p.n0) >> p.sh);
        p.w0 = (ka << em) | (lk & lmask);
        p.w1 = (kb << em) | ((lk >> em) & lmask);
        p.sh = 0u;
        const uint32_t n0 = (na << em) | (ln & lmask), n1 = (nb << em) | ((ln >> em) & lmask);
        p.h = exact_norm_h16(n0, flag, a.step) | (exact_norm_h16(n1, flag, a.step) << 16);
    };
    // the loop runs on a wave-uniform base, so that every lane takes part in
    // the exchange below (lanes past the range's end carry no flags and store
    // nothing)
    for (int64_t base = w0; base < w1; base += static_cast<int64_t>(kWaveStep) * kUnroll) {
        const int64_t c0 = base + 2 * lane;
        // the next 64 side-list entries (lane j: entry e_next + j), requested
        // with the records: the iteration's flagged chunks take their values
        // from this window by lane exchange instead of loads issued after
        // their flags are known
        const uint64_t wbase = e_next;
        uint2 wv = make_uint2(0u, 0u);
        if (wbase < e_end) {
            const uint64_t e = wbase + static_cast<uint64_t>(lane);
            wv = sval[e < e_end ? e : e_end - 1];
        }
        // entries are counted from wbase in 32 bits: wlim entries are left in
        // the list (saturated), wused have gone to earlier steps
        const uint64_t left = e_end - wbase;   // e_end >= wbase
        const uint32_t wlim = left > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(left);
        uint32_t wused = 0u;
        // side-list values of one step's flagged chunks, in order (a chunk
        // whose entry was dropped, past the capacity, keeps its bulk value)
        auto rank = [&](const DecPair &p, uint2 (&ov)[2], bool (&oh)[2]) {
            const bool f0 = (p.h & 0x8000u) != 0;
            const bool f1 = (p.h & 0x80000000u) != 0;
            const uint64_t m0 = __ballot(f0), m1 = __ballot(f1);
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m0 >> 32),
                                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m0), 0u)) +
                                   __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m1 >> 32),
                                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m1), 0u));
            const uint32_t q0 = wused + below;            // window lanes of the entries
            const uint32_t q1 = q0 + (f0 ? 1u : 0u);
            oh[0] = f0 && q0 < wlim;
            oh[1] = f1 && q1 < wlim;
            if ((m0 | m1) != 0u) {   // wave-uniform: every lane takes part in the exchange
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t q = i ? q1 : q0;
                    const int src = q < 64u ? static_cast<int>(q) : 0;
                    const uint2 v = make_uint2(static_cast<uint32_t>(__shfl(static_cast<int>(wv.x), src)),
                                               static_cast<uint32_t>(__shfl(static_cast<int>(wv.y), src)));
                    // entries past the window (more than 64 flags in one
                    // iteration) are loaded on their own; the empty asm
                    // takes the wait for that load inside this rare branch,
                    // so that the common path does not wait for every load
                    // in flight
                    const bool far = oh[i] && q >= 64u;
                    uint32_t vx = v.x, vy = v.y;
                    if (far) {
                        const uint2 t = sval[wbase + q];
                        vx = t.x;
                        vy = t.y;
                        asm volatile("" : "+v"(vx), "+v"(vy));
                    }
                    ov[i] = make_uint2(vx, vy);
                }
            }
            wused += static_cast<uint32_t>(__popcll(m0) + __popcll(m1));
        };
        // the two decoded chunks c, c + 1 of a step, one 16-byte store
        // (binary16 output: the bulk values rounded in pairs, an outlier's
        // side value taken as its binary16 words)
        auto emit = [&](int64_t c, const DecPair &cur, const uint2 (&ov)[2], const bool (&oh)[2]) {
            const uint64_t win = ((static_cast<uint64_t>(cur.w1) << 32) | cur.w0) >> cur.sh;
            f32x4 out[2];
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                uint32_t k = EXACT ? (i ? cur.w1 : cur.w0) : static_cast<uint32_t>(win >> (i * a.bits)) & kmask;
                k = min(k, static_cast<uint32_t>(ncw - 1));
                const uint16_t hi = static_cast<uint16_t>(cur.h >> (16 * i));
                const float r = 2.0f * f16_bits_to_f32(static_cast<uint16_t>(hi & 0x7FFFu));
                f32x4 cw;
                if constexpr (TABLE) {
                    cw = tab[k];
                } else {
                    const int s = static_cast<int>(k / 24u);
                    const f32x4 qv = tab[s];
                    const float qa[4] = {qv[0], qv[1], qv[2], qv[3]};
                    cw = codeword_f32(qa, static_cast<int>(k) - 24 * s);
                }
                out[i] = r * cw;
                if constexpr (F32OUT) {
                    if (oh[i]) {
                        const uint2 v = ov[i];
                        const f32x4 f = {f16_bits_to_f32(static_cast<uint16_t>(v.x)), f16_bits_to_f32(static_cast<uint16_t>(v.x >> 16)),
                                         f16_bits_to_f32(static_cast<uint16_t>(v.y)), f16_bits_to_f32(static_cast<uint16_t>(v.y >> 16))};
                        out[i] = f;
                    }
                } else {
                    const f16x4 hy = {static_cast<_Float16>(out[i][0]), static_cast<_Float16>(out[i][1]),
                                      static_cast<_Float16>(out[i][2]), static_cast<_Float16>(out[i][3])};
                    uint2 w = __builtin_bit_cast(uint2, hy);
                    if (oh[i]) w = ov[i];
                    o[2 * i] = w.x;
                    o[2 * i + 1] = w.y;
                }
            }
            // the iteration's wave-uniform output base plus a 32-bit lane offset
            const uint32_t rel = static_cast<uint32_t>(c - base);
            if constexpr (F32OUT) {
                f32x4 *yp = reinterpret_cast<f32x4 *>(a.y) + (sbase + base) + rel;
                __builtin_nontemporal_store(out[0], yp);
                __builtin_nontemporal_store(out[1], yp + 1);
            } else {
                uint16_t *yw = static_cast<uint16_t *>(a.y) + 4 * (sbase + base);
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(yw + 4 * rel));
            }
        };
        if constexpr (GROUPED) {
            // the group loads of every step first, then each step whole: its
            // pair from the group words, codes, ranking and store
            uint2 gw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) gw[u] = load_group(base + static_cast<int64_t>(u) * kWaveStep);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t c = c0 + static_cast<int64_t>(u) * kWaveStep;
                DecPair p = from_group(gw[u]);
                if (c >= w1) p = DecPair{};
                finish_exact(p);
                uint2 ov[2];
                bool oh[2];
                rank(p, ov, oh);
                if (c < w1) emit(c, p, ov, oh);
            }
            e_next = wbase + wused;
            continue;
        }
        // binary16 and packed norms: every step's loads are issued
        // unconditionally (lanes past the range's end read its last pair, w1
        // being even), so that the compiler waits for each step's loads
        // alone, not for all of them (exact-rate records: conditional loads,
        // which keep the register count)
        DecPair pd[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + static_cast<int64_t>(u) * kWaveStep;
            if constexpr (EXACT) pd[u] = c < w1 ? load(c) : DecPair{};
            else pd[u] = load(c < w1 ? c : w1 - 2);
        }
        if constexpr (NPACK) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const uint64_t nwin = ((static_cast<uint64_t>(pd[u].n1) << 32) | pd[u].n0) >> pd[u].sh;
                const uint32_t k0 = static_cast<uint32_t>(nwin) & kmask;
                const uint32_t k1 = static_cast<uint32_t>(nwin >> a.bits) & kmask;
                pd[u].h = compact_norm_h16(k0, a.bits) | (compact_norm_h16(k1, a.bits) << 16);
            }
        }
        if constexpr (EXACT) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) finish_exact(pd[u]);
        }
        // chunks past the range carry no flags
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (c0 + static_cast<int64_t>(u) * kWaveStep >= w1) pd[u].h = 0u;
        uint2 ov[kUnroll][2];
        bool oh[kUnroll][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) rank(pd[u], ov[u], oh[u]);
        e_next = wbase + wused;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + static_cast<int64_t>(u) * kWaveStep;
            if (c >= w1) break;
            emit(c, pd[u], ov[u], oh[u]);
        }
    }
}

// --------------------------------------------------------------------------
// Paged pool append.  The call's tokens are first encoded like any tensor
// (records in workspace, binary16 norms with Med3x flags); these kernels
// then move them into the pool.
// --------------------------------------------------------------------------
struct ScatterArgs {
    const uint64_t *offsets;   // the call's batch offsets, slice-major
    const uint32_t *out_pos;   // the call's side list (positions in the call's slice)
    const uint16_t *out_val;
    const int64_t *slots;      // [tokens] pool slot of each call token
    uint16_t *h16;             // the call's norms: flags of dropped entries are cleared
    uint32_t *side_count;
    uint32_t *side_pos;
    uint16_t *side_val;
    uint64_t *status;          // [2] outliers, dropped (may be null)
    int64_t slices, n_slice, num_pages, bps;
    int32_t log2_cpt, log2_page;
    uint32_t cap;
};

// One wave per slice walks the call's entries of that slice in list order
// (position order), 64 at a time.  The entries of one page form one run
// (the call writes a page's tokens consecutively and in order); a run's k-th
// entry goes to index count(page) + k of the page's list, and the run's end
// stores the new count.
__global__ __launch_bounds__(256) void paged_scatter_kernel(ScatterArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t s = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (s >= a.slices) return;   // whole waves
    const uint64_t e0 = a.offsets[s * a.bps], e1 = a.offsets[(s + 1) * a.bps];
    const int64_t nslot = a.num_pages << a.log2_page;
    const uint32_t cmask = (1u << a.log2_cpt) - 1u;
    const int64_t pmask = (int64_t{1} << a.log2_page) - 1;
    uint32_t *count_s = a.side_count + s * a.num_pages;
    int cur_page = -1;    // page of the previous entry (-1: none or skipped)
    uint32_t cur_idx = 0;  // list index the previous run would use next
    uint32_t found = 0, dropped = 0;
    for (uint64_t k = e0; k < e1; k += 64) {
        const uint64_t e = k + static_cast<uint64_t>(lane);
        const bool valid = e < e1;
        const uint32_t pos = valid ? a.out_pos[e] : 0u;
        const int64_t slot = valid ? a.slots[pos >> a.log2_cpt] : -1;
        const bool ok = slot >= 0 && slot < nslot;
        const int page = ok ? static_cast<int>(slot >> a.log2_page) : -1;
        int prev = __shfl_up(page, 1);
        if (lane == 0) prev = cur_page;
        const bool start = ok && page != prev;
        const uint64_t sm = __ballot(start);
        // a run that ended with the previous chunk stores its count now
        if (lane == 0 && cur_page >= 0 && page != cur_page)
            count_s[cur_page] = cur_idx < a.cap ? cur_idx : a.cap;
        const uint64_t upto = lane == 63 ? sm : (sm & ((uint64_t{2} << lane) - 1));
        const int j = upto ? 63 - __clzll(static_cast<long long>(upto)) : -1;
        uint32_t base = 0;
        if (start) {
            const uint32_t n = count_s[page];
            base = n < a.cap ? n : a.cap;
        }
        const uint32_t bj = __shfl(base, j < 0 ? 0 : j);
        const uint32_t idx = j >= 0 ? bj + static_cast<uint32_t>(lane - j) : cur_idx + static_cast<uint32_t>(lane);
        if (ok) {
            ++found;
            if (idx < a.cap) {
                const uint64_t d = static_cast<uint64_t>(s * a.num_pages + page) * a.cap + idx;
                a.side_pos[d] = (static_cast<uint32_t>(slot & pmask) << a.log2_cpt) + (pos & cmask);
                reinterpret_cast<uint2 *>(a.side_val)[d] = reinterpret_cast<const uint2 *>(a.out_val)[e];
            } else {
                ++dropped;   // the chunk keeps its bulk record
                a.h16[s * a.n_slice + pos] = static_cast<uint16_t>(a.h16[s * a.n_slice + pos] & 0x7FFFu);
            }
        }
        // a run that ends inside this chunk (or with the last entry) stores its count
        const int next_page = __shfl_down(page, 1);
        const bool ends = e + 1 == e1 || (lane < 63 && next_page != page);
        if (ok && ends) count_s[page] = idx + 1 < a.cap ? idx + 1 : a.cap;
        const int last = static_cast<int>(e1 - k > 64 ? 63 : e1 - k - 1);
        cur_page = __shfl(page, last);
        cur_idx = __shfl(idx, last) + 1u;
    }
    if (a.status) {
        for (int o = 32; o > 0; o >>= 1) {
            found += __shfl_xor(found, o);
            dropped += __shfl_xor(dropped, o);
        }
        if (lane == 0) {
            atomicAdd(reinterpret_cast<unsigned long long *>(a.status), static_cast<unsigned long long>(found));
            atomicAdd(reinterpret_cast<unsigned long long *>(a.status) + 1, static_cast<unsigned long long>(dropped));
        }
    }
}

struct RowsArgs {
    const uint32_t *idx;       // the call's index rows [slices][tokens][W]
    const uint16_t *h16;       // the call's norms [slices][tokens][cpt]
    const int64_t *slots;
    uint32_t *pool_idx;
    void *pool_norm;
    int64_t slices, tokens, num_pages;
    int32_t log2_page, cpt, bits, words, npack;
};

// Token rows of the call to the pool rows of their slots: one thread per
// output dword (a row is W index words, then cpt / 2 binary16 norm pairs or
// W packed norm words); blockIdx.y walks the slices.  Packed words are
// formed from the compact codes of the (at most five) chunks they hold.
__global__ __launch_bounds__(256) void paged_rows_kernel(RowsArgs a) {
    const int W = a.words;
    const int NH = a.npack ? W : a.cpt / 2;   // norm dwords per row
    const uint32_t per = static_cast<uint32_t>(W + NH);
    const uint32_t total = static_cast<uint32_t>(a.tokens) * per;   // dwords per slice (< 2^32)
    const int64_t nslot = a.num_pages << a.log2_page;
    for (int64_t s = blockIdx.y; s < a.slices; s += gridDim.y) {
        for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < total; e += gridDim.x * 256) {
            const uint32_t t = static_cast<uint32_t>(e) / per;
            const int w = static_cast<int>(static_cast<uint32_t>(e) - t * per);
            const int64_t slot = a.slots[t];
            if (slot < 0 || slot >= nslot) continue;
            const int64_t src = s * a.tokens + t;   // the call's row
            const int64_t dst = s * nslot + slot;   // the pool's row
            if (w < W) {
                a.pool_idx[dst * W + w] = a.idx[src * W + w];
            } else if (!a.npack) {
                const int j = w - W;
                reinterpret_cast<uint32_t *>(a.pool_norm)[dst * NH + j] =
                    reinterpret_cast<const uint32_t *>(a.h16)[src * NH + j];
            } else {
                const int j = w - W;
                const int b = a.bits;
                const uint16_t *hr = a.h16 + src * a.cpt;
                const int c_lo = (32 * j) / b, c_hi = min((32 * j + 31) / b, a.cpt - 1);
                uint32_t word = 0u;
                for (int c = c_lo; c <= c_hi; ++c) {
                    const uint32_t code = compact_norm_code(hr[c], b);
                    const int sft = c * b - 32 * j;
                    word |= sft >= 0 ? code << sft : code >> (-sft);
                }
                reinterpret_cast<uint32_t *>(a.pool_norm)[dst * W + j] = word;
            }
        }
    }
}

__global__ void paged_clear_kernel(uint32_t *side_count, int64_t slices, int64_t num_pages, const int32_t *pages,
                                   int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= slices * n) return;
    const int64_t s = i / n;
    const int32_t pg = pages[i - s * n];
    if (pg >= 0 && pg < num_pages) side_count[s * num_pages + pg] = 0u;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Batches small enough for the single-pass select (its bitmask is in LDS).
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace

bool med3_single_pass(const Geometry &g) { return g.batch_chunks <= kSel1MaxChunks; }

// --------------------------------------------------------------------------
// Launchers.
// --------------------------------------------------------------------------
namespace {
std::atomic<int> g_search_blocks_per_cu{0};
}  // namespace

void set_search_blocks_per_cu(int n) { g_search_blocks_per_cu.store(n, std::memory_order_relaxed); }
int search_blocks_per_cu() { return g_search_blocks_per_cu.load(std::memory_order_relaxed); }

hipError_t launch_encode_search(const Geometry &g, const void *x, const float *codebook,
                                uint32_t *idx, uint16_t *hnorm, const Med3Work *med, hipStream_t st) {
    const int64_t total = g.slices * g.n_slice;
    if (total == 0) return hipSuccess;
    EncArgs a = {};
    a.x = x;
    a.cb = codebook;
    a.idx = idx;
    a.hnorm = hnorm;
    a.n_slice = g.n_slice;
    a.tokens = g.tokens;
    a.S = g.S;
    a.NT = static_cast<int32_t>(ceil_div(g.S, 4));
    a.cpt = g.cpt;
    a.log2_cpt = __builtin_ctz(static_cast<unsigned>(g.cpt));
    a.bits = g.bits;
    a.words = g.words;
    int64_t blocks;
    if (med) {
        // tiles of at most 8192 chunks inside each batch
        int64_t tile = round_up(g.batch_chunks, 256);
        if (tile > 8192) tile = 8192;
        a.tile_chunks = static_cast<int32_t>(tile);
        a.tiles_per_batch = static_cast<int32_t>(ceil_div(g.batch_chunks, tile));
        a.batch_chunks = g.batch_chunks;
        a.bps = g.batches_per_slice;
        a.nbatch = g.slices * g.batches_per_slice;
        a.xcd_map = (a.nbatch % 8 == 0 && a.tiles_per_batch > 1) ? 1 : 0;
        a.hist = med->hist;
        a.tiles_per_slice = 0;
        blocks = a.nbatch * a.tiles_per_batch;
    } else {
        // tiles: multiples of 256 chunks (4 waves x 64), enough blocks to fill
        // 256 CUs several times, at most 8192 chunks so a block's codebook
        // setup stays amortised
        int64_t tile = round_up(ceil_div(total, 4096), 256);
        tile = tile < 256 ? 256 : (tile > 8192 ? 8192 : tile);
        a.tile_chunks = static_cast<int32_t>(tile);
        a.tiles_per_slice = ceil_div(g.n_slice, tile);
        a.batch_chunks = 0;
        blocks = g.slices * a.tiles_per_slice;
    }
    const dim3 grid(static_cast<unsigned>(blocks));
    const dim3 block(kEncThreads);
    const bool m = med != nullptr;
#define HQMQ_ENC(NT, F32, MED) hipLaunchKernelGGL((encode_search_kernel<NT, F32, MED>), grid, block, 0, st, a)
#define HQMQ_ENC_NT(NT)                          \
    do {                                         \
        if (m) HQMQ_ENC(NT, true, true);         \
        else HQMQ_ENC(NT, true, false);          \
    } while (0)
    if (g.f32) {
        if (a.NT == 2) HQMQ_ENC_NT(2);
        else if (a.NT == 8) HQMQ_ENC_NT(8);
        else HQMQ_ENC_NT(0);
    } else {
        return launch_search_h(a, blocks, (g.S + 7) / 8, m, search_blocks_per_cu(), st);
    }
#undef HQMQ_ENC_NT
#undef HQMQ_ENC
    return hipGetLastError();
}

hipError_t launch_med3_scan(int64_t batches, const uint32_t *counts, uint64_t *offsets,
                            uint64_t capacity, uint64_t *status, hipStream_t st) {
    hipLaunchKernelGGL(med3_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, batches, counts, offsets,
                       capacity, status);
    return hipGetLastError();
}

hipError_t launch_med3_select(const Geometry &g, const void *x, uint16_t *hnorm, const Med3Work &med,
                              uint32_t *pwords, hipStream_t st) {
    const int64_t nb = g.slices * g.batches_per_slice;
    if (nb == 0) return hipSuccess;
    SelArgs a;
    a.pwords = med3_single_pass(g) ? pwords : nullptr;
    a.tokens = g.tokens;
    a.log2_cpt = __builtin_ctz(static_cast<unsigned>(g.cpt));
    a.bits = g.bits;
    a.words = g.words;
    a.x = x;
    a.hnorm = hnorm;
    a.hist = med.hist;
    a.counts = med.counts;
    a.mask = med.mask;
    a.mask_words = med.mask_words;
    a.n_slice = g.n_slice;
    a.batch_chunks = g.batch_chunks;
    a.bps = g.batches_per_slice;
    a.C = g.med_C;
    a.f32 = g.f32;
    if (med3_single_pass(g))
        hipLaunchKernelGGL(med3_select1_kernel, dim3(static_cast<unsigned>(nb)), dim3(kSelThreads), 0, st, a);
    else
        hipLaunchKernelGGL(med3_select_kernel, dim3(static_cast<unsigned>(nb)), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_med3_gather(const Geometry &g, const void *x, const Med3Work &med,
                              const uint64_t *offsets, uint16_t *hnorm, uint32_t *out_pos,
                              uint16_t *out_val, uint64_t capacity, hipStream_t st) {
    const int64_t nb = g.slices * g.batches_per_slice;
    if (nb == 0) return hipSuccess;
    GatherArgs a;
    a.x = x;
    a.mask = med.mask;
    a.offsets = offsets;
    a.hnorm = hnorm;
    a.out_pos = out_pos;
    a.out_val = out_val;
    a.capacity = capacity;
    a.n_slice = g.n_slice;
    a.batch_chunks = g.batch_chunks;
    a.bps = g.batches_per_slice;
    a.mask_words = med.mask_words;
    a.f32 = g.f32;
    a.set_flags = med3_single_pass(g) ? 0 : 1;
    hipLaunchKernelGGL(med3_gather_kernel, dim3(static_cast<unsigned>(nb)), dim3(kFlagThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t *p, int64_t n, uint64_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_pack_norms(const Geometry &g, const uint16_t *h16, uint32_t *words, hipStream_t st) {
    const int64_t total = g.slices * g.n_slice;
    if (total == 0) return hipSuccess;
    const int64_t blocks = ceil_div(total, kPackChunks);
    hipLaunchKernelGGL(pack_norms_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPackThreads), 0, st, h16, words,
                       total, static_cast<int32_t>(__builtin_ctz(static_cast<unsigned>(g.cpt))), g.bits, g.words);
    return hipGetLastError();
}

hipError_t launch_paged_scatter(const Geometry &g, const uint64_t *offsets, const uint32_t *out_pos,
                                const uint16_t *out_val, const int64_t *slots, uint16_t *h16,
                                const PagedPool &pool, uint64_t *status, hipStream_t st) {
    if (g.slices == 0 || g.batches_per_slice == 0) return hipSuccess;
    ScatterArgs a;
    a.offsets = offsets;
    a.out_pos = out_pos;
    a.out_val = out_val;
    a.slots = slots;
    a.h16 = h16;
    a.side_count = pool.side_count;
    a.side_pos = pool.side_pos;
    a.side_val = pool.side_val;
    a.status = status;
    a.slices = g.slices;
    a.n_slice = g.n_slice;
    a.num_pages = pool.num_pages;
    a.bps = g.batches_per_slice;
    a.log2_cpt = __builtin_ctz(static_cast<unsigned>(g.cpt));
    a.log2_page = pool.log2_page;
    a.cap = pool.cap;
    hipLaunchKernelGGL(paged_scatter_kernel, dim3(static_cast<unsigned>(ceil_div(g.slices, 4))), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_paged_rows(const Geometry &g, const uint32_t *idx, const uint16_t *h16, const int64_t *slots,
                             const PagedPool &pool, hipStream_t st) {
    const int64_t rows = g.slices * g.tokens;
    if (rows == 0) return hipSuccess;
    RowsArgs a;
    a.idx = idx;
    a.h16 = h16;
    a.slots = slots;
    a.pool_idx = pool.idx;
    a.pool_norm = pool.hnorm;
    a.slices = g.slices;
    a.tokens = g.tokens;
    a.num_pages = pool.num_pages;
    a.log2_page = pool.log2_page;
    a.cpt = g.cpt;
    a.bits = g.bits;
    a.words = g.words;
    a.npack = g.npack;
    const int64_t per = g.words + (g.npack ? g.words : g.cpt / 2);
    const int64_t bx = ceil_div(g.tokens * per, 256);
    const dim3 grid(static_cast<unsigned>(bx < 65536 ? bx : 65536),
                    static_cast<unsigned>(g.slices < 65535 ? g.slices : 65535));
    hipLaunchKernelGGL(paged_rows_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_paged_clear(int64_t slices, const int32_t *pages, int64_t n, const PagedPool &pool,
                              hipStream_t st) {
    if (slices == 0 || n == 0) return hipSuccess;
    hipLaunchKernelGGL(paged_clear_kernel, dim3(static_cast<unsigned>(ceil_div(slices * n, 256))), dim3(256), 0, st,
                       pool.side_count, slices, pool.num_pages, pages, n);
    return hipGetLastError();
}

hipError_t launch_pack_exact(const Geometry &g, const uint32_t *idx32, const uint16_t *h16, uint32_t *groups,
                             hipStream_t st) {
    if (g.slices == 0 || g.tokens == 0) return hipSuccess;
    PackExArgs a;
    a.idx = idx32;
    a.h16 = h16;
    a.out = groups;
    a.tokens = g.tokens;
    a.gps = g.egps;
    a.log2_cpt = __builtin_ctz(static_cast<unsigned>(g.cpt));
    const int gpb = kPackExChunks >> (a.log2_cpt + 2);
    a.blocks_per_slice = ceil_div(g.egps, static_cast<int64_t>(gpb));
    a.bits = g.bits;
    a.words = g.words;
    a.m = g.em;
    a.wl = g.ewl;
    a.fh = g.efh;
    a.gw = g.egw;
    a.nmax = g.enmax;
    a.step = g.estep;
    a.gw_magic = static_cast<uint32_t>(((int64_t{1} << 24) + g.egw - 1) / g.egw);
    a.wl_magic = static_cast<uint32_t>(((int64_t{1} << 20) + g.ewl - 1) / g.ewl);
    a.m_recip = static_cast<uint32_t>(((int64_t{1} << 16) + g.em - 1) / g.em);
    a.log2_fh = __builtin_ctz(static_cast<unsigned>(g.efh));
    if (g.cpt == 32 && (g.em == 6 || g.em == 8)) {
        a.blocks_per_slice = ceil_div(g.egps, static_cast<int64_t>(kPackExThreads / 8));
        const dim3 grid(static_cast<unsigned>(g.slices * a.blocks_per_slice));
        if (g.em == 8) hipLaunchKernelGGL(pack_exact32_kernel<8>, grid, dim3(kPackExThreads), 0, st, a);
        else hipLaunchKernelGGL(pack_exact32_kernel<6>, grid, dim3(kPackExThreads), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(pack_exact_kernel, dim3(static_cast<unsigned>(g.slices * a.blocks_per_slice)),
                       dim3(kPackExThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode(const Geometry &g, const uint32_t *idx, const void *hnorm,
                         const uint64_t *offsets, const uint32_t *out_pos, const uint16_t *out_val,
                         uint64_t capacity, const float *codebook, void *y, hipStream_t st) {
    const int64_t total = g.slices * g.n_slice;
    if (total == 0) return hipSuccess;
    // block ranges: multiples of 512 chunks (4 waves x 128), enough blocks
    // to fill the chip, at most 16384 chunks
    int64_t wgc = round_up(ceil_div(total, 4096), 2 * kDecThreads);
    wgc = wgc < 2 * kDecThreads ? 2 * kDecThreads : (wgc > 16384 ? 16384 : wgc);
    DecArgs a;
    a.idx = idx;
    a.hnorm = hnorm;
    a.offsets = offsets;
    a.out_pos = out_pos;
    a.out_val = out_val;
    a.capacity = capacity;
    a.cb = codebook;
    a.y = y;
    a.n_slice = g.n_slice;
    a.tokens = g.tokens;
    a.wg_chunks = wgc;
    a.wg_per_slice = ceil_div(g.n_slice, wgc);
    a.batch_chunks = g.batch_chunks;
    a.bps = g.batch_chunks > 0 ? g.batches_per_slice : 0;
    a.S = g.S;
    a.cpt = g.cpt;
    a.log2_cpt = __builtin_ctz(static_cast<unsigned>(g.cpt));
    a.bits = g.bits;
    a.words = g.words;
    const dim3 grid(static_cast<unsigned>(g.slices * a.wg_per_slice));
    const dim3 block(kDecThreads);
    a.gps = g.egps;
    a.m = g.em;
    a.wl = g.ewl;
    a.fh = g.efh;
    a.gw = g.egw;
    a.step = g.estep;
    const bool table = g.S <= kTableMaxS;
    const size_t lds = (table ? 24 * static_cast<size_t>(g.S) : static_cast<size_t>(g.S)) * sizeof(f32x4);
    const int nf = g.exact ? kNormExact : (g.npack ? kNormPacked : kNormF16);
    const void *k = nullptr;
    // exact-rate records of head_dim 128 at m = 6 or 8 (S = 8, 32): whole
    // groups per wave step
    const bool grouped = g.exact && g.cpt == 32 && (g.em == 6 || g.em == 8) && g.ewl == g.em && g.efh == 4 &&
                         g.egw == 8 * g.em + 13;
    auto pick = [&](auto f32out) {
        constexpr bool F = decltype(f32out)::value;
        if (nf == kNormExact && grouped && table)
            k = g.em == 8 ? reinterpret_cast<const void *>(&decode_kernel<F, true, kNormExact, 8>)
                          : reinterpret_cast<const void *>(&decode_kernel<F, true, kNormExact, 6>);
        else if (nf == kNormExact)
            k = table ? reinterpret_cast<const void *>(&decode_kernel<F, true, kNormExact>)
                      : reinterpret_cast<const void *>(&decode_kernel<F, false, kNormExact>);
        else if (nf == kNormPacked)
            k = table ? reinterpret_cast<const void *>(&decode_kernel<F, true, kNormPacked>)
                      : reinterpret_cast<const void *>(&decode_kernel<F, false, kNormPacked>);
        else
            k = table ? reinterpret_cast<const void *>(&decode_kernel<F, true, kNormF16>)
                      : reinterpret_cast<const void *>(&decode_kernel<F, false, kNormF16>);
    };
    if (g.f32) pick(std::true_type{});
    else pick(std::false_type{});
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(k, grid, block, args, lds, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace hqmq
