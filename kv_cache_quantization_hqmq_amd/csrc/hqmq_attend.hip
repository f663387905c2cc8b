// Decode-step attention read straight from HQMQ records, for AMD Instinct
// MI355X (gfx950).
//
// The pages' latency result (gist.science/nl "Technische Samenvatting",
// "Memory en Latentie"; gist.science/pt "Memória e Latência") is a fused
// kernel that decodes K and V inside the attention loop instead of
// dequantising the whole cache every step.  This file is that operation:
// for one layer, every sequence b and query head j (reading KV head
// j / group),
//
//     out[b][j] = sum_t softmax_t(scale <q[b][j], k_t>) v_t,
//
// over the sequence's tokens of the encoded cache, where k_t and v_t are the
// fp16 values the decode kernel writes (bulk chunks 2 h (q_p * q_s) rounded
// to binary16, h the record's half-norm, stored as binary16 or as a packed
// compact code; Med3x outlier chunks their side-list values).
//
// Layout of the work.  A block takes one (sequence, KV head, token split);
// each of its 8 waves walks a contiguous eighth of the split in tiles of 16
// tokens: it decodes the tile's K and V chunks from the records into LDS
// (the same arithmetic as the decode kernel, so the values are bit-identical),
// computes the 16 x 16 score tile S[token][query head] with
// v_mfma_f32_16x16x16f16 (exact fp16 products, fp32 sums), updates an online
// softmax in fp32, and accumulates O^T[dim][head] += V^T P^T with the same
// MFMA, P in binary16 scaled by 2^15 (normal down to p = 2^-29).  The
// normaliser sums the same rounded weights, so the result is an exact convex
// combination of the v_t up to that weight rounding.  Waves and splits are
// merged by log-sum-exp; a second kernel combines the splits of each head.
#include <hip/hip_runtime.h>

#include "hqmq_device.h"
#include "hqmq_launch.h"

namespace hqmq {
namespace {

// 8 waves per block share the block's codeword tables: 66.6 KB of LDS, two
// blocks (16 waves) per CU, which the kernel's 128-VGPR budget allows
constexpr int kAttThreads = 512;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kTile = 16;            // tokens per wave step (one MFMA tile)
// Softmax weights enter the value sum as binary16 2^(s - m + kPScale), m a
// reference max that is raised only when a score exceeds it by more than
// kLazy (log2 units): weights stay below 2^(kPScale + kLazy) = 2^15 and stay
// normal down to 2^(-14 - kPScale) of the reference, and the accumulators are
// rescaled only when the reference moves.
constexpr float kPScale = 8.0f;
constexpr float kLazy = 7.0f;
constexpr int kAttTableMaxS = 64;    // the 24 S codewords of K and V in LDS up to here

// Code width of S secondary codewords (b = ceil(log2(24 S))) and the width
// the kernel is specialised for (0: any width).
inline int attend_code_bits(int S) {
    int b = 0;
    while ((1 << b) < 24 * S) ++b;
    return b;
}
inline int attend_kernel_bits(int S, bool table) {
    const int b = attend_code_bits(S);
    return table && (b == 10 || b == 8) ? b : 0;
}

struct AttArgs {
    AttRole r[2];               // K, V
    const uint16_t *q;          // [batch][heads * group][D] binary16
    const int64_t *seq_start;   // [batch] first token of each sequence in the slice
    const int32_t *seq_len;     // [batch]
    float *part;                // [batch][heads * group][nsplit][D + 2]: m, l, o[D]
    int64_t tokens;             // tokens per slice
    int64_t batch_chunks;       // Med3x batch length in chunks (0: off)
    int64_t bps;                // Med3x batches per slice
    int32_t layer, heads, group, nsplit, split_tokens, max_len, S, bits, words;
    float qscale;               // scale * log2(e)
    // paged pools (PAGED kernels): [batch][pt_stride] page ids, P = 2^log2_page
    const int32_t *page_table;
    int64_t num_pages;
    int32_t pt_stride, log2_page;
    uint32_t page_cap;          // side-list entries per (layer, head, page)
    // exact-rate records (NF == kNormExact): idx holds [slices][gps][gw] groups
    int64_t gps;
    int32_t m, wl, fh, gw;
    float step;
};  // r[].hnorm: binary16 half-norms, or packed compact codes (NF == kNormPacked)

// Norm formats: binary16 half-norms, packed compact codes, exact-rate groups.
constexpr int kNormF16 = 0, kNormPacked = 1, kNormExact = 2;

// First entry in [lo, hi) of a position-sorted side list whose position is
// at least p0 (hi when none): a 64-way search per round.
__device__ uint64_t search_first(const uint32_t *out_pos, uint64_t lo, uint64_t hi, int64_t p0, int lane) {
    while (hi > lo) {
        const uint64_t len = hi - lo;
        const uint64_t step = (len + 63) / 64;
        const uint64_t i = lo + static_cast<uint64_t>(lane) * step;
        const bool below = i < hi && static_cast<int64_t>(out_pos[i]) < p0;
        const int cnt = __popcll(__ballot(below));
        if (cnt == 0) break;
        const uint64_t nlo = lo + static_cast<uint64_t>(cnt - 1) * step + 1;
        const uint64_t nhi = lo + static_cast<uint64_t>(cnt) * step;
        hi = nhi < hi ? nhi : hi;
        lo = nlo;
    }
    return lo;
}

// First side-list entry of slice sl at or after position p0, among the
// entries of the Med3x batches that overlap [p0, p1); *e_end receives the
// end of those entries.
__device__ uint64_t first_entry(const AttRole &r, int64_t sl, int64_t bps, int64_t batch_chunks, int64_t p0,
                                int64_t p1, uint64_t *e_end, int lane) {
    *e_end = 0;
    if (bps <= 0 || p0 >= p1) return 0;
    const int64_t bl = p0 / batch_chunks;
    const int64_t bh = (p1 - 1) / batch_chunks;
    uint64_t lo = r.offsets[sl * bps + bl];
    uint64_t hi = r.offsets[sl * bps + bh + 1];
    hi = hi < r.capacity ? hi : r.capacity;
    lo = lo < hi ? lo : hi;
    *e_end = hi;
    return search_first(r.out_pos, lo, hi, p0, lane);
}

// Paged pool: the side list of page slot ps = slice * num_pages + page is
// entries [ps * cap, ps * cap + min(count, cap)).
__device__ __forceinline__ void page_list(const AttRole &r, int64_t ps, uint32_t cap, uint64_t *lo, uint64_t *hi) {
    const uint32_t n = r.side_count[ps];
    *lo = static_cast<uint64_t>(ps) * cap;
    *hi = *lo + (n < cap ? n : cap);
}

template <int D>
struct AttShape {
    static constexpr int CPT = D / 4;              // chunks per token
    static constexpr int CPL = CPT / 4;            // chunks per lane of a 16-token tile
    static constexpr int KB = D / 16;              // 16-dim blocks
    static constexpr int NU = D / 64;              // chunk groups per lane in the V operand
    // bytes per decoded token row: 8 bytes of padding put the 16 rows a
    // K-operand read touches on distinct LDS banks (measured: padding 0 is
    // 1.8x slower, 16 and 48 about 2-3% slower, 64 1.4x slower)
    static constexpr int ROWB = CPT * 8 + 8;
    static constexpr int TILEB = kTile * ROWB;     // bytes per decoded tile
    static constexpr int MERGEB = (32 + 16 * D) * 4;   // a wave's m, l and o for the merge
};

// Record words of one role's 16-token tile held by one lane: the half-norm
// codes of its CPL chunks and the index words holding their codes (BITS > 0:
// the NW consecutive row words from the first code's word; BITS = 0, any code
// width: two words per chunk pair).  Packed norms (NPACK) sit at the same word
// places as the index codes and are held the same way.
constexpr int max_code_shift(int cpl, int bits) {
    int m = 0;
    for (int q = 0; q < 4; ++q) m = ((q * cpl * bits) & 31) > m ? ((q * cpl * bits) & 31) : m;
    return m;
}

// Whether every lane's NW words lie inside its token row.
constexpr bool words_in_row(int cpl, int bits, int nw) {
    for (int q = 0; q < 4; ++q)
        if ((q * cpl * bits) / 32 + nw > (4 * cpl * bits + 31) / 32) return false;
    return true;
}

template <int D, int BITS, int NF>
struct TileRegs {
    static constexpr int CPL = D / 16;
    static constexpr bool EXACT = NF == kNormExact;
    // exact-rate records: BITS is m (0: any m up to 13); a window of NWL
    // words holds the lane's low bits of one plane, 2 words its digit fields
    static constexpr int NWL = BITS > 0 ? (max_code_shift(CPL, BITS) + CPL * BITS + 31) / 32
                                        : (31 + CPL * 13 + 31) / 32;
    static constexpr int NW = EXACT ? NWL + 2
                                    : (BITS > 0 ? (max_code_shift(CPL, BITS) + CPL * BITS + 31) / 32 : CPL);
    static_assert(EXACT || BITS == 0 || words_in_row(CPL, BITS, NW), "a lane's words must stay in its row");
    // binary16 code pairs, packed norm words, or (exact) the norm plane's
    // low-bit and digit windows
    uint32_t hw[NF == kNormF16 ? CPL / 2 : NW];
    uint32_t w[NW];   // index words (exact: low-bit window, then digit window)
    uint32_t dsh[EXACT ? 1 : 0];   // exact: bit offsets of the index | norm << 8 digit fields
};

// Waves per SIMD the register budget is set for: two 8-wave blocks per CU
// (128 VGPRs) where the LDS of two blocks fits, i.e. head_dim <= 128 with the
// 2^BITS-entry tables of a fixed code width; one block (256 VGPRs, no
// spills) otherwise.
constexpr int attend_waves_per_eu(int D, bool table, int bits) { return D <= 128 && table && bits > 0 ? 4 : 2; }

template <int D, bool TABLE, int BITS, int NF, bool PAGED>
__global__ __launch_bounds__(kAttThreads)
__attribute__((amdgpu_waves_per_eu(attend_waves_per_eu(D, TABLE, BITS), attend_waves_per_eu(D, TABLE, BITS))))
void attend_split_kernel(AttArgs a) {
    using Sh = AttShape<D>;
    constexpr int CPT = Sh::CPT, CPL = Sh::CPL, KB = Sh::KB, NU = Sh::NU, ROWB = Sh::ROWB, TILEB = Sh::TILEB;
    constexpr bool NPACK = NF == kNormPacked;
    constexpr bool EXACT = NF == kNormExact;   // BITS is then m (0: any)
    static_assert(!(EXACT && PAGED), "paged pools keep whole-bit token rows");

    extern __shared__ f32x4 smem[];
    // codeword tables: TABLE kernels of a fixed code width hold all 2^BITS
    // codes (zeros past 24 S), so a code read from the records needs no clamp
    const int ntab = TABLE ? ((BITS > 0 && !EXACT) ? (1 << BITS) : 24 * a.S) : a.S;
    f32x4 *tab = smem;                                                     // [2][ntab]
    unsigned char *tiles = reinterpret_cast<unsigned char *>(smem + 2 * ntab);   // [waves][TILEB]

    const int nsplit = a.nsplit;
    const int64_t bh = blockIdx.x / nsplit;
    const int split = static_cast<int>(blockIdx.x - bh * nsplit);
    const int b = static_cast<int>(bh / a.heads);
    const int h = static_cast<int>(bh - static_cast<int64_t>(b) * a.heads);
    const int G = a.group;
    const int64_t Hq = static_cast<int64_t>(a.heads) * G;
    const int64_t sl = static_cast<int64_t>(a.layer) * a.heads + h;

    // the sequence's tokens, clamped to the slice (paged: to its page table)
    int64_t start = 0;
    int64_t len = a.seq_len[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    if constexpr (PAGED) {
        const int64_t most = static_cast<int64_t>(a.pt_stride) << a.log2_page;
        len = len < most ? len : most;
    } else {
        start = a.seq_start[b];
        if (start < 0 || start > a.tokens) len = 0;
        else len = len < a.tokens - start ? len : a.tokens - start;
    }
    const int64_t t_lo = static_cast<int64_t>(split) * a.split_tokens;
    const int64_t t_hi = t_lo + a.split_tokens < len ? t_lo + a.split_tokens : len;
    float *part = a.part + ((static_cast<int64_t>(b) * Hq + static_cast<int64_t>(h) * G) * nsplit + split) * (D + 2);
    const int64_t pstride = static_cast<int64_t>(nsplit) * (D + 2);   // between query heads
    if (t_lo >= t_hi) {
        for (int i = threadIdx.x; i < G * (D + 2); i += kAttThreads) {
            const int n = i / (D + 2), e = i - n * (D + 2);
            part[n * pstride + e] = e == 0 ? -INFINITY : 0.0f;
        }
        return;
    }

    // codeword tables of K and V: TABLE: 2 (a_p * q_s) for the 24 S codes,
    // else the S secondary codewords
    for (int r = 0; r < 2; ++r) {
        const float *q = a.r[r].cb + sl * a.S * 4;
        for (int k = threadIdx.x; k < ntab; k += kAttThreads) {
            if constexpr (TABLE) {
                if (k >= 24 * a.S) {
                    tab[r * ntab + k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    continue;
                }
                const int s = k / 24;
                const float qe[4] = {double_f16(q[4 * s]), double_f16(q[4 * s + 1]), double_f16(q[4 * s + 2]),
                                     double_f16(q[4 * s + 3])};
                tab[r * ntab + k] = 2.0f * codeword_f32(qe, k - 24 * s);
            } else {
                const f32x4 v = {double_f16(q[4 * k]), double_f16(q[4 * k + 1]), double_f16(q[4 * k + 2]),
                                 double_f16(q[4 * k + 3])};
                tab[r * ntab + k] = v;
            }
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    // the wave index is uniform in a wave: say so, so that the wave's token
    // range, tile bases and side-list cursors live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t wq = a.split_tokens / kAttWaves;   // a multiple of the tile
    const int64_t w_lo = t_lo + wave * wq < t_hi ? t_lo + wave * wq : t_hi;
    const int64_t w_hi = w_lo + wq < t_hi ? w_lo + wq : t_hi;
    unsigned char *tt = tiles + wave * TILEB;   // this wave's decoded tile (K, then V)
    const int n = lane & 15;     // query head within the group (MFMA column)
    const int g = lane >> 4;     // lane group

    // query operand of S = K q: B[k = 4 g + j][n] = q[head n][16 kb + 4 g + j]
    f16x4 qv[KB];
    {
        const uint16_t *qp = a.q + (static_cast<int64_t>(b) * Hq + static_cast<int64_t>(h) * G + (n < G ? n : 0)) * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint2 u = n < G ? *reinterpret_cast<const uint2 *>(qp + 16 * kb + 4 * g) : make_uint2(0u, 0u);
            qv[kb] = __builtin_bit_cast(f16x4, u);
        }
    }

    // Paged pool: token t of the sequence lies on page page_of(t) (ids are
    // clamped into the pool), at row page_slot * P + t % P of the pool.
    const int32_t *ptab = PAGED ? a.page_table + static_cast<int64_t>(b) * a.pt_stride : nullptr;
    const int64_t page_mask = (int64_t{1} << a.log2_page) - 1;
    auto page_slot = [&](int64_t t) -> int64_t {
        int64_t pg = ptab[t >> a.log2_page];
        pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
        return sl * a.num_pages + pg;
    };

    // paged: the slot of the page the next tile lies on, and the slot and
    // side-list bounds of the page after it (requested a page ahead, so no
    // tile waits on the page table or a page's entry count)
    int64_t ps_now = 0, ps_ahead = 0;
    uint64_t ahead_lo[2] = {0, 0}, ahead_hi[2] = {0, 0};
    auto fetch_ahead = [&](int64_t t) {   // t: the first token of a page
        if (t < w_hi) {
            ps_ahead = page_slot(t);
            page_list(a.r[0], ps_ahead, a.page_cap, &ahead_lo[0], &ahead_hi[0]);
            page_list(a.r[1], ps_ahead, a.page_cap, &ahead_lo[1], &ahead_hi[1]);
        }
    };
    if constexpr (PAGED) {
        if (w_lo < w_hi) {
            ps_now = page_slot(w_lo);
            fetch_ahead((w_lo | page_mask) + 1);
        }
    }

    // side-list cursors of K and V for this wave's tokens
    uint64_t cur[2] = {0, 0}, end[2] = {0, 0};
    if constexpr (PAGED) {
        if (w_lo < w_hi) {
            const int64_t ps = page_slot(w_lo);
            const int64_t p0 = (w_lo & page_mask) * CPT;
            for (int r = 0; r < 2; ++r) {
                uint64_t lo, hi;
                page_list(a.r[r], ps, a.page_cap, &lo, &hi);
                cur[r] = search_first(a.r[r].out_pos, lo, hi, p0, lane);
                end[r] = hi;
            }
        }
    } else {
        const int64_t p0 = (start + w_lo) * CPT, p1 = (start + w_hi) * CPT;
        cur[0] = first_entry(a.r[0], sl, a.bps, a.batch_chunks, p0, p1, &end[0], lane);
        cur[1] = first_entry(a.r[1], sl, a.bps, a.batch_chunks, p0, p1, &end[1], lane);
    }

    const uint32_t kmask = (1u << a.bits) - 1u;
    const uint32_t kmax = static_cast<uint32_t>(24 * a.S - 1);
    const int last_word = a.words - 1;

    // Lane l decodes token l % 16 of a 16-token tile, chunks (l / 16) CPL ..
    // + CPL - 1: the 16 lanes that store together write 16 different rows,
    // so their stores fall on distinct LDS banks.  The records of tile t + 1
    // are loaded while tile t is decoded and used (two register sets, used in
    // turn), and each role keeps the next 64 side-list entries in registers
    // (one per lane), loaded one tile ahead.
    const int ti = lane & 15;
    const int c0 = (lane >> 4) * CPL;
    const int em = BITS > 0 ? BITS : a.m;   // exact-rate records: low bits per code
    const int cbits = BITS > 0 ? BITS : a.bits;
    const uint32_t sh0 = static_cast<uint32_t>(c0 * cbits) & 31u;
    const int w0 = (c0 * cbits) >> 5;
    const int64_t row0 = sl * a.tokens + start;   // the sequence's first token row (contiguous)
    // row of the sequence's token t (the first of a tile: a tile never
    // straddles pages)
    auto tile_row = [&](int64_t t) -> int64_t {
        if constexpr (PAGED) return (page_slot(t) << a.log2_page) + (t & page_mask);
        else return row0 + t;
    };

    // Loads are unconditional (lanes past a tile's end read the tile's last
    // valid row and are masked when decoded) and address a tile base common
    // to the wave plus a per-lane offset, so that the compiler keeps them in
    // flight across the decode of the current tile.
    auto load_tile = [&](int r, int64_t tb, int nvalid, TileRegs<D, BITS, NF> &tr) {
        const AttRole &R = a.r[r];
        const uint32_t ri = static_cast<uint32_t>(nvalid > 0 ? (ti < nvalid ? ti : nvalid - 1) : 0);
        if constexpr (EXACT) {
            // the tile's rows lie in at most 5 groups from the one holding
            // slice token tb - sl * tokens; lane token ri is row (st & 3) of
            // group st / 4 (the buffer resource's range spans those groups)
            using TR = TileRegs<D, BITS, NF>;
            const int64_t st0 = tb - sl * a.tokens;
            const uint32_t st = static_cast<uint32_t>(st0 & 3) + ri;   // token relative to the first group
            // (the range ends at the slice's last group: window words past it read 0)
            const int64_t ng = a.gps - (st0 >> 2) < 5 ? a.gps - (st0 >> 2) : 5;
            const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint32_t *>(R.idx + (sl * a.gps + (st0 >> 2)) * a.gw), 0,
                static_cast<int>(ng * a.gw * 4), kBufWord3);
            const uint32_t rr = st & 3u;
            const uint32_t gbase = __umul24(st >> 2, static_cast<uint32_t>(a.gw));
            const uint32_t lbit = static_cast<uint32_t>(c0 * em);
            const uint32_t lk = gbase + __umul24(rr, static_cast<uint32_t>(a.wl)) + (lbit >> 5);
            const uint32_t ln = lk + 4u * static_cast<uint32_t>(a.wl);
            const uint32_t fk = static_cast<uint32_t>(kFieldBits) *
                                (__umul24(2u * static_cast<uint32_t>(a.fh), rr) + static_cast<uint32_t>(c0 / kDigitsPerField));
            const uint32_t fn = fk + static_cast<uint32_t>(kFieldBits * a.fh);
            const uint32_t dbase = gbase + 8u * static_cast<uint32_t>(a.wl);
            tr.dsh[0] = (fk & 31u) | ((fn & 31u) << 8);
#pragma unroll
            for (int k = 0; k < TR::NWL; ++k) {
                tr.w[k] = __builtin_amdgcn_raw_buffer_load_b32(gr, static_cast<int>((lk + k) * 4u), 0, 0);
                tr.hw[k] = __builtin_amdgcn_raw_buffer_load_b32(gr, static_cast<int>((ln + k) * 4u), 0, 0);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                tr.w[TR::NWL + k] = __builtin_amdgcn_raw_buffer_load_b32(gr, static_cast<int>((dbase + (fk >> 5) + k) * 4u), 0, 0);
                tr.hw[TR::NWL + k] = __builtin_amdgcn_raw_buffer_load_b32(gr, static_cast<int>((dbase + (fn >> 5) + k) * 4u), 0, 0);
            }
            return;
        }
        // buffer resources over the tile's rows (wave-uniform bases; lanes
        // add 32-bit offsets, fixed word offsets go in the instructions)
        const int words = a.words;
        const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(R.idx + tb * words), 0, kTile * words * 4, kBufWord3);
        if constexpr (NPACK) {
            // the norm words at the index words' places (loaded below)
        } else {
            const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(R.hnorm + tb * CPT), 0, kTile * CPT * 2, kBufWord3);
            const int ho = static_cast<int>((__umul24(ri, static_cast<uint32_t>(CPT)) + static_cast<uint32_t>(c0)) * 2u);
            if constexpr (CPL == 4) {
                const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(hr, ho, 0, 0);
                tr.hw[0] = u[0];
                tr.hw[1] = u[1];
            } else {
#pragma unroll
                for (int v = 0; v < CPL / 8; ++v) {
                    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(hr, ho + 16 * v, 0, 0);
                    tr.hw[4 * v] = u[0];
                    tr.hw[4 * v + 1] = u[1];
                    tr.hw[4 * v + 2] = u[2];
                    tr.hw[4 * v + 3] = u[3];
                }
            }
        }
        const __amdgpu_buffer_rsrc_t nr = NPACK ? __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(reinterpret_cast<const uint32_t *>(R.hnorm) + tb * words), 0, kTile * words * 4,
            kBufWord3) : ir;
        const uint32_t ro = __umul24(ri, static_cast<uint32_t>(words));
        if constexpr (BITS > 0) {
            const int lo = static_cast<int>((ro + static_cast<uint32_t>(w0)) * 4u);
#pragma unroll
            for (int k = 0; k < TileRegs<D, BITS, NF>::NW; ++k) {
                tr.w[k] = __builtin_amdgcn_raw_buffer_load_b32(ir, lo + 4 * k, 0, 0);
                if constexpr (NPACK) tr.hw[k] = __builtin_amdgcn_raw_buffer_load_b32(nr, lo + 4 * k, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < CPL; j += 2) {
                const int w = ((c0 + j) * a.bits) >> 5;
                const int o0 = static_cast<int>((ro + static_cast<uint32_t>(w)) * 4u);
                const int o1 = static_cast<int>((ro + static_cast<uint32_t>(w + 1 < last_word ? w + 1 : last_word)) * 4u);
                tr.w[j] = __builtin_amdgcn_raw_buffer_load_b32(ir, o0, 0, 0);
                tr.w[j + 1] = __builtin_amdgcn_raw_buffer_load_b32(ir, o1, 0, 0);
                if constexpr (NPACK) {
                    tr.hw[j] = __builtin_amdgcn_raw_buffer_load_b32(nr, o0, 0, 0);
                    tr.hw[j + 1] = __builtin_amdgcn_raw_buffer_load_b32(nr, o1, 0, 0);
                }
            }
        }
    };

    // entries at and past end[r] are never used; lanes past it read a valid
    // address (the last entry, or, when there is none, the first 8 bytes of
    // the block's query rows, which every launch with work has: the exact
    // format has no norm plane to point at)
    uint64_t sv[2];   // side-list entries cur[r] + lane: values (4 x fp16)
    uint32_t sp[2];   // and positions
    auto load_window = [&](int r) {
        const uint64_t left = end[r] - cur[r];   // entries from cur[r] on (end >= cur)
        const uint32_t last = left > 64u ? 63u : (left > 0u ? static_cast<uint32_t>(left) - 1u : 0u);
        const bool any = left > 0u;
        const uint64_t *vb = any ? reinterpret_cast<const uint64_t *>(a.r[r].out_val) + cur[r]
                                 : reinterpret_cast<const uint64_t *>(a.q);
        const uint32_t *pb = any ? a.r[r].out_pos + cur[r] : reinterpret_cast<const uint32_t *>(a.q);
        const uint32_t li = static_cast<uint32_t>(lane);
        sv[r] = vb[li < last ? li : last];
        sp[r] = pb[li < last ? li : last];
    };
    load_window(0);
    load_window(1);

    // Decode a loaded tile of role r into dst[token][chunk] (fp16), with the
    // decoder's arithmetic: 2 hnorm (a_p * q_s) in fp32, rounded to binary16.
    // the lane's CPL codes from its record words (index or packed norm)
    using Words = uint32_t[TileRegs<D, BITS, NF>::NW];
    auto extract = [&](const Words &tw, uint32_t (&out)[CPL]) {
        if constexpr (BITS > 0) {
            constexpr int NW = TileRegs<D, BITS, NF>::NW;
            uint32_t nw[NW];   // the lane's codes from bit 0
#pragma unroll
            for (int k = 0; k + 1 < NW; ++k) nw[k] = __builtin_amdgcn_alignbit(tw[k + 1], tw[k], sh0);
            nw[NW - 1] = tw[NW - 1] >> sh0;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                constexpr uint32_t m = (1u << BITS) - 1u;
                const int p = j * BITS, k = p >> 5, sft = p & 31;
                if (sft + BITS <= 32) out[j] = (nw[k] >> sft) & m;
                else out[j] = __builtin_amdgcn_alignbit(nw[k + 1], nw[k], sft) & m;
            }
        } else {
#pragma unroll
            for (int j = 0; j < CPL; j += 2) {
                const int o = (c0 + j) * a.bits;
                const uint64_t win = ((static_cast<uint64_t>(tw[j + 1]) << 32) | tw[j]) >> (o & 31);
                out[j] = static_cast<uint32_t>(win) & kmask;
                out[j + 1] = static_cast<uint32_t>(win >> a.bits) & kmask;
            }
        }
    };

    // exact-rate records: the lane's CPL full codes of one plane from its
    // low-bit window (words 0 .. NWL-1, chunk c0's bits first) and digit
    // window (words NWL, NWL+1): code = 2^m d + l
    // (its body is compiled for exact-rate instantiations only: the others
    // hold no digit window)
    auto extract_exact = [&](const Words &tw, uint32_t dsh, uint32_t (&out)[CPL]) {
        using TR = TileRegs<D, BITS, NF>;
        if constexpr (TR::EXACT) {
            constexpr int NWL = TR::NWL;
            const uint32_t sh = static_cast<uint32_t>(c0 * em) & 31u;
            const uint32_t lmask = (1u << em) - 1u;
            if constexpr (BITS > 0) {
                // the window from the lane's first bit, then fields at fixed places
                uint32_t nw[NWL];
#pragma unroll
                for (int k = 0; k + 1 < NWL; ++k) nw[k] = __builtin_amdgcn_alignbit(tw[k + 1], tw[k], sh);
                nw[NWL - 1] = tw[NWL - 1] >> sh;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int p = j * BITS, k = p >> 5, sft = p & 31;
                    if (sft + BITS <= 32) out[j] = (nw[k] >> sft) & lmask;
                    else out[j] = __builtin_amdgcn_alignbit(nw[k + 1], nw[k], sft) & lmask;
                }
            } else {
                // any m: each field's two words picked from the window
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const uint32_t p = sh + static_cast<uint32_t>(j * em);
                    const uint32_t k = p >> 5;
                    uint32_t wlo = tw[0], whi = NWL > 1 ? tw[1] : 0u;
#pragma unroll
                    for (int q = 1; q < NWL; ++q) {
                        wlo = k == static_cast<uint32_t>(q) ? tw[q] : wlo;
                        whi = k + 1 == static_cast<uint32_t>(q) ? tw[q] : whi;
                    }
                    out[j] = __builtin_amdgcn_alignbit(whi, wlo, p & 31u) & lmask;
                }
            }
            // digit fields: CPL / 8 whole fields (CPL >= 8), or half of one
            uint32_t v = __builtin_amdgcn_alignbit(tw[NWL + 1], tw[NWL], dsh);
            if constexpr (CPL >= kDigitsPerField) {
#pragma unroll
                for (int f = 0; f < CPL / kDigitsPerField; ++f) {
                    uint32_t q = (v >> (kFieldBits * f)) & 0x1FFFu;
#pragma unroll
                    for (int i = 0; i < kDigitsPerField; ++i) {
                        const uint32_t q3 = div3_small(q);
                        out[f * kDigitsPerField + i] |= (q - 3u * q3) << em;
                        q = q3;
                    }
                }
            } else {
                uint32_t q = v & 0x1FFFu;
                if (c0 & 4) q = __umul24(q, 207127u) >> 24;   // skip digits 0..3: q / 81
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const uint32_t q3 = div3_small(q);
                    out[i] |= (q - 3u * q3) << em;
                    q = q3;
                }
            }
        }
    };

    // (after the tile: the cursor moves to the next page's list first when
    // the next tile starts a page, paged pools only)
    // (plo: slice position, or page position when paged, of the tile's
    // first chunk; rows at and past nvalid hold copies of a valid row)
    auto decode_tile = [&](int r, const TileRegs<D, BITS, NF> &tr, int nvalid, unsigned char *dst, uint32_t plo,
                           bool newpage, uint64_t nlo, uint64_t nhi) {
        uint32_t hw[CPL / 2];
        uint32_t code[CPL];
        if constexpr (EXACT) {
            uint32_t nc[CPL];
            extract_exact(tr.hw, (tr.dsh[0] >> 8) & 31u, nc);
            const uint32_t flag = (3u << em) - 1u;
#pragma unroll
            for (int v = 0; v < CPL / 2; ++v)
                hw[v] = exact_norm_h16(nc[2 * v], flag, a.step) | (exact_norm_h16(nc[2 * v + 1], flag, a.step) << 16);
            extract_exact(tr.w, tr.dsh[0] & 31u, code);
        } else {
            if constexpr (NPACK) {
                uint32_t nc[CPL];
                extract(tr.hw, nc);
                const int nbits = BITS > 0 ? BITS : a.bits;
#pragma unroll
                for (int v = 0; v < CPL / 2; ++v)
                    hw[v] = compact_norm_h16(nc[2 * v], nbits) | (compact_norm_h16(nc[2 * v + 1], nbits) << 16);
            } else {
#pragma unroll
                for (int v = 0; v < CPL / 2; ++v) hw[v] = tr.hw[v];
            }
            extract(tr.w, code);
        }
        if constexpr (!(TABLE && BITS > 0) || EXACT) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) code[j] = code[j] < kmax ? code[j] : kmax;
        }
        // two halves of the lane's chunks: lookups, products and stores of
        // one half at a time keep fewer values live
        uint2 *dp = reinterpret_cast<uint2 *>(dst + ti * ROWB + c0 * 8);
        constexpr int HC = CPL >= 8 ? CPL / 2 : CPL;
#pragma unroll
        for (int j0 = 0; j0 < CPL; j0 += HC) {
            f32x4 cw[HC];   // TABLE: 2 (a_p * q_s); else a_p * q_s
#pragma unroll
            for (int jj = 0; jj < HC; ++jj) {
                const int j = j0 + jj;
                if constexpr (TABLE) {
                    cw[jj] = tab[r * ntab + code[j]];
                } else {
                    const int s = static_cast<int>(code[j] / 24u);
                    const f32x4 qs = tab[r * ntab + s];
                    const float qa[4] = {qs[0], qs[1], qs[2], qs[3]};
                    cw[jj] = codeword_f32(qa, static_cast<int>(code[j]) - 24 * s);
                }
            }
#pragma unroll
            for (int jj = 0; jj < HC; ++jj) {
                const int j = j0 + jj;
                const float hv = f16_bits_to_f32(static_cast<uint16_t>((hw[j >> 1] >> (16 * (j & 1))) & 0x7FFFu));
                const f32x4 y = TABLE ? hv * cw[jj] : (2.0f * hv) * cw[jj];
                const f16x4 hy = {static_cast<_Float16>(y[0]), static_cast<_Float16>(y[1]), static_cast<_Float16>(y[2]),
                                  static_cast<_Float16>(y[3])};
                dp[j] = __builtin_bit_cast(uint2, hy);
            }
        }
        // Outlier chunks take their side-list values.  Lane i holds entry
        // cur + i (value and position); the list is sorted by position and cur
        // is its first entry at or after this tile, so the tile's entries are
        // a prefix of the window: each lane whose entry lies in the tile writes
        // it over the bulk value in LDS.  A tile with more than 64 entries reads
        // further windows (rare; those loads are used at once).  Chunks whose
        // entry was dropped (side list over capacity) keep the bulk value.
        {
            constexpr int LCPT = CPT == 16 ? 4 : (CPT == 32 ? 5 : 6);
            const uint64_t left = end[r] - cur[r];
            const uint32_t span = static_cast<uint32_t>(nvalid * CPT);   // the tile's positions
            const uint32_t lim = left < 64u ? static_cast<uint32_t>(left) : 64u;
            const uint32_t rel0 = sp[r] - plo;
            bool in = static_cast<uint32_t>(lane) < lim && rel0 < span;
            if (in) {
                const uint32_t rel = rel0;
                *reinterpret_cast<uint2 *>(dst + __umul24(rel >> LCPT, static_cast<uint32_t>(ROWB)) + (rel & (CPT - 1)) * 8) =
                    make_uint2(static_cast<uint32_t>(sv[r]), static_cast<uint32_t>(sv[r] >> 32));
            }
            uint32_t n = static_cast<uint32_t>(__popcll(__ballot(in)));
            if (n == 64u) {
                for (uint64_t base = 64u; left > base; base += 64u) {
                    const uint64_t rest = left - base;
                    const uint32_t l2 = rest < 64u ? static_cast<uint32_t>(rest) : 64u;
                    const uint32_t li = static_cast<uint32_t>(lane) < l2 ? static_cast<uint32_t>(lane) : l2 - 1u;
                    const uint64_t e = cur[r] + base + li;
                    const uint32_t pos = a.r[r].out_pos[e];
                    const uint64_t w = reinterpret_cast<const uint64_t *>(a.r[r].out_val)[e];
                    __builtin_amdgcn_s_waitcnt(0);
                    const uint32_t rel = pos - plo;
                    in = static_cast<uint32_t>(lane) < l2 && rel < span;
                    if (in) {
                        *reinterpret_cast<uint2 *>(dst + (rel >> LCPT) * ROWB + (rel & (CPT - 1)) * 8) =
                            make_uint2(static_cast<uint32_t>(w), static_cast<uint32_t>(w >> 32));
                    }
                    const uint32_t c = static_cast<uint32_t>(__popcll(__ballot(in)));
                    n += c;
                    if (c < 64u) break;
                }
            }
            cur[r] += n;
        }
        if (PAGED && newpage) {
            cur[r] = nlo;
            end[r] = nhi;
        }
        load_window(r);
    };

    float m_run = -INFINITY;   // running max of the scaled scores (log2 units), head n
    float l_run = 0.0f;        // this lane's part of the normaliser of head n
    f32x4 o[KB];               // O^T tiles: o[4 u + c][i] = dim 4 (4 g + i + 16 u) + c of head n
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) o[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // one 16-token tile: prefetch the next into nxt, decode cur, attend
    auto step = [&](int64_t t0, TileRegs<D, BITS, NF>(&cur_t)[2], TileRegs<D, BITS, NF>(&nxt_t)[2]) {
        const int nvalid = static_cast<int>(w_hi - t0 < kTile ? w_hi - t0 : kTile);
        const int64_t t1 = t0 + kTile;
        const int nv1 = t1 < w_hi ? static_cast<int>(w_hi - t1 < kTile ? w_hi - t1 : kTile) : 0;
        // paged: when the next tile starts a page, its slot and side lists
        // are the ones loaded a page ahead; then the page after is requested
        const bool newpage = PAGED && nv1 > 0 && (t1 & page_mask) == 0;
        uint64_t nlo[2] = {0, 0}, nhi[2] = {0, 0};
        int64_t tb1;
        if constexpr (PAGED) {
            if (newpage) {
                ps_now = ps_ahead;
                for (int r = 0; r < 2; ++r) {
                    nlo[r] = ahead_lo[r];
                    nhi[r] = ahead_hi[r];
                }
                fetch_ahead(t1 + (page_mask + 1));
            }
            tb1 = (ps_now << a.log2_page) + ((nv1 > 0 ? t1 : w_lo) & page_mask);
        } else {
            tb1 = tile_row(nv1 > 0 ? t1 : w_lo);
        }
        load_tile(0, tb1, nv1, nxt_t[0]);
        load_tile(1, tb1, nv1, nxt_t[1]);
        const uint32_t plo = static_cast<uint32_t>((PAGED ? (t0 & page_mask) : start + t0) * CPT);
        decode_tile(0, cur_t[0], nvalid, tt, plo, newpage, nlo[0], nhi[0]);
        wave_sync();

        // S[token 4 g + i][head n]: A[m = token n][k = 4 g + j] = K[token n][16 kb + 4 g + j]
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
        constexpr int KH = KB >= 8 ? KB / 2 : KB;   // reads in two halves: fewer live registers
#pragma unroll
        for (int k0 = 0; k0 < KB; k0 += KH) {
            uint2 ka[KH];   // the half's reads first, so their latencies overlap
#pragma unroll
            for (int kk = 0; kk < KH; ++kk)
                ka[kk] = *reinterpret_cast<const uint2 *>(tt + n * ROWB + (4 * (k0 + kk) + g) * 8);
#pragma unroll
            for (int kk = 0; kk < KH; ++kk)
                s = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, ka[kk]), qv[k0 + kk], s, 0, 0, 0);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = 4 * g + i < nvalid ? s[i] * a.qscale : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        // the max over the four lane groups: v_permlane16_swap pairs rows
        // 0-1 and 2-3 of 16 lanes, v_permlane32_swap the two halves of the
        // wave (VALU exchanges instead of two LDS-routed permutes)
        {
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
        }
        if (__ballot(tmax > m_run + kLazy)) {
            const float m_new = tmax > m_run + kLazy ? tmax : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 1 where unchanged, 0 from -inf
            l_run *= alpha;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) o[kb] *= alpha;
            m_run = m_new;
        }
        wave_sync();   // the K tile has been read: V goes into the same place
        decode_tile(1, cur_t[1], nvalid, tt, plo, newpage, nlo[1], nhi[1]);
        wave_sync();
        f16x4 ph;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // v_exp_f32 alone: arguments are at most kPScale + kLazy, and
            // results below the binary16 range become 0 either way
            const _Float16 p = static_cast<_Float16>(__builtin_amdgcn_exp2f(s[i] - m_run + kPScale));
            ph[i] = p;
            psum += static_cast<float>(p);
        }
        l_run += psum;

        // O^T += V^T P^T: A[m = n][k = 4 g + j] = V[token 4 g + j][dim 4 (n + 16 u) + c],
        // B[k = 4 g + j][n] = P[head n][token 4 g + j] (this lane's own weights)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            uint2 vv[4][1];   // one chunk group at a time: fewer live registers
#pragma unroll
            for (int j = 0; j < 4; ++j) vv[j][0] = *reinterpret_cast<const uint2 *>(tt + (4 * g + j) * ROWB + (n + 16 * u) * 8);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // halves c of tokens 4 g + 0..3: byte selectors of v_perm_b32
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t x0 = c < 2 ? vv[0][0].x : vv[0][0].y, x1 = c < 2 ? vv[1][0].x : vv[1][0].y;
                const uint32_t x2 = c < 2 ? vv[2][0].x : vv[2][0].y, x3 = c < 2 ? vv[3][0].x : vv[3][0].y;
                const uint2 pk = make_uint2(__builtin_amdgcn_perm(x1, x0, sel), __builtin_amdgcn_perm(x3, x2, sel));
                o[4 * u + c] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, pk), ph, o[4 * u + c], 0, 0, 0);
            }
        }
        wave_sync();
    };

    TileRegs<D, BITS, NF> ta[2], tb[2];
    if (w_lo < w_hi) {
        const int nv = static_cast<int>(w_hi - w_lo < kTile ? w_hi - w_lo : kTile);
        const int64_t tb0 = tile_row(w_lo);
        load_tile(0, tb0, nv, ta[0]);
        load_tile(1, tb0, nv, ta[1]);
    }
    for (int64_t t0 = w_lo; t0 < w_hi; t0 += 2 * kTile) {
        step(t0, ta, tb);
        if (t0 + kTile >= w_hi) break;
        step(t0 + kTile, tb, ta);
    }

    // merge the waves: each writes (m, l, o) of its 16 heads into its own
    // tile area, then the block combines them by log-sum-exp
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    __syncthreads();   // every wave is done with the tables and tiles
    unsigned char *merge = reinterpret_cast<unsigned char *>(smem);   // [waves][MERGEB]
    float *mw = reinterpret_cast<float *>(merge + wave * Sh::MERGEB);   // [16] m, [16] l, [16][D] o
    if (g == 0) {
        mw[n] = m_run;
        mw[16 + n] = l_tot;
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) mw[32 + n * D + 4 * (4 * g + i + 16 * u) + c] = o[4 * u + c][i];
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += kAttThreads) {
        const int hn = e / D, d = e - hn * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, reinterpret_cast<const float *>(merge + w * Sh::MERGEB)[hn]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) {
            const float *mv = reinterpret_cast<const float *>(merge + w * Sh::MERGEB);
            const float wt = mv[hn] == -INFINITY ? 0.0f : exp2f(mv[hn] - M);
            L += wt * mv[16 + hn];
            O += wt * mv[32 + hn * D + d];
        }
        float *ph = part + hn * pstride;
        ph[2 + d] = O;
        if (d == 0) {
            ph[0] = M;
            ph[1] = L;
        }
    }
}

// out[row][d] = sum_j w_j o_j[d] / sum_j w_j l_j, w_j = 2^(m_j - max m).
template <int D>
__global__ __launch_bounds__(D) void attend_combine_kernel(const float *part, int nsplit, float *out) {
    const int64_t row = blockIdx.x;
    const float *p = part + row * nsplit * (D + 2);
    float M = -INFINITY;
    for (int j = 0; j < nsplit; ++j) M = fmaxf(M, p[j * (D + 2)]);
    const int d = threadIdx.x;
    float L = 0.0f, O = 0.0f;
    for (int j = 0; j < nsplit; ++j) {
        const float mj = p[j * (D + 2)];
        const float w = mj == -INFINITY ? 0.0f : exp2f(mj - M);
        L += w * p[j * (D + 2) + 1];
        O += w * p[j * (D + 2) + 2 + d];
    }
    out[row * D + d] = L > 0.0f ? O / L : 0.0f;
}

template <int D>
size_t attend_lds(int S, bool table, bool exact) {
    const int bits = exact ? 0 : attend_kernel_bits(S, table);
    const int ntab = table ? (bits > 0 ? (1 << bits) : 24 * S) : S;
    const size_t loop = 2 * static_cast<size_t>(ntab) * sizeof(f32x4) + kAttWaves * static_cast<size_t>(AttShape<D>::TILEB);
    const size_t merge = kAttWaves * static_cast<size_t>(AttShape<D>::MERGEB);
    return loop > merge ? loop : merge;
}

template <int D, int NF, bool PAGED>
const void *split_kernel_for(bool table, int bits) {
    if (table && bits == 10) return reinterpret_cast<const void *>(&attend_split_kernel<D, true, 10, NF, PAGED>);
    if (table && bits == 8) return reinterpret_cast<const void *>(&attend_split_kernel<D, true, 8, NF, PAGED>);
    if (table) return reinterpret_cast<const void *>(&attend_split_kernel<D, true, 0, NF, PAGED>);
    return reinterpret_cast<const void *>(&attend_split_kernel<D, false, 0, NF, PAGED>);
}

// Exact-rate records: kernels of a fixed m for S = 8 (m = 6) and S = 32
// (m = 8), the general one for any other power of two.
template <int D>
const void *exact_kernel_for(bool table, int m) {
    if (table && m == 8) return reinterpret_cast<const void *>(&attend_split_kernel<D, true, 8, kNormExact, false>);
    if (table && m == 6) return reinterpret_cast<const void *>(&attend_split_kernel<D, true, 6, kNormExact, false>);
    if (table) return reinterpret_cast<const void *>(&attend_split_kernel<D, true, 0, kNormExact, false>);
    return reinterpret_cast<const void *>(&attend_split_kernel<D, false, 0, kNormExact, false>);
}

template <int D>
hipError_t launch_attend_d(const AttLaunch &L, hipStream_t st) {
    AttArgs a;
    a.r[0] = L.k;
    a.r[1] = L.v;
    a.q = L.q;
    a.seq_start = L.seq_start;
    a.seq_len = L.seq_len;
    a.part = L.part;
    a.tokens = L.tokens;
    a.batch_chunks = L.batch_chunks;
    a.bps = L.bps;
    a.layer = L.layer;
    a.heads = L.heads;
    a.group = L.group;
    a.nsplit = L.nsplit;
    a.split_tokens = L.split_tokens;
    a.max_len = L.max_len;
    a.S = L.S;
    a.bits = L.bits;
    a.words = L.words;
    a.qscale = L.scale * 1.4426950408889634f;
    const bool table = L.S <= kAttTableMaxS;
    const size_t lds = attend_lds<D>(L.S, table, L.exact != 0);
    a.gps = L.egps;
    a.m = L.em;
    a.wl = L.ewl;
    a.fh = L.efh;
    a.gw = L.egw;
    a.step = L.estep;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(L.batch) * L.heads * L.nsplit));
    // code widths of the common codebooks (S = 8: 8 bits, S = 32: 10) get
    // extraction at fixed bit positions; any other width the general path
    a.page_table = L.page_table;
    a.num_pages = L.num_pages;
    a.pt_stride = L.pt_stride;
    a.log2_page = L.log2_page;
    a.page_cap = L.page_cap;
    const bool paged = L.page_table != nullptr;
    const void *kern = L.exact ? exact_kernel_for<D>(table, L.em)
                       : paged ? (L.npack ? split_kernel_for<D, kNormPacked, true>(table, L.bits)
                                          : split_kernel_for<D, kNormF16, true>(table, L.bits))
                               : (L.npack ? split_kernel_for<D, kNormPacked, false>(table, L.bits)
                                          : split_kernel_for<D, kNormF16, false>(table, L.bits));
    // more than the default 64 KB of dynamic LDS must be asked for
    hipError_t e = hipSuccess;
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    void *args[] = {&a};
    e = hipLaunchKernel(kern, grid, dim3(kAttThreads), args, lds, st);
    if (e != hipSuccess) return e;
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attend_combine_kernel<D>), dim3(static_cast<unsigned>(static_cast<int64_t>(L.batch) * L.heads * L.group)),
                       dim3(D), 0, st, L.part, L.nsplit, L.out);
    return hipGetLastError();
}

}  // namespace

size_t attend_lds_bytes(int head_dim, int S, bool exact) {
    const bool table = S <= kAttTableMaxS;
    switch (head_dim) {
        case 64: return attend_lds<64>(S, table, exact);
        case 128: return attend_lds<128>(S, table, exact);
        case 256: return attend_lds<256>(S, table, exact);
        default: return 0;
    }
}

hipError_t launch_attend(const AttLaunch &L, hipStream_t st) {
    if (L.batch == 0 || L.group == 0) return hipSuccess;
    switch (L.head_dim) {
        case 64: return launch_attend_d<64>(L, st);
        case 128: return launch_attend_d<128>(L, st);
        case 256: return launch_attend_d<256>(L, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hqmq
