// C-ABI entry points of the HQMQ codec (declared in include/hqmq.h):
// argument validation, buffer sizes, the seeded codebook generator and the
// kernel launch sequence.  No device memory is allocated here.
#include "hqmq.h"

#include <algorithm>
#include <cmath>
#include <cstring>

#include "hqmq_launch.h"

namespace {

constexpr int64_t kMaxS = 1024;
constexpr uint64_t kWsAlign = 256;

bool head_dim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

int code_bits(int64_t S) {
    int b = 0;
    while ((int64_t{1} << b) < 24 * S) ++b;
    return b;
}

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validate a descriptor and derive the launch geometry.
int make_geometry(const hqmq_desc *d, hqmq::Geometry *g) {
    if (!d) return HQMQ_EINVAL;
    if (d->layers < 0 || d->kv_heads < 0 || d->tokens < 0) return HQMQ_EINVAL;
    if (!head_dim_ok(d->head_dim)) return HQMQ_EINVAL;
    if (d->S < 1 || d->S > kMaxS) return HQMQ_EINVAL;
    if (d->dtype != HQMQ_F16 && d->dtype != HQMQ_F32) return HQMQ_EINVAL;
    if (d->norm_format != HQMQ_NORM_F16 && d->norm_format != HQMQ_NORM_PACKED && d->norm_format != HQMQ_NORM_EXACT)
        return HQMQ_EINVAL;
    if (d->med_batch_tokens < 0) return HQMQ_EINVAL;
    if (d->med_batch_tokens > 0 && !(std::isfinite(d->med_C) && d->med_C > 0.0f)) return HQMQ_EINVAL;
    const int64_t cpt = d->head_dim / 4;
    // side-list positions are u32 chunk offsets within a slice
    if (d->tokens > (int64_t{1} << 32) / cpt - 1) return HQMQ_ENOTSUP;
    if (d->layers > (int64_t{1} << 31) || d->kv_heads > (int64_t{1} << 31)) return HQMQ_ENOTSUP;
    g->slices = d->layers * d->kv_heads;
    g->tokens = d->tokens;
    g->cpt = static_cast<int32_t>(cpt);
    g->n_slice = d->tokens * cpt;
    g->S = d->S;
    g->bits = code_bits(d->S);
    g->words = static_cast<int32_t>((static_cast<int64_t>(g->bits) * cpt + 31) / 32);
    g->f32 = d->dtype == HQMQ_F32 ? 1 : 0;
    if (d->med_batch_tokens > 0) {
        const int64_t B = d->med_batch_tokens < d->tokens ? d->med_batch_tokens : d->tokens;
        g->batch_chunks = (B > 0 ? B : 1) * cpt;
        g->batches_per_slice = d->tokens > 0 ? (d->tokens + B - 1) / B : 0;
    } else {
        g->batch_chunks = 0;
        g->batches_per_slice = 0;
    }
    g->med_C = d->med_C;
    g->npack = d->norm_format == HQMQ_NORM_PACKED ? 1 : 0;
    g->exact = d->norm_format == HQMQ_NORM_EXACT ? 1 : 0;
    if (g->exact) {
        // 24 S = 3 2^m needs S a power of two
        if ((d->S & (d->S - 1)) != 0) return HQMQ_ENOTSUP;
        const int m = 3 + __builtin_ctz(static_cast<unsigned>(d->S));
        g->em = m;
        g->ewl = static_cast<int32_t>((cpt * m + 31) / 32);
        g->efh = static_cast<int32_t>((cpt + 7) / 8);
        g->egw = 8 * g->ewl + (4 * 2 * g->efh * 13 + 31) / 32;
        g->egps = (d->tokens + 3) / 4;
        // levels n < R - 1 whose pattern floor((n 2^(15 - m) + 1) / 3) is below 0x7C00
        const uint32_t top = 95230u >> (15 - m);
        g->enmax = std::min((3u << m) - 2u, top);
        g->estep = static_cast<float>(std::ldexp(1.0, 15 - m) / 3.0);
    }
    // grids are one-dimensional: keep the block count well inside 2^31
    if (g->slices > 0 && g->n_slice / 256 + 1 > (int64_t{1} << 31) / g->slices) return HQMQ_ENOTSUP;
    return HQMQ_OK;
}

// Encode workspace.  Med3x: hist [batches][2048] u32 | counts [batches] u32 |
// mask [batches][mask_words] u32 (one bit per chunk).  Packed and exact
// norms: the binary16 half-norm plane [chunks] u16 that the search writes,
// Med3x flags, and the pack kernel reads.  Exact format: also the whole-bit
// code plane [slices][tokens][words] u32 of the search.
int64_t mask_words(const hqmq::Geometry &g) { return 2 * ((g.batch_chunks + 63) / 64); }

uint64_t workspace_layout(const hqmq::Geometry &g, void *base, hqmq::Med3Work *w) {
    uint64_t off = 0;
    uint64_t o_hist = 0, o_cnt = 0, o_mask = 0, o_h16 = 0, o_idx = 0;
    const uint64_t mw = static_cast<uint64_t>(mask_words(g));
    if (g.batch_chunks > 0) {
        const uint64_t nb = static_cast<uint64_t>(g.slices * g.batches_per_slice);
        o_hist = off;
        off = align_up(off + nb * 2048 * 4, kWsAlign);
        o_cnt = off;
        off = align_up(off + nb * 4, kWsAlign);
        o_mask = off;
        off = align_up(off + nb * mw * 4, kWsAlign);
    }
    if (g.npack || g.exact) {
        o_h16 = off;
        off = align_up(off + static_cast<uint64_t>(g.slices * g.n_slice) * 2, kWsAlign);
    }
    if (g.exact) {
        o_idx = off;
        off = align_up(off + static_cast<uint64_t>(g.slices * g.tokens) * g.words * 4, kWsAlign);
    }
    if (w) {
        char *b = static_cast<char *>(base);
        *w = hqmq::Med3Work{};
        if (g.batch_chunks > 0) {
            w->hist = reinterpret_cast<uint32_t *>(b + o_hist);
            w->counts = reinterpret_cast<uint32_t *>(b + o_cnt);
            w->mask = reinterpret_cast<uint32_t *>(b + o_mask);
            w->mask_words = static_cast<int64_t>(mw);
        }
        if (g.npack || g.exact) w->h16 = reinterpret_cast<uint16_t *>(b + o_h16);
        if (g.exact) w->idx32 = reinterpret_cast<uint32_t *>(b + o_idx);
    }
    return off;
}

// ----------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each round
// multiplies counter words 0 and 2 by the two round constants (full 128-bit
// products), and mixes the high halves with the other two words and the key;
// the key is bumped by two Weyl increments between rounds.
// ----------------------------------------------------------------------------
struct Philox4x64 {
    static constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
    static constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
    static constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
    static constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;

    static void block(const uint64_t in[4], uint64_t k0, uint64_t k1, uint64_t out[4]) {
        uint64_t c[4] = {in[0], in[1], in[2], in[3]};
        for (int r = 0; r < 10; ++r) {
            if (r) {
                k0 += kWeyl0;
                k1 += kWeyl1;
            }
            const unsigned __int128 p0 = static_cast<unsigned __int128>(kMul0) * c[0];
            const unsigned __int128 p1 = static_cast<unsigned __int128>(kMul1) * c[2];
            const uint64_t hi0 = static_cast<uint64_t>(p0 >> 64), lo0 = static_cast<uint64_t>(p0);
            const uint64_t hi1 = static_cast<uint64_t>(p1 >> 64), lo1 = static_cast<uint64_t>(p1);
            c[0] = hi1 ^ c[1] ^ k0;
            c[1] = lo1;
            c[2] = hi0 ^ c[3] ^ k1;
            c[3] = lo0;
        }
        std::memcpy(out, c, sizeof(c));
    }
};

// Nearest value on the double-binary16 grid used for codebooks: hi + lo with
// hi = fp16(q) and lo = fp16(q - hi), both rounded to nearest even (q - hi is
// exact in fp32, and so is the sum).  The encode kernels split a codebook
// value into exactly these two parts for the f16 matrix cores.
float double_f16(float q) {
    const _Float16 hi = static_cast<_Float16>(q);
    const _Float16 lo = static_cast<_Float16>(q - static_cast<float>(hi));
    return static_cast<float>(hi) + static_cast<float>(lo);
}

}  // namespace

// Validation and split plan of a decode-step attention request: enough
// (sequence, head, split) blocks to fill the chip several times, splits of a
// multiple of 128 tokens (8 waves x 16-token tiles).
static int attn_plan(const hqmq_desc *d, const hqmq::Geometry &g, const hqmq_attn_desc *a, int32_t *nsplit,
              int32_t *stok) {
    if (!a) return HQMQ_EINVAL;
    if (a->batch < 0 || a->group < 1 || a->group > 16 || a->max_len < 0 || a->reserved != 0 ||
        !std::isfinite(a->scale))
        return HQMQ_EINVAL;
    if (a->layer < 0 || (a->layer >= d->layers && !(d->layers == 0 && a->batch == 0))) return HQMQ_EINVAL;
    if (d->dtype != HQMQ_F16) return HQMQ_ENOTSUP;
    if (hqmq::attend_lds_bytes(static_cast<int>(d->head_dim), g.S, g.exact) == 0) return HQMQ_ENOTSUP;
    if (hqmq::attend_lds_bytes(static_cast<int>(d->head_dim), g.S, g.exact) > 160 * 1024) return HQMQ_ENOTSUP;
    if (d->kv_heads > 4096) return HQMQ_ENOTSUP;
    const int64_t pairs = std::max<int64_t>(1, static_cast<int64_t>(a->batch) * d->kv_heads);
    int64_t want = (1024 + pairs - 1) / pairs;
    const int64_t most = std::max<int64_t>(1, (static_cast<int64_t>(a->max_len) + 127) / 128);
    want = std::min(std::max<int64_t>(want, 1), most);
    int64_t st = ((a->max_len + want - 1) / want + 127) / 128 * 128;
    if (st < 128) st = 128;
    const int64_t ns = std::max<int64_t>(1, (a->max_len + st - 1) / st);
    if (pairs * ns > (int64_t{1} << 31) - 1) return HQMQ_ENOTSUP;
    *nsplit = static_cast<int32_t>(ns);
    *stok = static_cast<int32_t>(st);
    return HQMQ_OK;
}

// Paged pool geometry: validate p against the codec geometry g.
static int paged_geometry(const hqmq::Geometry &g, const hqmq_paged_desc *p, int32_t *log2_page) {
    if (!p) return HQMQ_EINVAL;
    if (g.exact) return HQMQ_ENOTSUP;   // pools keep whole-bit token rows
    const int64_t P = p->page_tokens;
    if (p->num_pages < 0 || p->page_capacity < 0 || P < 16 || (P & (P - 1)) != 0) return HQMQ_EINVAL;
    if (p->num_pages >= (int64_t{1} << 31) || P * g.cpt >= (int64_t{1} << 31)) return HQMQ_ENOTSUP;
    // pool rows and side entries stay well inside 2^62, grids inside 2^31 blocks
    if (g.slices > 0 && p->num_pages > 0 &&
        (p->num_pages * P > (int64_t{1} << 40) / g.slices ||
         p->num_pages * static_cast<int64_t>(p->page_capacity) > (int64_t{1} << 40) / g.slices))
        return HQMQ_ENOTSUP;
    *log2_page = __builtin_ctzll(static_cast<unsigned long long>(P));
    return HQMQ_OK;
}

// Append workspace: the encode scratch of the call's tensor, then its
// records (binary16 norms) with a worst-case side list.
struct AppendWork {
    void *enc_ws;
    uint64_t enc_ws_bytes;
    uint32_t *idx;
    uint16_t *h16;
    uint64_t *offsets;
    uint32_t *out_pos;
    uint16_t *out_val;
    uint64_t *status;
    uint64_t capacity;
};

static uint64_t append_layout(const hqmq_desc *dc, void *base, AppendWork *w) {
    hqmq_sizes_t sz;
    if (hqmq_sizes(dc, &sz) != HQMQ_OK) return 0;
    const uint64_t cap = static_cast<uint64_t>(sz.max_outliers);
    uint64_t off = 0;
    const uint64_t o_ws = off;
    off = align_up(off + sz.workspace_bytes, kWsAlign);
    const uint64_t o_idx = off;
    off = align_up(off + sz.idx_bytes, kWsAlign);
    const uint64_t o_h = off;
    off = align_up(off + sz.hnorm_bytes, kWsAlign);
    const uint64_t o_offs = off;
    off = align_up(off + sz.offsets_bytes, kWsAlign);
    const uint64_t o_pos = off;
    off = align_up(off + cap * 4, kWsAlign);
    const uint64_t o_val = off;
    off = align_up(off + cap * 8, kWsAlign);
    const uint64_t o_st = off;
    off = align_up(off + 16, kWsAlign);
    if (w) {
        char *b = static_cast<char *>(base);
        w->enc_ws = sz.workspace_bytes ? b + o_ws : nullptr;
        w->enc_ws_bytes = sz.workspace_bytes;
        w->idx = reinterpret_cast<uint32_t *>(b + o_idx);
        w->h16 = reinterpret_cast<uint16_t *>(b + o_h);
        w->offsets = reinterpret_cast<uint64_t *>(b + o_offs);
        w->out_pos = reinterpret_cast<uint32_t *>(b + o_pos);
        w->out_val = reinterpret_cast<uint16_t *>(b + o_val);
        w->status = reinterpret_cast<uint64_t *>(b + o_st);
        w->capacity = cap;
    }
    return off;
}

static bool pool_ok(const hqmq_pages *k, bool data) {
    if (!k) return false;
    if (!data) return true;
    return k->idx && k->hnorm && k->side_count && aligned(k->idx, 4) && aligned(k->hnorm, 16) &&
           aligned(k->side_count, 4) && (!k->side_pos || aligned(k->side_pos, 4)) &&
           (!k->side_val || aligned(k->side_val, 16));
}

extern "C" {

const char *hqmq_strerror(int code) {
    switch (code) {
        case HQMQ_OK: return "ok";
        case HQMQ_EINVAL: return "invalid argument (descriptor, pointer, size or alignment)";
        case HQMQ_ENOTSUP: return "request outside the supported limits";
        case HQMQ_ECAPACITY: return "Med3x side list exceeded out_capacity";
        case HQMQ_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int hqmq_sizes(const hqmq_desc *d, hqmq_sizes_t *out) {
    if (!out) return HQMQ_EINVAL;
    hqmq::Geometry g;
    const int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    std::memset(out, 0, sizeof(*out));
    out->code_bits = g.bits;
    out->words_per_token = g.words;
    out->chunks = g.slices * g.n_slice;
    out->batches = g.slices * g.batches_per_slice;
    int64_t mo = 0;
    if (g.batch_chunks > 0) {
        // s2 > fl(fl(C C) med) leaves at most floor(n / 2) chunks of a batch
        // above its lower median when fl(C C) >= 1; with a smaller multiplier
        // the median itself and everything above it can be outliers
        const int64_t full = g.n_slice / g.batch_chunks;
        const int64_t tail = g.n_slice - full * g.batch_chunks;
        const float cc = g.med_C * g.med_C;
        mo = cc >= 1.0f ? g.slices * (full * (g.batch_chunks / 2) + tail / 2) : g.slices * g.n_slice;
    }
    out->max_outliers = mo;
    out->input_bytes = static_cast<uint64_t>(out->chunks) * 4 * (g.f32 ? 4 : 2);
    if (g.exact) {
        out->idx_bytes = static_cast<uint64_t>(g.slices * g.egps) * g.egw * 4;
        out->hnorm_bytes = 0;
        out->group_rows = 4;
        out->group_words = g.egw;
    } else {
        out->idx_bytes = static_cast<uint64_t>(g.slices * g.tokens) * g.words * 4;
        out->hnorm_bytes = g.npack ? out->idx_bytes : static_cast<uint64_t>(out->chunks) * 2;
    }
    out->offsets_bytes = g.batch_chunks > 0 ? static_cast<uint64_t>(out->batches + 1) * 8 : 0;
    out->side_entry_bytes = 12;
    out->workspace_bytes = workspace_layout(g, nullptr, nullptr);
    out->codebook_bytes = static_cast<uint64_t>(g.slices) * g.S * 16;
    return HQMQ_OK;
}

int hqmq_make_codebook(uint64_t seed, int32_t layers, int32_t kv_heads, int32_t role, int32_t S,
                       float *out_host) {
    if (!out_host || layers < 0 || kv_heads < 0 || layers >= (1 << 24) || kv_heads >= (1 << 24) ||
        (role != HQMQ_ROLE_K && role != HQMQ_ROLE_V) || S < 1 || S > kMaxS)
        return HQMQ_EINVAL;
    for (int32_t l = 0; l < layers; ++l) {
        for (int32_t h = 0; h < kv_heads; ++h) {
            const uint64_t k1 = (static_cast<uint64_t>(l) << 32) | (static_cast<uint64_t>(h) << 8) |
                                static_cast<uint64_t>(role);
            float *q = out_host + (static_cast<int64_t>(l) * kv_heads + h) * S * 4;
            uint64_t ctr = 0;
            for (int32_t s = 0; s < S;) {
                const uint64_t in[4] = {ctr++, 0, 0, 0};
                uint64_t w[4];
                Philox4x64::block(in, seed, k1, w);
                double v[4];
                double n2 = 0.0;
                for (int m = 0; m < 4; ++m) {
                    // odd multiple of 2^-24 in (-1, 1) from the top 24 bits
                    v[m] = std::ldexp(static_cast<double>(static_cast<int64_t>(w[m] >> 40) * 2 - (int64_t{1} << 24) + 1), -24);
                    n2 += v[m] * v[m];
                }
                if (!(n2 <= 1.0)) continue;  // rejection: uniform in the ball
                const double r = std::sqrt(n2);
                for (int m = 0; m < 4; ++m) q[4 * s + m] = double_f16(static_cast<float>(v[m] / r));
                ++s;
            }
        }
    }
    return HQMQ_OK;
}

int hqmq_encode(const hqmq_desc *d, const void *x, const float *codebook, const hqmq_enc *enc,
                void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return hqmq_encode_timed(d, x, codebook, enc, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int hqmq_encode_timed(const hqmq_desc *d, const void *x, const float *codebook, const hqmq_enc *enc,
                      void *workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t search_begin, hipEvent_t search_end) {
    hqmq::Geometry g;
    int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    if (!enc) return HQMQ_EINVAL;
    const int64_t chunks = g.slices * g.n_slice;
    const bool med = g.batch_chunks > 0;
    const int64_t nb = g.slices * g.batches_per_slice;
    if (chunks > 0) {
        if (!x || !codebook || !enc->idx || (!enc->hnorm && !g.exact)) return HQMQ_EINVAL;
        if (!aligned(x, 16) || !aligned(codebook, 16) || !aligned(enc->idx, 4) ||
            (!g.exact && !aligned(enc->hnorm, 8)))
            return HQMQ_EINVAL;
    }
    hqmq::Med3Work ws{};
    if (med) {
        if (!enc->batch_offsets || !enc->status || !aligned(enc->batch_offsets, 8) || !aligned(enc->status, 8))
            return HQMQ_EINVAL;
        if (enc->out_capacity > 0 && (!enc->out_pos || !enc->out_val || !aligned(enc->out_val, 8)))
            return HQMQ_EINVAL;
    } else if (enc->status && !aligned(enc->status, 8)) {
        return HQMQ_EINVAL;
    }
    {
        const uint64_t need = workspace_layout(g, nullptr, nullptr);
        if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign)))
            return HQMQ_EINVAL;
        if (need > 0) workspace_layout(g, workspace, &ws);
    }
    // the binary16 half-norms: the record itself, or (packed, exact) the
    // scratch plane the pack kernels turn into norm codes at the end; the
    // whole-bit codes: the record, or (exact) a scratch plane
    uint16_t *h16 = (g.npack || g.exact) ? ws.h16 : static_cast<uint16_t *>(enc->hnorm);
    uint32_t *idx32 = g.exact ? ws.idx32 : enc->idx;

    hipError_t e = hipSuccess;
    if (med && nb > 0) {
        // clear the batch histograms the search accumulates and the outlier
        // bitmasks the select kernel ORs bits into (one contiguous range)
        const int64_t words = (reinterpret_cast<char *>(ws.mask + nb * ws.mask_words) -
                               reinterpret_cast<char *>(ws.hist)) / 4;
        e = hqmq::launch_fill_u32(ws.hist, words, 0u, stream);
        if (e != hipSuccess) return HQMQ_EHIP;
    }
    if (search_begin && hipEventRecord(search_begin, stream) != hipSuccess) return HQMQ_EHIP;
    if (chunks > 0) {
        e = hqmq::launch_encode_search(g, x, codebook, idx32, h16, med && nb > 0 ? &ws : nullptr, stream);
        if (e != hipSuccess) return HQMQ_EHIP;
    }
    if (search_end && hipEventRecord(search_end, stream) != hipSuccess) return HQMQ_EHIP;
    if (med) {
        if (nb > 0) {
            e = hqmq::launch_med3_select(g, x, h16, ws, g.npack ? static_cast<uint32_t *>(enc->hnorm) : nullptr,
                                         stream);
            if (e == hipSuccess)
                e = hqmq::launch_med3_scan(nb, ws.counts, enc->batch_offsets, enc->out_capacity, enc->status, stream);
            if (e == hipSuccess)
                e = hqmq::launch_med3_gather(g, x, ws, enc->batch_offsets, h16, enc->out_pos, enc->out_val,
                                             enc->out_capacity, stream);
        } else {
            e = hqmq::launch_fill_u64(enc->batch_offsets, 1, 0, stream);
            if (e == hipSuccess) e = hqmq::launch_fill_u64(enc->status, 2, 0, stream);
        }
    } else if (enc->status) {
        e = hqmq::launch_fill_u64(enc->status, 2, 0, stream);
    }
    // packed norms: the single-pass select has packed its batches already
    const bool packed_by_select = med && nb > 0 && hqmq::med3_single_pass(g);
    if (e == hipSuccess && g.npack && chunks > 0 && !packed_by_select)
        e = hqmq::launch_pack_norms(g, h16, static_cast<uint32_t *>(enc->hnorm), stream);
    if (e == hipSuccess && g.exact && chunks > 0) e = hqmq::launch_pack_exact(g, idx32, h16, enc->idx, stream);
    return e == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

int hqmq_encode_result(const hqmq_enc *enc, hipStream_t stream, uint64_t *n_outliers) {
    if (!enc || !n_outliers) return HQMQ_EINVAL;
    *n_outliers = 0;
    if (hipStreamSynchronize(stream) != hipSuccess) return HQMQ_EHIP;
    if (!enc->status) return HQMQ_OK;
    uint64_t st[2] = {0, 0};
    if (hipMemcpy(st, enc->status, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return HQMQ_EHIP;
    *n_outliers = st[0];
    return st[1] ? HQMQ_ECAPACITY : HQMQ_OK;
}

int hqmq_decode(const hqmq_desc *d, const hqmq_enc *enc, const float *codebook, void *y,
                hipStream_t stream) {
    hqmq::Geometry g;
    int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    if (!enc) return HQMQ_EINVAL;
    const int64_t chunks = g.slices * g.n_slice;
    if (chunks == 0) return HQMQ_OK;
    if (!y || !codebook || !enc->idx || (!enc->hnorm && !g.exact)) return HQMQ_EINVAL;
    if (!aligned(y, 16) || !aligned(codebook, 16) || !aligned(enc->idx, 4) || (!g.exact && !aligned(enc->hnorm, 8)))
        return HQMQ_EINVAL;
    if (g.batch_chunks > 0) {
        if (!enc->batch_offsets) return HQMQ_EINVAL;
        if (enc->out_capacity > 0 && (!enc->out_pos || !enc->out_val || !aligned(enc->out_val, 8)))
            return HQMQ_EINVAL;
    }
    const hipError_t e = hqmq::launch_decode(g, enc->idx, enc->hnorm,
                                             g.batch_chunks > 0 ? enc->batch_offsets : nullptr, enc->out_pos,
                                             enc->out_val, enc->out_capacity, codebook, y, stream);
    return e == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

int hqmq_set_search_blocks_per_cu(int32_t n) {
    if (n < 0 || n > 7) return HQMQ_EINVAL;
    hqmq::set_search_blocks_per_cu(n);
    return HQMQ_OK;
}

int hqmq_attn_sizes(const hqmq_desc *d, const hqmq_attn_desc *a, hqmq_attn_sizes_t *out) {
    if (!out) return HQMQ_EINVAL;
    hqmq::Geometry g;
    int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    int32_t nsplit = 0, stok = 0;
    rc = attn_plan(d, g, a, &nsplit, &stok);
    if (rc != HQMQ_OK) return rc;
    out->splits = nsplit;
    out->split_tokens = stok;
    out->workspace_bytes = static_cast<uint64_t>(a->batch) * d->kv_heads * a->group * nsplit *
                           (d->head_dim + 2) * 4;
    return HQMQ_OK;
}

int hqmq_attend(const hqmq_desc *d, const hqmq_attn_desc *a, const hqmq_enc *k, const float *codebook_k,
                const hqmq_enc *v, const float *codebook_v, const void *q, const int64_t *seq_start,
                const int32_t *seq_len, float *out, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
    hqmq_attn_sizes_t sz;
    int rc = hqmq_attn_sizes(d, a, &sz);
    if (rc != HQMQ_OK) return rc;
    if (!k || !v) return HQMQ_EINVAL;
    if (a->batch == 0 || d->kv_heads == 0) return HQMQ_OK;
    if (!q || !seq_start || !seq_len || !out || !workspace || workspace_bytes < sz.workspace_bytes)
        return HQMQ_EINVAL;
    if (!aligned(q, 8) || !aligned(seq_start, 8) || !aligned(seq_len, 4) || !aligned(out, 4) ||
        !aligned(workspace, 16))
        return HQMQ_EINVAL;
    hqmq::Geometry g;
    make_geometry(d, &g);
    const hqmq_enc *enc[2] = {k, v};
    const float *cb[2] = {codebook_k, codebook_v};
    hqmq::AttRole role[2];
    for (int r = 0; r < 2; ++r) {
        const hqmq_enc *e = enc[r];
        const bool data = g.tokens > 0;
        if (data && (!e->idx || (!g.exact && (!e->hnorm || !aligned(e->hnorm, 16))) || !cb[r] ||
                     !aligned(e->idx, 4) || !aligned(cb[r], 16)))
            return HQMQ_EINVAL;
        if (data && g.batch_chunks > 0) {
            if (!e->batch_offsets || !aligned(e->batch_offsets, 8)) return HQMQ_EINVAL;
            if (e->out_capacity > 0 && (!e->out_pos || !e->out_val || !aligned(e->out_pos, 4) ||
                                        !aligned(e->out_val, 8)))
                return HQMQ_EINVAL;
        }
        role[r] = hqmq::AttRole{e->idx, static_cast<const uint16_t *>(e->hnorm), g.batch_chunks > 0 ? e->batch_offsets : nullptr, e->out_pos,
                                e->out_val, g.batch_chunks > 0 ? e->out_capacity : 0, cb[r]};
    }
    hqmq::AttLaunch L{};
    L.k = role[0];
    L.v = role[1];
    L.q = static_cast<const uint16_t *>(q);
    L.seq_start = seq_start;
    L.seq_len = seq_len;
    L.part = static_cast<float *>(workspace);
    L.out = out;
    L.tokens = g.tokens;
    L.batch_chunks = g.batch_chunks;
    L.bps = g.batch_chunks > 0 ? g.batches_per_slice : 0;
    L.layer = a->layer;
    L.heads = static_cast<int32_t>(d->kv_heads);
    L.group = a->group;
    L.batch = a->batch;
    L.nsplit = sz.splits;
    L.split_tokens = sz.split_tokens;
    L.max_len = a->max_len;
    L.head_dim = static_cast<int32_t>(d->head_dim);
    L.S = g.S;
    L.bits = g.bits;
    L.words = g.words;
    L.npack = g.npack;
    L.exact = g.exact;
    L.em = g.em;
    L.ewl = g.ewl;
    L.efh = g.efh;
    L.egw = g.egw;
    L.egps = g.egps;
    L.estep = g.estep;
    L.scale = a->scale;
    return hqmq::launch_attend(L, stream) == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

int hqmq_paged_sizes(const hqmq_desc *d, const hqmq_paged_desc *p, hqmq_paged_sizes_t *out) {
    if (!out) return HQMQ_EINVAL;
    hqmq::Geometry g;
    int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    int32_t lp = 0;
    rc = paged_geometry(g, p, &lp);
    if (rc != HQMQ_OK) return rc;
    std::memset(out, 0, sizeof(*out));
    const uint64_t pages = static_cast<uint64_t>(g.slices) * static_cast<uint64_t>(p->num_pages);
    const uint64_t rows = pages * static_cast<uint64_t>(p->page_tokens);
    out->idx_bytes = rows * g.words * 4;
    out->hnorm_bytes = g.npack ? out->idx_bytes : rows * g.cpt * 2;
    out->side_count_bytes = pages * 4;
    out->side_pos_bytes = pages * p->page_capacity * 4;
    out->side_val_bytes = pages * p->page_capacity * 8;
    hqmq_desc dc = *d;
    dc.norm_format = HQMQ_NORM_F16;
    out->append_workspace_bytes = append_layout(&dc, nullptr, nullptr);
    return HQMQ_OK;
}

int hqmq_paged_clear(const hqmq_desc *d, const hqmq_paged_desc *p, const hqmq_pages *pool, const int32_t *pages,
                     int64_t n, hipStream_t stream) {
    hqmq::Geometry g;
    int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    int32_t lp = 0;
    rc = paged_geometry(g, p, &lp);
    if (rc != HQMQ_OK) return rc;
    if (!pool || n < 0) return HQMQ_EINVAL;
    if (n == 0 || g.slices == 0) return HQMQ_OK;
    if (!pages || !pool->side_count || !aligned(pages, 4) || !aligned(pool->side_count, 4)) return HQMQ_EINVAL;
    if (n > (int64_t{1} << 40) / g.slices) return HQMQ_ENOTSUP;
    hqmq::PagedPool pp{};
    pp.side_count = pool->side_count;
    pp.num_pages = p->num_pages;
    pp.log2_page = lp;
    return hqmq::launch_paged_clear(g.slices, pages, n, pp, stream) == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

int hqmq_append(const hqmq_desc *d, const hqmq_paged_desc *p, const void *x, const int64_t *slots,
                const float *codebook, const hqmq_pages *pool, uint64_t *status, void *workspace,
                size_t workspace_bytes, hipStream_t stream) {
    hqmq::Geometry g;
    int rc = make_geometry(d, &g);
    if (rc != HQMQ_OK) return rc;
    int32_t lp = 0;
    rc = paged_geometry(g, p, &lp);
    if (rc != HQMQ_OK) return rc;
    const bool med = g.batch_chunks > 0;
    const int64_t chunks = g.slices * g.n_slice;
    if (status && !aligned(status, 8)) return HQMQ_EINVAL;
    if (!pool_ok(pool, chunks > 0)) return HQMQ_EINVAL;
    if (chunks > 0 && med && p->page_capacity > 0 && (!pool->side_pos || !pool->side_val)) return HQMQ_EINVAL;
    if (chunks > 0 && (!slots || !aligned(slots, 8))) return HQMQ_EINVAL;
    hqmq_desc dc = *d;
    dc.norm_format = HQMQ_NORM_F16;
    const uint64_t need = append_layout(&dc, nullptr, nullptr);
    if (chunks > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))) return HQMQ_EINVAL;
    hipError_t e = hipSuccess;
    if (status) {
        e = hqmq::launch_fill_u64(status, 2, 0, stream);
        if (e != hipSuccess) return HQMQ_EHIP;
    }
    if (chunks == 0) return HQMQ_OK;
    AppendWork w;
    append_layout(&dc, workspace, &w);
    hqmq_enc enc{};
    enc.idx = w.idx;
    enc.hnorm = w.h16;
    enc.batch_offsets = med ? w.offsets : nullptr;
    enc.out_pos = med ? w.out_pos : nullptr;
    enc.out_val = med ? w.out_val : nullptr;
    enc.out_capacity = med ? w.capacity : 0;
    enc.status = w.status;
    // the call's records (the worst-case side list fits: no overflow)
    rc = hqmq_encode(&dc, x, codebook, &enc, w.enc_ws, w.enc_ws_bytes, stream);
    if (rc != HQMQ_OK) return rc;
    hqmq::PagedPool pp;
    pp.idx = pool->idx;
    pp.hnorm = pool->hnorm;
    pp.side_count = pool->side_count;
    pp.side_pos = pool->side_pos;
    pp.side_val = pool->side_val;
    pp.num_pages = p->num_pages;
    pp.log2_page = lp;
    pp.cap = static_cast<uint32_t>(p->page_capacity);
    if (med) {
        e = hqmq::launch_paged_scatter(g, w.offsets, w.out_pos, w.out_val, slots, w.h16, pp, status, stream);
        if (e != hipSuccess) return HQMQ_EHIP;
    }
    e = hqmq::launch_paged_rows(g, w.idx, w.h16, slots, pp, stream);
    return e == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

int hqmq_attend_paged(const hqmq_desc *d, const hqmq_paged_desc *p, const hqmq_attn_desc *a, const hqmq_pages *k,
                      const float *codebook_k, const hqmq_pages *v, const float *codebook_v, const void *q,
                      const int32_t *page_table, int32_t page_table_stride, const int32_t *seq_len, float *out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    hqmq_attn_sizes_t sz;
    int rc = hqmq_attn_sizes(d, a, &sz);
    if (rc != HQMQ_OK) return rc;
    hqmq::Geometry g;
    make_geometry(d, &g);
    int32_t lp = 0;
    rc = paged_geometry(g, p, &lp);
    if (rc != HQMQ_OK) return rc;
    if (page_table_stride < 1) return HQMQ_EINVAL;
    if (a->batch > 0 && d->kv_heads > 0 && static_cast<int64_t>(a->batch) * page_table_stride > (int64_t{1} << 40))
        return HQMQ_ENOTSUP;
    const bool data = p->num_pages > 0;
    if (!pool_ok(k, data) || !pool_ok(v, data)) return HQMQ_EINVAL;
    if (a->batch == 0 || d->kv_heads == 0) return HQMQ_OK;
    if (!q || !page_table || !seq_len || !out || !workspace || workspace_bytes < sz.workspace_bytes)
        return HQMQ_EINVAL;
    if (!aligned(q, 8) || !aligned(page_table, 4) || !aligned(seq_len, 4) || !aligned(out, 4) ||
        !aligned(workspace, 16))
        return HQMQ_EINVAL;
    if (!data) return HQMQ_EINVAL;   // sequences need pages
    const hqmq_pages *pools[2] = {k, v};
    const float *cb[2] = {codebook_k, codebook_v};
    hqmq::AttRole role[2];
    for (int r = 0; r < 2; ++r) {
        if (!cb[r] || !aligned(cb[r], 16)) return HQMQ_EINVAL;
        if (p->page_capacity > 0 && (!pools[r]->side_pos || !pools[r]->side_val)) return HQMQ_EINVAL;
        role[r] = hqmq::AttRole{pools[r]->idx, static_cast<const uint16_t *>(pools[r]->hnorm), nullptr,
                                pools[r]->side_pos, pools[r]->side_val, 0, cb[r], pools[r]->side_count};
    }
    hqmq::AttLaunch L{};
    L.k = role[0];
    L.v = role[1];
    L.q = static_cast<const uint16_t *>(q);
    L.seq_start = nullptr;
    L.seq_len = seq_len;
    L.part = static_cast<float *>(workspace);
    L.out = out;
    L.tokens = 0;
    L.batch_chunks = 0;
    L.bps = 0;
    L.layer = a->layer;
    L.heads = static_cast<int32_t>(d->kv_heads);
    L.group = a->group;
    L.batch = a->batch;
    L.nsplit = sz.splits;
    L.split_tokens = sz.split_tokens;
    L.max_len = a->max_len;
    L.head_dim = static_cast<int32_t>(d->head_dim);
    L.S = g.S;
    L.bits = g.bits;
    L.words = g.words;
    L.npack = g.npack;
    L.scale = a->scale;
    L.page_table = page_table;
    L.num_pages = p->num_pages;
    L.pt_stride = page_table_stride;
    L.log2_page = lp;
    L.page_cap = static_cast<uint32_t>(p->page_capacity);
    return hqmq::launch_attend(L, stream) == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

}  // extern "C"
