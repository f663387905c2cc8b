/*
 * hqmq.h -- C ABI of the HQMQ KV-cache codec for AMD Instinct MI355X (gfx950).
 *
 * HQMQ (Hurwitz Quaternion Multiplicative Quantization, arXiv 2605.27646)
 * treats every 4 consecutive elements of a K or V head vector as a
 * quaternion x, keeps its norm r = |x| and quantises its direction x / r to
 * the nearest of the 24 S products q_p * q_s, q_p in the binary tetrahedral
 * group 2T (the 24 unit Hurwitz quaternions) and q_s in a seeded codebook of S
 * random unit quaternions per (layer, head, role).  A per-batch Med3x step
 * first keeps every chunk with r > C * median(r) (C = 3) in fp16 on a side
 * list, flagged by one bit.  Sources: the paper's abstract (paperdance.org and
 * thelatestinai.com pages for 2605.27646); gist.science/nl/paper/2605.27646,
 * "Technische Samenvatting", Methodologie 1-3; signal-ia-rouge.vercel.app
 * article, sections "La mecanique" and "Le probleme des outliers : Med3x".
 *
 * Tensor layout.  x and y are contiguous [layers][kv_heads][tokens][head_dim]
 * (fp16 or fp32).  Chunk c of token t of slice (layer, head) is elements
 * 4c .. 4c+3 of that token's head vector; element 4c is the real part, then
 * i, j, k.  A (layer, head) pair is a "slice" of tokens * head_dim / 4 chunks.
 *
 * Encoded records (all caller-allocated device memory; sizes from hqmq_sizes):
 *   idx    [layers][kv_heads][tokens][words_per_token] u32.  Code k = 24 s + p
 *          of each chunk, b = ceil(log2(24 S)) bits, packed little-endian
 *          along the token row: bit i of code c is bit (c b + i) of the row,
 *          row bit j is bit j % 32 of word j / 32; unused high bits are 0.
 *          2T order p: +1, -1, +i, -i, +j, -j, +k, -k, then (s0,s1,s2,s3)/2
 *          with s_m = -1 iff bit m of p - 8 is set.  The record always holds
 *          the nearest codeword, also for an outlier chunk.
 *   hnorm  norm_format HQMQ_NORM_F16: [layers][kv_heads][tokens][head_dim / 4]
 *          u16, the binary16 half-norm h16 = binary16 of sqrt_rn(s2) / 2 with
 *          s2 = fma(x3,x3, fma(x2,x2, fma(x1,x1, x0*x0))) in fp32; bit 15 (the
 *          sign bit, free since norms are >= 0) is the Med3x outlier flag.
 *          norm_format HQMQ_NORM_PACKED: u32 words laid out exactly like idx
 *          (b bits per chunk, the same b), holding the compact norm code: h16
 *          rounded to nearest (a tie to the even code) to a float with 5
 *          exponent bits and b - 5 mantissa bits, capped at its largest
 *          finite value, as the top b bits of the binary16 pattern; the
 *          all-ones code is the outlier flag.  Then a chunk costs 2 b bits
 *          (S = 8: 4 bits per element, S = 32: 5), the pages' accounting of
 *          two log2(24 S)-bit codes per chunk (abstract: ~3.79 bits at S = 8,
 *          ~5 at S = 32) with whole bits.
 *   side list (Med3x only): out_pos[e] u32 = t * head_dim / 4 + c (position
 *          in its slice), out_val[4e..4e+3] = the chunk's values as binary16
 *          (fp32 inputs rounded to nearest even).  Ordered by (slice, batch,
 *          position); batch_offsets[b] .. batch_offsets[b+1] is batch b's
 *          range, batches numbered slice-major (slice * batches_per_slice +
 *          token_block).
 *   status [2] u64: status[0] = outliers found, status[1] = 1 when they did
 *          not fit out_capacity (entries past the capacity are dropped;
 *          their chunks decode to the bulk value of their record).
 *
 * Exact-rate records (norm_format HQMQ_NORM_EXACT, S a power of two): the
 * pages' rate of two log2(24 S)-bit codes per chunk (about 3.79 bits per
 * element at S = 8 and 4.79 at S = 32; the abstract, and the
 * signal-ia-rouge.vercel.app article, "La mecanique") without whole-bit
 * rounding.  The index k keeps its meaning; the norm code n has R = 24 S
 * levels: n = R - 1 is the Med3x flag, level n < R - 1 stands for the
 * binary16 half-norm pattern nearest n 2^15 / R (R / 32 levels per binade),
 * and n is the level whose value is nearest the binary16 half-norm h16 (a
 * tie to the even level, capped at the top finite level).  With R = 3 2^m
 * every code is 2^m d + l: m low bits l and a ternary digit d.  idx then
 * holds [layers][kv_heads][ceil(tokens / 4)][group_words] u32 (hnorm is
 * unused and may be NULL): one group per 4 token rows (rows past the end
 * are zero), wl = ceil(head_dim / 4 * m / 32), fh = ceil(head_dim / 32):
 *   words [0, 4 wl)      index low bits, row r's stream at word r wl, chunk c's
 *                        bits at stream bits c m .. c m + m - 1 (stream bit j is
 *                        bit j % 32 of word j / 32)
 *   words [4 wl, 8 wl)   norm low bits, the same way
 *   words [8 wl, end)    a stream of 13-bit fields: row r's 2 fh fields start
 *                        at bit 26 fh r; field f < fh holds the index digits of
 *                        chunks 8 f .. 8 f + 7, field fh + f their norm digits,
 *                        as sum_i d_i 3^i (3^8 <= 2^13).
 * At head_dim 128 a group is 61 words at S = 8 (3.8125 bits per element)
 * and 77 words at S = 32 (4.8125).
 *
 * Decoding: bulk chunk y = (2 * h) * (q_p * q_s) in fp32, rounded to the
 * output type, h the binary16 half-norm (packed format: the value the code
 * stands for); outlier chunk y = its side-list values.
 *
 * Codebook values.  Every call that takes a codebook (encode, decode,
 * attend, append, attend_paged) uses each fp32 value q on the
 * double-binary16 grid: q' = hi + lo with hi = binary16(q) and
 * lo = binary16(q - hi), both rounded to nearest even (q - hi and hi + lo
 * are exact in fp32; |q' - q| <= 2^-22 |q|).  The search splits each value
 * into exactly these two binary16 parts for the f16 matrix cores, so a
 * codebook off that grid encodes, decodes and attends exactly like its
 * rounded copy.  hqmq_make_codebook returns values already on the grid.
 *
 * Threading: every entry point is stateless and re-entrant; device work is
 * enqueued on the caller's stream and nothing is allocated.  Calls on
 * different streams that share output buffers race.
 */
#ifndef HQMQ_H_
#define HQMQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    HQMQ_OK = 0,
    HQMQ_EINVAL = -1,    /* bad descriptor, pointer, size or alignment */
    HQMQ_ENOTSUP = -2,   /* valid request outside this build's limits */
    HQMQ_ECAPACITY = -3, /* side list did not fit out_capacity */
    HQMQ_EHIP = -4       /* a HIP runtime call or kernel launch failed */
};

/* Element types of x and y. */
enum { HQMQ_F16 = 0, HQMQ_F32 = 1 };

/* Roles: which cache tensor a codebook belongs to. */
enum { HQMQ_ROLE_K = 0, HQMQ_ROLE_V = 1 };

/* Norm record formats (see hnorm above; HQMQ_NORM_EXACT: see below). */
enum { HQMQ_NORM_F16 = 0, HQMQ_NORM_PACKED = 1, HQMQ_NORM_EXACT = 2 };

/* Problem descriptor (a plain value, read only during the call).
 *   layers, kv_heads, tokens >= 0 (any of them 0 = empty input)
 *   head_dim in {16, 32, 64, 128, 256}
 *   S in [1, 1024]: secondary codewords per (layer, head)
 *   med_batch_tokens: Med3x batch length in tokens, 0 = Med3x off.  Batches
 *       start at token multiples of it within each slice; a final partial
 *       block is its own batch.  Median over the batch's chunks ("the
 *       current batch", gist.science/nl Methodologie 3).
 *   med_C: Med3x multiplier, the pages fix 3 (finite, > 0 when Med3x is on)
 *   dtype: HQMQ_F16 or HQMQ_F32 for x (and y)
 *   norm_format: HQMQ_NORM_F16, HQMQ_NORM_PACKED or HQMQ_NORM_EXACT (S a
 *       power of two, else HQMQ_ENOTSUP; not for paged pools). */
typedef struct hqmq_desc {
    int64_t layers;
    int64_t kv_heads;
    int64_t tokens;
    int64_t head_dim;
    int32_t S;
    int32_t dtype;
    int64_t med_batch_tokens;
    float med_C;
    int32_t norm_format;
} hqmq_desc;

/* Sizes of every buffer a call needs, in bytes (hqmq_sizes). */
typedef struct hqmq_sizes_t {
    int32_t code_bits;          /* b = ceil(log2(24 S)) */
    int32_t words_per_token;    /* ceil(b * head_dim / 4 / 32) */
    int64_t chunks;             /* layers * kv_heads * tokens * head_dim / 4 */
    int64_t batches;            /* Med3x batches (0 when Med3x is off) */
    int64_t max_outliers;       /* sum over batches of floor(n_batch / 2) (every
                                   chunk when fl(med_C * med_C) < 1) */
    uint64_t input_bytes;       /* x (and y) */
    uint64_t idx_bytes;         /* exact: slices * ceil(tokens / 4) * group_words * 4 */
    uint64_t hnorm_bytes;       /* chunks * 2 (binary16), idx_bytes (packed), 0 (exact) */
    uint64_t offsets_bytes;     /* (batches + 1) * 8, 0 when Med3x is off */
    uint64_t side_entry_bytes;  /* 12 bytes per outlier (4 pos + 8 values) */
    uint64_t workspace_bytes;   /* encode scratch: Med3x histograms and bitmasks, the
                                   binary16 half-norms when packed or exact, and the
                                   whole-bit codes when exact (0 if none) */
    uint64_t codebook_bytes;    /* layers * kv_heads * S * 16 */
    int32_t group_rows;         /* HQMQ_NORM_EXACT: 4 token rows per record group, else 0 */
    int32_t group_words;        /* HQMQ_NORM_EXACT: u32 words per group, else 0 */
} hqmq_sizes_t;

/* Encoded records: device pointers owned by the caller (see layout above).
 * hnorm is the norm plane in the descriptor's norm_format (u16 half-norms,
 * or the packed u32 words).  batch_offsets, out_pos, out_val and status may
 * be NULL when Med3x is off; out_pos/out_val may be NULL when out_capacity
 * is 0. */
typedef struct hqmq_enc {
    uint32_t *idx;
    void *hnorm;                /* 8-byte aligned (16 for hqmq_attend) */
    uint64_t *batch_offsets;
    uint32_t *out_pos;
    uint16_t *out_val;
    uint64_t out_capacity;
    uint64_t *status;
} hqmq_enc;

/* Message for a status code; never NULL. */
const char *hqmq_strerror(int code);

/* Buffer sizes for descriptor d.  Host only, no device work.
 * Errors: HQMQ_EINVAL for a NULL pointer or invalid descriptor. */
int hqmq_sizes(const hqmq_desc *d, hqmq_sizes_t *out);

/* Seeded secondary codebook ("S random unit quaternions" per (layer, head),
 * no calibration: the abstract; drawn per (layer, head, role): gist.science
 * Methodologie 1).  Writes [layers][kv_heads][S][4] fp32 into the caller's
 * HOST buffer out_host.  Uniform on S^3: Philox4x64-10 (Salmon et al., SC'11)
 * keyed (seed, layer << 32 | head << 8 | role), candidate j from counter
 * (j, 0, 0, 0), coordinates v_m = (2 (w_m >> 40) - 2^24 + 1) 2^-24, kept when
 * sum v^2 <= 1, q = v / sqrt(sum v^2) in fp64, rounded to fp32 and then to
 * the double-binary16 grid described above (q = hi + lo, 22 significant
 * bits), so that the stored values are the ones every kernel uses.
 * Bit-identical on every IEEE-754 host.  Host only.
 * Errors: HQMQ_EINVAL if out_host is NULL, layers or kv_heads < 0 or
 * >= 2^24, role not 0/1, or S outside [1, 1024]. */
int hqmq_make_codebook(uint64_t seed, int32_t layers, int32_t kv_heads, int32_t role,
                       int32_t S, float *out_host);

/* Encode x (device, [layers][kv_heads][tokens][head_dim] in d->dtype,
 * 16-byte aligned) with codebook (device, [layers][kv_heads][S][4] fp32,
 * used on the double-binary16 grid) into enc.  Steps: per chunk the fp32 norm and its binary16 half-norm code,
 * the nearest of the 24 S codewords <x, q_p q_s> (gist.science Methodologie
 * 1; the identity <x, q_p q_s> = <conj(q_p) x, q_s> of the isometry argument,
 * abstract), then, when Med3x is on, the exact lower median of s2 per batch,
 * outliers s2 > fl(fl(C*C) * median) flagged in hnorm and copied to the side
 * list in order; with HQMQ_NORM_PACKED the flagged half-norms are last turned
 * into packed compact codes.  workspace: device scratch of at least
 * hqmq_sizes().workspace_bytes, 256-byte aligned (may be NULL when that is 0).
 * Asynchronous on stream; nothing is enqueued when validation fails.  Ties
 * between exactly equal fp32 scores keep the smallest code.
 * Errors (synchronous): HQMQ_EINVAL (descriptor, NULL or misaligned pointer,
 * workspace too small), HQMQ_EHIP (launch failure).  Side-list overflow is
 * reported through status and hqmq_encode_result. */
int hqmq_encode(const hqmq_desc *d, const void *x, const float *codebook, const hqmq_enc *enc,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* hqmq_encode for profilers and benchmarks: identical work and results, and
 * additionally records search_begin immediately before and search_end
 * immediately after the launch of the nearest-codeword search kernel, on
 * stream, so that hipEventElapsedTime gives that kernel's duration.  Either
 * event may be NULL (not recorded).  Errors as hqmq_encode. */
int hqmq_encode_timed(const hqmq_desc *d, const void *x, const float *codebook,
                      const hqmq_enc *enc, void *workspace, size_t workspace_bytes,
                      hipStream_t stream, hipEvent_t search_begin, hipEvent_t search_end);

/* Wait for stream, read enc->status (16 bytes device to host) and return the
 * outlier count in *n_outliers.  Returns HQMQ_ECAPACITY (with the count
 * needed in *n_outliers) when the side list overflowed: re-allocate and
 * encode again.  Returns HQMQ_OK with 0 when Med3x was off (status NULL).
 * Errors: HQMQ_EINVAL (NULL enc or n_outliers), HQMQ_EHIP. */
int hqmq_encode_result(const hqmq_enc *enc, hipStream_t stream, uint64_t *n_outliers);

/* Decode enc into y (device, same shape as x, d->dtype, 16-byte aligned):
 * bulk chunks r^ (q_p q_s) with r^ = 2 h, h the half-norm of the record
 * (packed: the binary16 value its code stands for), computed in fp32 and
 * rounded to nearest even; outlier chunks take their side-list values (the decoder
 * the pages run before or inside attention: gist.science "Memory en
 * Latentie").  enc must come from hqmq_encode with the same descriptor and
 * codebook (used on the double-binary16 grid, as in the encode); after a
 * side-list overflow the chunks whose entries were dropped decode to their
 * bulk value.  Asynchronous on stream.
 * Errors: HQMQ_EINVAL, HQMQ_EHIP. */
int hqmq_decode(const hqmq_desc *d, const hqmq_enc *enc, const float *codebook, void *y,
                hipStream_t stream);

/* Scheduling, not part of the method: cap the blocks of the fp16 encode
 * search resident on one compute unit at n (1..7; 0, the default, removes
 * the cap).  Process-wide; it applies to the hqmq_encode, hqmq_encode_timed
 * and hqmq_append calls issued after it, and changes no output.  For callers
 * that run other work on a second stream during an encode (for example the
 * decode of the role encoded before): uncapped, the search fills every CU
 * and refills each slot a block frees, so the other stream's kernels wait
 * for its tail; at n = 7 a CU keeps one block slot (4 waves, about 16 KB of
 * LDS) for them.  The search blocks then reserve LDS they do not use.
 * Errors: HQMQ_EINVAL for n outside 0..7. */
int hqmq_set_search_blocks_per_cu(int32_t n);

/* ------------------------------------------------------------------------
 * Decode-step attention read straight from the records (gist.science/nl
 * "Technische Samenvatting", "Memory en Latentie": a fused kernel decodes K
 * and V inside the attention loop instead of dequantising the whole cache
 * each step).  For one layer of an encoded cache, every sequence b and query
 * head j (GQA: query head j reads KV head j / group):
 *
 *     out[b][j] = sum_t softmax_t(scale <q[b][j], k_t>) v_t,
 *
 * t over tokens [seq_start[b], seq_start[b] + seq_len[b]) of the (layer, KV
 * head) slice, k_t and v_t the binary16 values hqmq_decode would write.
 * Scores are fp32 sums of exact binary16 products; the softmax runs in fp32
 * and the weights enter the value sum rounded to binary16 (each within a
 * relative 2^-11), normalised by the sum of the same rounded weights.  An
 * empty sequence gives zeros.
 * ------------------------------------------------------------------------ */
typedef struct hqmq_attn_desc {
    int32_t batch;      /* sequences, >= 0 */
    int32_t group;      /* query heads per KV head, 1..16 */
    int32_t layer;      /* cache layer attended, 0 .. layers - 1 */
    int32_t max_len;    /* upper bound of every seq_len[b] (sizes the launch), >= 0 */
    float scale;        /* logit scale, finite (for example 1 / sqrt(head_dim)) */
    int32_t reserved;   /* must be 0 */
} hqmq_attn_desc;

typedef struct hqmq_attn_sizes_t {
    uint64_t workspace_bytes;   /* batch * kv_heads * group * splits * (head_dim + 2) * 4 */
    int32_t splits;             /* token splits per sequence */
    int32_t split_tokens;       /* tokens per split, a multiple of 128 */
} hqmq_attn_sizes_t;

/* Workspace size and split plan of hqmq_attend for cache d and request a.
 * Host only.  Errors: HQMQ_EINVAL (NULL pointer, invalid descriptor or
 * request), HQMQ_ENOTSUP (d->dtype not HQMQ_F16, head_dim not 64, 128 or
 * 256, or a launch beyond the kernel's limits). */
int hqmq_attn_sizes(const hqmq_desc *d, const hqmq_attn_desc *a, hqmq_attn_sizes_t *out);

/* Attention of one decode step over layer a->layer of the cache encoded as
 * k (role K, codebook_k) and v (role V, codebook_v), both from hqmq_encode
 * with descriptor d (codebooks used on the double-binary16 grid).  Device arrays: q [batch][kv_heads * group][head_dim]
 * binary16 (8-byte aligned); seq_start [batch] int64 and seq_len [batch]
 * int32 (token ranges within each slice; a range is clipped to the slice
 * and to max_len, a negative length counts as 0); out [batch][kv_heads *
 * group][head_dim] fp32; workspace of at least hqmq_attn_sizes()
 * .workspace_bytes, 16-byte aligned.  Asynchronous on stream; nothing is
 * enqueued when validation fails.  Errors: HQMQ_EINVAL, HQMQ_ENOTSUP (as
 * hqmq_attn_sizes), HQMQ_EHIP. */
int hqmq_attend(const hqmq_desc *d, const hqmq_attn_desc *a, const hqmq_enc *k, const float *codebook_k,
                const hqmq_enc *v, const float *codebook_v, const void *q, const int64_t *seq_start,
                const int32_t *seq_len, float *out, void *workspace, size_t workspace_bytes,
                hipStream_t stream);

/* hqmq_attend for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and results, with the split partials
 * kept in a library-owned device array of HQMQ_ATTEND_SCRATCH_BYTES per GPU
 * (a file-scope array each GPU holds until the process ends) instead of a
 * caller workspace.  The call allocates nothing; its first call on a device
 * looks the array's address up once.  stream must belong to the current
 * device.  Calls that overlap on one GPU share the array and race: order
 * them on one stream (or with events).  Errors: as hqmq_attend, and
 * HQMQ_ENOTSUP when hqmq_attn_sizes() gives a workspace larger than
 * HQMQ_ATTEND_SCRATCH_BYTES (nothing enqueued). */
#define HQMQ_ATTEND_SCRATCH_BYTES ((size_t)16 << 20)
int hqmq_attend_noalloc(const hqmq_desc *d, const hqmq_attn_desc *a, const hqmq_enc *k,
                        const float *codebook_k, const hqmq_enc *v, const float *codebook_v, const void *q,
                        const int64_t *seq_start, const int32_t *seq_len, float *out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Paged cache with streaming append.  A serving loop keeps each role's
 * records in a pool of fixed-size pages, appends every step's new tokens
 * into free slots and attends over each sequence's pages (the decode-step
 * use of gist.science/nl "Memory en Latentie").  An append call encodes its
 * tokens exactly as hqmq_encode encodes a tensor of that many tokens: the
 * Med3x batch is med_batch_tokens of the call's tokens of one (layer, head),
 * so a decode step's tokens form one batch per (layer, head) ("the current
 * batch", gist.science/nl Methodologie 3).
 *
 * Pool layout (P = page_tokens, W = words per token, cpt = head_dim / 4):
 *   idx        [layers][kv_heads][num_pages][P][W] u32, token rows as in idx
 *   hnorm      [layers][kv_heads][num_pages][P][cpt] u16 (HQMQ_NORM_F16), or
 *              [layers][kv_heads][num_pages][P][W] u32 (HQMQ_NORM_PACKED)
 *   side_count [layers][kv_heads][num_pages] u32: entries in each page's list
 *   side_pos   [layers][kv_heads][num_pages][page_capacity] u32: o * cpt + c
 *              for chunk c of the token at offset o of the page
 *   side_val   [layers][kv_heads][num_pages][page_capacity][4] binary16
 * Slot page * P + o is offset o of page `page`.  A page's side list holds
 * its outlier chunks in position order.  Each (layer, head) slice of the
 * pool is a record tensor of num_pages * P tokens in the layout above.
 * ------------------------------------------------------------------------ */
typedef struct hqmq_paged_desc {
    int64_t num_pages;        /* pages in the pool, >= 0 */
    int32_t page_tokens;      /* P: a multiple of 16, P * head_dim / 4 < 2^31 */
    int32_t page_capacity;    /* side-list entries per (layer, head, page), >= 0 */
} hqmq_paged_desc;

/* One role's pool: device pointers owned by the caller (layout above;
 * idx, side_count, side_pos 4-byte aligned, hnorm and side_val 16-byte
 * aligned). */
typedef struct hqmq_pages {
    uint32_t *idx;
    void *hnorm;
    uint32_t *side_count;
    uint32_t *side_pos;
    uint16_t *side_val;
} hqmq_pages;

typedef struct hqmq_paged_sizes_t {
    uint64_t idx_bytes;
    uint64_t hnorm_bytes;
    uint64_t side_count_bytes;
    uint64_t side_pos_bytes;
    uint64_t side_val_bytes;
    uint64_t append_workspace_bytes;   /* hqmq_append of d->tokens tokens */
} hqmq_paged_sizes_t;

/* Pool sizes for codec descriptor d and pool p, and the workspace of an
 * append of d->tokens tokens (the call's records with a worst-case side
 * list, plus the encode scratch).  Host only.
 * Errors: HQMQ_EINVAL (NULL pointer, invalid descriptor or pool),
 * HQMQ_ENOTSUP (pool beyond 32-bit positions or grid limits). */
int hqmq_paged_sizes(const hqmq_desc *d, const hqmq_paged_desc *p, hqmq_paged_sizes_t *out);

/* Empty the n pages listed in pages (device int32 page ids): zero their
 * side-list counts in every (layer, head), so they can take new tokens.
 * Ids outside [0, num_pages) are skipped.  A fresh pool needs its whole
 * side_count array zeroed (this call with every page, or a device fill).
 * Asynchronous on stream.  Errors: HQMQ_EINVAL, HQMQ_EHIP. */
int hqmq_paged_clear(const hqmq_desc *d, const hqmq_paged_desc *p, const hqmq_pages *pool,
                     const int32_t *pages, int64_t n, hipStream_t stream);

/* Append d->tokens tokens x [layers][kv_heads][tokens][head_dim] (d->dtype,
 * 16-byte aligned) to the pool: token t of every (layer, head) goes to slot
 * slots[t] (device int64).  The records are those hqmq_encode writes for x
 * with descriptor d (codes, norms in d->norm_format, Med3x flags); the
 * outlier chunks of each page go to the end of that page's side list.
 * Preconditions, not checked: slots are distinct; the tokens one call
 * writes to a page are consecutive in the call, in increasing offset order,
 * and come after every token already in the page (the way a sequence
 * grows).  A slot outside [0, num_pages * P) is skipped with its token.
 * Entries past page_capacity are dropped: their chunks keep the bulk record
 * (flag cleared).  status (device [2] u64, may be NULL) receives the
 * outlier chunks of the tokens written and how many of them were dropped.  workspace: at least
 * hqmq_paged_sizes().append_workspace_bytes for d, 256-byte aligned.
 * Asynchronous on stream; nothing is enqueued when validation fails.
 * Errors: HQMQ_EINVAL, HQMQ_ENOTSUP (as hqmq_paged_sizes), HQMQ_EHIP. */
int hqmq_append(const hqmq_desc *d, const hqmq_paged_desc *p, const void *x, const int64_t *slots,
                const float *codebook, const hqmq_pages *pool, uint64_t *status, void *workspace,
                size_t workspace_bytes, hipStream_t stream);

/* hqmq_attend over paged pools: sequence b's token t is at slot
 * page_table[b * page_table_stride + t / P] * P + t % P of k and v (device
 * int32 page table, ids in [0, num_pages)), and it has seq_len[b] tokens
 * (a negative length counts as 0; clipped to max_len and to
 * page_table_stride * P).  Scores, softmax, GQA and output as hqmq_attend;
 * d gives the codec parameters (d->tokens is not used).  The workspace and
 * split plan are hqmq_attn_sizes(d, a).  Errors: as hqmq_attend, and
 * HQMQ_EINVAL for an invalid pool or page_table_stride < 1. */
int hqmq_attend_paged(const hqmq_desc *d, const hqmq_paged_desc *p, const hqmq_attn_desc *a,
                      const hqmq_pages *k, const float *codebook_k, const hqmq_pages *v,
                      const float *codebook_v, const void *q, const int32_t *page_table,
                      int32_t page_table_stride, const int32_t *seq_len, float *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HQMQ_H_ */
