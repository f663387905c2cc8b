// Internal launch interface between the C-ABI host code (hqmq_api.cpp) and
// the gfx950 kernels (hqmq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace hqmq {

// Shape of one call after validation.
struct Geometry {
    int64_t slices;          // layers * kv_heads
    int64_t tokens;          // tokens per slice
    int64_t n_slice;         // chunks per slice = tokens * cpt
    int32_t cpt;             // chunks per token = head_dim / 4
    int32_t S;               // secondary codewords per slice
    int32_t bits;            // code width b
    int32_t words;           // u32 words per token row
    int32_t f32;             // 1: fp32 x / y, 0: fp16
    int64_t batch_chunks;    // Med3x batch length in chunks (0 = off)
    int64_t batches_per_slice;
    float med_C;
    int32_t npack;           // 1: norms as packed compact codes (b bits per chunk)
    // exact-rate records (norm_format HQMQ_NORM_EXACT; S a power of two):
    // groups of 4 token rows, each code m low bits plus a ternary digit
    int32_t exact;
    int32_t em;              // 24 S = 3 2^m
    int32_t ewl;             // words of low bits per row and plane: ceil(cpt m / 32)
    int32_t efh;             // digit fields per row and plane: ceil(cpt / 8)
    int32_t egw;             // words per group
    int64_t egps;            // groups per slice: ceil(tokens / 4)
    uint32_t enmax;          // top finite norm level
    float estep;             // fp32(2^(15 - m) / 3): norm level n sits at pattern round(n estep)
};

// Encode scratch (inside the caller's workspace).
struct Med3Work {
    uint32_t *hist;      // [batches][2048] histograms of the half-norm code >> 4
    uint32_t *counts;    // [batches] outliers per batch
    uint32_t *mask;      // [batches][mask_words] outlier bitmasks
    int64_t mask_words;
    uint16_t *h16;       // packed and exact formats: the binary16 half-norm plane
    uint32_t *idx32;     // exact format: the whole-bit code plane the search writes
};

// Encode: nearest codeword and norm code per chunk; with med != nullptr the
// launch also accumulates each batch's code histogram (med->hist must be
// zero).  The fp16 search keeps at most search_blocks_per_cu() blocks on a
// CU when that is above 0.
hipError_t launch_encode_search(const Geometry &g, const void *x, const float *codebook,
                                uint32_t *idx, uint16_t *hnorm, const Med3Work *med, hipStream_t st);

// The fp16 search's cap on resident blocks per CU (0: none), process-wide.
void set_search_blocks_per_cu(int n);
int search_blocks_per_cu();

// Med3x: per batch, exact median, threshold, outlier count and bitmask (and,
// for batches of at most 131072 chunks, the outlier flags in hnorm).  With
// pwords != nullptr and single-pass batches (med3_single_pass), the select
// also packs the batch's final codes into the record's norm words.
hipError_t launch_med3_select(const Geometry &g, const void *x, uint16_t *hnorm, const Med3Work &med,
                              uint32_t *pwords, hipStream_t st);

// Whether Med3x batches of this geometry take the single-pass select.
bool med3_single_pass(const Geometry &g);

// Exclusive scan of the per-batch counts into batch_offsets, total and
// overflow flag into status.
hipError_t launch_med3_scan(int64_t batches, const uint32_t *counts, uint64_t *offsets,
                            uint64_t capacity, uint64_t *status, hipStream_t st);

// Ordered side-list write from the bitmasks (and the outlier flags in hnorm
// where the select kernel has not set them).
hipError_t launch_med3_gather(const Geometry &g, const void *x, const Med3Work &med,
                              const uint64_t *offsets, uint16_t *hnorm, uint32_t *out_pos,
                              uint16_t *out_val, uint64_t capacity, hipStream_t st);

// Fill words with a kernel rather than a memset node (status / offsets of
// empty or Med3x-off calls, Med3x histograms).
hipError_t launch_fill_u64(uint64_t *p, int64_t n, uint64_t v, hipStream_t st);
hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st);

// Packed norm format: compact codes of the binary16 half-norms h16 (flag
// bit -> all-ones code), packed per token row like the index codes.
hipError_t launch_pack_norms(const Geometry &g, const uint16_t *h16, uint32_t *words, hipStream_t st);

// Exact-rate format: the group records of the whole-bit codes idx32 and the
// binary16 half-norms h16 (flags included).
hipError_t launch_pack_exact(const Geometry &g, const uint32_t *idx32, const uint16_t *h16, uint32_t *groups,
                             hipStream_t st);

// Decode: bulk gather-multiply plus outlier re-insertion (hnorm: the norm
// plane in the geometry's format; exact format: idx holds the groups).
hipError_t launch_decode(const Geometry &g, const uint32_t *idx, const void *hnorm,
                         const uint64_t *offsets, const uint32_t *out_pos, const uint16_t *out_val,
                         uint64_t capacity, const float *codebook, void *y, hipStream_t st);

// One encoded tensor (K or V) as the attention kernel reads it.
struct AttRole {
    const uint32_t *idx;
    const uint16_t *hnorm;
    const uint64_t *offsets;   // Med3x batch offsets (nullptr when off)
    const uint32_t *out_pos;
    const uint16_t *out_val;
    uint64_t capacity;
    const float *cb;           // [layers][kv_heads][S][4]
    const uint32_t *side_count;   // paged pools: entries per (slice, page)
};  // hnorm: binary16 half-norms, or packed compact codes (AttLaunch::npack)

// Decode-step attention over one layer of an encoded cache.
struct AttLaunch {
    AttRole k, v;
    const uint16_t *q;          // [batch][heads * group][head_dim] binary16
    const int64_t *seq_start;   // [batch]
    const int32_t *seq_len;     // [batch]
    float *part;                // [batch][heads * group][nsplit][head_dim + 2]
    float *out;                 // [batch][heads * group][head_dim]
    int64_t tokens;             // tokens per slice
    int64_t batch_chunks;       // Med3x batch length in chunks (0 = off)
    int64_t bps;                // Med3x batches per slice (0 = off)
    int32_t layer, heads, group, batch, nsplit, split_tokens, max_len, head_dim, S, bits, words, npack;
    // exact-rate records (see Geometry)
    int32_t exact, em, ewl, efh, egw;
    int64_t egps;
    float estep;
    float scale;
    // paged pools (page_table != nullptr): rows at (slice * num_pages + page) * P + offset,
    // side lists of page_cap entries per (slice, page); seq_start is not used
    const int32_t *page_table;  // [batch][pt_stride]
    int64_t num_pages;
    int32_t pt_stride, log2_page;
    uint32_t page_cap;
};

// Dynamic LDS of the attention kernel for this shape (0: unsupported head_dim).
size_t attend_lds_bytes(int head_dim, int S, bool exact);
hipError_t launch_attend(const AttLaunch &L, hipStream_t st);

// Paged pool of one role (device pointers), as the append kernels write it.
struct PagedPool {
    uint32_t *idx;          // [slices][num_pages * P][W]
    void *hnorm;            // [slices][num_pages * P][cpt] u16, or [..][W] u32 (npack)
    uint32_t *side_count;   // [slices][num_pages]
    uint32_t *side_pos;     // [slices][num_pages][cap]
    uint16_t *side_val;     // [slices][num_pages][cap][4]
    int64_t num_pages;
    int32_t log2_page;
    uint32_t cap;
};

// Append: the call's records (the encode of its tokens with geometry g,
// binary16 norms with flags in h16) moved into the pool at slots[t].  The
// side entries go to the end of their pages' lists (entries past the
// capacity are dropped and their flags cleared in h16); then the token rows
// are written (norms packed when g.npack).
hipError_t launch_paged_scatter(const Geometry &g, const uint64_t *offsets, const uint32_t *out_pos,
                                const uint16_t *out_val, const int64_t *slots, uint16_t *h16,
                                const PagedPool &pool, uint64_t *status, hipStream_t st);
hipError_t launch_paged_rows(const Geometry &g, const uint32_t *idx, const uint16_t *h16, const int64_t *slots,
                             const PagedPool &pool, hipStream_t st);
// Zero the side-list counts of the n pages listed (every slice).
hipError_t launch_paged_clear(int64_t slices, const int32_t *pages, int64_t n, const PagedPool &pool,
                              hipStream_t st);

}  // namespace hqmq
