// Encode-search pieces shared by the two search translation units: the
// fp32-input search (hqmq_kernels.hip, IEEE mode) and the fp16-input search
// on the f16 matrix cores (hqmq_search.hip, built with IEEE mode off and fp32
// denormals flushed).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqmq_device.h"

namespace hqmq {

// Arguments of one encode-search launch.
struct EncArgs {
    const void *x;
    const float *cb;
    uint32_t *idx;
    uint16_t *hnorm;
    int64_t n_slice;
    int64_t tiles_per_slice;
    int64_t tokens;
    int32_t tile_chunks;
    int32_t S;
    int32_t NT;     // ceil(S / 4) tiles of 4 secondary codewords
    int32_t cpt;
    int32_t log2_cpt;
    int32_t bits;
    int32_t words;
    // Med3x (batch_chunks == 0: off).  Tiles are grouped by batch and
    // accumulate the batch's histogram of half-norm codes.
    int32_t tiles_per_batch;
    int64_t batch_chunks;
    int64_t bps;            // batches per slice
    int64_t nbatch;         // slices * bps
    int32_t xcd_map;        // 1: a batch's tiles are dispatched to one XCD
    uint32_t *hist;         // [nbatch][2048] histograms of hnorm >> 4, zeroed
};

// fp16-input search launch (hqmq_search.hip): blocks of kEncThreads threads,
// nt8 = ceil(S / 8) tiles of 8 secondary codewords.  blocks_per_cu > 0 caps
// the blocks resident per CU at that many (each block then reserves LDS it
// does not use), leaving the rest of every CU to work on other streams.
hipError_t launch_search_h(const EncArgs &a, int64_t blocks, int nt8, bool med, int blocks_per_cu,
                           hipStream_t st);

namespace {

constexpr int kEncThreads = 256;   // 4 waves; each wave encodes 64 chunks per step
constexpr int kMaxS = 1024;

// Work-item and work-group ids straight from the hardware registers (the
// runtime's accessors are library functions, which are not inlined into a
// translation unit built in another floating-point mode).
__device__ __forceinline__ int thread_id() { return static_cast<int>(__builtin_amdgcn_workitem_id_x()); }
__device__ __forceinline__ int64_t block_id() { return static_cast<int64_t>(__builtin_amdgcn_workgroup_id_x()); }

// Correctly rounded fp32 square root of a >= 0.  v_sqrt_f32 is within one
// ulp; the result is then moved to the neighbour whose rounding interval
// holds sqrt(a), decided exactly in fp64: the midpoints between y and its
// neighbours have at most 25 significant bits, so their squares are exact.
// Inputs below 2^-100 are scaled by 2^100 first (exact) to stay in the
// normal range of v_sqrt_f32.
__device__ __forceinline__ float sqrt_rn(float a) {
    if (!(a > 0.0f)) return a;  // 0 (and the documented non-finite precondition)
    const bool tiny = a < 0x1p-100f;
    const float as = tiny ? a * 0x1p100f : a;
    float y = __builtin_amdgcn_sqrtf(as);
    const double ad = static_cast<double>(as);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const float yu = __uint_as_float(__float_as_uint(y) + 1u);
        const float yd = __uint_as_float(__float_as_uint(y) - 1u);
        const double hi = (static_cast<double>(y) + static_cast<double>(yu)) * 0.5;
        const double lo = (static_cast<double>(y) + static_cast<double>(yd)) * 0.5;
        if (ad > hi * hi) y = yu;
        else if (ad < lo * lo) y = yd;
    }
    return tiny ? y * 0x1p-50f : y;
}

// binary16 half-norm code fp16_rn(sqrt_rn(s2) / 2).  v_sqrt_f32 is within one
// ulp, so h = v_sqrt_f32(s2) / 2 and the exact half-root round to the same
// binary16 unless a rounding midpoint lies within one fp32 ulp of h: in the
// normal binary16 range [2^-14, 2^16) the midpoints are the fp32 values whose
// low 13 mantissa bits are 0x1000, so h is safe unless those bits are
// 0x0FFF..0x1001.  Only the others (about 3 in 8192 chunks, and any h outside
// that range) take the correctly rounded root.
// h: v_sqrt_f32(s2) / 2, formed by the caller.
__device__ __forceinline__ uint16_t half_norm_code(float s2, float h) {
    const uint32_t hb = __float_as_uint(h);
    const bool safe = (hb - 0x38800000u) < (0x47800000u - 0x38800000u) && ((hb & 0x1FFFu) - 0x0FFFu) > 2u;
    if (safe) return f32_to_f16_bits(h);
    return f32_to_f16_bits(sqrt_rn(s2) * 0.5f);
}
__device__ __forceinline__ uint16_t half_norm_code(float s2) {
    return half_norm_code(s2, __builtin_amdgcn_sqrtf(s2) * 0.5f);
}


// Chunk range of this block.  Without Med3x: tiles_per_slice tiles per
// slice.  With Med3x: tiles_per_batch tiles per batch, the last one partial
// or empty; blocks are dispatched to the 8 XCDs round-robin, so with
// xcd_map block b serves batch (b / 8 / tiles_per_batch) * 8 + b % 8 and the
// histogram atomics of a batch stay within one XCD.
struct TileCoords {
    int64_t slice, c_begin, c_end;
    int64_t batch, b_lo, b_n;   // Med3x: batch index, first chunk, chunk count
};

// The block's values, computed per lane but equal in every lane, as scalar
// registers: keeps the 64-bit arithmetic on them and the buffer resources
// built from them scalar (a value the compiler cannot prove uniform would
// otherwise make each buffer access a loop over the distinct resources).
__device__ __forceinline__ int64_t uniform(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T *uniform(T *p) {
    return reinterpret_cast<T *>(static_cast<uintptr_t>(uniform(static_cast<int64_t>(reinterpret_cast<uintptr_t>(p)))));
}

__device__ __forceinline__ TileCoords uniform(TileCoords t) {
    t.slice = uniform(t.slice);
    t.c_begin = uniform(t.c_begin);
    t.c_end = uniform(t.c_end);
    t.batch = uniform(t.batch);
    t.b_lo = uniform(t.b_lo);
    t.b_n = uniform(t.b_n);
    return t;
}

__device__ __forceinline__ TileCoords tile_coords(const EncArgs &a) {
    TileCoords t;
    const int64_t bid = block_id();
    if (a.batch_chunks == 0) {
        t.slice = bid / a.tiles_per_slice;
        t.c_begin = (bid - t.slice * a.tiles_per_slice) * a.tile_chunks;
        t.c_end = min(t.c_begin + static_cast<int64_t>(a.tile_chunks), a.n_slice);
        t.batch = -1;
        t.b_lo = 0;
        t.b_n = 0;
        return uniform(t);
    }
    const int64_t tpb = a.tiles_per_batch;
    int64_t batch, tile;
    if (a.xcd_map) {
        const int64_t j = bid >> 3;
        batch = (j / tpb) * 8 + (bid & 7);
        tile = j - (j / tpb) * tpb;
    } else {
        batch = bid / tpb;
        tile = bid - batch * tpb;
    }
    t.batch = batch;
    t.slice = batch / a.bps;
    t.b_lo = (batch - t.slice * a.bps) * a.batch_chunks;
    t.b_n = min(a.batch_chunks, a.n_slice - t.b_lo);
    t.c_begin = t.b_lo + tile * a.tile_chunks;
    t.c_end = min(t.c_begin + static_cast<int64_t>(a.tile_chunks), t.b_lo + t.b_n);
    return uniform(t);
}


// Called by every thread of a Med3x tile after its search loop: merge the
// tile's code histogram into its batch's (read by the next kernel).
__device__ void med3_after_tile(const EncArgs &a, const TileCoords &tc, uint32_t *shist, uint32_t *) {
    __syncthreads();
    uint32_t *gh = a.hist + tc.batch * 2048;
    for (int i = thread_id(); i < 2048; i += kEncThreads) {
        const uint32_t v = shist[i];
        if (v) atomicAdd(&gh[i], v);
    }
}


}  // namespace
}  // namespace hqmq
