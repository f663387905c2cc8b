// hqmq_attend_noalloc (declared in include/hqmq.h): decode-step attention
// for callers that cannot allocate (code under HIP graph capture, tight
// serving loops).  The per-split partial results that hqmq_attend keeps in
// the caller's workspace live here in a file-scope device array instead,
// one copy per GPU, found once per device with hipGetSymbolAddress.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hqmq.h"

// The attention partials of one call: batch * kv_heads * group * splits *
// (head_dim + 2) fp32 values (2.1 MB for 32 sequences x 32 query heads x 4
// splits at head_dim 128).  Every call on a device reuses this array.  In
// host code this name is only a handle for hipGetSymbolAddress: kernels get
// the address that call returns.
static __device__ __align__(256) unsigned char scratch[HQMQ_ATTEND_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void *g_scratch[kMaxDevices];   // the array's device address, per device

// The device address of `scratch` on the current device (looked up on the
// first call there, with that device current); nullptr on failure.
void *scratch_ptr(int *err) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = HQMQ_EHIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            *err = HQMQ_EHIP;
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int hqmq_attend_noalloc(const hqmq_desc *d, const hqmq_attn_desc *a, const hqmq_enc *k,
                                   const float *codebook_k, const hqmq_enc *v, const float *codebook_v,
                                   const void *q, const int64_t *seq_start, const int32_t *seq_len, float *out,
                                   hipStream_t stream) {
    hqmq_attn_sizes_t sz;
    const int rc = hqmq_attn_sizes(d, a, &sz);
    if (rc != HQMQ_OK) return rc;
    if (sz.workspace_bytes > HQMQ_ATTEND_SCRATCH_BYTES) return HQMQ_ENOTSUP;
    if (a->batch == 0 || d->kv_heads == 0) return hqmq_attend(d, a, k, codebook_k, v, codebook_v, q, seq_start,
                                                              seq_len, out, nullptr, 0, stream);
    int err = HQMQ_OK;
    void *ws = scratch_ptr(&err);
    if (ws == nullptr) return err;
    // the split kernel writes every partial it reads back (empty splits
    // included), so nothing needs clearing between calls
    return hqmq_attend(d, a, k, codebook_k, v, codebook_v, q, seq_start, seq_len, out, ws,
                       HQMQ_ATTEND_SCRATCH_BYTES, stream);
}
