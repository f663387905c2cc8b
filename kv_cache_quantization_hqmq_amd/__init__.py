"""HQMQ KV-cache codec for AMD Instinct MI355X (gfx950).

The codec runs in the HIP kernels of ``libhqmq.so`` behind the C ABI declared
in ``include/hqmq.h`` (and the measurement helpers of ``include/hqmq_ceiling.h``);
``kv_cache_quantization_hqmq_amd.hqmq`` is its ctypes
binding (same function names).  Build with
``python -m kv_cache_quantization_hqmq_amd.build``.
"""
from .hqmq import (AttnDesc, AttnSizes, CapacityError, Desc, HQMQError, PagedDesc, PagedSizes, Pages, Pool,
                   Records, Sizes, allocate_pool, allocate_records, append, append_workspace, attend,
                   attend_paged, decode, encode, hqmq_append, hqmq_attend, hqmq_attend_paged,
                   hqmq_attn_sizes, hqmq_decode, hqmq_paged_clear, hqmq_paged_sizes,
                   hqmq_encode, hqmq_encode_result, hqmq_encode_timed, hqmq_make_codebook, hqmq_sizes,
                   hqmq_set_search_blocks_per_cu, hqmq_strerror, workspace, HQMQ_F16, HQMQ_F32, HQMQ_NORM_F16, HQMQ_NORM_PACKED, HQMQ_NORM_EXACT,
                   HQMQ_ROLE_K, HQMQ_ROLE_V, hqmq_ceiling_compute, hqmq_ceiling_stream, HQMQ_CEIL_READ,
                   HQMQ_CEIL_WRITE, HQMQ_CEIL_COPY, HQMQ_CEIL_FMA_F32, HQMQ_CEIL_MFMA_F32, HQMQ_CEIL_MFMA_F16)

__all__ = ["AttnDesc", "AttnSizes", "CapacityError", "Desc", "HQMQError", "PagedDesc", "PagedSizes",
           "Pages", "Pool", "Records", "Sizes", "allocate_pool", "allocate_records", "append",
           "append_workspace", "attend", "attend_paged", "decode", "encode", "hqmq_append", "hqmq_attend",
           "hqmq_attend_paged", "hqmq_attn_sizes", "hqmq_paged_clear", "hqmq_paged_sizes",
           "hqmq_decode", "hqmq_encode", "hqmq_encode_result", "hqmq_encode_timed",
           "hqmq_make_codebook", "hqmq_sizes", "hqmq_set_search_blocks_per_cu", "hqmq_strerror", "workspace",
           "HQMQ_F16",
           "HQMQ_F32", "HQMQ_NORM_F16", "HQMQ_NORM_PACKED", "HQMQ_NORM_EXACT", "HQMQ_ROLE_K", "HQMQ_ROLE_V",
           "hqmq_ceiling_compute", "hqmq_ceiling_stream", "HQMQ_CEIL_READ", "HQMQ_CEIL_WRITE", "HQMQ_CEIL_COPY",
           "HQMQ_CEIL_FMA_F32", "HQMQ_CEIL_MFMA_F32", "HQMQ_CEIL_MFMA_F16"]
