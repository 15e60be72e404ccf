"""MI355X-native rotated INT4 paged KV cache (SAW-INT4 hot path).

The compute lives in ``libkvrq.so`` (HIP kernels for gfx950 behind the C ABI
of ``include/kvrq.h``); this package only marshals arguments.  Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built (``python -m int4_kv_cache_rotquant_amd.build``).
"""
from ._binding import (  # noqa: F401
    CacheBuffers,
    CacheDesc,
    HEAD_DIM,
    KVRQ_EHIP,
    KVRQ_EINVAL,
    KVRQ_ENOPAGES,
    KVRQ_EUNSUPPORTED,
    KVRQ_EWORKSPACE,
    KVRQ_OK,
    KVRQ_SPLIT_BALANCED,
    KvrqError,
    LIB_PATH,
    PagedInt4Cache,
    Pool,
    kv_int4_paged_decode,
    kv_int4_paged_decode_noalloc,
    kv_int4_paged_decode_workspace,
    kv_int4_paged_decode_step,
    kv_int4_paged_extend,
    kv_int4_paged_extend_workspace,
    kv_rotquant_write,
    kvrq_bf16_paged_write,
    kvrq_cache_sizes,
    kvrq_device_copy,
    kvrq_device_read,
    kvrq_paged_read,
    last_error,
    lib,
    status_str,
)
