"""MI355X (gfx950) dynamically quantized paged KV cache: quantize-on-write and
paged decode attention behind the C ABI of include/kvq.h (libkvq.so).

The Python layer marshals arguments only; every step runs in HIP kernels.
"""
from .kvq import (CacheDesc, KvqError, alloc_cache, alloc_workspace, kvq_calibrate_channel_scales,  # noqa: F401
                  kvq_decode_step, kvq_decode_workspace_size, kvq_gather_dequant,
                  kvq_paged_decode_attention, kvq_paged_decode_attention_noalloc,
                  kvq_paged_prefill_attention, kvq_prefill_workspace_size,
                  kvq_query_layout,
                  kvq_reshape_and_cache, kvq_workspace_init, KVQ_INT8_SYM, KVQ_INT4_ASYM,
                  KVQ_INT2_ASYM, KVQ_INT8_CHANNEL, KVQ_FP8_E4M3, KVQ_INT4_INLINE, KVQ_OUT_F32,
                  KVQ_OUT_BF16)
from ._lib import LIB_PATH, load as load_library  # noqa: F401
