"""MI355X-native Multi-head Latent Attention decode over a latent KV cache.

The compute lives in libmla.so (HIP kernels for gfx950 behind the C ABI of include/mla.h);
this package is its Python binding.
"""
from .binding import (  # noqa: F401
    BF16, F16, F32, FP6_E2M3, FP8_E4M3, DecodeStep, Dims, LatentCache, MLAError, PrecombinedStep, PrefillStep, absorb_out,
    absorb_out_noalloc, absorb_out_pre, combine_absorb_out, absorb_out_pre_workspace_bytes, absorb_out_workspace_bytes,
    absorb_q, absorb_q_pre, absorb_q_workspace_bytes, cache_store, combine, decode_attn, decode_workspace_bytes, lib,
    precombine, prefill_tables, rope, row_bytes,
    absorb_q_naive, output_proj, output_proj_workspace_bytes, prefill_naive_attn, prefill_naive_workspace_bytes,
    NAIVE_MIN_CHUNK, choose_prefill_form, naive_form_available, fused_output_suits,
    stream_read, STREAM_SINK_WORDS, version,
)
