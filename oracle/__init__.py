"""CPU oracle for MLA decode over a latent KV cache — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The GPU library never imports, links or calls it, and it shares no code with the GPU library.
"""
from .encodings import (  # noqa: F401
    bf16_encode, bf16_decode, fp16_encode, fp16_decode, e4m3_encode, e4m3_decode,
    quantize_row_e4m3, quantize_rows_e4m3, store_rows, load_rows,
    e2m3_encode, e2m3_decode, pack_e2m3, unpack_e2m3, quantize_rows_e2m3,
)
from .mla import (  # noqa: F401
    OracleDims, softmax, rope, rope_frequencies, score_scale, decode_step_explicit, decode_step_absorbed, decode_batch, prefill_chunk,
    head_slices, absorbed_query, output_projection, precombined_heads, precombined_weights, decode_step_precombined,
)
from .counts import cache_counts  # noqa: F401
