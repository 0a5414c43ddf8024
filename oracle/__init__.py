"""CPU oracle for exact scaled-dot-product attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may import
this package. The library (``io_aware_softmax_03_amd``) never imports it and has
no CPU fallback; the two share no code. Inputs come from ``synth``, which holds
no attention arithmetic.

Everything here is plain float64 numpy that materialises the full score matrix
S and probability matrix P, so a reader can check it against the definitions on
the pages by eye:

* ``attention``  — the definitions the GPU results are compared with:
  forward, packed variable-length forward, backward (exact gradient of the
  forward), single-token decode, decode against a paged cache.
* ``fp8``        — the FP8 forward emulated step by step (rotation, block
  quantization to e4m3, tiled online softmax with P quantized per block).
* ``algorithms`` — the pages' algorithms written out step by step in float64
  (tiled online softmax, two-pass softmax, split-and-merge decoding, a scalar
  brute force). They exist to pin the definitions above and the pages' claims
  about them; they are not compared with the GPU.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
scalar brute force, closed forms (identical keys, zero queries, constant
values), invariants the pages state (rows of P sum to one, shift invariance,
online = batch softmax, chunk merge = unsplit), finite differences for the
backward, and the figures the pages print (``tests/golden``). No function is
"parity unpinned".
"""
from .attention import (  # noqa: F401
    kv_head, band_keep, attention_head, attn_fwd, attn_fwd_window, attn_fwd_varlen, attn_bwd_head, attn_bwd,
    attn_decode, attn_decode_slice, attn_decode_paged,
)
from .fp8 import (  # noqa: F401
    round_e4m3, hadamard, rotation, fwht_f32, rotate_unnormalised, scale_exponent, block_exponents, quantize_rows, fp8_online_attention, fp8_operands, fp8_p_operand,
    fp8_attention_head,
    attn_fwd_fp8,
)
from .algorithms import (  # noqa: F401
    tiled_online_attention_head, softmax_two_pass, softmax_online,
    decode_chunk_partials, merge_partials, brute_force_attention,
)
