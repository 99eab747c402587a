"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package draws random numbers and lays out a block pool the way a host
block allocator would.  It holds none of the attention arithmetic: no softmax,
no dot products, no scatter kernel and no reading through block tables.
"""

from .generate import (  # noqa: F401
    NAN_BITS,
    DecodeCase,
    PrefillCase,
    normal_bits,
    make_decode_case,
    make_prefill_case,
    decode_tiny,
    decode_llama2_7b_layer,
    decode_gqa_shared_prefix,
    prefill_chunked,
    decode_long_context,
    CONFIG_BUILDERS,
)
