"""Plain, slow CPU oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this package: only the test suite, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library.
"""
from .sdpa_oracle import (  # noqa: F401
    to_bhsd, from_bhsd, kv_head_of, relpos_terms, relpos_bias, mask_bias,
    softmax_rows, sdpa, sdpa_rows,
)
from .sdpa_train_oracle import (  # noqa: F401
    philox4x32_10, dropout_threshold, dropout_keep, pack_keep_words, unpack_keep_words,
    sdpa_train_fwd, attention_weights, sdpa_bwd,
)
