"""fp64 CPU oracle for SANA's ReLU linear self-attention with QK-RMSNorm.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark may import or call this
package.  The product path (the HIP library and its Python binding) never
does, and shares no code with it.

The oracle is a plain, slow, obviously correct restatement of what the pages
define; every function names the passage it follows.  It is pinned by the
tests in ``tests/test_oracle_pins.py`` (hand-worked examples under
``tests/golden/``, exact rational and 40-digit brute force of the quadratic
form, closed forms and invariants) and, for the follow-on functions, in
``tests/test_oracle_w8a8.py``, ``tests/test_oracle_mix_ffn.py`` and
``tests/test_oracle_cross_attn.py``.
"""
from .linear_attn import (  # noqa: F401
    attend,
    feature_map,
    kv_state,
    linear_attn,
    qkv_linear_attn,
    qkv_project,
    rms_inverse,
    split_heads,
)
from .cross_attn import cross_attn, rms_normalize  # noqa: F401
from .mix_ffn import depthwise_conv3x3, expand, glu, mix_ffn  # noqa: F401
from .w8a8 import qkv_w8a8_linear_attn, quantize_rows, quantize_weight, w8a8_project  # noqa: F401
