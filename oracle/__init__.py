"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP path and never imports it.
"""

from .attention import attention_ref, online_ref, brute_ref, softmax_weights_ref, visible_keys  # noqa: F401
from .attention_bwd import attention_bwd_ref, row_dot_ref  # noqa: F401
from .attention_varlen import attention_varlen_ref, brute_varlen_ref, causal_offset  # noqa: F401
from .attention_dropout import (attention_dropout_ref, attention_dropout_bwd_ref, dropout_threshold,  # noqa: F401
                                keep_mask, keep_mask_loop, _philox_np)
from .philox import philox4x32  # noqa: F401
from .attention_fp8 import attention_fp8_ref, dequantize, e4m3_decode  # noqa: F401
from . import accounting  # noqa: F401
