"""CPU oracle (test infrastructure only; never imported by the library)."""
from .saga_oracle import (DecodeResult, attention_logits, dense_gqa, key_head_of,  # noqa: F401
                          nth_largest, refresh_threshold, saga_decode_step,
                          sparse_softmax_pv, threshold_select, value_head_of)
