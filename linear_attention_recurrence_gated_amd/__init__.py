"""MI355X-native gated delta-rule recurrence (Gated DeltaNet mixer core).

The compute lives in libgdn.so (hand-written HIP for gfx950, C ABI in
include/gdn.h); ``gdn`` is its thin Python binding.
"""
from .gdn import (GdnError, decode_step, decode_step_slots, prefill, prefill_algorithm,  # noqa: F401
                  prefill_set_marks, prefill_workspace_bytes, preprocess, state_bytes, state_init, state_reset)
