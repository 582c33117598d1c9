"""CPU float64 oracle for exact scaled-dot-product attention (TEST INFRASTRUCTURE).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python
binding) never calls it, shares no code with it, and fails loudly when its
native library is missing instead of falling back to anything here.

Contents:
  attention.py  plain definition: explicit S, mask, row softmax, P.V, LSE, and
                the analytic backward (NumPy, float64); attn_fwd_kv is the same
                forward for Nq queries against Nk >= Nq keys.
  brute.py      pure-Python triple loops with math.exp / math.fsum for tiny
                shapes (an independent second statement of the forward).
  online.py     the blocked online-softmax recurrence, step by step, used only
                to show that the recurrence the fused kernel runs is exact.
  masked.py     the same definition under a general boolean visibility mask, with builders
                for padded variable-length batches, per-sequence key/value cache lengths and
                block-sparse maps (empty rows: O = 0, LSE = -inf).
  dropout.py    the Philox4x32-10 keep mask of attention dropout (from the generator's published
                definition) and attention forward / backward with a given keep mask.

Every function cites the passage of the pages it follows. Parity pins (closed
forms, invariants, brute force, library special cases, finite differences)
live in tests/test_oracle.py, tests/test_oracle_masked.py and tests/test_oracle_dropout.py.
"""
from .attention import attn_bwd, attn_bwd_keys, attn_bwd_rows, attn_fwd, attn_fwd_kv, attn_fwd_rows, softmax_rows
from .brute import brute_fwd
from .dropout import attn_bwd_dropout, attn_fwd_dropout, keep_mask, keep_threshold, philox4x32_10, random_bytes
from .masked import attn_bwd_masked, attn_fwd_masked, kv_cache_visible, padded_batch_visible
from .online import online_fwd

__all__ = ["attn_fwd", "attn_fwd_kv", "attn_fwd_rows", "attn_bwd", "attn_bwd_rows", "attn_bwd_keys", "softmax_rows",
           "brute_fwd", "online_fwd",
           "attn_fwd_masked", "attn_bwd_masked", "padded_batch_visible", "kv_cache_visible",
           "attn_fwd_dropout", "attn_bwd_dropout", "keep_mask", "keep_threshold", "philox4x32_10", "random_bytes"]
