"""Oracle for exact attention: plain, slow, float64 CPU code.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package; only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

Sources (the three web pages the method is taken from):
  * "What is FlashAttention?" (interview.clozo.ai), sections "Step 2: How
    online softmax keeps tiled attention exact", "Step 3", "Step 4" and
    "Worked example".
  * "FlashAttention" (deepconcepts.dev), sections "Why it is allowed to be
    exact" and "What it does not do".
  * "Explain FlashAttention and why it is IO-aware" (aiinfrainterviews.com),
    sections "Keep only the state needed for the final weighted average" and
    "Executable recurrence, with an empty-state policy".
"""

from .attention import (
    visible_mask,
    scaled_scores,
    attention_materialised,
    attention_rows,
    online_row,
    attention_online,
    attention_backward,
    finite_difference_grads,
    merge_states,
    attention_decode,
    attention_packed,
    attention_backward_packed,
)

__all__ = [
    "visible_mask",
    "scaled_scores",
    "attention_materialised",
    "attention_rows",
    "online_row",
    "attention_online",
    "attention_backward",
    "finite_difference_grads",
    "merge_states",
    "attention_decode",
    "attention_packed",
    "attention_backward_packed",
]
