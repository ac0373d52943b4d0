"""CPU oracle for speculative-decoding verification: TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 definitions of what the verification library computes,
written from the pages' descriptions of the method:

* "PipeSpec: Breaking Stage Dependencies in Hierarchical LLM Decoding"
  (Pith review page) -- greedy longest-matching-prefix verification, per-stage
  buffers and rollback ("What carries the argument"), the expected-token
  formula and the steady-state verification probability ("Core claim",
  "Assumptions & free parameters").
* "Accelerating LLM Inference with Staged Speculative Decoding" (abstract) --
  the tree-shaped speculative batch and the second speculative stage.
* "CLaSp: In-Context Layer Skip for Self-Speculative Decoding" (Pith review
  page, "Assumptions & free parameters") -- speculative sampling is lossless.

The stochastic accept/residual/bonus rule (accept when u < min(1, p/q); on a
rejection resample from the renormalised max(0, p - q); after a full window
draw a bonus token from p) is the speculative-sampling rule those pages cite
by name; it is written out here as its plain definition.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or generators) and imports nothing from
it.  Every function is pinned by a ``-m "not gpu"`` test in ``tests/``
against something other than itself (numpy's Philox, scipy, brute force,
closed forms from the pages); see each module's header for its pins.
"""

from .philox import philox4x64_10, uniform24, window_uniforms, tree_uniforms
from .verify import (
    decode,
    softmax,
    first_argmax,
    inverse_cdf,
    verify_window,
    verify_greedy,
    tree_meta,
    verify_tree,
    verify_tree_multiround,
    lmhead_logits,
    verify_window_lmhead,
    rollback,
    hierarchy_three_stage,
)

__all__ = [
    "philox4x64_10",
    "uniform24",
    "window_uniforms",
    "tree_uniforms",
    "decode",
    "softmax",
    "first_argmax",
    "inverse_cdf",
    "verify_window",
    "verify_greedy",
    "tree_meta",
    "verify_tree",
    "verify_tree_multiround",
    "lmhead_logits",
    "verify_window_lmhead",
    "rollback",
    "hierarchy_three_stage",
]
