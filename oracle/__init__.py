"""CPU oracle for the DDTree tree-verify step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy/Python implementations of the four
steps of the verify path and of the draft top-K that feeds it.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path (the
HIP library and its Python binding) never does, and shares no code with it.

Sources (blog pages on DDTree speculative decoding):
  * topk    -- "The Architecture of Speculative Decoding: Dissecting DDTree's
               Tree-Parallel Evaluation Strategy", Section 1 step 1 (per-depth
               top-k log-probs of the draft head).
  * build   -- "The Architecture of Speculative Decoding: Dissecting DDTree's
               Tree-Parallel Evaluation Strategy", Section 1 (five-step flow,
               steps 2-3); "The Tree That Couldn't Branch", "Context: The Road
               to DDTree" and "Hypothesis 4".
  * attention -- same first page, Section 1 step 4 and Section 2 (context
               loaded once, shared by every tree node); "The Pivot Point",
               "The Design Constraint: Load Contexts Once".
  * vocab   -- Section 1 step 4 (per-node argmax); Section 3 (softmax over the
               verify logits at temperature T).
  * linear  -- Section 3 (linear DFlash at temperature T: accept with
               min(1, p_target / p_draft), else the residual) and "Mistakes and
               Incorrect Assumptions" (the draft's full probabilities are needed).
  * topp    -- Section 3 (top_p threaded through to the verify walk): the
               nucleus of the integer target law.
  * commit  -- Section 1 step 5 and its summary (the longest verified path is
               committed) and Section 2 (the context cache grows by the
               committed tokens and is read once by later steps).
  * verify  -- Section 1 step 5 (greedy walk, bonus token); Section 3 and
               "Implementing Temperature-Aware Tree Sampling for DDTree",
               "Path B: CPU-Side Tree Rejection Sampling" (tree rejection
               sampling with residual renormalisation).

Parity status: every function here is pinned by tests under tests/ that check
it against brute force, closed forms, library routines or a statistical test
(see the test modules' docstrings); none is "parity unpinned".
"""
from .topk import attach_draft_topk, draft_topk, log_sum_exp
from .build import build_tree, N_WORDS
from .attention import tree_attention, to_f64
from .vocab import vocab_reduce, weight_constants, weights
from .verify import verify_greedy, verify_sample
from .linear import verify_linear_sample
from .commit import commit_path
from .topp import keep_mask, nucleus_row, top_p_fixed, vocab_top_p

__all__ = ["attach_draft_topk", "draft_topk", "log_sum_exp", "build_tree", "N_WORDS", "tree_attention", "to_f64",
           "vocab_reduce", "weight_constants", "weights", "verify_greedy", "verify_sample",
           "verify_linear_sample", "commit_path", "keep_mask", "nucleus_row", "top_p_fixed",
           "vocab_top_p"]
