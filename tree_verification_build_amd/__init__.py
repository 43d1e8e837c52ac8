"""libddtree: the DDTree tree-verify step on AMD MI355X (gfx950).

Thin ctypes binding over the C-ABI in include/ddtree.h.  The functions carry
the C names (ddtree_draft_topk, ddtree_build,
ddtree_tree_attention[_ranges, _tuned, _noalloc],
ddtree_vocab_reduce, ddtree_verify_greedy, ddtree_vocab_verify_greedy, ddtree_verify_sample,
ddtree_verify_sample_lazy, ddtree_verify_linear_sample, ddtree_vocab_top_p,
ddtree_verify_sample_top_p, ddtree_commit); they only check and marshal
arguments -- torch tensors on the GPU in, device pointers and the current
stream out -- and every step of the path runs in the HIP kernels of
libddtree.so.  There is no fallback: if the library is missing, importing this
package raises.
"""
from ._lib import (  # noqa: F401
    DDTREE_BF16, DDTREE_F32, DdtreeError, Tree, alloc_tree, ddtree_build, ddtree_commit,
    ddtree_draft_topk,
    ddtree_draft_topk_workspace_size, ddtree_last_error,
    ddtree_sampling_constants, ddtree_tree_attention, ddtree_tree_attention_ranges,
    ddtree_tree_attention_ranges_capped,
    ddtree_tree_attention_ranges_workspace_size, ddtree_tree_attention_workspace_size,
    ddtree_tree_attention_tuned, ddtree_tree_attention_tuned_workspace_size,
    ddtree_tree_attention_noalloc,
    ddtree_verify_greedy, ddtree_verify_linear_sample, ddtree_verify_sample,
    ddtree_verify_sample_lazy, ddtree_verify_sample_top_p, ddtree_version, ddtree_vocab_top_p,
    ddtree_vocab_reduce, ddtree_vocab_verify_greedy,
    ddtree_vocab_reduce_workspace_size, library_path, lib,
)
