"""fp64 CPU oracle of the verify step (test infrastructure only; see verify.py)."""
from .verify import (FLAG_BAND, MIX_SPACES, BatchResult, ChainResult, GreedyResult, InvalidRow,  # noqa: F401
                     accept_prob, as_f32_scalar, chain_verify, chain_verify_one, enhanced_logits,
                     inverse_cdf,
                     mixture, pack_mask_rows, path_rows, residual_weights, softmax_T,
                     tree_attention_mask, tree_attention_mask_one, tree_greedy,
                     tree_greedy_one, tree_multi, tree_multi_one, tree_path, tree_path_one)
