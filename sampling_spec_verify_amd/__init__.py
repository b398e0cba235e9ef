"""libspecverify: the speculative-decoding verify step on MI355X (gfx950).

The compute path is the HIP library ``libspecverify.so`` (C ABI declared in
``include/specverify.h``); ``specverify`` is its ctypes binding.
"""
from .specverify import (AcceptanceRateCall, ChainCall, ChainOut, KernelTimer,  # noqa: F401
                         SpecVerifyError, TreeGreedyCall, TreeGreedyOut, TreeMaskCall,
                         TreeMaskOut, TreeMultiOut, TreePathCall, chain_acceptance_rate, chain_verify,
                         chain_workspace_bytes, decode_flags, lib, status_string,
                         tree_attention_mask, tree_verify_greedy, tree_verify_multi,
                         tree_verify_path, tree_workspace_bytes)
