"""MI355X (gfx950) implementation of the HypeNet RNN mixer, Lightning Attention.

The mixer itself is the C-ABI library ``liblightning.so`` (HIP kernels, built by
``long_context_hybrid_amd.build``); ``long_context_hybrid_amd.lightning`` is its Python binding.
"""
