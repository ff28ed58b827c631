"""MI355X-native DeepSeek Sparse Attention (DSA) hot path.

The compute lives in ``libdsa.so`` (hand-written gfx950 HIP kernels behind a
C ABI, declared in ``include/dsa.h``).  This package only marshals arguments:
``sparse_attention_18_amd.binding`` loads the library and exposes the same
entry points over torch tensors.  Importing the package does not load the
library; the first binding call does, and fails loudly if it is missing.
"""
__all__ = ["workloads"]
