"""MI355X-native AB-Attention sparse attention layer (HIP kernels behind a C ABI).

Importing the package does not load the HIP library; the first call into
``block_sparse_attention_38_amd.aba`` does, and raises if it is missing.
"""
from . import workloads  # noqa: F401
