"""MI355X-native DSpark vocabulary-wide propose / dyadic24 / verify.

The compute lives in the HIP library ``libdspark.so`` (built from ``csrc/``);
``binding`` marshals torch tensors into its C ABI.  Importing the package
does not load the library; the first call does, and fails loudly if it is
missing.
"""
from .binding import (  # noqa: F401
    DTYPE_BF16, DTYPE_F32, GREEDY, SAMPLED, STATUS_NAMES, abi_version, fused, library_path,
    load_library, propose, q_alloc, q_alloc_weights, q_semantic_id, sample, status_name,
    verify_greedy, cr_expf, workspace_bytes,
)
