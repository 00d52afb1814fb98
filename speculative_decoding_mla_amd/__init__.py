"""MI355X (gfx950) verify attention for tree speculative decoding over a paged
MLA latent KV cache: a C-ABI library (include/mla_verify.h) and its thin
Python binding."""

from .binding import (  # noqa: F401
    DEVERR_BAD_PARENT,
    DEVERR_SEQ_LEN,
    DEVERR_SLOT_RANGE,
    MlaError,
    MlaVerifyDesc,
    VerifyPlan,
    alloc_workspace,
    build_tree_mask,
    desc_for,
    device_error,
    library_path,
    load_library,
    make_desc,
    verify_attention,
    verify_combine,
    verify_partial,
    workspace_bytes,
)
