"""CPU oracles for tree-masked MLA verify attention over a paged latent KV pool
(mla_oracle) and for the steps next to it (spec_ops_oracle: sparse top-k
decode, tree accept, KV append and commit, sliding-window gather, fp8 indexer
logits).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package. The
product path (the HIP library and its Python binding) never touches it, and it
shares no code with that path.
"""

from .mla_oracle import (  # noqa: F401
    ancestor_mask,
    ancestor_sets,
    bf16_bits_to_f64,
    brute_force_verify,
    oracle_case,
    oracle_split_combine,
    oracle_verify,
    request_slots,
    visible_positions,
)
