"""MI355X-native batched draft-token verification (speculative sampling).

The compute path is the C-ABI library libspecverify.so (hand-written HIP for
gfx950, declared in include/spec_verify.h).  This package is its thin Python
binding (`binding`, re-exported here) plus the seeded input generators
(`synth`).  Importing the package does not load the library; the first call
does, and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    SV_BF16, SV_F32, SV_MAX_GAMMA, SV_MAX_TREE_NODES, SV_MAX_VOCAB,
    SV_SEQ_BAD_PARENT, SV_SEQ_D2T, SV_SEQ_NO_MASS, SV_SEQ_TOKEN_RANGE, SpecVerifyError, lib,
    spec_draft_sample, spec_fanout_lookup, spec_lmhead_verify_greedy, spec_lmhead_verify_tree, spec_verify_count,
    spec_vocab_trim, sv_workspace_bytes_draft, sv_workspace_bytes_lmhead,
    sv_workspace_bytes_vocab_trim,
    spec_verify_greedy, spec_verify_sample, spec_verify_sample_noalloc, spec_verify_tree_greedy,
    sv_workspace_bytes_greedy, sv_workspace_bytes_sample, sv_workspace_bytes_tree,
)
