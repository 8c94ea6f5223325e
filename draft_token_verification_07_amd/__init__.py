"""MI355X-native batched draft-token verification (speculative sampling).

The compute path is the C-ABI library libspecverify.so (hand-written HIP for
gfx950).  This package is its thin Python binding; see `binding` for the
calls.  `synth` holds the seeded input generators.
"""
