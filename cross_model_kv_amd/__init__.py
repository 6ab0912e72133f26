"""MI355X-native cross-model KV handoff: factorized linear mapper, rank-disagreement
selection and contextual recompute-attention as hand-written HIP kernels for gfx950
behind a C-ABI library (``libkvx.so``); ``kvx`` is its thin Python binding."""
