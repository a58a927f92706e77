"""hash_scored_top_amd: hash-scored top-k sparse decode attention on MI355X.

The compute path is libhst.so (hand-written HIP for gfx950, C ABI in
include/hst.h); this package only marshals torch tensors into it.
"""
from ._lib import (  # noqa: F401
    DecodeHamming, DecodeSoftLSH, DecodeSoftLSHMass, DecodeSoftLSHRouted, DecodeSoftLSHShared,
    EXPORTED, HST_BF16, HST_F16, HST_F32, HST_I32, HstError, HstShape, LIB_PATH,
    debug_status, hst_append_kv_binary, hst_append_kv_softlsh, hst_build_cards_softlsh, hst_decode_step_hamming,
    hst_decode_step_softlsh, hst_decode_step_softlsh_noalloc, hst_hash_keys_binary,
    hst_hash_keys_softlsh, hst_query_tables_softlsh,
    hst_score_keys_hamming, hst_score_keys_softlsh, hst_score_scan_softlsh, hst_select_mass,
    hst_select_topk, hst_sparse_decode_attention, make_shape, workspace_size,
)
