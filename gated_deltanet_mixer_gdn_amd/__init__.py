"""MI355X (gfx950) Gated DeltaNet decode mixer: a C-ABI HIP library and its binding.

The binding loads ``libgdn_hip.so`` lazily (on the first call), so importing the
package does not need a GPU. There is no CPU or PyTorch fallback.
"""
from .gdn import (  # noqa: F401
    EXPORTS, GDN_ERR_ARG, GDN_ERR_HIP, GDN_ERR_UNSUPPORTED, GDN_FLAG_BAD_NTOK, GDN_FLAG_BAD_SLOT,
    GDN_OK, GdnError, Geom, LIB_PATH, StatePool, gdn_conv_silu_norm,
    gdn_decode_fused, gdn_decode_step, gdn_decode_step_norm, gdn_gated_rmsnorm, gdn_mixer, gdn_state_pool_bytes, gdn_state_pool_zero,
    gdn_ab_project, gdn_check_slots, set_slot_checks, gdn_commit, gdn_commit_window, gdn_verify_window, load_library, gdn_split_bf16, gdn_pack_bf16, gdn_project_bf16,
    gdn_project_bf16_noalloc,
    gdn_project2_bf16, gdn_project, gdn_project_workspace_bytes, gdn_project_multi_bf16, SplitX, PackedW, gdn_geom,
)
