"""Target-verify path of tree-structured speculative decoding over compressed-attention
KV, for AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI (include/tv.h) and
a thin ctypes binding with the same entry-point names."""
from .tv import (TvError, DeviceState, DeviceScratch, lib, header_symbols, to_device, to_host,
                 round_cap, tv_build_tree_mask, tv_verify_attn_workspace_bytes, tv_verify_attn, tv_verify_attn_noalloc,
                 tv_accept, tv_refresh_state, tv_accept_refresh, tv_compress_prefix, tv_build_draft_tree, tv_draft_attn, tv_version,
                 TV_OK, TV_EINVAL, TV_EUNSUPPORTED, TV_EWORKSPACE, TV_EHIP, TV_SEQ_OK,
                 TV_SEQ_BAD_PARENT, TV_SEQ_POOL_FULL, TV_SEQ_BAD_PREFIX, TV_SEQ_BAD_PATH, TV_SEQ_BAD_PAGE,
                 TV_MAX_D)

__all__ = ["TvError", "DeviceState", "DeviceScratch", "lib", "header_symbols", "to_device", "to_host",
           "round_cap", "tv_build_tree_mask", "tv_verify_attn_workspace_bytes", "tv_verify_attn", "tv_verify_attn_noalloc",
           "tv_accept", "tv_refresh_state", "tv_accept_refresh", "tv_compress_prefix", "tv_build_draft_tree", "tv_draft_attn",
           "tv_version"]
