"""SCAPE per-worker optimizer step on AMD Instinct MI355X (gfx950).

The data-parallel hot path of SCAPE ("SCAPE: Accurate and Efficient LLM
Training with Extreme Sparse Communication") as hand-written HIP kernels
behind a C ABI (include/scape.h, libscape.so); this package is the Python
binding with the same entry-point names.
"""
from ._scape import (  # noqa: F401
    LIB_PATH, PHASES, Context, Layout, Mask, ScapeConfig, ScapeError, alloc_mask, lib, scape_dense_step, scape_destroy,
    scape_init,
    scape_last_error, scape_layout, scape_mask_build, scape_mask_index, scape_mask_union_add, scape_owner_map, scape_pack,
    scape_copy_probe, scape_stream_probe, scape_profile_enable, scape_profile_read, scape_reduce_sparse, scape_step, scape_step_offload, scape_unpack,
    scape_step_interleaved, scape_dense_step_interleaved, interleaved_view, scape_workspace_bytes,
    scape_mask_index_static, scape_selection_flags, SELECT_EXACT_HISTOGRAM, SELECT_KEY_PASSES,
    scape_set_select_path, SELECT_PATH_AUTO, SELECT_PATH_SAMPLED, SELECT_PATH_COMPACT, scape_set_update_in_dense_pass,
    scape_set_offload_path, OFFLOAD_PATH_AUTO, OFFLOAD_PATH_STAGED,
    scape_version)


def build(verbose: bool = False) -> str:
    from .build import build as _build
    return _build(verbose)
