"""MoLE (Mixture-of-Lookup-Experts) inference hot path for AMD MI355X.

Thin Python binding over the C ABI of ``libmole.so`` (declared in
``include/mole.h``).  Every computation runs in the library's HIP kernels;
this module only turns torch tensors into pointers and sizes and raises
:class:`MoleError` on a non-zero status.  torch supplies device memory and
streams.

The native library is loaded on first use; if it has not been built the
first call raises ``MoleLibraryMissing`` (build it with
``python -m mixture_lookup_experts_amd.build``).
"""
from __future__ import annotations

from ._native import (  # noqa: F401
    MOLE_BF16,
    MOLE_F32,
    MoleError,
    MoleLibraryMissing,
    library,
    library_path,
    mole_build_lut,
    mole_build_lut_workspace_size,
    mole_gather_nf3_host,
    mole_layer_forward,
    mole_lookup_combine_int8,
    mole_lookup_combine_nf4,
    mole_nf4_levels,
    mole_pack_int8,
    mole_pack_nf4,
    mole_layer_workspace_size,
    mole_lookup_combine,
    mole_lookup_combine_nf3,
    mole_lookup_combine_nf3_host,
    mole_lookup_combine_nf3_mapped,
    mole_lookup_combine_mapped,
    mole_lookup_combine_grouped_mapped,
    mole_lookup_combine_nf3_grouped,
    mole_lookup_combine_nf3_grouped_mapped,
    mole_nf3_host_staging_size,
    mole_nf3_host_stack_staging_size,
    mole_prefetch_nf3_host_stack,
    mole_gather_nf3_file,
    mole_lookup_combine_grouped_workspace_size,
    mole_check_ids,
    mole_lookup_combine_grouped,
    mole_lookup_combine_nf3_file,
    mole_nf3_file_shape,
    mole_nf3_file_write,
    mole_nf3_levels,
    mole_pack_nf3,
    mole_status_string,
    mole_train_backward,
    mole_train_forward,
    mole_train_index,
    mole_train_workspace_size,
)

__all__ = [
    "MOLE_F32", "MOLE_BF16", "MoleError", "MoleLibraryMissing", "library", "library_path",
    "mole_build_lut", "mole_build_lut_workspace_size", "mole_lookup_combine", "mole_pack_nf3",
    "mole_lookup_combine_nf3", "mole_gather_nf3_host", "mole_lookup_combine_nf3_host",
    "mole_lookup_combine_nf3_mapped", "mole_lookup_combine_mapped", "mole_lookup_combine_grouped_mapped",
    "mole_lookup_combine_nf3_grouped", "mole_lookup_combine_nf3_grouped_mapped",
    "mole_nf3_host_staging_size", "mole_nf3_host_stack_staging_size", "mole_prefetch_nf3_host_stack",
    "mole_nf3_levels", "mole_status_string", "mole_layer_forward", "mole_layer_workspace_size",
    "mole_nf4_levels", "mole_pack_nf4", "mole_lookup_combine_nf4", "mole_pack_int8", "mole_lookup_combine_int8",
    "mole_train_index", "mole_train_workspace_size", "mole_train_forward", "mole_train_backward",
    "mole_nf3_file_write", "mole_nf3_file_shape", "mole_gather_nf3_file", "mole_lookup_combine_nf3_file",
    "mole_lookup_combine_grouped", "mole_lookup_combine_grouped_workspace_size", "mole_check_ids",
]
