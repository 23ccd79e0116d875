"""MI355X (gfx950) Gated DeltaNet chunkwise forward and backward passes.

Thin Python binding of libgdn.so (C ABI in include/gdn.h).  It only marshals
arguments: every step of both passes runs in the library's HIP kernels.
PyTorch is used for device memory and streams.  Importing the package does not
load the library; the first call does, and raises if it was not built
(``python -m gated_deltanet_chunkwise_amd.build``).
"""
from ._binding import (  # noqa: F401
    BWD_NUM_STAGES,
    BWD_STAGES,
    GDN_BF16,
    GDN_F16,
    GDN_F32,
    GDN_SCRATCH_BYTES,
    GDN_SEG_AUTO,
    GdnBackward,
    GdnError,
    GdnForward,
    NUM_STAGES,
    Params,
    STAGES,
    STAGE_ALL,
    STAGE_BITS,
    WorkspaceLayout,
    bwd,
    check,
    decode,
    decode_launcher,
    fuses_output,
    fwd,
    fwd_noalloc,
    gated_delta_rule,
    kda_gate,
    kda_gate_launcher,
    lib_path,
    load_library,
    make_params,
    seg_chunks,
    status_string,
    workspace_layout,
    workspace_size,
)

__all__ = [
    "BWD_NUM_STAGES", "BWD_STAGES", "GdnBackward", "bwd",
    "GDN_BF16", "GDN_F16", "GDN_F32", "GDN_SCRATCH_BYTES", "GDN_SEG_AUTO", "GdnError", "GdnForward", "NUM_STAGES", "Params", "STAGES", "STAGE_ALL", "STAGE_BITS", "WorkspaceLayout",
    "check", "decode", "decode_launcher", "fuses_output", "fwd", "fwd_noalloc", "gated_delta_rule", "kda_gate", "kda_gate_launcher", "lib_path", "load_library", "make_params", "seg_chunks", "status_string",
    "workspace_layout", "workspace_size",
]
