"""Chunked gated delta-rule forward (KDA / Gated DeltaNet) for MI355X (gfx950).

The forward runs in hand-written HIP kernels behind the C interface of
include/chunk_dr.h (libchunkdr.so); this package is its thin Python binding.
"""
from .ops import (chunk_dr_fwd, PreparedForward, load_library, workspace_bytes, make_problem, check,  # noqa: F401
                  STAGE_INTRA, STAGE_CHAIN, STAGE_OUTPUT, STAGE_ALL, fused_recurrent_fwd, PreparedRecurrent,
                  chunk_dr_bwd, PreparedBackward, bwd_workspace_bytes,
                  BWD_PREP, BWD_CHAINS, BWD_LOCAL, BWD_ALL, segment_map, merge_states,
                  chunk_dr_fwd_noalloc, NOALLOC_SCRATCH_BYTES, check_cu_seqlens)
