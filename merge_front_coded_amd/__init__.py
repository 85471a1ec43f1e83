"""MI355X (gfx950) replacement merge into a front-coded bit payload.

The hot path runs in hand-written HIP kernels behind the C ABI of
include/em.h (libem.so); ``binding`` marshals arguments to it and
``pipeline`` orders the calls.  PyTorch supplies device memory and streams.
"""
from .binding import (COLLISION_MODES, EM_COLLISION_512, EM_COLLISION_512_COMPACT, EM_COLLISION_512_TILED,
                      EM_COLLISION_2048, EM_NONE, DeviceSide, EmError, em_collision_rank, em_collision_rank_mode,
                      em_collision_workspace_bytes, em_emit, em_emit_merged, em_fc_lengths, em_merge_fc, em_merge_fc_onepass,
                      em_merge_fc_workspace_bytes, em_merge_keep, em_merge_lengths, em_onepass_workspace_bytes, em_partition,
                      em_payload_bound_bits, em_rank512_probe, em_rank512_workspace_bytes, em_rank2048_probe,
                      em_rank2048_workspace_bytes, em_scan, em_scan_noalloc, em_workspace_bytes, lib, load_library,
                      EF_INFO_FIELDS, EfSections, em_ef_capacity, em_ef_encode, em_ef_entry_count,
                      em_ef_navigation, em_ef_workspace_bytes, em_fcin_compare, em_fcin_materialize, em_fcin_parse,
                      em_fcin_prefix8,
                      em_fcin_workspace_bytes, fcin_decode, em_bp_emit, em_bp_lengths, em_bp_navigation,
                      em_bp_workspace_bytes)
from .pipeline import Pipeline

__all__ = ["COLLISION_MODES", "EM_COLLISION_512", "EM_COLLISION_512_COMPACT", "EM_COLLISION_512_TILED",
           "EM_COLLISION_2048", "EM_NONE", "DeviceSide", "EmError", "Pipeline", "em_collision_rank",
           "em_collision_rank_mode", "em_collision_workspace_bytes", "em_rank2048_probe",
           "em_rank2048_workspace_bytes", "EF_INFO_FIELDS", "EfSections", "em_ef_capacity", "em_ef_encode",
           "em_ef_entry_count", "em_ef_navigation", "em_ef_workspace_bytes", "em_fcin_compare", "em_fcin_materialize",
           "em_fcin_prefix8",
           "em_fcin_parse", "em_fcin_workspace_bytes", "fcin_decode", "em_bp_emit", "em_bp_lengths",
           "em_bp_navigation", "em_bp_workspace_bytes", "em_emit",
           "em_emit_merged", "em_fc_lengths", "em_merge_fc", "em_merge_fc_onepass", "em_merge_fc_workspace_bytes",
           "em_merge_keep", "em_merge_lengths", "em_onepass_workspace_bytes",
           "em_partition", "em_payload_bound_bits",
           "em_rank512_probe", "em_rank512_workspace_bytes", "em_scan", "em_scan_noalloc", "em_workspace_bytes", "lib",
           "load_library"]
