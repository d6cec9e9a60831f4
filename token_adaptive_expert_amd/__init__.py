"""MI355X (gfx950) forward of a routed SwiGLU MoE layer with ACE per-token
expert-slot skipping.  The arithmetic lives in the HIP library built from
``csrc/``; this package holds its ctypes binding and a buffer-owning layer
wrapper (torch supplies device memory and streams)."""
from ._lib import (ACE_BF16, ACE_F32, ACE_PATH_AUTO, ACE_PATH_GROUPED, ACE_PATH_STREAM, ACE_STAGE_DOWN,
                   ACE_STAGE_GATEUP, AceMoeError, MoeDesc,
                   ACE_LAYOUT_LINEAR, ACE_LAYOUT_PACKED, load, make_desc, moe_abi_version, moe_calibrate_thresholds, moe_calibrate_workspace_bytes, moe_combine,
                   moe_dispatch, moe_expert_forward, moe_pack_router, moe_pack_weights, moe_router_packed_bytes,
                   moe_last_error, moe_route_skip, moe_set_kernel_events, moe_workspace_bytes,
                   moe_build_tables, moe_tables_workspace_bytes, moe_forward, moe_forward_static,
                   ACE_STATIC_SCRATCH_BYTES, moe_hbm_read_probe, moe_l2_load_probe)
from .layer import AceMoeLayer, LayerBuffers, build_tables
from .stack import AceMoeStack

__all__ = ["ACE_BF16", "ACE_F32", "ACE_PATH_AUTO", "ACE_PATH_GROUPED", "ACE_PATH_STREAM", "ACE_STAGE_DOWN",
           "ACE_STAGE_GATEUP", "AceMoeError", "MoeDesc",
           "ACE_LAYOUT_LINEAR", "ACE_LAYOUT_PACKED", "load", "make_desc", "moe_pack_router", "moe_pack_weights", "moe_router_packed_bytes", "moe_abi_version", "moe_calibrate_thresholds", "moe_calibrate_workspace_bytes", "moe_combine", "moe_dispatch", "moe_expert_forward",
           "moe_last_error", "moe_route_skip", "moe_set_kernel_events", "moe_workspace_bytes", "AceMoeLayer",
           "LayerBuffers", "moe_build_tables", "moe_tables_workspace_bytes", "build_tables", "AceMoeStack", "moe_forward",
           "moe_forward_static", "ACE_STATIC_SCRATCH_BYTES", "moe_hbm_read_probe", "moe_l2_load_probe"]
