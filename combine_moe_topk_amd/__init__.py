"""MI355X-native MoE token dispatch and combine (one GPU's share).

The compute path is the HIP library ``libmoe_topk.so`` (C ABI in
``include/moe_topk.h``); this package is its thin ctypes binding.  Names
match the C entry points: :func:`moe_topk_gate`, :func:`moe_dispatch_layout`,
:func:`moe_dispatch_pack`, :func:`moe_combine`, :func:`moe_dispatch_combine`,
and the node-level two-leg path :func:`moe_dispatch_pack_nodes`,
:func:`moe_dispatch_forward`, :func:`moe_combine_partial`,
:func:`moe_combine_nodes`, :func:`moe_dispatch_combine_nodes`, and the FP8
dispatch :func:`moe_dispatch_pack_fp8`, :func:`moe_combine_fp8`,
:func:`moe_dispatch_combine_fp8`, and the capacity-padded / bucketed layout
:func:`moe_dispatch_layout_capacity`, :func:`moe_dispatch_pack_capacity`,
:func:`moe_combine_capacity`, :func:`moe_dispatch_combine_capacity`, and the
communication-aware task assignment :func:`moe_assign_tasks`, and
:func:`moe_dispatch_combine_noalloc`, the fused call with its workspace in
the library's static device scratch, for callers that cannot allocate.
"""
from ._lib import (  # noqa: F401
    LAYOUT_FIELDS, Layout, MoeError, MOE_BF16, MOE_DEVERR_DUP_EXPERT,
    MOE_DEVERR_EXPERT_RANGE, MOE_EINVAL, MOE_ELAUNCH, MOE_EUNSUPPORTED,
    MOE_EWORKSPACE, MOE_F32, MOE_F_NO_RENORM, MOE_OK, alloc_layout,
    alloc_workspace, lib, make_cfg, moe_cfg, moe_combine,
    moe_dispatch_combine, moe_dispatch_combine_noalloc, MOE_ESCRATCH,
    MOE_SCRATCH_BYTES, moe_dispatch_layout, moe_dispatch_pack,
    moe_layout, moe_read_device_error, moe_strerror, moe_topk_gate,
    moe_validate_cfg, moe_version, moe_workspace_bytes, moe_workspace_init,
    moe_node_rows_max, moe_dispatch_pack_nodes, moe_dispatch_forward,
    moe_combine_partial, moe_combine_nodes, moe_dispatch_combine_nodes,
    moe_fp8_row_bytes, moe_dispatch_pack_fp8, moe_combine_fp8,
    moe_dispatch_combine_fp8,
    MOE_MAX_LEVELS, CapacityLayout, moe_capacity_layout,
    alloc_capacity_layout, alloc_capacity_workspace,
    moe_dispatch_layout_capacity, moe_dispatch_pack_capacity,
    moe_combine_capacity, moe_dispatch_combine_capacity,
    MOE_DEVERR_NO_REPLICA, MOE_DEVERR_SRC_RANK, alloc_assign_workspace,
    moe_assign_tasks,
)
