"""MI355X-native routed-experts MoE decode step (MXFP8 activations x FP4 weights).

The compute lives in ``libmoe_mx.so`` (HIP, gfx950) behind the C ABI of
``include/moe_mx.h``; ``_lib`` binds it with ctypes under the same names, and
``layer`` holds a small convenience wrapper that owns the device buffers of one layer.
"""
from ._lib import (EXPORTED, MoeError, moe_combine, moe_decode_run, moe_decode_run_noalloc, moe_experts_run, moe_group, moe_pack_weights,  # noqa: F401
                   moe_packed_weight_bytes, moe_plan, moe_plan_bytes, moe_plan_group, moe_run_opts_t, moe_units_bytes, moe_units_export,
                   moe_weights_t, moe_work_split, moe_grouped_runs, moe_workspace_bytes, moe_workspace_init, status_string)
