"""MI355X (gfx950) 3D-windowed joint attention: window planner, layout
relayout and bf16-MFMA window attention behind a C ABI (libwsp.so).

The Python surface is a thin ctypes binding with the C entry points' names;
all device work runs in libwsp's HIP kernels.
"""
from ._lib import (BF16, CANONICAL, F32, IO_CANONICAL, IO_LAYOUT, ORDER_ID, ORDER_LPT, ORDER_LPT_XCD, REGULAR, SHIFTED,
                   SCHED_AUTO, SCHED_PER_ITEM, SCHED_PER_ITEM_128, SCHED_QUEUE, SCHED_QUEUE_128,
                   set_attn_schedule,
                   LIB_PATH, Plan, WspError, canonical, fp8_amax, fp8_quantize, lib, linear, linear_rope, plan, relayout,
                   rope_relayout, rope_text, set_attn_order, version, window_attn, window_attn_noalloc, noalloc_per_window, window_attn_qk8,
                   window_attn_rope, window_attn_rope_workspace, device_info,
                   window_attn_workspace)

__all__ = ["BF16", "CANONICAL", "F32", "IO_CANONICAL", "IO_LAYOUT", "ORDER_ID", "ORDER_LPT", "ORDER_LPT_XCD", "REGULAR",
           "SHIFTED", "LIB_PATH", "Plan", "WspError", "canonical", "lib", "plan", "relayout",
           "rope_relayout", "rope_text", "set_attn_order", "version", "window_attn", "window_attn_noalloc", "noalloc_per_window", "window_attn_workspace",
           "fp8_amax", "fp8_quantize", "window_attn_qk8", "window_attn_rope", "window_attn_rope_workspace", "device_info", "SCHED_AUTO", "SCHED_PER_ITEM", "SCHED_PER_ITEM_128", "SCHED_QUEUE", "SCHED_QUEUE_128",
           "set_attn_schedule", "linear", "linear_rope"]
