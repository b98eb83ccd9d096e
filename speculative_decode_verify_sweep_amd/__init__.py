"""Small-window paged attention for speculative-decoding verify and draft blocks
on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libsmallw.so (include/smallw.h) with
hand-written HIP kernels; this package only marshals arguments to it.
"""
from .binding import (SMALLW_EDEVICE, SMALLW_EINVAL, SMALLW_ENOMEM, SMALLW_EUNSUPPORTED,
                      SMALLW_EWORKSPACE, SMALLW_KV_BF16, SMALLW_KV_FP8_E4M3, SMALLW_KV_MXFP4, SMALLW_OK,
                      Plan,
                      SmallwError, make_problem, small_w_attention_plan,
                      small_w_attention_check_pages,
                      small_w_attention_plan_export, small_w_attention_plan_max_unit_pages,
                      small_w_attention_run, small_w_attention_run_noalloc,
                      small_w_attention_strerror,
                      small_w_attention_trace_pages, small_w_attention_workspace_bytes,
                      small_w_kv_append, small_w_stream_read, smallw_problem)

__all__ = ["SMALLW_EDEVICE", "SMALLW_EINVAL", "SMALLW_ENOMEM", "SMALLW_EUNSUPPORTED",
           "SMALLW_EWORKSPACE", "SMALLW_KV_BF16", "SMALLW_KV_FP8_E4M3", "SMALLW_KV_MXFP4", "SMALLW_OK", "Plan",
           "SmallwError", "make_problem", "small_w_attention_check_pages", "small_w_attention_plan",
           "small_w_attention_plan_export", "small_w_attention_plan_max_unit_pages",
           "small_w_attention_run", "small_w_attention_run_noalloc", "small_w_attention_strerror", "small_w_attention_trace_pages",
           "small_w_attention_workspace_bytes", "small_w_kv_append", "small_w_stream_read",
           "smallw_problem"]
