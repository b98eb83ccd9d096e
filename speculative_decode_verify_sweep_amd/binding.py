"""ctypes binding over libsmallw.so (include/smallw.h): argument marshalling only.

Every step of the attention runs in the HIP kernels of the library.  PyTorch
tensors are used only as device memory and for the current HIP stream.  There
is no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmallw.so")

SMALLW_OK = 0
SMALLW_EINVAL = -1
SMALLW_EUNSUPPORTED = -2
SMALLW_EWORKSPACE = -3
SMALLW_EDEVICE = -4
SMALLW_ENOMEM = -5
SMALLW_KV_BF16 = 0
SMALLW_KV_FP8_E4M3 = 1
SMALLW_KV_MXFP4 = 2


class SmallwError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {small_w_attention_strerror(code)} ({code})")


class smallw_problem(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("num_cus", ctypes.c_int32),
                ("force_splits", ctypes.c_int32),
                ("split_pages", ctypes.c_int32),
                ("window_left", ctypes.c_int32)]


_lib = None


def lib():
    """Load libsmallw.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with "
                          "`python -m speculative_decode_verify_sweep_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_size_t
        L.small_w_attention_plan.argtypes = [ctypes.POINTER(smallw_problem), i32p,
                                             ctypes.POINTER(vp)]
        L.small_w_attention_plan.restype = ctypes.c_int
        L.small_w_attention_workspace_bytes.argtypes = [vp]
        L.small_w_attention_workspace_bytes.restype = sz
        L.small_w_attention_plan_max_unit_pages.argtypes = [vp]
        L.small_w_attention_plan_max_unit_pages.restype = sz
        run_args = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.small_w_attention_run.argtypes = run_args
        L.small_w_attention_run.restype = ctypes.c_int
        L.small_w_attention_run_events.argtypes = run_args + [vp, vp, vp]
        L.small_w_attention_run_events.restype = ctypes.c_int
        L.small_w_attention_plan_export.argtypes = [vp, i32p, sz, ctypes.POINTER(sz)]
        L.small_w_attention_plan_export.restype = ctypes.c_int
        L.small_w_attention_trace_pages.argtypes = [vp, vp, vp, vp, sz, vp]
        L.small_w_kv_append.argtypes = [vp] * 10
        L.small_w_attention_trace_pages.restype = ctypes.c_int
        L.small_w_attention_plan_destroy.argtypes = [vp]
        L.small_w_attention_plan_destroy.restype = None
        L.small_w_attention_strerror.argtypes = [ctypes.c_int]
        L.small_w_attention_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


class Plan:
    """Owns a smallw_plan* and destroys it when collected."""

    def __init__(self, handle: int, problem: smallw_problem):
        self.handle = ctypes.c_void_p(handle)
        self.problem = problem

    def __del__(self):
        if getattr(self, "handle", None) and self.handle.value and _lib is not None:
            _lib.small_w_attention_plan_destroy(self.handle)
            self.handle = None


def make_problem(*, num_reqs, window, num_q_heads, num_kv_heads, head_dim, num_pages,
                 max_pages_per_req, causal, kv_dtype=SMALLW_KV_BF16, scale=0.0, num_cus=0,
                 force_splits=0, split_pages=0, window_left=0, page_size=16) -> smallw_problem:
    return smallw_problem(num_reqs, window, num_q_heads, num_kv_heads, head_dim, page_size,
                          num_pages, max_pages_per_req, int(causal), int(kv_dtype),
                          float(scale), num_cus, force_splits, split_pages, window_left)


def small_w_attention_plan(problem: smallw_problem, seq_lens_host) -> Plan:
    seq = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    h = ctypes.c_void_p()
    rc = lib().small_w_attention_plan(ctypes.byref(problem),
                                      seq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      ctypes.byref(h))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_plan")
    return Plan(h.value, problem)


def small_w_attention_workspace_bytes(plan: Plan) -> int:
    return int(lib().small_w_attention_workspace_bytes(plan.handle))


def small_w_attention_plan_max_unit_pages(plan: Plan) -> int:
    return int(lib().small_w_attention_plan_max_unit_pages(plan.handle))


def small_w_attention_plan_export(plan: Plan) -> np.ndarray:
    need = ctypes.c_size_t()
    lib().small_w_attention_plan_export(plan.handle, None, 0, ctypes.byref(need))
    buf = np.zeros(need.value, dtype=np.int32)
    rc = lib().small_w_attention_plan_export(
        plan.handle, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), buf.size,
        ctypes.byref(need))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_plan_export")
    return buf


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def small_w_attention_run(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table,
                          seq_lens, out, lse, workspace=None, stream=None, events=None) -> None:
    """Enqueue one attention call.  Tensors are device tensors in the documented
    layouts; `workspace` is a uint8 device tensor of at least
    small_w_attention_workspace_bytes(plan) bytes (or None when that is 0).
    `events`: optional 3 raw hipEvent_t handles (ints) recorded around the kernels."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
            _stream(stream)]
    if events is None:
        rc = lib().small_w_attention_run(*args)
    else:
        rc = lib().small_w_attention_run_events(*args, *events)
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_run")


def small_w_attention_trace_pages(plan: Plan, block_table, seq_lens, pages_out,
                                  stream=None) -> None:
    maxp = pages_out.shape[-1]
    rc = lib().small_w_attention_trace_pages(plan.handle, _ptr(block_table), _ptr(seq_lens),
                                             _ptr(pages_out), maxp, _stream(stream))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_trace_pages")


def small_w_kv_append(plan: Plan, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                      block_table, seq_lens, stream=None) -> None:
    """Write the plan's W window tokens (bf16 [P][W][Hkv][D] device tensors) into
    their pool slots, quantising to e4m3 with per-(token, KV-head) scales for an
    fp8 or MXFP4 pool.  Tensors are device tensors in the documented layouts."""
    rc = lib().small_w_kv_append(plan.handle, _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                 _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                 _ptr(seq_lens), _stream(stream))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_kv_append")


def small_w_attention_strerror(code: int) -> str:
    return lib().small_w_attention_strerror(int(code)).decode()


# raw HIP events for in-place kernel timing (plumbing around the library calls)
_hip = None


def _hip_rt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return _hip


def hip_event_create() -> int:
    ev = ctypes.c_void_p()
    rc = _hip_rt().hipEventCreate(ctypes.byref(ev))
    if rc != 0:
        raise RuntimeError(f"hipEventCreate failed ({rc})")
    return ev.value


def hip_event_elapsed_ms(a: int, b: int) -> float:
    ms = ctypes.c_float()
    _hip_rt().hipEventSynchronize(ctypes.c_void_p(b))
    rc = _hip_rt().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return float(ms.value)


def hip_event_record(ev: int, stream) -> None:
    rc = _hip_rt().hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(_stream(stream)))
    if rc != 0:
        raise RuntimeError(f"hipEventRecord failed ({rc})")


def hip_event_destroy(ev: int) -> None:
    _hip_rt().hipEventDestroy(ctypes.c_void_p(ev))
