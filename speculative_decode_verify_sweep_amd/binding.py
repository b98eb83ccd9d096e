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
SMALLW_V_DMAJOR = 0
SMALLW_V_TOKEN_MAJOR = 1


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
                ("window_left", ctypes.c_int32),
                ("v_layout", ctypes.c_int32)]


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
        L.small_w_attention_run_noalloc.argtypes = [vp] * 11
        L.small_w_attention_run_noalloc.restype = ctypes.c_int
        L.small_w_attention_run_events.restype = ctypes.c_int
        L.small_w_attention_plan_export.argtypes = [vp, i32p, sz, ctypes.POINTER(sz)]
        L.small_w_attention_plan_export.restype = ctypes.c_int
        L.small_w_attention_trace_pages.argtypes = [vp, vp, vp, vp, sz, vp]
        L.small_w_kv_append.argtypes = [vp] * 10
        L.small_w_attention_trace_pages.restype = ctypes.c_int
        L.small_w_attention_check_pages.argtypes = [vp] * 5
        L.small_w_attention_check_pages.restype = ctypes.c_int
        L.small_w_attention_plan_destroy.argtypes = [vp]
        L.small_w_attention_plan_destroy.restype = None
        L.small_w_stream_read.argtypes = [vp, sz, vp, vp, vp, vp]
        L.small_w_stream_read.restype = ctypes.c_int
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
                 force_splits=0, split_pages=0, window_left=0, page_size=16,
                 v_layout=0) -> smallw_problem:
    return smallw_problem(num_reqs, window, num_q_heads, num_kv_heads, head_dim, page_size,
                          num_pages, max_pages_per_req, int(causal), int(kv_dtype),
                          float(scale), num_cus, force_splits, split_pages, window_left,
                          int(v_layout))


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


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(t, name, dtypes, numel=None, min_bytes=None, device=None):
    """Raise ValueError unless tensor t has one of `dtypes` (names such as
    "bfloat16"), exactly `numel` elements or at least `min_bytes` bytes, and
    sits on `device`.  Raw integer device pointers pass unchecked: the caller
    vouches for them."""
    if t is None or isinstance(t, int):
        return
    dt = str(t.dtype).replace("torch.", "")
    if dt not in dtypes:
        raise ValueError(f"{name}: dtype {dt}, expected {' or '.join(dtypes)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_bytes is not None and _nbytes(t) < min_bytes:
        raise ValueError(f"{name}: {_nbytes(t)} bytes, the plan needs at least {min_bytes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device} (the current device)")


# bf16 tensors may also arrive as 16-bit integer tensors holding the bits
BF16_BITS = ("bfloat16", "int16", "uint16")


def _page_head_bytes(pr) -> tuple[int, int, tuple]:
    """(pool bytes per page-head, scale bytes per page-head, scale dtypes)."""
    D = pr.head_dim
    if pr.kv_dtype == SMALLW_KV_FP8_E4M3:
        return 16 * D, 16 * 4, ("float32",)
    if pr.kv_dtype == SMALLW_KV_MXFP4:
        return 8 * D, 16 * (D // 32), ("uint8",)
    return 32 * D, 0, ()


def _check_pools(pr, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, dev):
    pool_b, scale_b, scale_dt = _page_head_bytes(pr)
    heads = pr.num_pages * pr.num_kv_heads
    pool_dt = BF16_BITS if pr.kv_dtype == SMALLW_KV_BF16 else \
        ("uint8", "int8", "float8_e4m3fn")
    _check(k_pool, "k_pool", pool_dt, min_bytes=heads * pool_b, device=dev)
    _check(v_pool, "v_pool", pool_dt, min_bytes=heads * pool_b, device=dev)
    if scale_b:
        if k_scale is None or v_scale is None:
            raise ValueError("k_scale and v_scale are required for this KV format")
        _check(k_scale, "k_scale", scale_dt, min_bytes=heads * scale_b, device=dev)
        _check(v_scale, "v_scale", scale_dt, min_bytes=heads * scale_b, device=dev)
    _check(block_table, "block_table", ("int32",), numel=pr.num_reqs * pr.max_pages_per_req,
           device=dev)
    _check(seq_lens, "seq_lens", ("int32",), numel=pr.num_reqs, device=dev)


def _current_device():
    import torch
    return torch.device("cuda", torch.cuda.current_device())


def small_w_attention_run(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table,
                          seq_lens, out, lse, workspace=None, stream=None, events=None) -> None:
    """Enqueue one attention call.  Tensors are device tensors in the documented
    layouts; `workspace` is a uint8 device tensor of at least
    small_w_attention_workspace_bytes(plan) bytes (or None when that is 0).
    `events`: optional 3 raw hipEvent_t handles (ints) recorded around the kernels.
    Raises ValueError when a tensor's dtype, size or device does not fit the
    plan (an int32 table read as int64 pairs, or a short pool, would otherwise
    give wrong numbers or out-of-bounds reads on the device)."""
    pr = plan.problem
    dev = _current_device()
    rows = pr.num_reqs * pr.window * pr.num_q_heads
    _check(q, "q", BF16_BITS, numel=rows * pr.head_dim, device=dev)
    _check(out, "out", BF16_BITS, numel=rows * pr.head_dim, device=dev)
    _check(lse, "lse", ("float32",), numel=rows, device=dev)
    _check_pools(pr, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, dev)
    _check(workspace, "workspace", ("uint8",), device=dev)
    ws_bytes = 0 if workspace is None else _nbytes(workspace) if not isinstance(workspace, int) \
        else small_w_attention_workspace_bytes(plan)
    args = [plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
            _stream(stream)]
    if events is None:
        rc = lib().small_w_attention_run(*args)
    else:
        rc = lib().small_w_attention_run_events(*args, *events)
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_run")


def small_w_attention_run_noalloc(plan: Plan, q, k_pool, v_pool, k_scale, v_scale,
                                  block_table, seq_lens, out, lse, stream=None) -> None:
    """small_w_attention_run without a workspace: the library's own per-GPU
    scratch holds the split partials (calls that overlap on one GPU race)."""
    pr = plan.problem
    dev = _current_device()
    rows = pr.num_reqs * pr.window * pr.num_q_heads
    _check(q, "q", BF16_BITS, numel=rows * pr.head_dim, device=dev)
    _check(out, "out", BF16_BITS, numel=rows * pr.head_dim, device=dev)
    _check(lse, "lse", ("float32",), numel=rows, device=dev)
    _check_pools(pr, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, dev)
    rc = lib().small_w_attention_run_noalloc(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                             _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                             _ptr(seq_lens), _ptr(out), _ptr(lse),
                                             _stream(stream))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_run_noalloc")


def small_w_attention_trace_pages(plan: Plan, block_table, seq_lens, pages_out,
                                  stream=None) -> None:
    pr = plan.problem
    dev = _current_device()
    _check(block_table, "block_table", ("int32",), numel=pr.num_reqs * pr.max_pages_per_req,
           device=dev)
    _check(seq_lens, "seq_lens", ("int32",), numel=pr.num_reqs, device=dev)
    maxp = pages_out.shape[-1]
    units = int(small_w_attention_plan_export(plan)[2])
    _check(pages_out, "pages_out", ("int32",), numel=units * maxp, device=dev)
    if maxp < small_w_attention_plan_max_unit_pages(plan):
        raise ValueError("pages_out: fewer columns than the plan's largest unit")
    rc = lib().small_w_attention_trace_pages(plan.handle, _ptr(block_table), _ptr(seq_lens),
                                             _ptr(pages_out), maxp, _stream(stream))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_trace_pages")


def small_w_attention_check_pages(plan: Plan, block_table, seq_lens, bad_out,
                                  stream=None) -> None:
    """Enqueue the table check: bad_out (device int32 [P]) receives, per
    request, the count of block-table entries the call reads that lie outside
    the pool, or -1 for a device length outside the rules."""
    pr = plan.problem
    dev = _current_device()
    _check(block_table, "block_table", ("int32",), numel=pr.num_reqs * pr.max_pages_per_req,
           device=dev)
    _check(seq_lens, "seq_lens", ("int32",), numel=pr.num_reqs, device=dev)
    _check(bad_out, "bad_out", ("int32",), numel=pr.num_reqs, device=dev)
    rc = lib().small_w_attention_check_pages(plan.handle, _ptr(block_table), _ptr(seq_lens),
                                             _ptr(bad_out), _stream(stream))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_attention_check_pages")


def small_w_kv_append(plan: Plan, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                      block_table, seq_lens, stream=None) -> None:
    """Write the plan's W window tokens (bf16 [P][W][Hkv][D] device tensors) into
    their pool slots: copied for a bf16 pool, quantised to e4m3 with a
    per-(token, KV-head) fp32 scale for an fp8 pool, or to E2M1 codes with an
    E8M0 scale per 32 elements for an MXFP4 pool.  Tensors are device tensors
    in the documented layouts; ValueError when one does not fit the plan."""
    pr = plan.problem
    dev = _current_device()
    n_new = pr.num_reqs * pr.window * pr.num_kv_heads * pr.head_dim
    _check(k_new, "k_new", BF16_BITS, numel=n_new, device=dev)
    _check(v_new, "v_new", BF16_BITS, numel=n_new, device=dev)
    _check_pools(pr, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, dev)
    rc = lib().small_w_kv_append(plan.handle, _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                 _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                 _ptr(seq_lens), _stream(stream))
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_kv_append")


def small_w_stream_read(buf, sink, stream=None, events=None) -> None:
    """Read the whole device tensor `buf` once with 16-byte loads (the HBM read
    ceiling reference); `sink` is a device uint32 tensor of at least one element;
    `events`: optional 2 raw hipEvent_t handles (start, end of the kernel)."""
    _check(sink, "sink", ("uint32", "int32"), device=buf.device)
    ev = events or (None, None)
    rc = lib().small_w_stream_read(_ptr(buf), _nbytes(buf), _ptr(sink), _stream(stream), *ev)
    if rc != SMALLW_OK:
        raise SmallwError(rc, "small_w_stream_read")


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
