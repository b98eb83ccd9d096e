"""Oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU reference for small-window paged attention.
Only `tests/`, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code, header, table or constant generator with the
HIP library and never imports it.

  attention.c   fp64 attention over the gathered pages (C, OpenMP)
  _lib.py       builds and loads attention.c through ctypes
  append.py     the paged KV append, the e4m3fn round-to-nearest-even encoder
                and the MXFP4 (E2M1 + E8M0 block scale) quantizer
  ref.py        the split planner restated from its written specification,
                the log-sum-exp combine, the per-unit page gather and the
                closed-form work and byte counts
"""
from ._lib import (attention, build_oracle, decode_bf16, decode_e2m1, decode_e4m3, decode_e8m0,
                   oracle_threads)
from .append import (E4M3_MAX, e2m1_encode, e4m3_encode, e4m3_row_quantize, kv_append,
                     mxfp4_row_quantize)
from .ref import (PLAN_MIN_PAGES, attention_pairs, gather_unit_pages, kv_bytes, lse_combine,
                  plan, plan_export, split_range)

__all__ = ["attention", "decode_bf16", "decode_e4m3", "decode_e2m1", "decode_e8m0",
           "build_oracle", "oracle_threads", "e2m1_encode", "mxfp4_row_quantize",
           "PLAN_MIN_PAGES", "attention_pairs", "gather_unit_pages", "kv_bytes", "lse_combine",
           "plan", "plan_export", "split_range", "E4M3_MAX", "e4m3_encode", "e4m3_row_quantize",
           "kv_append"]
