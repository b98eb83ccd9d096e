"""Device plumbing for callers that hold inputs as host arrays.

Copies host arrays in the library's documented layouts into device tensors,
builds a plan and enqueues calls.  PyTorch provides memory and the stream; all
attention arithmetic happens in libsmallw.so.  Inputs are duck-typed: any
object with the attributes P, W, Hq, Hkv, D, causal, kv ("bf16"/"fp8"/"mxfp4"),
scale, num_pages, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

KV_DTYPES = {"bf16": B.SMALLW_KV_BF16, "fp8": B.SMALLW_KV_FP8_E4M3, "mxfp4": B.SMALLW_KV_MXFP4}


def upload(w, device: str = "cuda:0") -> dict:
    dev = torch.device(device)
    raw = w.kv != "bf16"      # byte pools (e4m3 codes, MXFP4 nibbles) and their scales

    def t(a, dtype=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            x = x.view(dtype)
        return x.to(dev)

    d = {
        "q": t(w.q.view(np.int16), torch.bfloat16),
        "k_pool": t(w.k_pool) if raw else t(w.k_pool.view(np.int16), torch.bfloat16),
        "v_pool": t(w.v_pool) if raw else t(w.v_pool.view(np.int16), torch.bfloat16),
        "k_scale": t(w.k_scale) if raw else None,
        "v_scale": t(w.v_scale) if raw else None,
        "block_table": t(w.block_table),
        "seq_lens": t(w.seq_lens),
    }
    d["out"] = torch.empty((w.P, w.W, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    d["lse"] = torch.empty((w.P, w.W, w.Hq), dtype=torch.float32, device=dev)
    return d


def plan_for(w, *, num_cus: int = 0, force_splits: int = 0, split_pages: int = 0) -> B.Plan:
    pr = B.make_problem(num_reqs=w.P, window=w.W, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                        head_dim=w.D, num_pages=w.num_pages,
                        max_pages_per_req=w.block_table.shape[1], causal=w.causal,
                        kv_dtype=KV_DTYPES[w.kv],
                        scale=w.scale, num_cus=num_cus, force_splits=force_splits,
                        split_pages=split_pages, window_left=getattr(w, "window_left", 0),
                        v_layout=getattr(w, "v_layout", 0))
    return B.small_w_attention_plan(pr, w.seq_lens)


def workspace_for(plan: B.Plan, device: str = "cuda:0"):
    n = B.small_w_attention_workspace_bytes(plan)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def run(plan: B.Plan, d: dict, workspace=None, stream=None, events=None) -> None:
    B.small_w_attention_run(plan, d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                            d["block_table"], d["seq_lens"], d["out"], d["lse"], workspace,
                            stream=stream, events=events)
