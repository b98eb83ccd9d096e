"""A plan fixed on the host, lengths that move on the device, and graph replay.

The sweep recomputes every unit's page range from the device seq_lens and the
plan's split counts, so one plan (and one captured graph) serves later steps
whose lengths changed.  Their block-table rows must cover the new lengths, and
the lengths must fit the table's row stride.  Results then follow the device
lengths; only the split balance (and, in row-exact mode, the grouping into
pieces) comes from the plan.  Each case is checked against the fp64 oracle for
the device lengths.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_sweep_amd import binding as B
from speculative_decode_verify_sweep_amd import device as dv
from test_gpu_parity import announce, check
from workloads import make_workload

pytestmark = pytest.mark.gpu

HOST = [500, 1200, 40]                 # lengths the plan is built from
DEVICE = [[700, 1000, 40], [31, 1360, 300], [500, 1200, 40], [8, 8, 1400]]


def _workload(kv, causal=True):
    D = 128
    longest = [max(c) for c in zip(HOST, *DEVICE)]
    npg = sum(-(-L // 16) for L in longest)
    return make_workload(None, P=3, Hq=12, Hkv=2, D=D, ctx=(0, 0, 0), W=8, causal=causal,
                         kv=kv, placement="permuted", pool_pages=npg + 3, seed=811,
                         seq_lens=tuple(longest))


def _plan(w, host, split_pages=0):
    pr = B.make_problem(num_reqs=w.P, window=w.W, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                        head_dim=w.D, num_pages=w.num_pages,
                        max_pages_per_req=w.block_table.shape[1], causal=w.causal,
                        kv_dtype=dv.KV_DTYPES[w.kv], scale=w.scale, split_pages=split_pages)
    return B.small_w_attention_plan(pr, np.asarray(host, dtype=np.int32))


def _result(d):
    o = d["out"].float().cpu().numpy().astype(np.float64)
    l = d["lse"].cpu().numpy().astype(np.float64)
    return o, l


@pytest.mark.parametrize("kv,split_pages", [("bf16", 0), ("fp8", 0), ("mxfp4", 0), ("bf16", 9)])
def test_device_lengths_may_move_under_a_fixed_plan(kv, split_pages):
    w = _workload(kv)
    d = dv.upload(w)
    pl = _plan(w, HOST, split_pages)
    ws = dv.workspace_for(pl)
    for dev_lens in DEVICE:
        wl = dataclasses.replace(w, seq_lens=np.asarray(dev_lens, dtype=np.int32))
        d["seq_lens"].copy_(torch.from_numpy(wl.seq_lens))
        announce(f"{kv} split_pages={split_pages}: plan {HOST}, device lengths {dev_lens}")
        dv.run(pl, d, ws)
        torch.cuda.synchronize()
        o, l = _result(d)
        check(wl, o, l, *oracle.attention(wl))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_replays_follow_the_device_lengths(kv):
    w = _workload(kv)
    d = dv.upload(w)
    pl = _plan(w, HOST)
    ws = dv.workspace_for(pl)
    announce(f"{kv}: capture one call in a graph")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dv.run(pl, d, ws)                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dv.run(pl, d, ws)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for dev_lens in DEVICE:
            wl = dataclasses.replace(w, seq_lens=np.asarray(dev_lens, dtype=np.int32))
            d["seq_lens"].copy_(torch.from_numpy(wl.seq_lens))
            d["out"].zero_()
            scratch.mul_(0.5).add_(1.0)        # eager work between the replays
            torch.cuda.synchronize()
            announce(f"{kv} replay {rep}, device lengths {dev_lens}")
            g.replay()
            torch.cuda.synchronize()
            o, l = _result(d)
            check(wl, o, l, *oracle.attention(wl))


def test_calls_on_two_streams_overlap_safely():
    """One plan shared by two streams, each call with its own workspace and
    outputs, plus a second plan of another format on a third stream; all
    enqueued interleaved, then checked against the oracle."""
    wa = _workload("bf16")
    wb = _workload("fp8", causal=False)
    da, da2, db = dv.upload(wa), dv.upload(wa), dv.upload(wb)
    pa, pb = _plan(wa, HOST), _plan(wb, HOST)
    wsa, wsa2, wsb = dv.workspace_for(pa), dv.workspace_for(pa), dv.workspace_for(pb)
    for d, w in ((da, wa), (da2, wa), (db, wb)):
        d["seq_lens"].copy_(torch.from_numpy(np.asarray(HOST, dtype=np.int32)))
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    announce("three streams, two plans, separate workspaces")
    for _ in range(5):
        for s, (pl, d, ws) in zip(streams, ((pa, da, wsa), (pa, da2, wsa2), (pb, db, wsb))):
            with torch.cuda.stream(s):
                dv.run(pl, d, ws)
    torch.cuda.synchronize()
    for d, w in ((da, wa), (da2, wa), (db, wb)):
        wl = dataclasses.replace(w, seq_lens=np.asarray(HOST, dtype=np.int32))
        o, l = _result(d)
        check(wl, o, l, *oracle.attention(wl))
    np.testing.assert_array_equal(da["out"].view(torch.int16).cpu().numpy(),
                                  da2["out"].view(torch.int16).cpu().numpy())
