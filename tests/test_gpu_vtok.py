"""Token-major value pages (bf16): V stored [page][head][16][D] like K.

The kernel reads such pages with LDS transpose reads and hands the PV product
the same operand elements, in the same order, as it reads from d-major pages,
so every output is bitwise the d-major run on the same values, and both match
the oracle (which gathers V from either layout) under the parity bound.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_sweep_amd as sw
from speculative_decode_verify_sweep_amd import device as dv
from test_gpu_parity import EDGE, WINDOW, announce, check, gpu_run
from workloads import make_workload
from workloads.synth import to_bf16_bits

pytestmark = pytest.mark.gpu


def pair(name=None, **kw):
    """The same seeded values in both layouts."""
    wd = make_workload(name, v_layout=0, **kw)
    wt = make_workload(name, v_layout=1, **kw)
    assert wt.v_layout == 1 and wd.v_layout == 0
    np.testing.assert_array_equal(wt.v_pool.transpose(0, 1, 3, 2), wd.v_pool)
    return wd, wt


def same_as_dmajor(wd, wt, **run):
    o, l = gpu_run(wt, **run)
    od, ld = gpu_run(wd, **run)
    np.testing.assert_array_equal(o, od)
    np.testing.assert_array_equal(l, ld)
    check(wt, o, l, *oracle.attention(wt))


@pytest.mark.parametrize("name,W,force", [("tiny", None, 0), ("tiny", None, 3),
                                          ("verify16k", 16, 0), ("verify64k", 16, 0),
                                          ("verify64k", 1, 0), ("draft", None, 0),
                                          ("mixed", None, 0)])
def test_token_major_named_workloads(name, W, force):
    wd, wt = pair(name, **({} if W is None else {"W": W}))
    announce(f"token-major {name} W={wt.W} force={force}")
    same_as_dmajor(wd, wt, force_splits=force)


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("force", [0, 2])
def test_token_major_edge_shapes(case, force):
    spec = EDGE[case]
    npg = sum(-(-(c + spec["W"]) // 16) for c in spec["ctx"])
    wd, wt = pair(kv="bf16", placement="permuted", pool_pages=npg + 7, seed=300 + case, **spec)
    announce(f"token-major edge {case} {spec} force={force}")
    same_as_dmajor(wd, wt, force_splits=force)


@pytest.mark.parametrize("case", range(len(WINDOW)))
@pytest.mark.parametrize("mode", ["auto", "exact"])
def test_token_major_sliding_window(case, mode):
    spec = dict(WINDOW[case])
    name = spec.pop("name")
    if name is None:
        npg = sum(-(-(c + spec["W"]) // 16) for c in spec["ctx"])
        spec.update(kv="bf16", placement="permuted", pool_pages=npg + 7, seed=90 + case)
    wd, wt = pair(name, **spec)
    announce(f"token-major window {case} {mode}")
    same_as_dmajor(wd, wt, split_pages=13 if mode == "exact" else 0)


def test_token_major_row_exact_rows_do_not_depend_on_the_window():
    wd, wt = pair(None, P=2, Hq=24, Hkv=4, D=256, ctx=(1500, 333), W=16, causal=True,
                  kv="bf16", placement="permuted", pool_pages=140, seed=61, poison=False)
    announce("token-major row-exact window independence")
    o, l = gpu_run(wt, split_pages=8)
    for i in (0, 7, 15):
        w1 = dataclasses.replace(wt, W=1, q=np.ascontiguousarray(wt.q[:, i:i + 1]),
                                 seq_lens=(wt.seq_lens - wt.W + i + 1).astype(np.int32))
        o1, l1 = gpu_run(w1, split_pages=8)
        np.testing.assert_array_equal(o[:, i], o1[:, 0])
        np.testing.assert_array_equal(l[:, i], l1[:, 0])
    check(wt, o, l, *oracle.attention(wt))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_token_major_append_then_verify(D):
    """Append the window's K/V rows into token-major pages (bitwise the
    oracle's append), then verify over the updated pool against the oracle."""
    W, Hkv = 8, 2
    w = make_workload(None, P=3, Hq=8, Hkv=Hkv, D=D, ctx=(40, 300, 5), W=W, causal=True,
                      kv="bf16", placement="permuted", pool_pages=40, seed=470 + D, v_layout=1)
    rng = np.random.default_rng(D)
    kn = to_bf16_bits(rng.standard_normal((w.P, W, Hkv, D), dtype=np.float32))
    vn = to_bf16_bits(rng.standard_normal((w.P, W, Hkv, D), dtype=np.float32))
    announce(f"token-major append + verify D={D}")
    d = dv.upload(w)
    plan = dv.plan_for(w)
    sw.small_w_kv_append(plan, torch.from_numpy(kn.view(np.int16)).cuda(),
                         torch.from_numpy(vn.view(np.int16)).cuda(), d["k_pool"], d["v_pool"],
                         None, None, d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    kp, vp, _, _ = oracle.kv_append(P=w.P, W=W, Hkv=Hkv, D=D, kv="bf16", k_new_bits=kn,
                                    v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                    k_scale=None, v_scale=None, block_table=w.block_table,
                                    seq_lens=w.seq_lens, num_pages=w.num_pages, v_layout=1)
    np.testing.assert_array_equal(d["k_pool"].view(torch.int16).cpu().numpy().view(np.uint16), kp)
    np.testing.assert_array_equal(d["v_pool"].view(torch.int16).cpu().numpy().view(np.uint16), vp)
    w2 = dataclasses.replace(w, k_pool=kp, v_pool=vp)
    ws = dv.workspace_for(plan)
    dv.run(plan, d, ws)
    torch.cuda.synchronize()
    o = d["out"].float().cpu().numpy().astype(np.float64)
    l = d["lse"].cpu().numpy().astype(np.float64)
    check(w2, o, l, *oracle.attention(w2))
