"""Pools past 4 GiB: page offsets beyond 2^32 bytes (and 2^31 pool elements).

A small seeded workload's pages are spread over both ends of a pool a little
larger than 4 GiB (even pages keep their index, odd ones move to the top), and
every other page of the big pool is poison (NaN bf16, e4m3 NaN codes with NaN
scales, NaN E8M0 scales).  The call must give bitwise the outputs of the same
workload in its own small pool, which match the oracle; the append must write,
at the top of the big pool, the bytes the oracle's append writes in the small
one.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_sweep_amd as sw
from speculative_decode_verify_sweep_amd import device as dv
from test_gpu_parity import announce, check, gpu_run
from workloads import make_workload
from workloads.synth import to_bf16_bits

pytestmark = pytest.mark.gpu

PAGE_BYTES = {"bf16": 2.0, "fp8": 1.0, "mxfp4": 0.5}   # bytes per element of a pool


def small_case(kv):
    return make_workload(None, P=2, Hq=24, Hkv=4, D=256, ctx=(2500, 900), W=16, causal=True,
                         kv=kv, placement="permuted", pool_pages=230, seed=811, poison=True)


def page_map(w, nb):
    n = w.num_pages
    i = np.arange(n)
    return np.where(i % 2 == 0, i, nb - n + i).astype(np.int64)


def big_pools(w, d, nb):
    """Device tensors of nb pages holding w's pool pages at page_map(w, nb),
    every other page poisoned, and the block table rewritten to match."""
    m = page_map(w, nb)
    mt = torch.from_numpy(m).cuda()
    out = dict(d)
    for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
        x = d[key]
        if x is None:
            continue
        big = torch.empty((nb,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
        if x.dtype == torch.bfloat16 or x.dtype == torch.float32:
            big.fill_(float("nan"))
        else:  # byte pools: e4m3 NaN codes, E2M1 codes under NaN E8M0 scales
            big.fill_(0xFF if (key.endswith("scale") or w.kv == "fp8") else 0x77)
        big.index_copy_(0, mt, x)
        out[key] = big
    bt = w.block_table.astype(np.int64)
    ok = (bt >= 0) & (bt < w.num_pages)
    bt[ok] = m[bt[ok]]
    out["block_table"] = torch.from_numpy(bt.astype(np.int32)).cuda()
    return out, bt.astype(np.int32)


def pool_pages_past_4gib(w):
    per_page = int(w.Hkv * 16 * w.D * PAGE_BYTES[w.kv])
    return (1 << 32) // per_page + 64


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_pages_past_4gib_give_the_small_pool_outputs(kv):
    w = small_case(kv)
    nb = pool_pages_past_4gib(w)
    announce(f"big pool {kv}: {nb} pages")
    o_small, l_small = gpu_run(w)
    d, bt = big_pools(w, dv.upload(w), nb)
    assert d["k_pool"].numel() * d["k_pool"].element_size() > 1 << 32
    wb = dataclasses.replace(w, num_pages=nb, block_table=bt)
    plan = dv.plan_for(wb)
    ws = dv.workspace_for(plan)
    d["out"].fill_(float("nan"))
    d["lse"].fill_(float("nan"))
    dv.run(plan, d, ws)
    torch.cuda.synchronize()
    o = d["out"].float().cpu().numpy().astype(np.float64)
    l = d["lse"].cpu().numpy().astype(np.float64)
    del d, ws
    torch.cuda.empty_cache()
    np.testing.assert_array_equal(o, o_small)
    np.testing.assert_array_equal(l, l_small)
    check(w, o, l, *oracle.attention(w))


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_append_past_4gib_writes_the_oracle_bytes(kv):
    w = small_case(kv)
    nb = pool_pages_past_4gib(w)
    rng = np.random.default_rng(5)
    shape = (w.P, w.W, w.Hkv, w.D)
    kn = to_bf16_bits(rng.normal(0, 1, size=shape).astype(np.float32))
    vn = to_bf16_bits(rng.normal(0, 1, size=shape).astype(np.float32))
    announce(f"big pool append {kv}: {nb} pages")
    d, bt = big_pools(w, dv.upload(w), nb)
    wb = dataclasses.replace(w, num_pages=nb, block_table=bt)
    plan = dv.plan_for(wb)
    sw.small_w_kv_append(plan, torch.from_numpy(kn.view(np.int16)).cuda(),
                         torch.from_numpy(vn.view(np.int16)).cuda(), d["k_pool"], d["v_pool"],
                         d["k_scale"], d["v_scale"], d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    scaled = kv != "bf16"
    want = oracle.kv_append(P=w.P, W=w.W, Hkv=w.Hkv, D=w.D, kv=kv, k_new_bits=kn,
                            v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                            k_scale=w.k_scale if scaled else None,
                            v_scale=w.v_scale if scaled else None,
                            block_table=w.block_table, seq_lens=w.seq_lens,
                            num_pages=w.num_pages)
    mt = torch.from_numpy(page_map(w, nb)).cuda()
    for key, ref in zip(("k_pool", "v_pool", "k_scale", "v_scale"), want):
        if ref is None:
            continue
        got = d[key].index_select(0, mt).cpu()
        if got.dtype == torch.bfloat16:
            got = got.view(torch.int16).numpy().view(np.uint16)
        else:
            got = got.numpy()
        np.testing.assert_array_equal(got, ref, err_msg=key)
    del d
    torch.cuda.empty_cache()
