"""Pins for the oracle: each test ties it to something other than itself.

* brute force: a dense numpy/torch formulation (vectorised gather, torch's own
  bf16 / float8_e4m3fn decoders, an explicit mask matrix) and torch's
  scaled_dot_product_attention in float64;
* closed forms (Q = 0, equal keys, constant V, one key, W = 1);
* invariants (window split, page relabelling, GQA = replicated MHA, batch =
  singles, NaN poison, split partials + log-sum-exp combine);
* format tables (all bf16, e4m3fn and E8M0 codes against torch; the sixteen
  E2M1 codes against the value table of the OCP MX format);
* numbers the pages print (tests/golden/).
"""
import dataclasses
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(P=1, Hq=4, Hkv=2, D=8, ctx=(20,), W=3, causal=True, kv="bf16", seed=1, pool=None,
         poison=True, **kw):
    npg = sum(math.ceil((c + W) / 16) for c in ctx)
    return make_workload(None, P=P, Hq=Hq, Hkv=Hkv, D=D, ctx=tuple(ctx), W=W, causal=causal,
                         kv=kv, placement="permuted", pool_pages=pool or npg + 5, seed=seed,
                         poison=poison, **kw)


# ---------------------------------------------------------------- brute force
def dense_kv(w):
    """Dense K, V [P][Hkv][Lmax][D] in float64 via vectorised gather + torch decoders."""
    Lmax = max(1, int(w.seq_lens.max()))
    K = np.zeros((w.P, w.Hkv, Lmax, w.D))
    V = np.zeros((w.P, w.Hkv, Lmax, w.D))
    for p in range(w.P):
        L = int(w.seq_lens[p])
        if L == 0:
            continue
        t = np.arange(L)
        phys = w.block_table[p, t // 16]
        slot = t % 16
        if w.kv == "mxfp4":
            kd, vd = dense_mxfp4(w, phys, slot)
            K[p, :, :L] = kd.transpose(1, 0, 2)
            V[p, :, :L] = vd.transpose(1, 0, 2)
            continue
        kc = w.k_pool[phys, :, slot, :]                  # [L][Hkv][D]
        if getattr(w, "v_layout", 0) == 1:               # token-major value pages
            vc = w.v_pool[phys, :, slot, :]
        else:
            vc = w.v_pool[phys, :, :, slot]              # [L][Hkv][D]
        if w.kv == "fp8":
            kd = torch.from_numpy(np.ascontiguousarray(kc)).view(torch.float8_e4m3fn).double()
            vd = torch.from_numpy(np.ascontiguousarray(vc)).view(torch.float8_e4m3fn).double()
            kd = kd * torch.from_numpy(w.k_scale[phys, :, slot]).double()[..., None]
            vd = vd * torch.from_numpy(w.v_scale[phys, :, slot]).double()[..., None]
        else:
            kd = torch.from_numpy(np.ascontiguousarray(kc).view(np.int16)).view(torch.bfloat16).double()
            vd = torch.from_numpy(np.ascontiguousarray(vc).view(np.int16)).view(torch.bfloat16).double()
        K[p, :, :L] = kd.numpy().transpose(1, 0, 2)
        V[p, :, :L] = vd.numpy().transpose(1, 0, 2)
    return K, V


# E2M1 magnitudes of codes 0..7 as the OCP MX format tabulates them
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def dense_mxfp4(w, phys, slot):
    """K, V [L][Hkv][D] of the tokens at (phys[t], slot[t]): nibbles unpacked
    with numpy, E2M1 by the table above, E8M0 by torch's float8_e8m0fnu."""
    table = np.array(E2M1_TABLE + [-x for x in E2M1_TABLE])
    kb = w.k_pool[phys, :, slot, :]                          # [L][Hkv][D/2]
    kn = np.stack([kb & 15, kb >> 4], axis=-1).reshape(kb.shape[0], w.Hkv, w.D)
    vb = w.v_pool[phys, :, :, slot // 2]                     # [L][Hkv][D]
    vn = np.where((slot % 2 == 1)[:, None, None], vb >> 4, vb & 15)

    def e8m0(b):
        return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e8m0fnu).double().numpy()

    ks = np.repeat(e8m0(w.k_scale[phys, :, slot, :]), 32, axis=-1)   # [L][Hkv][D]
    vs = np.repeat(e8m0(w.v_scale[phys, :, :, slot]), 32, axis=-1)   # block-major V scales
    return table[kn] * ks, table[vn] * vs


def q_f64(w):
    return torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).double().numpy()


def mask_matrix(L, W, causal, Lmax, window_left=0):
    i = np.arange(W)[:, None]
    j = np.arange(Lmax)[None, :]
    vis = np.broadcast_to(j < L, (W, Lmax))
    hi = (L - W + i) if causal else np.full((W, 1), L - 1)
    if causal:
        vis = vis & (j <= hi)
    if window_left > 0:
        vis = vis & (j >= hi - window_left + 1)
    return vis


def brute(w):
    K, V = dense_kv(w)
    Q = q_f64(w)
    G = w.G
    Lmax = K.shape[2]
    out = np.zeros((w.P, w.W, w.Hq, w.D))
    lse = np.full((w.P, w.W, w.Hq), -np.inf)
    for p in range(w.P):
        M = mask_matrix(int(w.seq_lens[p]), w.W, w.causal, Lmax, w.window_left)
        for h in range(w.Hq):
            S = (Q[p, :, h, :] @ K[p, h // G].T) * w.scale      # [W][Lmax]
            S = np.where(M, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            E = np.where(M, np.exp(S - np.where(np.isfinite(m), m, 0.0)), 0.0)
            l = E.sum(axis=1)
            out[p, ok, h] = (E[ok] @ V[p, h // G]) / l[ok, None]
            lse[p, ok, h] = m[ok, 0] + np.log(l[ok])
    return out, lse


CASES = [
    dict(P=1, Hq=4, Hkv=1, D=64, ctx=(256,), W=4, causal=True),            # the tiny config
    dict(P=3, Hq=4, Hkv=2, D=8, ctx=(5, 40, 66), W=5, causal=True),
    dict(P=2, Hq=6, Hkv=3, D=16, ctx=(1, 33), W=2, causal=False),
    dict(P=2, Hq=4, Hkv=4, D=8, ctx=(15, 16), W=1, causal=True),
    dict(P=1, Hq=12, Hkv=2, D=64, ctx=(300,), W=16, causal=True),
    dict(P=2, Hq=4, Hkv=1, D=8, ctx=(17, 31), W=3, causal=True, kv="fp8"),
    dict(P=2, Hq=8, Hkv=2, D=16, ctx=(50, 9), W=4, causal=False, kv="fp8"),
    dict(P=2, Hq=4, Hkv=2, D=8, ctx=(40, 70), W=5, causal=True, window_left=20),
    dict(P=1, Hq=4, Hkv=1, D=16, ctx=(50,), W=6, causal=True, window_left=3),   # window < W
    dict(P=2, Hq=4, Hkv=2, D=8, ctx=(33, 10), W=3, causal=False, window_left=17),
    dict(P=2, Hq=4, Hkv=1, D=8, ctx=(90, 4), W=4, causal=True, kv="fp8", window_left=33),
    dict(P=2, Hq=4, Hkv=2, D=32, ctx=(17, 45), W=3, causal=True, kv="mxfp4"),
    dict(P=2, Hq=6, Hkv=1, D=64, ctx=(60, 3), W=5, causal=False, kv="mxfp4"),
    dict(P=1, Hq=4, Hkv=2, D=96, ctx=(70,), W=4, causal=True, kv="mxfp4", window_left=21),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_oracle_matches_dense_brute_force(case):
    w = tiny(seed=10 + case, **CASES[case])
    o, l = oracle.attention(w)
    ob, lb = brute(w)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=1e-13, atol=1e-12)


VTOK_CASES = [c for c in CASES if c.get("kv", "bf16") == "bf16"]


@pytest.mark.parametrize("case", range(len(VTOK_CASES)))
def test_oracle_reads_token_major_value_pages(case):
    """bf16 value pages stored token-major ([page][head][16][D], like K): the
    generator lays the same values out as the transpose of the d-major pool,
    the oracle matches the brute force (which gathers V by its own indexing)
    and is bitwise its own d-major result on those values."""
    spec = VTOK_CASES[case]
    wt = tiny(seed=40 + case, v_layout=1, **spec)
    wd = tiny(seed=40 + case, v_layout=0, **spec)
    np.testing.assert_array_equal(wt.v_pool.transpose(0, 1, 3, 2), wd.v_pool)
    o, l = oracle.attention(wt)
    ob, lb = brute(wt)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=1e-13, atol=1e-12)
    od, ld = oracle.attention(wd)
    np.testing.assert_array_equal(o, od)
    np.testing.assert_array_equal(l, ld)
    if spec["D"] != 16:   # reading a d-major pool as token-major changes the output
        wrong = dataclasses.replace(wt, v_pool=np.ascontiguousarray(
            wd.v_pool.reshape(wt.v_pool.shape)))
        assert not np.array_equal(oracle.attention(wrong)[0], o)


def test_oracle_rejects_token_major_low_precision_pools():
    w = tiny(kv="fp8", D=16)
    with pytest.raises(ValueError):
        oracle.attention(dataclasses.replace(w, v_layout=1))


def test_oracle_append_token_major_is_the_transposed_append():
    wt = tiny(P=2, Hq=4, Hkv=2, D=32, ctx=(40, 5), W=4, seed=72, v_layout=1)
    wd = tiny(P=2, Hq=4, Hkv=2, D=32, ctx=(40, 5), W=4, seed=72, v_layout=0)
    rng = np.random.default_rng(5)
    kn = to_bf16_bits(rng.standard_normal((2, 4, 2, 32), dtype=np.float32))
    vn = to_bf16_bits(rng.standard_normal((2, 4, 2, 32), dtype=np.float32))
    out = {}
    for lay, w in ((1, wt), (0, wd)):
        out[lay] = oracle.kv_append(P=2, W=4, Hkv=2, D=32, kv="bf16", k_new_bits=kn,
                                    v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                    k_scale=None, v_scale=None, block_table=w.block_table,
                                    seq_lens=w.seq_lens, num_pages=w.num_pages, v_layout=lay)
    np.testing.assert_array_equal(out[1][0], out[0][0])
    np.testing.assert_array_equal(out[1][1].transpose(0, 1, 3, 2), out[0][1])
    pos = int(wt.seq_lens[0]) - 4 + 2                 # token 2 of request 0
    pg = int(wt.block_table[0, pos // 16])
    np.testing.assert_array_equal(out[1][1][pg, 1, pos % 16, :], vn[0, 2, 1])


@pytest.mark.parametrize("case", range(len(CASES)))
def test_oracle_matches_torch_sdpa_fp64(case):
    w = tiny(seed=20 + case, **CASES[case])
    o, _ = oracle.attention(w)
    K, V = dense_kv(w)
    Q = q_f64(w)
    for p in range(w.P):
        L = int(w.seq_lens[p])
        M = torch.from_numpy(np.array(mask_matrix(L, w.W, w.causal, K.shape[2], w.window_left)))
        kk = torch.from_numpy(K[p]).repeat_interleave(w.G, dim=0)[None]     # [1][Hq][L][D]
        vv = torch.from_numpy(V[p]).repeat_interleave(w.G, dim=0)[None]
        qq = torch.from_numpy(Q[p]).permute(1, 0, 2)[None]                   # [1][Hq][W][D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=M, scale=w.scale)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o[p], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_zero_query_gives_log_count_and_mean_value():
    w = tiny(P=2, Hq=4, Hkv=2, D=16, ctx=(29, 70), W=6, causal=True, seed=3)
    w.q[...] = 0
    o, l = oracle.attention(w)
    _, V = dense_kv(w)
    for p in range(w.P):
        L = int(w.seq_lens[p])
        for i in range(w.W):
            n = L - w.W + i + 1
            np.testing.assert_allclose(l[p, i], math.log(n), rtol=0, atol=1e-13)
            for h in range(w.Hq):
                np.testing.assert_allclose(o[p, i, h], V[p, h // w.G, :n].mean(axis=0),
                                           rtol=0, atol=1e-13)


def test_equal_keys_give_uniform_weights():
    w = tiny(P=1, Hq=2, Hkv=1, D=8, ctx=(40,), W=3, causal=True, seed=4)
    key = to_bf16_bits(np.linspace(-1, 1, 8, dtype=np.float32))
    for n in range(math.ceil(int(w.seq_lens[0]) / 16)):
        w.k_pool[w.block_table[0, n], 0, :, :] = key
    o, l = oracle.attention(w)
    K, V = dense_kv(w)
    Q = q_f64(w)
    for i in range(w.W):
        n = int(w.seq_lens[0]) - w.W + i + 1
        for h in range(w.Hq):
            s = w.scale * float(Q[0, i, h] @ K[0, 0, 0])
            assert abs(l[0, i, h] - (s + math.log(n))) < 1e-12
            np.testing.assert_allclose(o[0, i, h], V[0, 0, :n].mean(axis=0), atol=1e-13)


def test_constant_value_rows_return_the_constant():
    w = tiny(P=2, Hq=4, Hkv=2, D=8, ctx=(21, 50), W=4, causal=False, seed=5)
    c = 0.375
    w.v_pool[...] = to_bf16_bits(np.float32(c))
    o, _ = oracle.attention(w)
    np.testing.assert_allclose(o, c, rtol=0, atol=1e-15)


def test_single_key_returns_its_value_and_score():
    w = tiny(P=1, Hq=2, Hkv=1, D=8, ctx=(0,), W=1, causal=False, seed=6)
    o, l = oracle.attention(w)
    K, V = dense_kv(w)
    Q = q_f64(w)
    for h in range(2):
        np.testing.assert_array_equal(o[0, 0, h], V[0, 0, 0])
        assert abs(l[0, 0, h] - w.scale * float(Q[0, 0, h] @ K[0, 0, 0])) < 1e-14


def test_one_row_causal_equals_non_causal():
    w = tiny(P=2, Hq=4, Hkv=2, D=8, ctx=(10, 45), W=1, causal=True, seed=7)
    a = oracle.attention(w)
    b = oracle.attention(dataclasses.replace(w, causal=False))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_empty_request_gives_zero_and_minus_inf():
    w = tiny(P=3, Hq=2, Hkv=1, D=8, ctx=(10, 0, 20), W=2, causal=True, seed=8,
             seq_lens=(12, 0, 22))
    o, l = oracle.attention(w)
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
    ob, lb = brute(w)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(l[[0, 2]], lb[[0, 2]], atol=1e-12)


def test_causal_shorter_than_window_is_rejected():
    w = tiny(P=1, Hq=2, Hkv=1, D=8, ctx=(5,), W=4, causal=True, seq_lens=(3,))
    with pytest.raises(ValueError):
        oracle.attention(w)


# ---------------------------------------------------------------- invariants
def test_window_rows_equal_single_row_calls():
    w = tiny(P=2, Hq=6, Hkv=2, D=16, ctx=(37, 80), W=7, causal=True, seed=11)
    o, l = oracle.attention(w)
    for i in range(w.W):
        one = dataclasses.replace(w, W=1, q=np.ascontiguousarray(w.q[:, i:i + 1]),
                                  seq_lens=(w.seq_lens - w.W + i + 1).astype(np.int32))
        o1, l1 = oracle.attention(one)
        np.testing.assert_array_equal(o[:, i], o1[:, 0])
        np.testing.assert_array_equal(l[:, i], l1[:, 0])


def test_sixteen_rows_equal_two_eight_row_calls():
    w = tiny(P=1, Hq=4, Hkv=1, D=8, ctx=(100,), W=16, causal=True, seed=12)
    o, l = oracle.attention(w)
    lo = dataclasses.replace(w, W=8, q=np.ascontiguousarray(w.q[:, :8]),
                             seq_lens=(w.seq_lens - 8).astype(np.int32))
    hi = dataclasses.replace(w, W=8, q=np.ascontiguousarray(w.q[:, 8:]))
    np.testing.assert_array_equal(o[:, :8], oracle.attention(lo)[0])
    np.testing.assert_array_equal(o[:, 8:], oracle.attention(hi)[0])


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_page_relabelling_is_bitwise_invariant(kv):
    w = tiny(P=2, Hq=4, Hkv=2, D=32, ctx=(50, 77), W=5, causal=True, kv=kv, seed=13, pool=20)
    perm = np.random.default_rng(0).permutation(w.num_pages)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(w.num_pages)
    w2 = dataclasses.replace(
        w, k_pool=np.ascontiguousarray(w.k_pool[inv]), v_pool=np.ascontiguousarray(w.v_pool[inv]),
        k_scale=None if w.k_scale is None else np.ascontiguousarray(w.k_scale[inv]),
        v_scale=None if w.v_scale is None else np.ascontiguousarray(w.v_scale[inv]),
        block_table=np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
        .astype(np.int32))
    a, b = oracle.attention(w), oracle.attention(w2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_gqa_equals_replicated_mha():
    w = tiny(P=2, Hq=6, Hkv=2, D=8, ctx=(30, 47), W=3, causal=True, seed=14)
    rep = np.repeat(np.arange(w.Hkv), w.G)
    w2 = dataclasses.replace(w, Hkv=w.Hq, k_pool=np.ascontiguousarray(w.k_pool[:, rep]),
                             v_pool=np.ascontiguousarray(w.v_pool[:, rep]))
    a, b = oracle.attention(w), oracle.attention(w2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_batch_equals_single_requests():
    w = tiny(P=3, Hq=4, Hkv=2, D=8, ctx=(12, 60, 33), W=4, causal=False, seed=15)
    o, l = oracle.attention(w)
    for p in range(w.P):
        one = dataclasses.replace(w, P=1, q=np.ascontiguousarray(w.q[p:p + 1]),
                                  block_table=np.ascontiguousarray(w.block_table[p:p + 1]),
                                  seq_lens=np.ascontiguousarray(w.seq_lens[p:p + 1]))
        o1, l1 = oracle.attention(one)
        np.testing.assert_array_equal(o[p], o1[0])
        np.testing.assert_array_equal(l[p], l1[0])


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_nan_in_stale_slots_and_free_pages_is_never_read(kv):
    D = 32 if kv == "mxfp4" else 8
    a = tiny(P=2, Hq=4, Hkv=2, D=D, ctx=(19, 42), W=3, kv=kv, seed=16, poison=True, pool=12)
    b = tiny(P=2, Hq=4, Hkv=2, D=D, ctx=(19, 42), W=3, kv=kv, seed=16, poison=False, pool=12)
    assert np.isnan(oracle.decode_bf16(a.k_pool)).any() if kv == "bf16" else True
    oa, la = oracle.attention(a)
    ob, lb = oracle.attention(b)
    assert np.isfinite(oa).all() and np.isfinite(la).all()
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


@pytest.mark.parametrize("force", [1, 2, 3, 7, 0])
def test_split_partials_combine_to_the_full_result(force):
    w = tiny(P=1, Hq=4, Hkv=2, D=16, ctx=(200,), W=6, causal=True, seed=17)
    n = math.ceil(int(w.seq_lens[0]) / 16)
    pl = oracle.plan(P=1, Hkv=w.Hkv, D=w.D, kv_fp8=False, seq_lens=w.seq_lens, num_cus=1,
                     force_splits=force or n)
    o, l = oracle.attention(w)
    S = pl["splits"][0]
    parts_o, parts_l = [], []
    for s in range(S):
        pb, pe = oracle.split_range(n, S, s)
        po, plse = oracle.attention(w, key_lo=pb * 16, key_hi=pe * 16)
        parts_o.append(po)
        parts_l.append(plse)
    co, cl = oracle.lse_combine(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(co, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(cl, l, rtol=1e-13, atol=1e-12)


def test_sampled_rows_equal_full_rows():
    w = tiny(P=2, Hq=6, Hkv=3, D=16, ctx=(40, 90), W=5, causal=True, seed=18)
    o, l = oracle.attention(w)
    rows = np.array([[0, 0, 0], [1, 4, 5], [1, 2, 3], [0, 3, 1]])
    os_, ls_ = oracle.attention(w, rows=rows)
    for k, (p, i, h) in enumerate(rows):
        np.testing.assert_array_equal(os_[k], o[p, i, h])
        assert ls_[k] == l[p, i, h]


# ---------------------------------------------------------------- formats
def test_bf16_decode_matches_torch_for_every_code():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_bf16(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert np.nanmax(mine) == 448.0 and mine[1] == 2.0 ** -9


def test_e2m1_decode_matches_the_format_table():
    codes = np.arange(16, dtype=np.uint8)
    mine = oracle.decode_e2m1(codes)
    np.testing.assert_array_equal(mine[:8], E2M1_TABLE)
    np.testing.assert_array_equal(mine[8:], [-x for x in E2M1_TABLE])
    assert np.signbit(mine[8]) and not np.signbit(mine[0])
    # only the low nibble of each byte is a code
    np.testing.assert_array_equal(oracle.decode_e2m1(codes | 0xF0), mine)


def test_e8m0_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    mine = oracle.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(mine[255]) and np.isnan(ref[255]) and not np.isnan(mine[:255]).any()
    np.testing.assert_array_equal(mine[:255], ref[:255])
    assert mine[127] == 1.0 and mine[0] == 2.0 ** -127


def test_mxfp4_pools_decode_like_the_same_values_stored_as_bf16():
    """Every E2M1 value times a power of two in bf16 range is a bf16 value, so
    an MXFP4 workload re-stored as bf16 (decoded here with the test's own table)
    must give bitwise the oracle's MXFP4 result."""
    w = tiny(P=2, Hq=6, Hkv=2, D=64, ctx=(40, 21), W=4, causal=True, kv="mxfp4", seed=31,
             poison=False)
    npg, Hkv, D = w.num_pages, w.Hkv, w.D
    pages = np.repeat(np.arange(npg), 16)
    slots = np.tile(np.arange(16), npg)
    kd, vd = dense_mxfp4(w, pages, slots)                        # [npg*16][Hkv][D]
    kbits = to_bf16_bits(kd.astype(np.float32)).reshape(npg, 16, Hkv, D).transpose(0, 2, 1, 3)
    vbits = to_bf16_bits(vd.astype(np.float32)).reshape(npg, 16, Hkv, D).transpose(0, 2, 3, 1)
    np.testing.assert_array_equal(oracle.decode_bf16(kbits).transpose(0, 2, 1, 3).reshape(-1, Hkv, D), kd)
    w2 = dataclasses.replace(w, kv="bf16", k_pool=np.ascontiguousarray(kbits),
                             v_pool=np.ascontiguousarray(vbits), k_scale=None, v_scale=None)
    a, b = oracle.attention(w), oracle.attention(w2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_mxfp4_kv_byte_count():
    # per token and KV head: K and V at half a byte per element, one scale byte
    # per 32 elements each
    assert oracle.kv_bytes([16384 + 16], 4, 256, kv="mxfp4") == (16384 + 16) * 4 * (256 + 16)
    assert oracle.kv_bytes([10], 1, 64, kv="mxfp4") == 10 * (64 + 4)


# ---------------------------------------------------------------- counts and the pages' numbers
def test_attention_pairs_equal_mask_population():
    for L, W, causal in [(260, 4, True), (9, 9, True), (1309, 9, False), (70, 16, True)]:
        M = mask_matrix(L, W, causal, L)
        assert oracle.attention_pairs([L], W, 3, causal) == 3 * int(M.sum())
    # closed forms: causal H*(W*L - W(W-1)/2), non-causal H*W*L
    assert oracle.attention_pairs([100, 50], 5, 2, True) == 2 * (5 * 150 - 2 * 10)
    assert oracle.attention_pairs([100, 50], 5, 2, False) == 2 * 5 * 150


def _rows(fname):
    rows = []
    for line in open(os.path.join(GOLDEN, fname)):
        line = line.split("#")[0].strip()
        if line:
            rows.append([float(x) for x in line.split()])
    return rows


def test_kv_byte_count_reproduces_the_pages_bandwidth_figures():
    for ctx, _W, us, gbps in _rows("p1_measurement.txt"):
        b = oracle.kv_bytes([int(ctx)], Hkv=4, D=256)
        assert abs(b / (us * 1e-6) / 1e9 - gbps) / gbps < 0.005


def test_draft_work_blowup_matches_the_pages_ratio():
    for ctx, k, ratio, tol in _rows("p2_work.txt"):
        from oracle.ref import materialised_pairs, paged_pairs
        r = materialised_pairs([int(ctx)], int(k)) / paged_pairs([int(ctx)], int(k))
        assert abs(r - ratio) / ratio < tol


# ---------------------------------------------------------------- planner specification
def test_plan_partitions_every_request_into_balanced_splits():
    rng = np.random.default_rng(5)
    for trial in range(200):
        P = int(rng.integers(1, 9))
        seq = [int(x) for x in rng.integers(0, 5000, size=P)]
        Hkv = int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128, 256]))
        fp8 = bool(rng.integers(0, 2))
        force = int(rng.choice([0, 0, 1, 3, 50]))
        pl = oracle.plan(P=P, Hkv=Hkv, D=D, kv_fp8=fp8, seq_lens=seq, num_cus=256,
                         force_splits=force)
        assert pl["U"] == Hkv * sum(pl["splits"]) == len(pl["units"])
        if force == 0 and P * Hkv <= 256:                   # never a second round
            assert pl["U"] <= 256 * (1 if D == 256 or fp8 else 2)
        k = 0
        for p in range(P):
            n, S = pl["n_pg"][p], pl["splits"][p]
            assert n == math.ceil(seq[p] / 16)
            assert 1 <= S <= max(n, 1)
            if force == 0 and n >= 8:
                assert n // S >= 8                    # at least 8 pages a split
            for kvh in range(Hkv):
                edge = 0
                for s in range(S):
                    up, ukvh, us, pb, pe = pl["units"][k]
                    assert (up, ukvh, us) == (p, kvh, s) and pb == edge
                    assert n // S <= pe - pb <= -(-n // S)
                    edge = pe
                    k += 1
                assert edge == n


def test_plan_at_the_long_context_shapes():
    # 64K verify: 256 slots (D=256: one per CU), 4 heads -> a round holds 64
    # splits, all for the one request (floor(4097/8) = 512 does not bind) ->
    # 256 units, one per compute unit.
    pl = oracle.plan(P=1, Hkv=4, D=256, kv_fp8=False, seq_lens=[65552], num_cus=256)
    assert pl["splits"] == [64] and pl["U"] == 256
    # 16K verify: the same 64, and floor(1025/8) = 128 does not bind
    pl = oracle.plan(P=1, Hkv=4, D=256, kv_fp8=False, seq_lens=[16400], num_cus=256)
    assert pl["splits"] == [64]
    # fp8 batch: pages 513/1025/2049/4097, 64 splits.  Pages per split at most
    # x needs S_p >= n_p / x: x = 4097/33 = 124.15 needs 5 + 9 + 17 + 33 = 64
    # splits, and any x below it needs S_4 = 34 and still 5 + 9 + 17, 65 in all.
    # So [5, 9, 17, 33] is the one allocation with the smallest largest split.
    pl = oracle.plan(P=4, Hkv=4, D=256, kv_fp8=True, seq_lens=[8208, 16400, 32784, 65552],
                     num_cus=256)
    assert pl["splits"] == [5, 9, 17, 33] and pl["U"] == 256
    # tiny: 17 pages, one head, 512 slots (D=64) -> the 8-page floor: floor(17/8) = 2
    pl = oracle.plan(P=1, Hkv=1, D=64, kv_fp8=False, seq_lens=[260], num_cus=256)
    assert pl["splits"] == [2] and [u[3:] for u in pl["units"]] == [(0, 8), (8, 17)]
    # draft block at D = 128: a bf16 unit leaves room for a second on its CU, an
    # e4m3 or MXFP4 one does not.  8 requests x 8 heads; with 1000 pages each the
    # 8-page floor never binds, so the budget is spent evenly: 512 slots -> 64
    # splits (8 a request), 256 slots -> 32 (4 a request)
    for kv, S in (("bf16", 8), ("fp8", 4), ("mxfp4", 4)):
        pl = oracle.plan(P=8, Hkv=8, D=128, kv_fp8=kv == "fp8", kv=kv, seq_lens=[16000] * 8,
                         num_cus=256)
        assert pl["splits"] == [S] * 8 and pl["U"] == 64 * S


def test_plan_minimises_the_largest_split_by_brute_force():
    """On tiny problems, the automatic split counts reach the smallest possible
    largest pages-per-split over every allocation that fits the budget (found by
    enumeration), and they spend the budget while any request may still grow."""
    rng = np.random.default_rng(17)
    checked = 0
    for trial in range(300):
        P = int(rng.integers(1, 5))
        Hkv = int(rng.choice([1, 2]))
        cus = int(rng.integers(1, 7))
        seq = [int(x) for x in rng.integers(0, 16 * 70, size=P)]
        pl = oracle.plan(P=P, Hkv=Hkv, D=256, kv_fp8=False, seq_lens=seq, num_cus=cus)
        n = [-(-L // 16) for L in seq]
        cap = [max(1, x // 8) if x > 0 else 1 for x in n]
        rnd = max(1, cus // Hkv)
        budget = rnd if P <= rnd else P + rnd
        best = None
        for S in itertools.product(*[range(1, c + 1) for c in cap]):
            if sum(S) <= budget:
                worst = max(Fraction(a, b) for a, b in zip(n, S))
                best = worst if best is None or worst < best else best
        got = pl["splits"]
        assert all(1 <= g <= c for g, c in zip(got, cap))
        assert max(Fraction(a, b) for a, b in zip(n, got)) == best, (seq, cus, Hkv, got)
        assert sum(got) == min(budget, sum(cap)), (seq, cus, Hkv, got)
        checked += 1
    assert checked == 300


def test_plan_with_more_requests_than_one_round_holds():
    # 2 slots, one head: a round holds 2 splits; 5 requests exceed it, so the
    # budget is 5 + 2 = 7.  Request 0 has 100 pages (up to 12 splits), the others
    # 8 pages (one split each): both extra splits go to request 0 -> [3, 1, 1, 1, 1].
    pl = oracle.plan(P=5, Hkv=1, D=256, kv_fp8=False, seq_lens=[1600, 128, 128, 128, 128],
                     num_cus=2)
    assert pl["splits"] == [3, 1, 1, 1, 1] and pl["U"] == 7
    # equal requests take the extra splits in index order: 4 x 64 pages, 3 slots -> [2, 2, 2, 1]
    pl = oracle.plan(P=4, Hkv=1, D=256, kv_fp8=False, seq_lens=[1024] * 4, num_cus=3)
    assert pl["splits"] == [2, 2, 2, 1]


def test_row_exact_plan_splits_at_fixed_page_multiples():
    # tiny, B = 8: 17 pages -> ceil(17/8) = 3 splits [0,8) [8,16) [16,17)
    pl = oracle.plan(P=1, Hkv=1, D=64, kv_fp8=False, seq_lens=[260], num_cus=256, split_pages=8)
    assert pl["splits"] == [3] and [u[3:] for u in pl["units"]] == [(0, 8), (8, 16), (16, 17)]
    assert pl["combine"] and pl["any_split"]
    # one split only: still finished by the combine (row-exactness across W)
    pl = oracle.plan(P=1, Hkv=1, D=64, kv_fp8=False, seq_lens=[260], num_cus=256,
                     split_pages=64)
    assert pl["splits"] == [1] and pl["combine"] and not pl["any_split"]
    # 64K, B = 65: 4097 pages -> 64 splits of 65 pages except the last (2 pages)
    pl = oracle.plan(P=1, Hkv=4, D=256, kv_fp8=False, seq_lens=[65552], num_cus=256,
                     split_pages=65)
    assert pl["splits"] == [64] and pl["U"] == 256
    assert pl["units"][62][3:] == (4030, 4095) and pl["units"][63][3:] == (4095, 4097)
    # boundaries do not move with the length or with other requests
    a = oracle.plan(P=2, Hkv=2, D=128, kv_fp8=False, seq_lens=[1000, 37], num_cus=8,
                    split_pages=10)
    b = oracle.plan(P=1, Hkv=2, D=128, kv_fp8=False, seq_lens=[990], num_cus=256,
                    split_pages=10)
    ua = [u[3:] for u in a["units"] if u[0] == 0 and u[1] == 0]
    ub = [u[3:] for u in b["units"] if u[1] == 0]
    assert ua[:-1] == ub[:-1] and ua[-1] == (60, 63) and ub[-1] == (60, 62)
    # with a sliding window the first piece starts below the window's first page,
    # on the grid of the pages one arithmetic step groups: L = 1000, W = 4, causal,
    # window 700 -> row 0's first key 996 - 700 + 1 = 297, page 18; B = 20 -> k = 0.
    # bf16 groups page pairs: piece 0 starts at 18; e4m3 and MXFP4 group 8 pages: at 16
    for kv, start in (("bf16", 18), ("fp8", 16), ("mxfp4", 16)):
        pl = oracle.plan(P=1, Hkv=1, D=128, kv_fp8=kv == "fp8", kv=kv, seq_lens=[1000],
                         num_cus=256, split_pages=20, W=4, causal=True, window_left=700)
        assert pl["splits"] == [4] and pl["units"][0][3:] == (start, 20)
        assert [u[3:] for u in pl["units"][1:]] == [(20, 40), (40, 60), (60, 63)]


def test_row_exact_split_partials_combine_to_the_full_result():
    w = tiny(P=1, Hq=4, Hkv=2, D=16, ctx=(200,), W=6, causal=True, seed=18)
    pl = oracle.plan(P=1, Hkv=w.Hkv, D=w.D, kv_fp8=False, seq_lens=w.seq_lens, num_cus=1,
                     split_pages=4)
    o, l = oracle.attention(w)
    parts_o, parts_l = [], []
    for (_, kvh, _, pb, pe) in pl["units"]:
        if kvh == 0:
            po, plse = oracle.attention(w, key_lo=pb * 16, key_hi=pe * 16)
            parts_o.append(po)
            parts_l.append(plse)
    assert len(parts_o) == 4                  # 13 pages -> [0,4) [4,8) [8,12) [12,13)
    co, cl = oracle.lse_combine(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(co, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(cl, l, rtol=1e-13, atol=1e-12)


# ---------------------------------------------------------------- sliding window
def test_window_of_one_key_returns_the_rows_own_value_and_score():
    w = tiny(P=2, Hq=4, Hkv=2, D=16, ctx=(45, 20), W=5, causal=True, seed=81, window_left=1)
    o, l = oracle.attention(w)
    K, V = dense_kv(w)
    Q = q_f64(w)
    for p in range(w.P):
        L = int(w.seq_lens[p])
        for i in range(w.W):
            j = L - w.W + i
            for h in range(w.Hq):
                np.testing.assert_array_equal(o[p, i, h], V[p, h // w.G, j])
                assert l[p, i, h] == pytest.approx(w.scale * Q[p, i, h] @ K[p, h // w.G, j],
                                                   abs=1e-12)


def test_window_covering_every_key_changes_nothing():
    w = tiny(P=2, Hq=4, Hkv=2, D=16, ctx=(45, 20), W=5, causal=True, seed=82)
    o, l = oracle.attention(w)
    o2, l2 = oracle.attention(dataclasses.replace(w, window_left=int(w.seq_lens.max())))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_plan_skips_the_pages_before_the_window():
    # 64K verify, window 4096: row 0's window starts at 65536 - 4096 + 1 = 61441
    # -> page 3840; 4097 - 3840 = 257 pages streamed per head; 4*257 = 1028
    # page-heads on 256 slots -> S = min(floor(257*256/1028), floor(257/8)) = 32
    pl = oracle.plan(P=1, Hkv=4, D=256, kv_fp8=False, seq_lens=[65552], num_cus=256, W=16,
                     causal=True, window_left=4096)
    assert pl["splits"] == [32] and pl["U"] == 128
    # split 31: 3840 + floor(31*257/32) = 3840 + 248
    assert pl["units"][0][3:] == (3840, 3848) and pl["units"][31][3:] == (4088, 4097)
    # row-exact pieces stay on the absolute grid: B = 100 -> pieces from 3800
    pl = oracle.plan(P=1, Hkv=4, D=256, kv_fp8=False, seq_lens=[65552], num_cus=256, W=16,
                     causal=True, window_left=4096, split_pages=100)
    assert pl["splits"] == [41 - 38]
    assert [u[3:] for u in pl["units"][:3]] == [(3840, 3900), (3900, 4000), (4000, 4097)]
