"""Paged KV append: the oracle's e4m3 encoder and append pinned on the CPU,
then the HIP kernel (through the C ABI) against the oracle, bit for bit.

The e4m3 encoder is pinned against torch's own float8_e4m3fn cast (a library
routine with the same round-to-nearest-even definition), against every finite
code's exact value, and against the midpoints between codes (ties to even).
The MXFP4 quantizer (OCP Microscaling Formats v1.0: E2M1 elements, one E8M0
scale per 32 elements) is pinned by the E2M1 value table, midpoints and
saturation, worked blocks derived by hand from the format's rules, and the
error bound and block-maximum range that those rules imply.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload
from workloads.synth import quantize_e4m3, to_bf16_bits


# ---------------------------------------------------------------- CPU: oracle pins
def test_e4m3_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.decode_e4m3(codes).astype(np.float32)
    vals[codes == 0x80] = -0.0
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_encoder_sends_midpoints_to_the_even_code():
    pos = np.array([c for c in range(0x7F)], dtype=np.uint8)
    v = oracle.decode_e4m3(pos)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)   # exact in fp32
    got = oracle.e4m3_encode(mids)
    want = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    np.testing.assert_array_equal(got, want)
    # a hair above / below a midpoint goes to the nearer code
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    np.testing.assert_array_equal(oracle.e4m3_encode(up), pos[1:])
    np.testing.assert_array_equal(oracle.e4m3_encode(dn), pos[:-1])


def test_e4m3_encoder_agrees_with_torch_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 60000), rng.normal(0, 1, 60000),
                        rng.normal(0, 2 ** -8, 60000)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(x), want)


def test_oracle_append_bf16_writes_exactly_the_window_slots():
    w = make_workload(None, P=2, Hq=8, Hkv=2, D=64, ctx=(40, 5), W=4, causal=True, kv="bf16",
                      placement="permuted", pool_pages=12, seed=71, poison=False)
    rng = np.random.default_rng(3)
    kn = to_bf16_bits(rng.normal(size=(2, 4, 2, 64)).astype(np.float32))
    vn = to_bf16_bits(rng.normal(size=(2, 4, 2, 64)).astype(np.float32))
    kp, vp, _, _ = oracle.kv_append(P=2, W=4, Hkv=2, D=64, kv="bf16", k_new_bits=kn,
                                    v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                    k_scale=None, v_scale=None, block_table=w.block_table,
                                    seq_lens=w.seq_lens, num_pages=w.num_pages)
    touched = np.zeros(kp.shape[:3], bool)
    for p in range(2):
        for i in range(4):
            pos = int(w.seq_lens[p]) - 4 + i
            pg, sl = int(w.block_table[p, pos // 16]), pos % 16
            np.testing.assert_array_equal(kp[pg, :, sl, :], kn[p, i])
            np.testing.assert_array_equal(vp[pg, :, :, sl], vn[p, i])
            touched[pg, :, sl] = True
    np.testing.assert_array_equal(kp[~touched], w.k_pool[~touched])
    np.testing.assert_array_equal(vp.transpose(0, 1, 3, 2)[~touched],
                                  w.v_pool.transpose(0, 1, 3, 2)[~touched])


def test_oracle_fp8_row_quantizer_matches_the_input_generator():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 3, size=(64, 256)).astype(np.float32)
    x = (to_bf16_bits(x).astype(np.uint32) << 16).view(np.float32)   # bf16-exact rows
    x[5] = 0.0                                                         # all-zero row
    codes, scales = quantize_e4m3(x)
    for r in range(64):
        c, s = oracle.e4m3_row_quantize(x[r])
        np.testing.assert_array_equal(c, codes[r])
        assert np.float32(s) == scales[r]
    assert scales[5] == 1.0


# MXFP4 (OCP Microscaling Formats v1.0): E2M1 magnitudes of codes 0..7
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_encoder_round_trips_every_code():
    vals = np.array(E2M1 + [-x for x in E2M1])
    vals[8] = -0.0
    np.testing.assert_array_equal(oracle.e2m1_encode(vals), np.arange(16, dtype=np.uint8))


def test_e2m1_encoder_sends_midpoints_to_the_even_code_and_saturates():
    # midpoints of neighbouring values and the code that holds them
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]
    np.testing.assert_array_equal(oracle.e2m1_encode(mids), want)
    np.testing.assert_array_equal(oracle.e2m1_encode([-x for x in mids]),
                                  [8 | c for c in want])
    eps = 1e-9
    np.testing.assert_array_equal(oracle.e2m1_encode([m + eps for m in mids]), [1, 2, 3, 4, 5, 6, 7])
    np.testing.assert_array_equal(oracle.e2m1_encode([m - eps for m in mids]), [0, 1, 2, 3, 4, 5, 6])
    # past the largest value (6) everything below 8 saturates to it
    np.testing.assert_array_equal(oracle.e2m1_encode([6.5, 7.0, 7.99, -7.5]), [7, 7, 7, 15])


def _blk(vals):
    x = np.zeros(32)
    x[:len(vals)] = vals
    return x


def test_mxfp4_block_quantizer_worked_examples():
    # amax 5 -> floor(log2 5) = 2 -> X = 0, scale byte 127; 5 ties to 4 (even)
    c, s = oracle.mxfp4_row_quantize(_blk([5.0, 1.0, 0.3, -2.5, -0.0]))
    assert list(s) == [127]
    assert list(c[:6]) == [6, 2, 1, 8 | 4, 8, 0]
    # amax 0.75 -> floor(log2 0.75) = -1 -> X = -3 (byte 124), 0.75 * 8 = 6
    c, s = oracle.mxfp4_row_quantize(_blk([0.75, -0.1, 0.0625]))
    assert list(s) == [124]
    assert list(c[:3]) == [7, 8 | 2, 1]     # -0.8 is nearer -1.0 than -0.5; 0.5 exact
    # amax exactly 4 -> X = 0; amax just under 8 saturates to 6
    c, s = oracle.mxfp4_row_quantize(_blk([4.0, 7.96875]))
    assert list(s) == [127] and list(c[:2]) == [6, 7]
    # all-zero block -> scale byte 0, codes 0 (negative zero keeps its sign)
    c, s = oracle.mxfp4_row_quantize(_blk([0.0, -0.0]))
    assert list(s) == [0] and list(c[:3]) == [0, 8, 0]
    # tiny block: X = floor(log2 2^-130) - 2 = -132 clamps to -127
    c, s = oracle.mxfp4_row_quantize(_blk([2.0 ** -130, 2.0 ** -126]))
    assert list(s) == [0] and list(c[:2]) == [0, 4]   # y = 2^-3 -> 0 and y = 2 -> 2.0
    # two blocks of one row get their own scales
    c, s = oracle.mxfp4_row_quantize(np.concatenate([_blk([1.0]), _blk([96.0])]))
    assert list(s) == [127 - 2, 127 + 4] and c[0] == 6 and c[32] == 7   # y = 4 and y = 6


def test_mxfp4_block_quantizer_error_bound_and_block_maximum():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, size=(500, 256)) * rng.choice([1e-3, 1.0, 40.0], size=(500, 1))
    x = (to_bf16_bits(x.astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    table = np.array(E2M1 + [-v for v in E2M1])
    for row in x.astype(np.float64):
        c, s = oracle.mxfp4_row_quantize(row)
        scale = np.repeat(2.0 ** (s.astype(np.int64) - 127), 32)
        y = row / scale
        deq = table[c]
        # the largest |y| of each block is in [4, 8)
        amax = np.abs(y).reshape(-1, 32).max(axis=1)
        assert ((amax >= 4) & (amax < 8)).all()
        # error: at most half the spacing of the grid around |y| (0.5 below 2,
        # 1 up to 4, 2 up to 6), or the distance to 6 when saturated
        a = np.abs(y)
        half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
        err = np.abs(deq - y)
        assert (err <= np.where(a > 6, a - 6, half)).all()
        assert (np.sign(deq) * np.sign(y) >= 0).all()


def test_oracle_append_mxfp4_writes_only_the_window_nibbles():
    w = make_workload(None, P=2, Hq=8, Hkv=2, D=64, ctx=(41, 6), W=5, causal=True, kv="mxfp4",
                      placement="permuted", pool_pages=12, seed=75, poison=True)
    rng = np.random.default_rng(5)
    kn = to_bf16_bits(rng.normal(size=(2, 5, 2, 64)).astype(np.float32))
    vn = to_bf16_bits(rng.normal(size=(2, 5, 2, 64)).astype(np.float32))
    kp, vp, ks, vs = oracle.kv_append(P=2, W=5, Hkv=2, D=64, kv="mxfp4", k_new_bits=kn,
                                      v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                      k_scale=w.k_scale, v_scale=w.v_scale,
                                      block_table=w.block_table, seq_lens=w.seq_lens,
                                      num_pages=w.num_pages)
    table = np.array(E2M1 + [-v for v in E2M1])
    touched = np.zeros((w.num_pages, 2, 16), bool)
    for p in range(2):
        for i in range(5):
            pos = int(w.seq_lens[p]) - 5 + i
            pg, sl = int(w.block_table[p, pos // 16]), pos % 16
            touched[pg, :, sl] = True
            for h in range(2):
                kx = (kn[p, i, h].astype(np.uint32) << 16).view(np.float32)
                vx = (vn[p, i, h].astype(np.uint32) << 16).view(np.float32)
                kc, ksc = oracle.mxfp4_row_quantize(kx)
                vc, vsc = oracle.mxfp4_row_quantize(vx)
                kcodes = np.stack([kp[pg, h, sl] & 15, kp[pg, h, sl] >> 4], -1).reshape(-1)
                vcodes = (vp[pg, h, :, sl // 2] >> (4 * (sl % 2))) & 15
                np.testing.assert_array_equal(kcodes, kc)
                np.testing.assert_array_equal(vcodes, vc)
                np.testing.assert_array_equal(ks[pg, h, sl], ksc)
                np.testing.assert_array_equal(vs[pg, h, :, sl], vsc)
                # the stored values are the quantised row
                deq = table[kcodes] * np.repeat(2.0 ** (ksc.astype(int) - 127), 32)
                assert np.abs(deq - kx).max() <= np.abs(kx).max() / 4 + 1e-30
    # everything else is untouched: K rows and scales of other slots, and the
    # other token's nibble of every value byte
    np.testing.assert_array_equal(kp[~touched], w.k_pool[~touched])
    np.testing.assert_array_equal(ks[~touched], w.k_scale[~touched])
    np.testing.assert_array_equal(vs.transpose(0, 1, 3, 2)[~touched],
                                  w.v_scale.transpose(0, 1, 3, 2)[~touched])
    for sl in range(16):
        keep = ~touched[:, :, sl]                                       # [pages][Hkv]
        old = (w.v_pool[:, :, :, sl // 2] >> (4 * (sl % 2))) & 15
        new = (vp[:, :, :, sl // 2] >> (4 * (sl % 2))) & 15
        np.testing.assert_array_equal(new[keep], old[keep])


# ---------------------------------------------------------------- GPU: kernel parity
def host_bits(t):
    """Device pool tensor -> host array of its raw bits (uint16 bf16 or uint8 codes)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint8)


def _append_case(kv, D=128, W=16, ctx=(700, 45, 0), seed=72, Hq=8):
    w = make_workload(None, P=len(ctx), Hq=Hq, Hkv=4, D=D, ctx=ctx, W=W, causal=True, kv=kv,
                      placement="permuted", pool_pages=sum(-(-(c + W) // 16) for c in ctx) + 6,
                      seed=seed, seq_lens=tuple(c + W if c > 0 else 0 for c in ctx))
    rng = np.random.default_rng(seed)
    shape = (w.P, W, w.Hkv, D)
    kn = to_bf16_bits(rng.normal(0, 1, size=shape).astype(np.float32))   # same draw as the
    vn = to_bf16_bits(rng.normal(0, 1, size=shape).astype(np.float32))   # workloads' K and V
    kn[0, 3, 1] = 0                              # an all-zero row: scale 1
    if kv == "mxfp4":
        # blocks the MX exponent must clamp: bf16 denormals and the smallest normals
        kn[0, 4, 2, :32] = np.arange(1, 33, dtype=np.uint16)                  # 2^-133 ..
        vn[0, 4, 2, 32:64] = (0x0080 + np.arange(32)).astype(np.uint16)       # 2^-126 ..
        vn[0, 5, 3, :] = 0x8000                                                # all -0.0
    return w, kn, vn


@pytest.mark.gpu
@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_append_kernel_matches_oracle_bitwise(kv, D):
    from speculative_decode_verify_sweep_amd import device as dv
    import speculative_decode_verify_sweep_amd as sw
    if kv == "mxfp4" and D == 64:
        pytest.skip("MXFP4 pools serve head_dim 128 and 256")
    w, kn, vn = _append_case(kv, D=D)
    print(f"[case] append {kv} D={D}", flush=True)
    d = dv.upload(w)
    plan = dv.plan_for(w)
    kt = torch.from_numpy(kn.view(np.int16)).cuda()
    vt = torch.from_numpy(vn.view(np.int16)).cuda()
    sw.small_w_kv_append(plan, kt, vt, d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                         d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    scaled = kv != "bf16"
    kp, vp, ks, vs = oracle.kv_append(P=w.P, W=w.W, Hkv=w.Hkv, D=D, kv=kv, k_new_bits=kn,
                                      v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                      k_scale=w.k_scale if scaled else None,
                                      v_scale=w.v_scale if scaled else None,
                                      block_table=w.block_table, seq_lens=w.seq_lens,
                                      num_pages=w.num_pages)
    np.testing.assert_array_equal(host_bits(d["k_pool"]), kp)
    np.testing.assert_array_equal(host_bits(d["v_pool"]), vp)
    if scaled:
        np.testing.assert_array_equal(d["k_scale"].cpu().numpy(), ks)
        np.testing.assert_array_equal(d["v_scale"].cpu().numpy(), vs)


@pytest.mark.gpu
def test_append_mxfp4_rounds_every_tie_to_even_and_saturates():
    """Blocks holding 4.0 have X = 0, so the codes are the E2M1 rounding of the
    bf16 inputs themselves: every value, every midpoint and their bf16
    neighbours, and values past 6 up to just under 8 (saturation)."""
    from speculative_decode_verify_sweep_amd import device as dv
    import speculative_decode_verify_sweep_amd as sw
    grid = np.array(E2M1, np.float32)
    mids = (grid[:-1] + grid[1:]) / 2
    cand = np.concatenate([grid, mids, [6.5, 7.0, 7.5, 7.96875]]).astype(np.float32)
    bits = to_bf16_bits(np.concatenate([cand, -cand]))
    near = np.concatenate([bits, bits + 1, bits - 1]).astype(np.uint16)
    vals = (near.astype(np.uint32) << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 8)]
    per_block = 31
    nblk = -(-vals.size // per_block)
    D, W = 256, 16
    blocks = np.zeros((nblk, 32), np.float32)
    blocks[:, 0] = 4.0                                           # amax in [4, 8): X = 0
    flat = np.zeros(nblk * per_block, np.float32)
    flat[:vals.size] = vals
    blocks[:, 1:] = flat.reshape(nblk, per_block)
    rows = -(-nblk // (D // 32))
    assert rows <= W * 4
    full = np.zeros((W * 4 * (D // 32), 32), np.float32)
    full[:, 0] = 4.0
    full[:nblk] = blocks
    full = full.reshape(1, W, 4, D)
    w = make_workload(None, P=1, Hq=4, Hkv=4, D=D, ctx=(48,), W=W, causal=True, kv="mxfp4",
                      placement="in_order", pool_pages=5, seed=76)
    kn = to_bf16_bits(full)
    d = dv.upload(w)
    plan = dv.plan_for(w)
    kt = torch.from_numpy(kn.view(np.int16)).cuda()
    print("[case] append MXFP4 ties", flush=True)
    sw.small_w_kv_append(plan, kt, kt, d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                         d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    kp, vp, ks, vs = oracle.kv_append(P=1, W=W, Hkv=4, D=D, kv="mxfp4", k_new_bits=kn,
                                      v_new_bits=kn, k_pool=w.k_pool, v_pool=w.v_pool,
                                      k_scale=w.k_scale, v_scale=w.v_scale,
                                      block_table=w.block_table, seq_lens=w.seq_lens,
                                      num_pages=w.num_pages)
    assert np.all(ks[3] == 127)                                  # X = 0 everywhere
    np.testing.assert_array_equal(host_bits(d["k_pool"]), kp)
    np.testing.assert_array_equal(host_bits(d["v_pool"]), vp)
    np.testing.assert_array_equal(d["k_scale"].cpu().numpy(), ks)
    np.testing.assert_array_equal(d["v_scale"].cpu().numpy(), vs)


@pytest.mark.gpu
def test_append_kernel_rounds_every_tie_to_even():
    """Rows holding 448 have scale exactly 1, so the codes are the e4m3 rounding
    of the bf16 inputs themselves: every code value, every midpoint and their
    bf16 neighbours go through the kernel's conversion."""
    from speculative_decode_verify_sweep_amd import device as dv
    import speculative_decode_verify_sweep_amd as sw
    pos = np.arange(0x7F, dtype=np.uint8)
    v = oracle.decode_e4m3(pos)
    mids = (v[:-1] + v[1:]) / 2
    cand = np.concatenate([v, mids, -v, -mids]).astype(np.float32)
    bits = to_bf16_bits(cand)
    near = np.concatenate([bits, bits + 1, bits - 1]).astype(np.uint16)
    vals = (near.astype(np.uint32) << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    D, W = 256, 16
    per_row = D - 1
    rows = -(-vals.size // per_row)
    assert rows <= W * 4
    data = np.zeros((rows * per_row,), np.float32)
    data[:vals.size] = vals
    data = data.reshape(rows, per_row)
    data = np.concatenate([np.full((rows, 1), 448, np.float32), data], axis=1)   # amax = 448
    full = np.zeros((1, W, 4, D), np.float32)
    full.reshape(W * 4, D)[:rows] = data
    full.reshape(W * 4, D)[rows:, 0] = 448
    w = make_workload(None, P=1, Hq=4, Hkv=4, D=D, ctx=(48,), W=W, causal=True, kv="fp8",
                      placement="in_order", pool_pages=5, seed=73)
    kn = to_bf16_bits(full)
    d = dv.upload(w)
    plan = dv.plan_for(w)
    kt = torch.from_numpy(kn.view(np.int16)).cuda()
    print("[case] append e4m3 ties", flush=True)
    sw.small_w_kv_append(plan, kt, kt, d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                         d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    assert int(w.block_table[0, 3]) == 3 and np.all(d["k_scale"].cpu().numpy()[3] == 1.0)
    kp, _, _, _ = oracle.kv_append(P=1, W=W, Hkv=4, D=D, kv="fp8", k_new_bits=kn,
                                   v_new_bits=kn, k_pool=w.k_pool, v_pool=w.v_pool,
                                   k_scale=w.k_scale, v_scale=w.v_scale,
                                   block_table=w.block_table, seq_lens=w.seq_lens,
                                   num_pages=w.num_pages)
    np.testing.assert_array_equal(host_bits(d["k_pool"]), kp)


@pytest.mark.gpu
@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_append_then_verify_matches_oracle(kv):
    """The step pair a verify does: append the window's K/V, then attend."""
    from speculative_decode_verify_sweep_amd import device as dv
    import speculative_decode_verify_sweep_amd as sw
    from test_gpu_parity import check
    w, kn, vn = _append_case(kv, D=256, W=16, ctx=(3000, 200, 0), seed=74, Hq=24)
    scaled = kv != "bf16"
    d = dv.upload(w)
    plan = dv.plan_for(w)
    ws = dv.workspace_for(plan)
    print(f"[case] append + verify {kv}", flush=True)
    sw.small_w_kv_append(plan, torch.from_numpy(kn.view(np.int16)).cuda(),
                         torch.from_numpy(vn.view(np.int16)).cuda(), d["k_pool"], d["v_pool"],
                         d["k_scale"], d["v_scale"], d["block_table"], d["seq_lens"])
    dv.run(plan, d, ws)
    torch.cuda.synchronize()
    kp, vp, ks, vs = oracle.kv_append(P=w.P, W=w.W, Hkv=w.Hkv, D=w.D, kv=kv, k_new_bits=kn,
                                      v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                      k_scale=w.k_scale if scaled else None,
                                      v_scale=w.v_scale if scaled else None,
                                      block_table=w.block_table, seq_lens=w.seq_lens,
                                      num_pages=w.num_pages)
    w2 = dataclasses.replace(w, k_pool=kp, v_pool=vp, k_scale=ks if scaled else w.k_scale,
                             v_scale=vs if scaled else w.v_scale)
    o = d["out"].float().cpu().numpy().astype(np.float64)
    l = d["lse"].cpu().numpy().astype(np.float64)
    check(w2, o, l, *oracle.attention(w2))


@pytest.mark.gpu
@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_append_in_a_replayed_graph_matches_oracle_bitwise(kv):
    """The append captured in a HIP graph, as a caller capturing a decode step
    does (bench.py times it that way), replayed three times.  Before each replay
    the pools go back to their state before the append and eager work runs, so a
    replay that wrote nothing, or wrote stale values, would fail."""
    from speculative_decode_verify_sweep_amd import device as dv
    import speculative_decode_verify_sweep_amd as sw
    w, kn, vn = _append_case(kv, D=256, seed=75)
    d = dv.upload(w)
    plan = dv.plan_for(w)
    kt = torch.from_numpy(kn.view(np.int16)).cuda()
    vt = torch.from_numpy(vn.view(np.int16)).cuda()
    names = [n for n in ("k_pool", "v_pool", "k_scale", "v_scale") if d.get(n) is not None]
    fresh = {n: d[n].clone() for n in names}

    def call():
        sw.small_w_kv_append(plan, kt, vt, d["k_pool"], d["v_pool"], d["k_scale"],
                             d["v_scale"], d["block_table"], d["seq_lens"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    scaled = kv != "bf16"
    kp, vp, ks, vs = oracle.kv_append(P=w.P, W=w.W, Hkv=w.Hkv, D=w.D, kv=kv, k_new_bits=kn,
                                      v_new_bits=vn, k_pool=w.k_pool, v_pool=w.v_pool,
                                      k_scale=w.k_scale if scaled else None,
                                      v_scale=w.v_scale if scaled else None,
                                      block_table=w.block_table, seq_lens=w.seq_lens,
                                      num_pages=w.num_pages)
    assert not np.array_equal(host_bits(fresh["k_pool"]), kp)   # the append changes the pool
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for n in names:
            d[n].copy_(fresh[n])
        scratch.mul_(0.5).add_(1.0)             # eager work between the replays
        torch.cuda.synchronize()
        print(f"[case] append {kv} graph replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(d["k_pool"]), kp)
        np.testing.assert_array_equal(host_bits(d["v_pool"]), vp)
        if scaled:
            np.testing.assert_array_equal(d["k_scale"].cpu().numpy(), ks)
            np.testing.assert_array_equal(d["v_scale"].cpu().numpy(), vs)
