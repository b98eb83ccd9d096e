"""Host-side checks of the C-ABI library: no GPU needed.

* libsmallw.so loads and exports every function include/smallw.h declares;
* small_w_attention_plan rejects each malformed or unsupported problem with
  the documented status code (all checks run on the host);
* the integer plan export is bit-exact against the oracle's restatement of
  the written split specification, over a seeded sweep of problems;
* small_w_attention_run rejects null pointers and short or misaligned
  workspaces before touching the device;
* the header serves a C11 caller: tests/c_abi_host.c builds with every
  warning an error, links against the library and passes its host checks.
"""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import speculative_decode_verify_sweep_amd as sw
from speculative_decode_verify_sweep_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smallw.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(small_w_\w+)\s*\(", text)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_serves_a_c11_caller(tmp_path):
    exe = str(tmp_path / "c_abi_host")
    pkg = os.path.dirname(B.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_host.c"),
           "-o", exe, "-L", pkg, "-lsmallw", f"-Wl,-rpath,{pkg}"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.stdout, run.stderr)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "small_w_attention_plan" in names and "small_w_attention_run" in names
    assert "small_w_kv_append" in names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def base_problem(**kw):
    d = dict(num_reqs=1, window=4, num_q_heads=4, num_kv_heads=1, head_dim=64, num_pages=32,
             max_pages_per_req=32, causal=1, kv_dtype=0, scale=0.0, num_cus=256,
             force_splits=0, split_pages=0, window_left=0)
    d.update(kw)
    return B.make_problem(**d)


@pytest.mark.parametrize("field,value,code", [
    ("num_reqs", 0, B.SMALLW_EINVAL),
    ("num_reqs", 257, B.SMALLW_EUNSUPPORTED),
    ("window", 0, B.SMALLW_EINVAL),
    ("window", 17, B.SMALLW_EUNSUPPORTED),
    ("num_q_heads", 6, B.SMALLW_EINVAL),            # 6 % 4 kv heads != 0 (set below)
    ("num_kv_heads", 0, B.SMALLW_EINVAL),
    ("head_dim", 96, B.SMALLW_EUNSUPPORTED),
    ("head_dim", 0, B.SMALLW_EINVAL),
    ("page_size", 32, B.SMALLW_EUNSUPPORTED),
    ("num_pages", 0, B.SMALLW_EINVAL),
    ("max_pages_per_req", 0, B.SMALLW_EINVAL),
    ("causal", 2, B.SMALLW_EINVAL),
    ("kv_dtype", 7, B.SMALLW_EINVAL),
    ("scale", float("nan"), B.SMALLW_EINVAL),
    ("num_cus", -1, B.SMALLW_EINVAL),
    ("force_splits", -2, B.SMALLW_EINVAL),
    ("split_pages", -1, B.SMALLW_EINVAL),
    ("window_left", -5, B.SMALLW_EINVAL),
    ("v_layout", 2, B.SMALLW_EINVAL),
])
def test_plan_rejects_bad_problems(field, value, code):
    kw = {field: value}
    if field == "num_q_heads":
        kw["num_kv_heads"] = 4
    pr = base_problem(**kw)
    with pytest.raises(B.SmallwError) as e:
        sw.small_w_attention_plan(pr, [260])
    assert e.value.code == code


def test_plan_rejects_forced_and_row_exact_splits_together():
    with pytest.raises(B.SmallwError) as e:
        sw.small_w_attention_plan(base_problem(force_splits=2, split_pages=4), [260])
    assert e.value.code == B.SMALLW_EINVAL


def test_plan_rejects_bad_lengths_and_too_many_rows():
    with pytest.raises(B.SmallwError) as e:      # causal window longer than the request
        sw.small_w_attention_plan(base_problem(), [3])
    assert e.value.code == B.SMALLW_EINVAL
    with pytest.raises(B.SmallwError) as e:      # longer than the block-table row
        sw.small_w_attention_plan(base_problem(max_pages_per_req=2), [33])
    assert e.value.code == B.SMALLW_EINVAL
    with pytest.raises(B.SmallwError) as e:
        sw.small_w_attention_plan(base_problem(), [-1])
    assert e.value.code == B.SMALLW_EINVAL
    with pytest.raises(B.SmallwError) as e:      # W * G = 16 * 9 = 144 rows > 128
        sw.small_w_attention_plan(base_problem(window=16, num_q_heads=9, num_kv_heads=1), [260])
    assert e.value.code == B.SMALLW_EUNSUPPORTED
    # empty request is a valid idle slot, W * G = 128 is the limit
    sw.small_w_attention_plan(base_problem(num_reqs=2, window=16, num_q_heads=8), [0, 16])


def test_plan_export_matches_oracle_plan_bit_exactly():
    rng = np.random.default_rng(2024)
    for trial in range(300):
        P = int(rng.integers(1, 12))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 6]))
        W = int(rng.integers(1, 17))
        if W * G > 128:
            W = 128 // G
        D = int(rng.choice([64, 128, 256]))
        fp8 = int(rng.integers(0, 3))       # storage format code: bf16, e4m3, MXFP4
        if fp8 == 2 and D == 64:
            fp8 = 0                          # MXFP4 serves D = 128 and 256
        causal = int(rng.integers(0, 2))
        force = int(rng.choice([0, 0, 0, 1, 2, 5, 64]))
        spg = int(rng.choice([0, 0, 0, 1, 7, 64])) if force == 0 else 0
        win = int(rng.choice([0, 0, 0, 1, 37, 1000]))
        cus = int(rng.choice([1, 8, 80, 256, 304]))
        hi = int(rng.choice([40, 3000, 70000]))
        seq = rng.integers(W if causal else 0, hi, size=P).astype(np.int32)
        if rng.integers(0, 4) == 0:
            seq[rng.integers(0, P)] = 0
        maxp = int(-(-int(seq.max()) // 16)) + int(rng.integers(0, 3)) or 1
        pr = B.make_problem(num_reqs=P, window=W, num_q_heads=Hkv * G, num_kv_heads=Hkv,
                            head_dim=D, num_pages=100000, max_pages_per_req=maxp, causal=causal,
                            kv_dtype=fp8, num_cus=cus, force_splits=force, split_pages=spg,
                            window_left=win)
        plan = sw.small_w_attention_plan(pr, seq)
        mine = sw.small_w_attention_plan_export(plan)
        pl = oracle.plan(P=P, Hkv=Hkv, D=D, kv_fp8=fp8 == 1, seq_lens=seq, num_cus=cus,
                         kv=("bf16", "fp8", "mxfp4")[fp8],
                         force_splits=force, split_pages=spg, W=W, causal=bool(causal),
                         window_left=win)
        np.testing.assert_array_equal(mine, oracle.plan_export(pl, R=W * G))
        biggest = max(pe - pb for (_, _, _, pb, pe) in pl["units"])
        assert sw.small_w_attention_plan_max_unit_pages(plan) == biggest
        # workspace: fp16 partial outputs in whole 16-row tiles and a {lse, scale}
        # pair per unit and row, each region 256-byte aligned
        U, R = pl["U"], W * G
        a256 = lambda x: (x + 255) // 256 * 256
        want = a256(U * (-(-R // 16) * 16) * D * 2) + a256(U * R * 8) if pl["combine"] else 0
        assert sw.small_w_attention_workspace_bytes(plan) == want


def test_plan_export_matches_oracle_on_large_batches():
    """Batches of 64..256 requests (the request limit), with repeated lengths so
    the apportionment meets many equal pages-per-split ties, one round or more."""
    rng = np.random.default_rng(2025)
    for trial in range(24):
        P = int(rng.choice([64, 200, 256]))
        Hkv = int(rng.choice([1, 2, 8]))
        D = int(rng.choice([128, 256]))
        cus = int(rng.choice([8, 80, 256]))
        seq = rng.choice([0, 16, 160, 1600, 16000, int(rng.integers(1, 30000))], size=P)
        seq = seq.astype(np.int32)
        maxp = int(-(-int(seq.max()) // 16)) or 1
        pr = B.make_problem(num_reqs=P, window=1, num_q_heads=Hkv, num_kv_heads=Hkv,
                            head_dim=D, num_pages=100000, max_pages_per_req=maxp, causal=0,
                            kv_dtype=0, num_cus=cus)
        plan = sw.small_w_attention_plan(pr, seq)
        pl = oracle.plan(P=P, Hkv=Hkv, D=D, kv_fp8=False, seq_lens=seq, num_cus=cus, W=1,
                         causal=False)
        np.testing.assert_array_equal(sw.small_w_attention_plan_export(plan),
                                      oracle.plan_export(pl, R=1))


def test_run_rejects_null_pointers_and_bad_workspace_before_any_launch():
    pr = base_problem(force_splits=3)
    plan = sw.small_w_attention_plan(pr, [260])
    need = sw.small_w_attention_workspace_bytes(plan)
    assert need > 0
    lib = B.lib()
    fake = 1 << 40  # never dereferenced: every check below fails before a launch
    args = [plan.handle, fake, fake, fake, None, None, fake, fake, fake, fake, fake, need, None]
    for k in (1, 2, 3, 6, 7, 8, 9):
        bad = list(args)
        bad[k] = None
        assert lib.small_w_attention_run(*bad) == B.SMALLW_EINVAL
    short = list(args)
    short[11] = need - 1
    assert lib.small_w_attention_run(*short) == B.SMALLW_EWORKSPACE
    noptr = list(args)
    noptr[10] = None
    assert lib.small_w_attention_run(*noptr) == B.SMALLW_EWORKSPACE
    misaligned = list(args)
    misaligned[10] = fake + 16
    assert lib.small_w_attention_run(*misaligned) == B.SMALLW_EWORKSPACE
    assert lib.small_w_attention_run(None, *args[1:]) == B.SMALLW_EINVAL


def test_kv_append_rejects_null_pointers_before_any_launch():
    lib = B.lib()
    plan = sw.small_w_attention_plan(base_problem(), [260])
    fake = 1 << 40  # never dereferenced
    args = [plan.handle, fake, fake, fake, fake, None, None, fake, fake, None]
    for k in (1, 2, 3, 4, 7, 8):
        bad = list(args)
        bad[k] = None
        assert lib.small_w_kv_append(*bad) == B.SMALLW_EINVAL
    assert lib.small_w_kv_append(None, *args[1:]) == B.SMALLW_EINVAL
    fp8 = sw.small_w_attention_plan(base_problem(kv_dtype=1), [260])
    assert lib.small_w_kv_append(fp8.handle, *args[1:]) == B.SMALLW_EINVAL   # scales missing


@pytest.mark.parametrize("kv", [B.SMALLW_KV_FP8_E4M3, B.SMALLW_KV_MXFP4])
def test_scaled_formats_require_scales(kv):
    plan = sw.small_w_attention_plan(base_problem(kv_dtype=kv, head_dim=128), [260])
    fake = 1 << 40
    rc = B.lib().small_w_attention_run(plan.handle, fake, fake, fake, None, None, fake, fake,
                                       fake, fake, None, 0, None)
    assert rc == B.SMALLW_EINVAL


def test_token_major_values_are_a_bf16_layout():
    for kv in (B.SMALLW_KV_FP8_E4M3, B.SMALLW_KV_MXFP4):
        with pytest.raises(B.SmallwError) as e:
            sw.small_w_attention_plan(base_problem(kv_dtype=kv, head_dim=128, v_layout=1), [260])
        assert e.value.code == B.SMALLW_EUNSUPPORTED
    sw.small_w_attention_plan(base_problem(v_layout=1), [260])


def test_mxfp4_needs_head_dim_128_or_256():
    with pytest.raises(B.SmallwError) as e:
        sw.small_w_attention_plan(base_problem(kv_dtype=B.SMALLW_KV_MXFP4, head_dim=64), [260])
    assert e.value.code == B.SMALLW_EUNSUPPORTED
    for D in (128, 256):
        sw.small_w_attention_plan(base_problem(kv_dtype=B.SMALLW_KV_MXFP4, head_dim=D), [260])


def test_strerror_names_every_code():
    for code in (0, -1, -2, -3, -4, -5):
        assert len(sw.small_w_attention_strerror(code)) >= 2
    assert "unknown" in sw.small_w_attention_strerror(-99)


def test_package_has_no_fallback_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(OSError):
        B.lib()


def _cpu_call_tensors(pr, kv="bf16"):
    """CPU stand-ins with the shapes and dtypes a call with problem pr takes."""
    import torch
    P, W, Hq, Hkv, D, n = (pr.num_reqs, pr.window, pr.num_q_heads, pr.num_kv_heads,
                           pr.head_dim, pr.num_pages)
    if kv == "bf16":
        pool = torch.zeros((n, Hkv, 16, D), dtype=torch.bfloat16)
        sc = None
    elif kv == "fp8":
        pool = torch.zeros((n, Hkv, 16, D), dtype=torch.uint8)
        sc = torch.zeros((n, Hkv, 16), dtype=torch.float32)
    else:
        pool = torch.zeros((n, Hkv, 16, D // 2), dtype=torch.uint8)
        sc = torch.zeros((n, Hkv, 16, D // 32), dtype=torch.uint8)
    return dict(q=torch.zeros((P, W, Hq, D), dtype=torch.bfloat16), k_pool=pool,
                v_pool=pool.clone(), k_scale=sc, v_scale=None if sc is None else sc.clone(),
                block_table=torch.zeros((P, pr.max_pages_per_req), dtype=torch.int32),
                seq_lens=torch.zeros((P,), dtype=torch.int32),
                out=torch.zeros((P, W, Hq, D), dtype=torch.bfloat16),
                lse=torch.zeros((P, W, Hq), dtype=torch.float32))


@pytest.mark.parametrize("kv,code", [("bf16", 0), ("fp8", 1), ("mxfp4", 2)])
def test_binding_rejects_tensors_that_do_not_fit_the_plan(monkeypatch, kv, code):
    """Wrong dtypes (an int64 table, fp32 queries), wrong element counts and
    short pools raise ValueError in the binding, before the library is called."""
    import torch
    monkeypatch.setattr(B, "_current_device", lambda: torch.device("cpu"))
    called = []
    monkeypatch.setattr(B, "lib", lambda: called.append(1))
    pr = base_problem(kv_dtype=code, head_dim=128, num_pages=30)
    plan = B.Plan(0, pr)
    good = _cpu_call_tensors(pr, kv)
    bad_cases = {
        "seq_lens": good["seq_lens"].long(),
        "block_table": good["block_table"].long(),
        "q": good["q"].float(),
        "out": good["out"][:, :1].contiguous(),
        "lse": good["lse"].double(),
        "k_pool": good["k_pool"][:-1].contiguous(),
        "v_pool": good["v_pool"][:-1].contiguous(),
    }
    if kv != "bf16":
        bad_cases["k_scale"] = good["k_scale"][:-1].contiguous()
    for name, t in bad_cases.items():
        args = dict(good)
        args[name] = t
        with pytest.raises(ValueError, match=name):
            B.small_w_attention_run(plan, args["q"], args["k_pool"], args["v_pool"],
                                    args["k_scale"], args["v_scale"], args["block_table"],
                                    args["seq_lens"], args["out"], args["lse"], stream=0)
    if kv != "bf16":
        with pytest.raises(ValueError, match="scale"):
            B.small_w_attention_run(plan, good["q"], good["k_pool"], good["v_pool"], None, None,
                                    good["block_table"], good["seq_lens"], good["out"],
                                    good["lse"], stream=0)
    kn = torch.zeros((pr.num_reqs, pr.window, pr.num_kv_heads, pr.head_dim), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_new"):
        B.small_w_kv_append(plan, kn[:, :1].contiguous(), kn, good["k_pool"], good["v_pool"],
                            good["k_scale"], good["v_scale"], good["block_table"],
                            good["seq_lens"], stream=0)
    with pytest.raises(ValueError, match="seq_lens"):
        B.small_w_kv_append(plan, kn, kn, good["k_pool"], good["v_pool"], good["k_scale"],
                            good["v_scale"], good["block_table"], good["seq_lens"].long(),
                            stream=0)
    assert not called, "the library was called despite a bad argument"


def test_noalloc_rejects_plans_beyond_its_scratch_before_any_launch():
    """A plan whose partials exceed the library's scratch gets SMALLW_EWORKSPACE
    from the allocation-free entry point; a null plan gets SMALLW_EINVAL."""
    lib = B.lib()
    fake = 1 << 40  # never dereferenced
    pr = base_problem(num_reqs=1, window=16, num_q_heads=24, num_kv_heads=4, head_dim=256,
                      num_pages=1100, max_pages_per_req=1100, force_splits=1025)
    plan = sw.small_w_attention_plan(pr, [16400])
    assert sw.small_w_attention_workspace_bytes(plan) > 32 << 20
    args = [fake, fake, fake, None, None, fake, fake, fake, fake, None]
    assert lib.small_w_attention_run_noalloc(plan.handle, *args) == B.SMALLW_EWORKSPACE
    assert lib.small_w_attention_run_noalloc(None, *args) == B.SMALLW_EINVAL
