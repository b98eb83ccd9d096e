"""Invariants of the compiled gfx950 device code (CPU only: hipcc cross-compiles).

* No kernel spills registers to scratch: the sweep's ring and accumulators are
  sized to fit 256 VGPRs at eight waves per CU.
* No packed fp32 VALU forms (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the
  build turns the packed-fp32 feature off for every device function.
* M0 is written only by the DMA statements (an M0 write, its wait state and
  the LDS DMA load that reads it), so the inline asm that sets M0 without
  declaring it clobbered cannot overwrite a value the compiler keeps there.
* The softmax's reductions across the four 16-lane groups use the VALU lane
  swaps, not LDS permutes: every sweep has v_permlane16_swap and
  v_permlane32_swap, and the bf16 sweeps no ds_bpermute at all (the 8- and
  4-bit ones keep a few in their Q quantisation, before the loop).  The
  combine merges each row's 16 lanes with DPP row moves, also without LDS
  permutes.
"""
import os
import re
import shutil
import subprocess

import pytest

from speculative_decode_verify_sweep_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in ("smallw.hip", "append.hip"):
        dst = d / (src + ".s")
        flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
        cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"),
               "-I", B.CSRC, "-o", str(dst), os.path.join(B.CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        out[src] = dst.read_text()
    return out


def kernels(text):
    """(name, body) of every kernel in a device assembly file."""
    found = []
    funcs = set(re.findall(r"\.type\s+(_Z\w+),@function", text))
    for m in re.finditer(r"^(_Z\w+):", text, re.M):
        if m.group(1) not in funcs:      # a device variable, not a kernel
            continue
        end = text.find(".Lfunc_end", m.start())
        found.append((m.group(1), text[m.start():end]))
    return found


def instructions(body):
    for line in body.split("\n"):
        t = line.strip()
        if t and not t.startswith((";", ".")) and not t.endswith(":"):
            yield t


def test_every_kernel_is_present(asm):
    names = [n for n, _ in kernels(asm["smallw.hip"])]
    for k in ("sweep_kernel", "combine_kernel", "trace_kernel", "check_kernel"):
        assert any(k in n for n in names), (k, names)
    # bf16 sweeps at D = 64 / 128 / 256 for d-major and token-major value pages,
    # the e4m3 sweep at the three head dims, the MXFP4 sweep at D = 128 / 256 in
    # both load-issue forms (waves 4 and 5 spared or not)
    assert sum("sweep_kernel" in n for n in names) == 2 * 3
    assert sum("sweep8_kernel" in n for n in names) == 3
    assert sum("sweep4_kernel" in n for n in names) == 2 * 2
    # the combine with clamped and with skipped loads, at D = 64 / 128 / 256
    assert sum("combine_kernel" in n for n in names) == 2 * 3
    assert any("append_kernel" in n for n, _ in kernels(asm["append.hip"]))


def test_no_register_spills(asm):
    for src, text in asm.items():
        for name, _ in kernels(text):
            sz = re.search(re.escape(name) + r"\.private_seg_size, (\d+)", text)
            assert sz is not None, name
            assert int(sz.group(1)) == 0, f"{name} uses {sz.group(1)} bytes of scratch"
            nv = int(re.search(re.escape(name) + r"\.num_vgpr, (\d+)", text).group(1))
            na = int(re.search(re.escape(name) + r"\.num_agpr, (\d+)", text).group(1))
            assert nv + na <= 256, (name, nv, na)


def test_no_packed_fp32_valu(asm):
    bad = re.compile(r"^v_pk_(add|mul|fma)_f32\b")
    for src, text in asm.items():
        for name, body in kernels(text):
            hits = [i for i in instructions(body) if bad.match(i)]
            assert not hits, (name, hits[:3])


def test_m0_written_only_by_the_dma_statements(asm):
    for src, text in asm.items():
        for name, body in kernels(text):
            ins = list(instructions(body))
            for k, i in enumerate(ins):
                if not re.search(r"\bm0\b", i):
                    continue
                assert i.startswith("s_mov_b32 m0,"), (name, i)
                assert ins[k + 1] == "s_nop 0", (name, ins[k:k + 3])
                assert ins[k + 2].startswith("global_load_lds_dword"), (name, ins[k:k + 3])


def test_group_reductions_use_lane_swaps(asm):
    for name, body in kernels(asm["smallw.hip"]):
        if not any(k in name for k in ("sweep_kernel", "sweep8_kernel", "sweep4_kernel")):
            continue
        ins = [i.split()[0] for i in instructions(body)]
        assert any(i.startswith("v_permlane16_swap_b32") for i in ins), name
        assert any(i.startswith("v_permlane32_swap_b32") for i in ins), name
        if "sweep_kernel" in name:     # bf16 sweeps: <D, 4, VT>
            assert not any(i.startswith("ds_bpermute") for i in ins), name
            # token-major value pages (VT = true): the PV operand comes from
            # transpose reads, and only there
            vt = any(i.startswith("ds_read_b64_tr_b16") for i in ins)
            assert vt == ("ELi4ELb1EEE" in name), name


def test_combine_merges_rows_with_dpp(asm):
    for name, body in kernels(asm["smallw.hip"]):
        if "combine_kernel" not in name:
            continue
        ins = list(instructions(body))
        assert not any(i.startswith("ds_bpermute") for i in ins), name
        assert sum("row_ror:8" in i for i in ins) >= 2, name
        assert sum("row_ror:4" in i for i in ins) >= 2, name
