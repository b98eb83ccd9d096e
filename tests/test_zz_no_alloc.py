"""GPU: small_w_attention_run_noalloc (the entry point for callers that cannot
allocate) against small_w_attention_run on the same plan and inputs, on calls
in a row through the C ABI: a 64K verify call, then a smaller draft batch
(different head dim and plan, over what the first call left in the scratch),
then the first call again.  Same kernels, so the outputs must be bitwise
equal, and both within the oracle bounds."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_sweep_amd as sw
from speculative_decode_verify_sweep_amd import binding as B
from speculative_decode_verify_sweep_amd import device as dv
from test_gpu_parity import announce, check
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _both(w, force_splits=0):
    plan = dv.plan_for(w, force_splits=force_splits)
    need = sw.small_w_attention_workspace_bytes(plan)
    assert 0 < need <= 32 << 20
    d = dv.upload(w)
    ws = dv.workspace_for(plan)
    d["out"].fill_(float("nan"))
    d["lse"].fill_(float("nan"))
    dv.run(plan, d, ws)
    torch.cuda.synchronize()
    ref = (d["out"].float().cpu().numpy(), d["lse"].cpu().numpy())
    d["out"].fill_(float("nan"))
    d["lse"].fill_(float("nan"))
    sw.small_w_attention_run_noalloc(plan, d["q"], d["k_pool"], d["v_pool"], d["k_scale"],
                                     d["v_scale"], d["block_table"], d["seq_lens"], d["out"],
                                     d["lse"])
    torch.cuda.synchronize()
    got = (d["out"].float().cpu().numpy(), d["lse"].cpu().numpy())
    return need, ref, got


def test_noalloc_matches_run_on_calls_in_a_row():
    cases = [("verify64k W=16", make_workload("verify64k", W=16), 0),
             ("draft P=8 W=9 (smaller)", make_workload("draft"), 0),
             ("verify64k W=16 again", make_workload("verify64k", W=16), 0)]
    sizes = []
    for label, w, force in cases:
        announce(f"noalloc vs run: {label}")
        need, (ro, rl), (go, gl) = _both(w, force)
        sizes.append(need)
        np.testing.assert_array_equal(go, ro)
        np.testing.assert_array_equal(gl, rl)
        check(w, go.astype(np.float64), gl.astype(np.float64), *oracle.attention(w))
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_a_plan_larger_than_the_scratch():
    w = make_workload("verify16k", W=16)
    plan = dv.plan_for(w, force_splits=1025)      # 4100 units of 48 KiB partials
    assert sw.small_w_attention_workspace_bytes(plan) > 32 << 20
    d = dv.upload(w)
    announce("noalloc oversized plan")
    with pytest.raises(B.SmallwError) as e:
        sw.small_w_attention_run_noalloc(plan, d["q"], d["k_pool"], d["v_pool"], None, None,
                                         d["block_table"], d["seq_lens"], d["out"], d["lse"])
    assert e.value.code == B.SMALLW_EWORKSPACE
