"""CPU checks of the per-element output bound the GPU parity tests apply.

The bound is max(1e-2, 2^-7 A) with A[d] = sum_j p_j |v_j[d]| / sum_j p_j,
computed by the oracle on the same workload with every V sign bit cleared.
These tests pin that construction: the magnitude workload really yields the
softmax-weighted mean |v| (against a dense brute force), it dominates |o|,
and an emulation of the kernels' two bf16 roundings (each weight before the
PV product, then the output) stays inside 2^-7 A on few-key and many-key rows.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import BF16_U, magnitude_workload, o_bound
from test_oracle_pins import CASES, dense_kv, mask_matrix, q_f64, tiny


def bf16_round(x):
    """fp64 -> nearest bf16 (ties to even, through fp32), back to fp64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def weighted_mean_abs_v(w):
    """Brute force A[p][i][h][d] from dense K, V and an explicit mask."""
    K, V = dense_kv(w)
    Q = q_f64(w)
    A = np.zeros((w.P, w.W, w.Hq, w.D))
    for p in range(w.P):
        M = mask_matrix(int(w.seq_lens[p]), w.W, w.causal, K.shape[2], w.window_left)
        for h in range(w.Hq):
            S = np.where(M, (Q[p, :, h] @ K[p, h // w.G].T) * w.scale, -np.inf)
            m = S.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            E = np.where(M, np.exp(S - np.where(np.isfinite(m), m, 0.0)), 0.0)
            A[p, ok, h] = (E[ok] @ np.abs(V[p, h // w.G])) / E[ok].sum(axis=1)[:, None]
    return A


def emulate_kernel_rounding(w):
    """Exact scores, each weight rounded to bf16 before the PV sum (normalised
    by the unrounded sum, as the kernels do), the output rounded to bf16."""
    K, V = dense_kv(w)
    Q = q_f64(w)
    out = np.zeros((w.P, w.W, w.Hq, w.D))
    for p in range(w.P):
        M = mask_matrix(int(w.seq_lens[p]), w.W, w.causal, K.shape[2], w.window_left)
        for h in range(w.Hq):
            S = np.where(M, (Q[p, :, h] @ K[p, h // w.G].T) * w.scale, -np.inf)
            m = S.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            E = np.where(M, np.exp(S - np.where(np.isfinite(m), m, 0.0)), 0.0)
            o = (bf16_round(E[ok]) @ V[p, h // w.G]) / E[ok].sum(axis=1)[:, None]
            out[p, ok, h] = bf16_round(o)
    return out


@pytest.mark.parametrize("case", range(len(CASES)))
def test_magnitude_workload_gives_the_weighted_mean_abs_value(case):
    w = tiny(**CASES[case])
    A, _ = oracle.attention(magnitude_workload(w))
    np.testing.assert_allclose(A, weighted_mean_abs_v(w), rtol=1e-12, atol=1e-12)
    o, _ = oracle.attention(w)
    assert np.all(np.abs(o) <= A + 1e-12)
    assert np.any(A > np.abs(o) + 1e-3), "V signs were not cleared"


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("ctx,W,window", [((3, 700), 4, 0), ((1, 2000), 16, 5),
                                          ((300,), 8, 2)])
def test_two_bf16_roundings_stay_inside_the_bound(kv, ctx, W, window):
    """Few-key rows (1..5 keys, narrow windows) and a many-key row: the
    emulated kernel roundings keep every element within 2^-7 A, and the
    bound the tests apply (never below 1e-2) holds them too."""
    D = 32 if kv == "mxfp4" else 16
    w = tiny(P=len(ctx), Hq=4, Hkv=2, D=D, ctx=ctx, W=W, causal=True, kv=kv, seed=7,
             window_left=window)
    ref, _ = oracle.attention(w)
    A, _ = oracle.attention(magnitude_workload(w))
    err = np.abs(emulate_kernel_rounding(w) - ref)
    assert np.all(err <= 2.0 * BF16_U * A * (1 + 1e-9) + 1e-15)
    assert np.all(err <= o_bound(w))
