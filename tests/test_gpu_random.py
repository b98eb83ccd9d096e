"""GPU parity on seeded random configurations: every storage format, head dim,
window size, grouping, causal or not, ragged contexts (including empty
requests), sliding windows and all three split modes, each case against the
fp64 oracle with the tolerances of test_gpu_parity."""
import numpy as np
import pytest

import oracle
from test_gpu_parity import announce, check, gpu_run
from workloads import make_workload

pytestmark = pytest.mark.gpu


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    kv = ["bf16", "fp8", "mxfp4"][seed % 3]
    D = int(rng.choice([128, 256] if kv == "mxfp4" else [64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    W = int(rng.integers(1, 17))
    W = min(W, 128 // G)
    causal = bool(rng.integers(0, 2))
    P = int(rng.integers(1, 5))
    ctx = [int(rng.choice([0, int(rng.integers(1, 40)), int(rng.integers(40, 3000))]))
           for _ in range(P)]
    if all(c == 0 for c in ctx):
        ctx[0] = int(rng.integers(1, 500))
    window = int(rng.choice([0, 0, int(rng.integers(1, 64)), int(rng.integers(64, 2000))]))
    mode = ["auto", "force", "exact"][int(rng.integers(0, 3))]
    seq = tuple(c + W if c > 0 else 0 for c in ctx)
    npg = sum(-(-L // 16) for L in seq)
    w = make_workload(None, P=P, Hq=Hkv * G, Hkv=Hkv, D=D, ctx=tuple(ctx), W=W, causal=causal,
                      kv=kv, placement="permuted", pool_pages=npg + 7, seed=2000 + seed,
                      seq_lens=seq, window_left=window)
    force = int(rng.integers(1, 9)) if mode == "force" else 0
    spg = int(rng.choice([1, 3, 8, 33])) if mode == "exact" else 0
    return w, force, spg, (kv, D, Hkv, G, W, causal, ctx, window, mode)


@pytest.mark.parametrize("seed", range(36))
def test_random_configuration_matches_oracle(seed):
    w, force, spg, desc = random_case(seed)
    announce(f"random {seed}: {desc} force={force} split_pages={spg}")
    o, l = gpu_run(w, force_splits=force, split_pages=spg)
    check(w, o, l, *oracle.attention(w))
