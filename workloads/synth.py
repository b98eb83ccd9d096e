"""Seeded synthetic workloads with the shapes of the pages' verify and draft calls.

Storage layout (the library's documented layout):
  q         bf16 bits, uint16 [P][W][Hq][D]
  k_pool    [num_pages][Hkv][16][D]     uint16 bf16 bits, or uint8 e4m3fn codes
  v_pool    [num_pages][Hkv][D][16]     each page-head stored transposed, or
            [num_pages][Hkv][16][D]     like K (bf16, v_layout = 1: token-major)
  k_scale   fp32 [num_pages][Hkv][16]   fp8 only (dequantised value = code * scale)
  v_scale   fp32 [num_pages][Hkv][16]
  MXFP4 (kv = "mxfp4"): uint8, two E2M1 codes per byte, the even element in the
  low nibble; k_pool [num_pages][Hkv][16][D/2] (byte i of token t: elements 2i,
  2i+1), v_pool [num_pages][Hkv][D][8] (byte i of row d: tokens 2i, 2i+1),
  E8M0 bytes, one per 32-element block of a token's row: k_scale
  [num_pages][Hkv][16][D/32], v_scale block-major [num_pages][Hkv][D/32][16]
  block_table int32 [P][max_pages_per_req]   (-1 past a request's last page)
  seq_lens    int32 [P]   (context + window: the window's own K/V rows are
              already in the pool, so a verify row i sits at position L - W + i)

Pool pages that no block table references, and the slots of a request's last
page past its length, hold NaN so a read of them would show in the output (for
MXFP4, whose codes have no NaN, the NaN scale byte 0xFF).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

PAGE = 16
E4M3_MAX = 448.0

# name -> shape recipe.  "ctx" is the context before the window; "pool" names
# the page placement; W may be overridden per call.
CONFIGS = {
    # batch 1, 4 q / 1 KV head, D 64, context 256 + W=4 causal, contiguous pages
    "tiny": dict(P=1, Hq=4, Hkv=1, D=64, ctx=(256,), W=4, causal=True, kv="bf16",
                 placement="in_order", pool_pages=None),
    # batch 1, 24 q / 4 KV heads, D 256, 16K context, pages in order
    "verify16k": dict(P=1, Hq=24, Hkv=4, D=256, ctx=(16384,), W=16, causal=True, kv="bf16",
                      placement="in_order", pool_pages=None),
    # batch 1, 24 q / 4 KV heads, D 256, 64K context, pages a seeded permutation
    # of a 5000-page pool
    "verify64k": dict(P=1, Hq=24, Hkv=4, D=256, ctx=(65536,), W=16, causal=True, kv="bf16",
                      placement="permuted", pool_pages=5000),
    # P=8 draft blocks, contexts ~ U[1000,1600], 9 block rows, non-causal,
    # 32 q / 8 KV heads, D 128, disjoint pages of a shared 1024-page pool
    "draft": dict(P=8, Hq=32, Hkv=8, D=128, ctx=("uniform", 1000, 1600), W=9, causal=False,
                  kv="bf16", placement="permuted", pool_pages=1024),
    # batch 4, 24 q / 4 KV heads, D 256, contexts 8K..64K, W=16 causal, fp8 KV,
    # pages randomly placed in a 10000-page pool
    "fp8": dict(P=4, Hq=24, Hkv=4, D=256, ctx=(8192, 16384, 32768, 65536), W=16, causal=True,
                kv="fp8", placement="permuted", pool_pages=10000),
    # batch 1, 24 q / 4 KV heads, D 256, 16K context, W=16 causal, 4-bit (MXFP4)
    # KV, pages in order
    "fp4_16k": dict(P=1, Hq=24, Hkv=4, D=256, ctx=(16384,), W=16, causal=True, kv="mxfp4",
                    placement="in_order", pool_pages=None),
    # the same at 64K context, pages a seeded permutation of a 5000-page pool
    "fp4_64k": dict(P=1, Hq=24, Hkv=4, D=256, ctx=(65536,), W=16, causal=True, kv="mxfp4",
                    placement="permuted", pool_pages=5000),
    # a mixed-length verify batch: 16 requests, contexts ~ U[100, 24000], W=16
    # causal, 32 q / 8 KV heads, D 128, bf16, pages a seeded permutation of the
    # pool (the varlen batching the split planner has to balance)
    "mixed": dict(P=16, Hq=32, Hkv=8, D=128, ctx=("uniform", 100, 24000), W=16, causal=True,
                  kv="bf16", placement="permuted", pool_pages=None),
}

CONFIG_SEED_BASE = 20261202


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def quantize_e4m3(x: np.ndarray):
    """Per-row (last axis) e4m3fn codes and fp32 scales: scale = amax / 448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1, keepdims=True)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale, -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale[..., 0]


@dataclasses.dataclass
class Workload:
    name: str
    P: int
    W: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    kv: str                      # "bf16" | "fp8" | "mxfp4"
    scale: float
    num_pages: int
    max_pages: int
    q: np.ndarray                # uint16 [P][W][Hq][D]
    k_pool: np.ndarray           # uint16 or uint8 [num_pages][Hkv][16][D]
    v_pool: np.ndarray           # uint16 or uint8 [num_pages][Hkv][D][16]
    k_scale: np.ndarray | None   # fp32 [num_pages][Hkv][16]
    v_scale: np.ndarray | None
    block_table: np.ndarray      # int32 [P][max_pages]
    seq_lens: np.ndarray         # int32 [P]
    seed: int
    window_left: int = 0         # sliding window (keys per row); 0 = none
    v_layout: int = 0            # 0: value pages d-major; 1: token-major (bf16)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kv_fp8(self) -> bool:
        return self.kv == "fp8"


def _contexts(spec, P, rng):
    if spec[0] == "uniform":
        return [int(c) for c in rng.integers(spec[1], spec[2] + 1, size=P)]
    assert len(spec) == P
    return [int(c) for c in spec]


def make_workload(name: str | None = None, *, W: int | None = None, seed: int | None = None,
                  poison: bool = True, **over) -> Workload:
    """Build a seeded workload.  Any recipe field may be overridden by keyword,
    e.g. make_workload("tiny", W=2, Hq=2, Hkv=1, D=8, ctx=(5,)) for tiny cases.

    Value draws: Q, K, V ~ N(0, 1) in fp32, rounded to the storage format
    (bf16, or e4m3 with a per-row scale).  MXFP4 K and V are drawn as codes:
    every E2M1 code equally likely, E8M0 block scales uniform over 2^-3 .. 2^0.
    """
    spec = dict(CONFIGS[name]) if name else {}
    spec.update(over)
    if W is not None:
        spec["W"] = W
    if seed is None:
        seed = CONFIG_SEED_BASE + (list(CONFIGS).index(name) if name in CONFIGS else 99)
    rng = np.random.default_rng(seed)
    P, Hq, Hkv, D, Wn = spec["P"], spec["Hq"], spec["Hkv"], spec["D"], spec["W"]
    ctx = _contexts(spec["ctx"], P, rng)
    seq = [c + Wn for c in ctx]
    if spec.get("seq_lens") is not None:          # explicit lengths (edge cases)
        seq = [int(x) for x in spec["seq_lens"]]
    npg = [math.ceil(L / PAGE) for L in seq]
    max_pages = max(1, spec.get("max_pages") or max(npg + [1]))
    need = sum(npg)
    pool_pages = spec.get("pool_pages") or max(need, 1)
    pool_pages = max(pool_pages, need)
    fp8 = spec["kv"] == "fp8"
    fp4 = spec["kv"] == "mxfp4"
    vtok = int(spec.get("v_layout", 0)) == 1
    assert not vtok or spec["kv"] == "bf16", "token-major value pages are a bf16 layout"

    q = to_bf16_bits(rng.standard_normal((P, Wn, Hq, D), dtype=np.float32))

    # physical placement of every request's logical pages
    if spec["placement"] == "in_order":
        order = np.arange(pool_pages)
    else:
        order = rng.permutation(pool_pages)
    bt = np.full((P, max_pages), -1, dtype=np.int32)
    pos = 0
    for p in range(P):
        bt[p, :npg[p]] = order[pos:pos + npg[p]]
        pos += npg[p]

    if fp4:
        k_pool = np.full((pool_pages, Hkv, PAGE, D // 2), 0x77, dtype=np.uint8)
        v_pool = np.full((pool_pages, Hkv, D, PAGE // 2), 0x77, dtype=np.uint8)
        k_scale = np.full((pool_pages, Hkv, PAGE, D // 32), 0xFF, dtype=np.uint8)
        v_scale = np.full((pool_pages, Hkv, D // 32, PAGE), 0xFF, dtype=np.uint8)
    elif fp8:
        k_pool = np.full((pool_pages, Hkv, PAGE, D), 0x7F, dtype=np.uint8)
        v_pool = np.full((pool_pages, Hkv, D, PAGE), 0x7F, dtype=np.uint8)
        k_scale = np.full((pool_pages, Hkv, PAGE), np.nan, dtype=np.float32)
        v_scale = np.full((pool_pages, Hkv, PAGE), np.nan, dtype=np.float32)
    else:
        k_pool = np.full((pool_pages, Hkv, PAGE, D), 0x7FC0, dtype=np.uint16)
        v_pool = np.full((pool_pages, Hkv, PAGE, D) if vtok else (pool_pages, Hkv, D, PAGE),
                         0x7FC0, dtype=np.uint16)
        k_scale = v_scale = None
    if not poison:
        k_pool[...] = 0
        v_pool[...] = 0
        if fp8:
            k_scale[...] = 1.0
            v_scale[...] = 1.0
        if fp4:
            k_scale[...] = 127
            v_scale[...] = 127

    for p in range(P):
        L = seq[p]
        if L == 0:
            continue
        if fp4:
            # codes [Hkv][L][D], scales [Hkv][L][D/32]
            kc = rng.integers(0, 16, size=(Hkv, L, D), dtype=np.uint8)
            vc = rng.integers(0, 16, size=(Hkv, L, D), dtype=np.uint8)
            ksc = rng.integers(124, 128, size=(Hkv, L, D // 32), dtype=np.uint8)
            vsc = rng.integers(124, 128, size=(Hkv, L, D // 32), dtype=np.uint8)
            for n in range(npg[p]):
                t0, t1 = n * PAGE, min(L, (n + 1) * PAGE)
                phys = bt[p, n]
                k_pool[phys, :, :t1 - t0, :] = kc[:, t0:t1, 0::2] | (kc[:, t0:t1, 1::2] << 4)
                k_scale[phys, :, :t1 - t0, :] = ksc[:, t0:t1]
                v_scale[phys, :, :, :t1 - t0] = vsc[:, t0:t1].transpose(0, 2, 1)
                for t in range(t0, t1):
                    slot = t - t0
                    sh = 4 * (slot & 1)
                    cur = v_pool[phys, :, :, slot // 2] & np.uint8(0xF0 >> sh)
                    v_pool[phys, :, :, slot // 2] = cur | (vc[:, t, :] << sh)
            continue
        kl = rng.standard_normal((Hkv, L, D), dtype=np.float32)
        vl = rng.standard_normal((Hkv, L, D), dtype=np.float32)
        for name_, logical in (("k", kl), ("v", vl)):
            if fp8:
                codes, sc = quantize_e4m3(logical)          # [Hkv][L][D], [Hkv][L]
            else:
                codes, sc = to_bf16_bits(logical), None
            for n in range(npg[p]):
                t0, t1 = n * PAGE, min(L, (n + 1) * PAGE)
                phys = bt[p, n]
                blk = codes[:, t0:t1, :]                      # [Hkv][slots][D]
                if name_ == "k":
                    k_pool[phys, :, :t1 - t0, :] = blk
                    if fp8:
                        k_scale[phys, :, :t1 - t0] = sc[:, t0:t1]
                elif vtok:
                    v_pool[phys, :, :t1 - t0, :] = blk
                else:
                    v_pool[phys, :, :, :t1 - t0] = blk.transpose(0, 2, 1)
                    if fp8:
                        v_scale[phys, :, :t1 - t0] = sc[:, t0:t1]

    return Workload(name=name or "custom", P=P, W=Wn, Hq=Hq, Hkv=Hkv, D=D,
                    causal=bool(spec["causal"]), kv=spec["kv"], scale=1.0 / math.sqrt(D),
                    num_pages=pool_pages, max_pages=max_pages, q=q, k_pool=k_pool,
                    v_pool=v_pool, k_scale=k_scale, v_scale=v_scale, block_table=bt,
                    seq_lens=np.asarray(seq, dtype=np.int32), seed=seed,
                    window_left=int(spec.get("window_left", 0)), v_layout=int(vtok))
