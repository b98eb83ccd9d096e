"""Oracle (test infrastructure only): integer planning, page gather, combine, counts.

Everything here is restated from written definitions, in plain Python/numpy:

* The split planner follows the library's written planner specification
  (the pages give no split formula; key splitting and its reduce kernel are
  only named in "ChunkedSmallT re-streams full KV per query chunk", section
  Finding).  It is an independent restatement, never a call into the library.
* The log-sum-exp combine is the exact merge of softmax partials over disjoint
  key ranges (the "reduce kernel" of the same section).
* kv_bytes follows the same page's section Measurement: GB/s there is the KV
  bytes of one sweep over the visible context divided by the call time.
* attention_pairs follows "DFlash2 leaves the paged graph fast path ...",
  section The cost (its work-per-draft-step table).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

PAGE = 16
PLAN_MIN_PAGES = 8          # a split never holds fewer pages than this (auto mode)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def first_page(L: int, W: int, causal: bool, window_left: int) -> int:
    """First page any row of the request needs: with a sliding window of N keys,
    row 0 (the lowest) sees keys from (L - W if causal else L - 1) - N + 1 on."""
    if window_left <= 0 or L <= 0:
        return 0
    hi0 = (L - W) if causal else (L - 1)
    return max(0, hi0 - window_left + 1) // PAGE


def plan(*, P, Hkv, D, kv_fp8, seq_lens, num_cus, force_splits=0, split_pages=0, W=1,
         causal=True, window_left=0, kv=None):
    """Split plan for one call.

    n_pg(p)     = ceil(L_p / 16);  n_lo(p) = first page any row needs (0 without a
                  sliding window);  n_eff(p) = n_pg - n_lo  pages streamed
    slots       = num_cus * (2 if bf16 and D < 256 else 1)  units resident per CU
    round       = max(1, floor(slots / Hkv))     splits that one round of units holds
    S_p         = 1                          if n_pg(p) == 0
                = ceil(n_pg/B) - floor(n_lo/B) if split_pages = B > 0 (row-exact mode)
                = min(force_splits, n_eff)   if force_splits > 0
                  otherwise apportioned: every request starts with one split; then,
                  while the splits number fewer than the budget (round if P <= round,
                  so one round and no second; else P + round), the request with the
                  most pages per split, n_eff / S_p, gets one more (the lowest index
                  among equals), as long as that leaves it 8 pages a split
                  (S_p < floor(n_eff / 8)); stop early when no request may grow
    unit_off[p] = Hkv * sum_{q<p} S_q;  unit u = unit_off[p] + kvh*S_p + s
    split s covers pages n_lo + [floor(s*n_eff/S), floor((s+1)*n_eff/S)), or in
    row-exact mode the s-th piece of the absolute grid [k*B, (k+1)*B), the last
    split ending at n_pg and the first starting at n_lo moved down to a multiple
    of 2 pages from its k*B, or of 8 pages for e4m3 and MXFP4 pools (the pages
    the sweep groups into one step then line up in every call); kv names the
    storage format ("bf16", "fp8", "mxfp4"), by default fp8 if kv_fp8 else bf16
    """
    seq = [int(x) for x in seq_lens]
    assert len(seq) == P
    n_pg = [_ceil_div(L, PAGE) for L in seq]
    n_lo = [first_page(L, W, causal, window_left) for L in seq]
    n_eff = [n - lo for n, lo in zip(n_pg, n_lo)]
    fmt = kv or ("fp8" if kv_fp8 else "bf16")
    slots = num_cus * (2 if fmt == "bf16" and D < 256 else 1)
    splits = []
    for n, lo, ne in zip(n_pg, n_lo, n_eff):
        if n == 0:
            splits.append(1)
        elif split_pages > 0:
            splits.append(_ceil_div(n, split_pages) - lo // split_pages)
        elif force_splits > 0:
            splits.append(min(force_splits, ne))
        else:
            splits.append(1)            # apportioned below
    if split_pages == 0 and force_splits == 0:
        rnd = max(1, slots // Hkv)
        budget = rnd if P <= rnd else P + rnd
        while sum(splits) < budget:
            may_grow = [p for p in range(P)
                        if n_pg[p] > 0 and splits[p] < max(1, n_eff[p] // PLAN_MIN_PAGES)]
            if not may_grow:
                break
            best = may_grow[0]
            for p in may_grow[1:]:
                if Fraction(n_eff[p], splits[p]) > Fraction(n_eff[best], splits[best]):
                    best = p
            splits[best] += 1
    unit_off = [0]
    for s in splits:
        unit_off.append(unit_off[-1] + Hkv * s)
    # pages one step of the sweep's arithmetic groups: 128-token steps for e4m3
    # and MXFP4 pools, two-page chunks for bf16 (the library's written specification)
    align = 2 if fmt == "bf16" else 8
    units = []
    for p in range(P):
        S, n, lo, ne = splits[p], n_pg[p], n_lo[p], n_eff[p]
        for kvh in range(Hkv):
            for s in range(S):
                if split_pages > 0:
                    k = lo // split_pages + s
                    b0 = k * split_pages
                    pb = (b0 + ((lo - b0) // align) * align) if s == 0 else b0
                    pe = n if s + 1 == S else (k + 1) * split_pages
                else:
                    pb, pe = split_range(ne, S, s)
                    pb, pe = pb + lo, pe + lo
                units.append((p, kvh, s, pb, pe))
    any_split = any(s > 1 for s in splits)
    return {"P": P, "Hkv": Hkv, "n_pg": n_pg, "splits": splits, "unit_off": unit_off,
            "units": units, "U": unit_off[-1], "any_split": any_split,
            "combine": any_split or split_pages > 0}


def split_range(n: int, S: int, s: int):
    """Balanced split s of n pages into S (the automatic and forced modes)."""
    return (s * n) // S, ((s + 1) * n) // S


def plan_export(pl, R: int) -> np.ndarray:
    """Integer export layout: [P, Hkv, U, R] + S_p[P] + unit_off[P+1] + U*(p,kvh,s,pb,pe)."""
    head = [pl["P"], pl["Hkv"], pl["U"], R]
    flat = head + list(pl["splits"]) + list(pl["unit_off"])
    for u in pl["units"]:
        flat.extend(u)
    return np.asarray(flat, dtype=np.int32)


def gather_unit_pages(pl, block_table: np.ndarray) -> list[list[int]]:
    """Physical page ids each work unit streams, in logical order."""
    out = []
    for (p, _kvh, _s, pb, pe) in pl["units"]:
        out.append([int(block_table[p, n]) for n in range(pb, pe)])
    return out


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge partials over disjoint key ranges.

    o_parts [S][..., D] (each normalised by its own sum), lse_parts [S][...].
    M = max_s lse_s; lse = M + ln sum_s exp(lse_s - M); o = sum_s exp(lse_s - lse) o_s.
    A part with lse_s = -inf has weight 0; all parts -inf gives o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    Ms = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse_parts - Ms)                      # exp(-inf) = 0
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, Ms + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    wn = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


def kv_bytes(seq_lens, Hkv: int, D: int, kv_fp8: bool = False, kv: str | None = None) -> int:
    """Bytes of one sweep over every visible K and V element plus their scales
    (fp8: one fp32 per token and head; MXFP4: half a byte per element and one
    byte per 32 elements)."""
    tokens = int(sum(int(L) for L in seq_lens))
    kv = kv or ("fp8" if kv_fp8 else "bf16")
    per_token_head = {"bf16": 2 * D * 2, "fp8": 2 * D + 2 * 4,
                      "mxfp4": 2 * (D // 2) + 2 * (D // 32)}[kv]
    return tokens * Hkv * per_token_head


def attention_pairs(seq_lens, W: int, Hq: int, causal: bool) -> int:
    """(query row, key) pairs the exact method scores: sum over rows of visible keys."""
    total = 0
    for L in seq_lens:
        L = int(L)
        for i in range(W):
            n = (L - W + i + 1) if causal else L
            total += max(n, 0)
    return total * Hq


def materialised_pairs(ctxs, k: int) -> int:
    """Pairs of the fallback that attends every context row too: sum_r (ctx_r+1+k)^2."""
    return sum((int(c) + 1 + k) ** 2 for c in ctxs)


def paged_pairs(ctxs, k: int) -> int:
    """Pairs of the block-only route: (1+k) * C, C = sum of contexts."""
    return (1 + k) * sum(int(c) for c in ctxs)
