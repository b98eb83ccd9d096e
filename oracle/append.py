"""Oracle (test infrastructure only): paged KV append and the e4m3fn encoder.

Restated from the definitions the library documents for small_w_kv_append:
* "perf(dflash): widen the verify window past the compact graph's four-row
  limit", section What changed: the window's K/V rows are written into the
  paged cache at their positions; "DFlash2 leaves the paged graph fast path
  ...", section Scope: one pool addressed by a batched block table and
  per-request lengths.
* e4m3 rows: scale = amax|x| / 448 in float32 (1.0 for an all-zero row) and
  codes = x / scale (float32 IEEE division), clamped to +-448 and rounded to
  the nearest OCP e4m3fn value, ties to the even code.  The encoder below finds
  that value by comparing against every finite code's exact value, which is
  slow and plainly correct.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    """Exact value of a finite OCP e4m3fn code (bias 7; S.1111.111 is NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# non-negative finite codes 0x00..0x7E in increasing value
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = np.array([_e4m3_value(int(c)) for c in _POS_CODES], dtype=np.float64)


def e4m3_encode(x) -> np.ndarray:
    """Round float32 values in [-448, 448] to the nearest e4m3fn code, ties to
    the even code; the sign bit follows the sign of x (so -0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    a = np.abs(flat.astype(np.float64))
    if (a > E4M3_MAX).any():
        raise ValueError("e4m3_encode expects values clamped to +-448")
    out = np.empty(flat.shape, dtype=np.uint8)
    for lo in range(0, flat.size, 4096):
        d = np.abs(_POS_VALUES[None, :] - a[lo:lo + 4096, None])   # distance to every code
        near = d == d.min(axis=1, keepdims=True)                    # the nearest (1 or 2)
        # among the nearest, prefer an even code; codes are in increasing order
        pick = np.where(near & (_POS_CODES[None, :] % 2 == 0), 1, 0) * 2 + near
        out[lo:lo + 4096] = _POS_CODES[pick.argmax(axis=1)]
    out |= np.where(np.signbit(flat), 0x80, 0).astype(np.uint8)
    return out.reshape(x.shape)


def e4m3_row_quantize(x) -> tuple[np.ndarray, np.float32]:
    """One (token, KV head) row of bf16-exact values -> (codes, fp32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max())
    scale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    y = np.clip(x / scale, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(y), scale


def kv_append(*, P, W, Hkv, D, kv_fp8, k_new_bits, v_new_bits, k_pool, v_pool, k_scale,
              v_scale, block_table, seq_lens, num_pages):
    """Return updated copies of the pools after appending the window tokens.

    k_new_bits / v_new_bits: uint16 bf16 bits [P][W][Hkv][D].  Pools in the
    library's layouts (uint16 for bf16, uint8 codes for e4m3)."""
    kp, vp = k_pool.copy(), v_pool.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    cap = block_table.shape[1] * 16
    for p in range(P):
        L = min(max(int(seq_lens[p]), 0), cap)
        for i in range(W):
            pos = L - W + i
            if pos < 0:
                continue
            page = int(block_table[p, pos // 16])
            page = min(max(page, 0), num_pages - 1)
            slot = pos % 16
            for h in range(Hkv):
                kb = k_new_bits[p, i, h]
                vb = v_new_bits[p, i, h]
                if not kv_fp8:
                    kp[page, h, slot, :] = kb
                    vp[page, h, :, slot] = vb
                else:
                    kx = (kb.astype(np.uint32) << 16).view(np.float32)
                    vx = (vb.astype(np.uint32) << 16).view(np.float32)
                    kc, kscl = e4m3_row_quantize(kx)
                    vc, vscl = e4m3_row_quantize(vx)
                    kp[page, h, slot, :] = kc
                    vp[page, h, :, slot] = vc
                    ks[page, h, slot] = kscl
                    vs[page, h, slot] = vscl
    return kp, vp, ks, vs
