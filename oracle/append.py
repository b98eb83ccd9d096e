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
* MXFP4 rows (OCP Microscaling Formats v1.0, the conversion of a vector of
  scalars to an MX block, with E2M1 elements and an E8M0 scale): each block of
  32 consecutive elements of one (token, KV head) row gets the shared exponent
  X = floor(log2(amax)) - 2 (2 is E2M1's largest exponent), clamped to E8M0's
  [-127, 127], stored as the byte X + 127; an all-zero block stores 0 (2^-127).
  Each element x becomes the E2M1 value nearest to x / 2^X, ties to the even
  code, values past 6 saturating to 6; the sign bit is the sign of x.
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


# E2M1 magnitudes of codes 0..7 (sign in bit 3)
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_encode(y) -> np.ndarray:
    """Round values with |y| < 8 to the nearest E2M1 code (ties to the even
    code, past 6 to 6); the sign bit follows the sign of y.  One code per byte."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y.reshape(-1))
    if (a >= 8).any():
        raise ValueError("e2m1_encode expects |y| < 8")
    d = np.abs(_E2M1_POS[None, :] - a[:, None])
    near = d == d.min(axis=1, keepdims=True)
    pick = np.where(near & (np.arange(8)[None, :] % 2 == 0), 1, 0) * 2 + near
    codes = pick.argmax(axis=1).astype(np.uint8)
    codes |= np.where(np.signbit(y.reshape(-1)), 8, 0).astype(np.uint8)
    return codes.reshape(y.shape)


def mxfp4_row_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """One row of bf16-exact values (length a multiple of 32) -> (E2M1 codes,
    one per element, uint8; E8M0 scale bytes, one per 32-element block)."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(-1, 32)
    codes = np.empty(blocks.shape, dtype=np.uint8)
    scales = np.empty(blocks.shape[0], dtype=np.uint8)
    for b, blk in enumerate(blocks):
        amax = np.abs(blk).max()
        if amax == 0:
            X = -127
        else:
            _, e = np.frexp(amax)          # amax = f * 2^e, f in [0.5, 1)
            X = min(max(int(e) - 1 - 2, -127), 127)
        scales[b] = X + 127
        codes[b] = e2m1_encode(blk / 2.0 ** X)
    return codes.reshape(x.shape), scales


def kv_append(*, P, W, Hkv, D, k_new_bits, v_new_bits, k_pool, v_pool, k_scale,
              v_scale, block_table, seq_lens, num_pages, kv="bf16", v_layout=0):
    """Return updated copies of the pools after appending the window tokens.

    k_new_bits / v_new_bits: uint16 bf16 bits [P][W][Hkv][D].  Pools and scales
    in the library's layouts for kv = "bf16" | "fp8" | "mxfp4" (uint8 bytes
    for the last two; the MXFP4 value pool packs tokens 2i, 2i+1 of a row d
    into byte i, the even token in the low nibble, and its scales are
    block-major [page][head][D/32][16]).  v_layout=1: a bf16 value pool laid
    out token-major [page][head][16][D], written like K."""
    assert kv in ("bf16", "fp8", "mxfp4")
    assert v_layout in (0, 1) and (v_layout == 0 or kv == "bf16")
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
                if kv == "bf16":
                    kp[page, h, slot, :] = kb
                    if v_layout:
                        vp[page, h, slot, :] = vb
                    else:
                        vp[page, h, :, slot] = vb
                elif kv == "mxfp4":
                    kx = (kb.astype(np.uint32) << 16).view(np.float32)
                    vx = (vb.astype(np.uint32) << 16).view(np.float32)
                    kc, kscl = mxfp4_row_quantize(kx)
                    vc, vscl = mxfp4_row_quantize(vx)
                    kp[page, h, slot, :] = kc[0::2] | (kc[1::2] << 4)
                    sh = 4 * (slot & 1)
                    keep = np.uint8(0xF0 >> sh)
                    vp[page, h, :, slot // 2] = (vp[page, h, :, slot // 2] & keep) | (vc << sh)
                    ks[page, h, slot, :] = kscl
                    vs[page, h, :, slot] = vscl          # V scales block-major
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
