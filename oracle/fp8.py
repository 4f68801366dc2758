"""CPU oracle of the FP8 KV cache (test infrastructure only).

Page "vLLM 部署深度指南" lists an FP8 KV cache (``--kv-cache-dtype fp8`` in the FP8
deployment command; FP8 halves the memory in the quantisation table). The pages name no
format and no scaling, so the plainest reading is taken (each reading is listed here):

* The stored format is OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the all-ones pattern
  S.1111.111 is NaN; there are no infinities; the largest finite magnitude is
  1.75 * 2^8 = 448.
* One scale per tensor: ``k_scale`` for keys, ``v_scale`` for values (fp32, > 0). A stored
  element is ``e4m3(fp32(x) * fp32(1 / scale))``, the product computed in fp32 and
  rounded once, then rounded to E4M3 to nearest with ties to the even code, magnitudes
  at or above 448 saturating to 448 (NaN stays NaN).
* Attention reads ``decode(code) * scale`` in place of the fp16 element; everything after
  that is the fp16 cache's definition (``oracle.decode``).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """Values (fp64) of E4M3 codes (uint8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# magnitudes of the non-negative finite codes 0x00 .. 0x7E, increasing with the code
_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
assert np.all(np.diff(_POS) > 0)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of fp32 values: nearest code, ties to the even code, magnitudes
    of 448 and more saturate to 448, NaN gives 0x7F with the input's sign."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)  # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo & (hi > 0), lo, hi).astype(np.int64)
    code = np.where(nan, E4M3_NAN, code)
    sign = np.signbit(np.asarray(x)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Stored codes of fp16 (or fp32) elements ``x`` under a per-tensor ``scale``."""
    inv = np.float32(1.0) / np.float32(scale)
    return e4m3_encode(np.asarray(x, dtype=np.float32) * inv)


def kv_append_fp8(pool_u8: np.ndarray, key, value, slot_mapping, k_scale: float,
                  v_scale: float) -> np.ndarray:
    """Copy of the uint8 pool ``[NB, bs, 2, Hkv, D]`` with token t's quantized key and
    value at slot ``slot_mapping[t]`` (negative: skipped)."""
    out = pool_u8.copy()
    bs = pool_u8.shape[1]
    kq = quantize(key, k_scale)
    vq = quantize(value, v_scale)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        out[slot // bs, slot % bs, 0] = kq[t]
        out[slot // bs, slot % bs, 1] = vq[t]
    return out


def dequantize_pool(pool_u8: np.ndarray, k_scale: float, v_scale: float) -> np.ndarray:
    """The pool as the attention reads it (fp64): code values times their scale."""
    vals = e4m3_decode(pool_u8)
    vals[:, :, 0] *= float(np.float32(k_scale))
    vals[:, :, 1] *= float(np.float32(v_scale))
    return vals
