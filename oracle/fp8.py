"""Oracle for the FP8 (e4m3) KV cache: encode / decode of the 8-bit format, the quantising cache
scatter, and decode attention over the dequantised cache.

TEST INFRASTRUCTURE ONLY (tests, smoke check); never imported by the product path, and it shares no
code with the HIP library.

Source, by page title and section:
  [vLLM-PA] paged_attn.py (vLLM-derived fork ported to Iluvatar BI-V100), ``PagedAttention``:
            ``write_to_paged_cache`` and ``forward_decode`` take ``kv_cache_dtype`` with per-tensor
            ``k_scale`` / ``v_scale`` floats next to the caches; the page names the arguments but not
            the format or the arithmetic.

Readings where the page leaves the step open:
  * format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities and the
    largest finite magnitude is 448;
  * a stored code is e4m3(x / scale), with x the bf16 input widened to fp32 and the quotient rounded
    to fp32 (IEEE division); the fp32 -> e4m3 step rounds to the nearest representable value, ties to
    the even mantissa, saturates magnitudes of 448 and above to 448 (infinities included), keeps the
    sign of zero, and stores every NaN as 0x7F;
  * the cache is read back as decode(code) * scale, and attention over the cache is the plain
    definition over those dequantised keys and values.
"""
from __future__ import annotations

import numpy as np

from .attention import paged_decode, _ints

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The value a code stands for, straight from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# every code's value, and the non-negative finite codes 0x00 .. 0x7E in increasing value
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS_CODES = np.arange(0x7F)
_POS_VALUES = E4M3_TABLE[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


def e4m3_encode(x) -> np.ndarray:
    """fp32 values -> e4m3 codes (uint8): nearest representable magnitude, ties to the even
    mantissa (even code), saturation at 448, sign kept (zero included), NaN -> 0x7F."""
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(v)
    sign = np.signbit(v)
    a = np.where(nan, 0.0, np.abs(v))
    # neighbours in the ordered table of magnitudes: vals[lo] <= a <= vals[hi]
    hi = np.clip(np.searchsorted(_POS_VALUES, a), 1, len(_POS_VALUES) - 1)
    lo = hi - 1
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    tie_pick = np.where(lo % 2 == 0, lo, hi)  # the even code has the even mantissa
    c = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, tie_pick))
    c = np.where(a >= E4M3_MAX, 0x7E, c)
    codes = (c | np.where(sign, 0x80, 0)).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), codes).astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Codes of e4m3(fp32(x) / fp32(scale)), x given in bf16 (or any float array)."""
    if torch is not None and isinstance(x, torch.Tensor):
        xf = x.detach().to("cpu").to(torch.float32).numpy()
    else:
        xf = np.asarray(x, dtype=np.float32)
    q = (xf / np.float32(scale)).astype(np.float32)
    return e4m3_encode(q)


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale: float, v_scale: float):
    """[vLLM-PA] ``write_to_paged_cache`` with an fp8 cache: the scatter of the bf16 path, storing
    quantize(row, scale). Caches are uint8 code arrays [NB, Hkv, bs, D]; returns the new caches."""
    def codes(t):
        if torch is not None and isinstance(t, torch.Tensor):
            return t.detach().to("cpu").contiguous().view(torch.uint8).numpy().copy()
        return np.array(t, dtype=np.uint8, copy=True)
    kc, vc = codes(k_cache), codes(v_cache)
    kq, vq = quantize(k, k_scale), quantize(v, v_scale)
    nb, _, bs, _ = kc.shape
    slots = _ints(slot_mapping).reshape(-1)
    live = slots[slots >= 0]
    if live.size and live.max() >= nb * bs:
        raise IndexError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slot in slot_mapping")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        kc[s // bs, :, s % bs, :] = kq[t]
        vc[s // bs, :, s % bs, :] = vq[t]
    return kc, vc


def dequantize(codes, scale: float) -> np.ndarray:
    if torch is not None and isinstance(codes, torch.Tensor):
        codes = codes.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    return e4m3_decode(codes) * float(np.float32(scale))


def paged_decode_fp8(q, k_codes, v_codes, block_tables, seq_lens, scale: float, k_scale: float,
                     v_scale: float, return_lse: bool = False):
    """Decode attention over the dequantised fp8 cache (the plain definition of paged_decode with
    K = decode(code) * k_scale and V = decode(code) * v_scale)."""
    return paged_decode(q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), block_tables,
                        seq_lens, scale, return_lse=return_lse)
