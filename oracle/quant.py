"""Float64 CPU oracle of the quantised compressed-KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it, and it imports nothing from the product path.

Source: "Lab tổng hợp DeepSeek-V4.1-Flash", section "3 Giải pháp" (the 890
B/token budget of block 6A is priced with FP4 E2M1 for the latent and FP8
E4M3 for the RoPE tail) and section "1 Định nghĩa" (block 3B: the cache
keeps the compressed form only).  "LLM Atlas: DeepSeek", section "FP8 训练
真正难在哪" (low-precision tensors need fine-grained scaling).

The two element formats are the standard ones:

* E2M1 (4 bits): sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity, no NaN.
* E4M3 (8 bits, the "fn" variant): sign, 4 exponent bits (bias 7), 3
  mantissa bits; normal magnitudes 2^(e-7) * (1 + m/8), subnormals
  2^-6 * m/8; the all-ones pattern S.1111.111 is NaN, so the largest
  magnitude is 448; no infinity.

Readings (the pages name only the element formats):

* Block scaling: every 32 consecutive channels share one power-of-two scale
  2^x, stored as the biased exponent byte x + 127 (an E8M0 byte).  x is the
  smallest integer with max|v| / 2^x <= the format's largest magnitude (6 or
  448), so no element of a block is clipped; an all-zero block stores 0
  (scale 2^-127).  The latent (channels 0 .. D-rope-1) uses E2M1, the RoPE
  tail (the last rope_dim channels) E4M3; both widths are multiples of 32.
* Elements round to the nearest representable value, ties to the even code
  (the code whose lowest bit is 0); a value that rounds to zero keeps its
  sign (the negative-zero code).
* Row layout (bytes): latent codes, two per byte (even channel in the low
  nibble); tail codes, one byte each; latent scales, one byte per block;
  tail scales; zero padding to a multiple of 16 bytes.  The codes come
  first so that every group of codes a reader takes at once starts on its
  own alignment.  D = 512 with a 64-wide tail takes 224 + 64 + 14 + 2 = 304
  bytes instead of 1024 in bf16.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_decode(code):
    """Value of an E2M1 code (0..15): sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0 or 0.5)."""
    code = np.asarray(code, dtype=np.int64)
    s = np.where(code & 8, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return s * mag


def e4m3_decode(code):
    """Value of an E4M3 ("fn") code (0..255); the two NaN codes give NaN."""
    code = np.asarray(code, dtype=np.int64)
    s = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def _nearest_code(y, codes, values, sign_bit):
    """Code of the representable value nearest to each y, searching the
    whole table (the definition of round-to-nearest): among equally near
    codes the one whose sign bit is the sign of y (so that a value rounding
    to zero keeps its sign), then the even one."""
    y = np.asarray(y, dtype=np.float64)
    d = np.abs(y[..., None] - values)                 # distance to every code
    best = np.min(d, axis=-1, keepdims=True)
    nearest = d == best
    sign_match = ((codes & sign_bit) != 0) == np.signbit(y)[..., None]
    even = (codes & 1) == 0
    score = nearest * (4 + 2 * sign_match + even)
    return codes[np.argmax(score, axis=-1)]


_E2M1_CODES = np.arange(16)
_E2M1_VALUES = e2m1_decode(_E2M1_CODES)
_E4M3_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])   # the finite codes
_E4M3_VALUES = e4m3_decode(_E4M3_CODES)


def block_scale_exp(block, fmt_max):
    """Exponent x of the block scale 2^x: the smallest integer with
    max|v| / 2^x <= fmt_max (-127 for an all-zero block)."""
    a = float(np.max(np.abs(block)))
    if a == 0.0:
        return -127
    x = max(int(np.ceil(np.log2(a / fmt_max))), -127)
    # guard the floating-point log against an off-by-one at exact powers
    while a / 2.0 ** x > fmt_max:
        x += 1
    while x > -127 and a / 2.0 ** (x - 1) <= fmt_max:
        x -= 1
    return x


def quantize_blocks(v, fmt):
    """Codes and scale exponents of v (length a multiple of 32) in blocks of
    32 channels: fmt 'e2m1' or 'e4m3'."""
    v = np.asarray(v, dtype=np.float64).reshape(-1, BLOCK)
    fmt_max, codes, values, sign_bit = ((E2M1_MAX, _E2M1_CODES, _E2M1_VALUES, 8) if fmt == "e2m1"
                                        else (E4M3_MAX, _E4M3_CODES, _E4M3_VALUES, 0x80))
    xs = np.array([block_scale_exp(b, fmt_max) for b in v], dtype=np.int64)
    y = v / np.exp2(xs.astype(np.float64))[:, None]
    return _nearest_code(y, codes, values, sign_bit).reshape(-1), xs


def dequantize_blocks(codes, xs, fmt):
    dec = e2m1_decode if fmt == "e2m1" else e4m3_decode
    vals = dec(np.asarray(codes)).reshape(-1, BLOCK)
    return (vals * np.exp2(np.asarray(xs, dtype=np.float64))[:, None]).reshape(-1)


def row_bytes(D, rope_dim):
    """Bytes of one quantised cache row (a multiple of 16)."""
    lat = D - rope_dim
    raw = lat // 2 + lat // BLOCK + rope_dim + rope_dim // BLOCK
    return (raw + 15) // 16 * 16


def quantize_row(v, rope_dim):
    """One compressed entry (D values) as its quantised cache row (uint8)."""
    v = np.asarray(v, dtype=np.float64)
    D = v.shape[-1]
    lat = D - rope_dim
    assert lat % BLOCK == 0 and rope_dim % BLOCK == 0
    out = np.zeros(row_bytes(D, rope_dim), dtype=np.uint8)
    c4, x4 = quantize_blocks(v[:lat], "e2m1")
    out[:lat // 2] = (c4[0::2] | (c4[1::2] << 4)).astype(np.uint8)
    o = lat // 2
    s = o + rope_dim                                    # the scale bytes follow all codes
    out[s:s + lat // BLOCK] = (x4 + 127).astype(np.uint8)
    if rope_dim:
        c8, x8 = quantize_blocks(v[lat:], "e4m3")
        out[o:o + rope_dim] = c8.astype(np.uint8)
        out[s + lat // BLOCK:s + lat // BLOCK + rope_dim // BLOCK] = (x8 + 127).astype(np.uint8)
    return out


def dequantize_row(row, D, rope_dim):
    """The D values a quantised cache row stands for."""
    row = np.asarray(row, dtype=np.uint8).astype(np.int64)
    lat = D - rope_dim
    c4 = np.empty(lat, dtype=np.int64)
    c4[0::2] = row[:lat // 2] & 15
    c4[1::2] = row[:lat // 2] >> 4
    o = lat // 2
    s = o + rope_dim
    x4 = row[s:s + lat // BLOCK] - 127
    out = np.empty(D, dtype=np.float64)
    out[:lat] = dequantize_blocks(c4, x4, "e2m1")
    if rope_dim:
        c8 = row[o:o + rope_dim]
        x8 = row[s + lat // BLOCK:s + lat // BLOCK + rope_dim // BLOCK] - 127
        out[lat:] = dequantize_blocks(c8, x8, "e4m3")
    return out
