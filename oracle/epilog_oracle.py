"""CPU oracle of the quantised cache write that follows the Compressor
(compressor_epilog).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Page cited (by title):
  [PyPTO] "CANN PyPTO 算子实战：Compressor 长序列 KV Cache 压缩算子的原理、参数与调用方法",
          section DeepSeek-V4 整网集成方式.

That section says only that the network's Compressor module hands its
compressed rows to compressor_epilog, which writes them into the Lightning
Indexer and Sparse Flash Attention compressed caches, and that those caches
may be quantised to float8 or hifloat8.  Everything below is a reading of
that sentence (each is listed, with the reasoning, in the design notes):

E1  Format: the OCP 8-bit floating point format E4M3 (sign bit 7, exponent
    bits 6..3 with bias 7, mantissa bits 2..0; exponent field 0 holds the
    subnormals m * 2^-9; S.1111.111 is NaN, there is no infinity; the largest
    finite magnitude is 448).  hifloat8 is not built: no definition of it is
    at hand.
E2  Scaling: one fp32 scale per block of 128 consecutive channels of a row:
    amax = max |x| over the block, scale = amax / 448, and each element's code
    is the E4M3 value nearest to q = clamp(x * (448 / amax), -448, 448), ties
    to the even code (round to nearest even); a block with amax = 0 stores
    scale 0 and q = x * 0.  The code is an integer decided by floating point,
    so the decision is taken in the kernel's precision: 448 / amax, x times
    that and amax / 448 are IEEE fp32 operations (correctly rounded) here as
    there; only the rounding of q to E4M3 is done in fp64, where it is exact.
E3  Placement: row i goes to slot slot_mapping[i] of a cache of num_slots
    rows (codes [num_slots, D] bytes, scales [num_slots, D / 128] fp32);
    slot -1 means "no slot" and writes nothing; any other slot outside
    [0, num_slots) is an error and writes nothing.  Other slots keep their
    contents.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128
SLOT_ERROR = 16          # device error bit of a slot outside [-1, num_slots)


def e4m3_value(code) -> np.ndarray:
    """Real value of E4M3 codes from the format definition (E1): NaN for
    S.1111.111, -0.0 for 0x80."""
    c = np.asarray(code, dtype=np.int64)
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


# the finite non-negative values, in increasing order: codes 0 .. 126
_POS = e4m3_value(np.arange(127))


def e4m3_encode(q) -> np.ndarray:
    """Code of the E4M3 value nearest to each q (|q| <= 448), ties to the even
    code, the sign of q kept (-0.0 -> 0x80).  Codes increase with magnitude,
    so the candidates are the two neighbours of |q| in the value table."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    if np.any(~(a <= E4M3_MAX)):
        raise ValueError("e4m3_encode: |q| above 448 or NaN")
    hi = np.minimum(np.searchsorted(_POS, a, side="left"), 126)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(_POS[hi] == a, hi, code)
    return (code | (np.signbit(q).astype(np.int64) << 7)).astype(np.uint8)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Codes uint8 [rows, D] and scales fp32 [rows, D / 128] of rows x (fp32
    values; the bf16 rows of the Compressor output are exact in fp32), per
    E2."""
    x = np.asarray(x, dtype=np.float32)
    rows, d = x.shape
    if d % BLOCK:
        raise ValueError("row length must be a multiple of 128")
    xb = x.reshape(rows, d // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)                                   # exact
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(0.0)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    q = (xb * inv[:, :, None]).astype(np.float32)                       # fp32 products
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode(q.astype(np.float64)).reshape(rows, d)
    return codes, scale


def epilog(rows_f32, slot_mapping, cache_codes, cache_scale):
    """The cache after one call (E3): returns (codes, scales, error bits);
    the inputs are not modified."""
    codes, scales = quantize_rows(rows_f32)
    out_c, out_s = np.array(cache_codes, copy=True), np.array(cache_scale, copy=True)
    num_slots = out_c.shape[0]
    err = 0
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot == -1:
            continue
        if slot < -1 or slot >= num_slots:
            err |= SLOT_ERROR
            continue
        out_c[slot] = codes[i]
        out_s[slot] = scales[i]
    return out_c, out_s, err
