"""Pins of the FP8 cache-write oracle (oracle/epilog_oracle.py) to things
other than itself: the E4M3 format definition (OCP 8-bit floating point
specification: bias 7, largest finite 448, subnormals down to 2^-9, NaN at
S.1111.111), PyTorch's own float32 -> float8_e4m3fn conversion (a library
routine, round to nearest even), and closed-form properties of per-block
absmax scaling."""
import numpy as np
import pytest
import torch

from oracle import epilog_oracle as E


def torch_e4m3(q):
    t = torch.from_numpy(np.asarray(q, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_format_definition_values():
    # the special encodings the format defines
    v = E.e4m3_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9                  # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9              # largest subnormal, 0.875 * 2^-6
    assert v(0x08) == 2.0 ** -6                  # smallest normal
    assert v(0x38) == 1.0 and v(0x3F) == 1.875 and v(0x40) == 2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    pos = v(np.arange(127))
    assert np.all(np.diff(pos) > 0)              # codes 0 .. 126 increase


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(E.e4m3_encode(E.e4m3_value(codes)), codes.astype(np.uint8))


def test_ties_go_to_the_even_code():
    pos = E.e4m3_value(np.arange(127))
    mid = (pos[:-1] + pos[1:]) / 2                     # exact in fp64
    got = E.e4m3_encode(mid)
    k = np.arange(126)
    assert np.array_equal(got, np.where(k % 2 == 0, k, k + 1).astype(np.uint8))
    # a hair off the midpoint goes to the nearer value
    eps = (pos[1:] - pos[:-1]) * 1e-3
    assert np.array_equal(E.e4m3_encode(mid - eps), k.astype(np.uint8))
    assert np.array_equal(E.e4m3_encode(mid + eps), (k + 1).astype(np.uint8))
    # worked cases: 1.0625 lies halfway between 1 (0x38) and 1.125 (0x39)
    assert E.e4m3_encode(1.0625) == 0x38 and E.e4m3_encode(1.1875) == 0x3A
    assert E.e4m3_encode(2.0 ** -10) == 0x00 and E.e4m3_encode(3 * 2.0 ** -10) == 0x02


def test_encoder_matches_the_library_conversion():
    rng = np.random.default_rng(20260 + 700)
    pos = E.e4m3_value(np.arange(127)).astype(np.float32)
    mid = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    q = np.concatenate([
        rng.uniform(-448, 448, 200000).astype(np.float32),
        (rng.standard_normal(100000) * rng.choice([1e-3, 1e-2, 1, 30], 100000)).astype(np.float32),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 50000).astype(np.float32),   # subnormal range
        pos, -pos, mid, -mid, np.float32([0.0, -0.0, 448.0, -448.0]),
    ])
    q = np.clip(q, -448, 448).astype(np.float32)
    assert np.array_equal(E.e4m3_encode(q.astype(np.float64)), torch_e4m3(q))


def test_encoder_picks_a_nearest_value():
    rng = np.random.default_rng(20260 + 701)
    q = rng.uniform(-448, 448, 50000)
    c = E.e4m3_encode(q)
    err = np.abs(q - E.e4m3_value(c))
    pos = E.e4m3_value(np.arange(127))
    best = np.min(np.abs(np.abs(q)[:, None] - pos[None, :]), axis=1)
    assert np.array_equal(err, best)


def _blocks(rng, rows, d):
    x = rng.standard_normal((rows, d)).astype(np.float32)
    x *= rng.choice([1e-3, 1.0, 50.0], (rows, d // 128, 1)).repeat(128, axis=2).reshape(rows, d)
    return x


def test_block_scaling_closed_forms():
    rng = np.random.default_rng(20260 + 702)
    x = _blocks(rng, 64, 512)
    codes, scale = E.quantize_rows(x)
    xb = x.reshape(64, 4, 128)
    amax = np.abs(xb).max(axis=2)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest magnitude of every block lands on +-448
    cb = codes.reshape(64, 4, 128)
    idx = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(cb, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # dequantised values within half a step of the E4M3 grid (relative 2^-4
    # for normals, 2^-10 absolute in units of the scale below 2^-6)
    deq = E.e4m3_value(cb) * scale[:, :, None]
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, scale[:, :, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - xb) <= bound)


def test_block_scaling_invariances():
    rng = np.random.default_rng(20260 + 703)
    x = _blocks(rng, 32, 256)
    codes, scale = E.quantize_rows(x)
    # a power-of-two factor moves only the scale
    c2, s2 = E.quantize_rows(x * np.float32(8.0))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale * np.float32(8.0))
    # negation flips the sign bits only
    c3, s3 = E.quantize_rows(-x)
    assert np.array_equal(c3, codes ^ np.uint8(0x80)) and np.array_equal(s3, scale)
    # blocks are independent: changing one block leaves the others alone
    y = x.copy()
    y[:, :128] *= np.float32(3.0)
    c4, s4 = E.quantize_rows(y)
    assert np.array_equal(c4[:, 128:], codes[:, 128:]) and np.array_equal(s4[:, 1:], scale[:, 1:])


def test_zero_block_and_single_spike():
    x = np.zeros((2, 128), np.float32)
    x[1, 5] = -3.0
    codes, scale = E.quantize_rows(x)
    assert scale[0, 0] == 0 and not codes[0].any()
    assert scale[1, 0] == np.float32(3.0) / np.float32(448) and codes[1, 5] == 0xFE
    assert not np.delete(codes[1], 5).any()


def test_placement_by_slot_mapping():
    rng = np.random.default_rng(20260 + 704)
    x = _blocks(rng, 6, 128)
    cache = rng.integers(0, 256, (5, 128), dtype=np.uint8)
    cscale = rng.standard_normal((5, 1)).astype(np.float32)
    slots = np.array([3, -1, 0, 7, -5, 4])
    c, s, err = E.epilog(x, slots, cache, cscale)
    codes, scale = E.quantize_rows(x)
    assert err == E.SLOT_ERROR
    assert np.array_equal(c[3], codes[0]) and np.array_equal(c[0], codes[2])
    assert np.array_equal(c[4], codes[5]) and s[4, 0] == scale[5, 0]
    for untouched in (1, 2):
        assert np.array_equal(c[untouched], cache[untouched]) and s[untouched, 0] == cscale[untouched, 0]
    with pytest.raises(ValueError):
        E.quantize_rows(np.zeros((1, 100), np.float32))
