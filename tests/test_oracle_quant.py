"""Pins of the quantised-cache oracle (FP4 E2M1 latent, FP8 E4M3 RoPE tail,
power-of-two scales per 32 channels) against facts fixed by the formats and
by an independent library (torch's float8_e4m3fn), a hand-worked row, and
invariants (no clipping, minimal scale, idempotence).  Source: "Lab tổng hợp
DeepSeek-V4.1-Flash", section "3 Giải pháp" (FP4 E2M1 latent, FP8 E4M3 rope
tail); the block scaling and the row layout are readings stated in
oracle/quant.py."""
import numpy as np
import pytest
import torch

from oracle import quant as Q
from tests.conftest import read_golden


def test_e2m1_codes_decode_to_the_format_table():
    """Sign, 2 exponent bits (bias 1), 1 mantissa bit: the eight magnitudes of
    the format, positive codes 0..7 and their negatives 8..15."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = Q.e2m1_decode(np.arange(16))
    assert list(got[:8]) == mags
    assert list(got[8:]) == [-m for m in mags]
    assert np.signbit(got[8])                        # code 8 is negative zero


def test_e4m3_codes_match_torch_float8_e4m3fn():
    """All 256 codes against torch's float8_e4m3fn (an independent decoder):
    the same finite values, NaN exactly at S.1111.111, largest 448."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = Q.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.nanmax(got) == 448.0 and set(np.nonzero(np.isnan(got))[0]) == {0x7F, 0xFF}


def test_e4m3_rounding_matches_torch_conversion():
    """Round to nearest, ties to even, negative values that round to zero
    keep their sign: the oracle's table search against torch's float ->
    float8_e4m3fn conversion on random values, every midpoint between
    neighbouring codes and the subnormal range."""
    rng = np.random.default_rng(0)
    vals = Q.e4m3_decode(np.arange(256))
    fin = np.sort(np.unique(vals[~np.isnan(vals)]))
    mids = (fin[1:] + fin[:-1]) / 2
    y = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.02, 0.02, 2000), mids,
                        [0.0, -0.0, 1e-9, -1e-9, 448.0, -448.0]])
    direct = Q._nearest_code(y, Q._E4M3_CODES, Q._E4M3_VALUES, 0x80)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(direct, ref)


def test_e2m1_midpoints_round_to_the_even_code():
    """Every midpoint between neighbouring E2M1 magnitudes goes to the code
    whose last bit is 0: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4,
    5->4 (and the same with a minus sign); values just off a midpoint go to
    the nearer side."""
    mid = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    for sign in (1.0, -1.0):
        y = sign * np.array(mid)
        got = Q.e2m1_decode(Q._nearest_code(y, Q._E2M1_CODES, Q._E2M1_VALUES, 8))
        assert list(got) == [sign * w for w in want]
        lo = Q.e2m1_decode(Q._nearest_code(y - sign * 1e-9, Q._E2M1_CODES, Q._E2M1_VALUES, 8))
        hi = Q.e2m1_decode(Q._nearest_code(y + sign * 1e-9, Q._E2M1_CODES, Q._E2M1_VALUES, 8))
        assert list(lo) == [sign * v for v in [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]]
        assert list(hi) == [sign * v for v in [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]]


@pytest.mark.parametrize("fmt,fmax", [("e2m1", 6.0), ("e4m3", 448.0)])
def test_block_scale_is_the_smallest_without_clipping(fmt, fmax):
    """max|v| / 2^x <= the format's largest value, and 2^(x-1) would clip;
    exact boundary cases by hand (a block max of exactly 6 scales by 2^0, a
    hair above by 2^1, 3 by 2^-1)."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        b = rng.standard_normal(32) * np.exp2(rng.integers(-20, 20))
        x = Q.block_scale_exp(b, fmax)
        a = np.max(np.abs(b))
        assert a / 2.0 ** x <= fmax < a / 2.0 ** (x - 1)
    if fmt == "e2m1":
        assert Q.block_scale_exp(np.r_[6.0, np.zeros(31)], 6.0) == 0
        assert Q.block_scale_exp(np.r_[6.0 + 1e-12, np.zeros(31)], 6.0) == 1
        assert Q.block_scale_exp(np.r_[-3.0, np.zeros(31)], 6.0) == -1
    assert Q.block_scale_exp(np.zeros(32), fmax) == -127


def test_hand_worked_row():
    """A 64-wide entry with a 32-wide RoPE tail, worked by hand
    (tests/golden/quant_row.txt)."""
    g = read_golden("quant_row.txt")
    v = np.array([float(t) for t in g["values"]])
    want = np.array([int(t, 16) for t in g["bytes"]], dtype=np.uint8)
    got = Q.quantize_row(v, int(g["rope_dim"][0]))
    assert got.shape == (int(g["row_bytes"][0]),)
    assert np.array_equal(got, want)
    deq = Q.dequantize_row(got, len(v), int(g["rope_dim"][0]))
    assert np.array_equal(deq, np.array([float(t) for t in g["dequantized"]]))


def test_quantisation_is_idempotent_and_bounded():
    """Values a row stands for are representable: quantising them again
    gives back the same values (the bytes may differ only in a block whose
    largest value rounded down to half the format's maximum, which then takes
    a scale one step smaller); every element lands within half a code step
    (times the block scale) of its value; the Flash row (512 wide, 64-wide
    tail) takes 304 bytes."""
    rng = np.random.default_rng(2)
    assert Q.row_bytes(512, 64) == 304
    for _ in range(20):
        v = rng.standard_normal(512)
        v /= np.sqrt(np.mean(v * v))
        row = Q.quantize_row(v, 64)
        deq = Q.dequantize_row(row, 512, 64)
        assert np.array_equal(Q.dequantize_row(Q.quantize_row(deq, 64), 512, 64), deq)
        for lo, hi, fmt, step in ((0, 448, "e2m1", 1.0), (448, 512, "e4m3", 1 / 16)):
            for b in range(lo, hi, 32):
                blk = v[b:b + 32]
                x = Q.block_scale_exp(blk, 6.0 if fmt == "e2m1" else 448.0)
                # half the widest relative spacing of the format (E2M1: 4 -> 6;
                # E4M3: 2^-3 of the value) times the scale
                bound = 2.0 ** x * step if fmt == "e2m1" else np.abs(blk) / 16 + 2.0 ** (x - 9)
                assert np.all(np.abs(deq[b:b + 32] - blk) <= bound + 1e-15)
