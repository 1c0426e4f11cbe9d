"""CPU pins of the oracle's FP8 cache rows ("图解DeepSeek V4：详细计算流程解析" 2:
the non-RoPE part of a KV row is quantised).  The E4M3 decode and the
round-to-nearest-even encode are checked against PyTorch's float8_e4m3fn on
the CPU (a library routine), the block exponent against brute force, the row
layout and round trip against closed forms."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc


def _torch_codes(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9 and got[8] == 2.0 ** -6


def test_e4m3_encode_matches_torch_on_ties_and_random_values():
    vals = orc.e4m3_value(np.arange(127, dtype=np.uint8))          # every non-negative finite value
    mids = (vals[:-1] + vals[1:]) / 2                                # exact ties (representable in fp32)
    rng = np.random.default_rng(0)
    rand = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 20000),
                           np.ldexp(rng.uniform(1, 2, 5000), rng.integers(-12, 9, 5000))])
    rand = np.clip(rand, -448, 448).astype(np.float32).astype(np.float64)
    for v in (vals, -vals, mids, -mids, rand):
        got = orc.e4m3_rne(v)
        ref = _torch_codes(v)
        # +0 and -0 both decode to zero; torch keeps the sign bit, so compare values
        assert np.array_equal(orc.e4m3_value(got), orc.e4m3_value(ref))
    # a tie goes to the even code: halfway between 1.0 (code 0x38) and 1.125 (0x39) -> 0x38,
    # between 1.125 and 1.25 (0x3A) -> 0x3A
    assert orc.e4m3_rne(np.array([1.0625, 1.1875])).tolist() == [0x38, 0x3A]
    with pytest.raises(ValueError):
        orc.e4m3_rne(np.array([449.0]))


def test_block_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 3000), rng.integers(-30, 30, 3000)),
                           np.ldexp(448.0, np.arange(-20, 20)), np.ldexp(448.0, np.arange(-20, 20)) * (1 + 1e-12)])
    k = orc.fp8_block_exp(amax)
    for a, kk in zip(amax, k):
        assert a <= 448.0 * 2.0 ** kk
        assert a > 448.0 * 2.0 ** (kk - 1)
    assert orc.fp8_block_exp(np.array([0.0]))[0] == 0


def test_row_layout_and_round_trip():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 512)) * np.array([0.01, 1.0, 30.0, 1e-3, 7.0])[:, None]
    x[3, :64] = 0.0                                                  # an all-zero block
    rows = orc.quantize_rows_fp8(x)
    assert rows.shape == (5, 640) and rows.dtype == np.uint8
    k = rows[:, 576:583].view(np.int8).astype(np.int64)
    assert np.all(rows[:, 583:] == 0)
    assert k[3, 0] == 0 and np.all(rows[3, :64] == 0)
    # rope dims: the bf16 rounding of the value, bit for bit
    assert np.array_equal(rows[:, 448:576].view(np.uint16), orc.round_bf16(x[:, 448:]))
    # codes: E4M3 of x / 2^k per 64-dim block, so the dequantised value is within half a step
    d = orc.dequantize_rows_fp8(rows)
    xb = x[:, :448].reshape(5, 7, 64)
    a = np.abs(xb) / np.ldexp(1.0, k)[..., None]
    _, E = np.frexp(np.maximum(a, 2.0 ** -6))
    half_step = np.ldexp(1.0, k)[..., None] * np.ldexp(1.0, E - 1 - 3) / 2
    assert np.all(np.abs(d[:, :448].reshape(5, 7, 64) - xb) <= half_step * (1 + 1e-12))
    # the block maximum maps into (224, 448]: the exponent uses the whole range
    top = np.max(a, axis=-1)
    nz = np.max(np.abs(xb), axis=-1) > 0
    assert np.all((top[nz] > 224.0) & (top[nz] <= 448.0))
    # values already on the grid survive exactly (the codes may change with the
    # block exponent when the rounded maximum crosses a power of two)
    assert np.array_equal(orc.dequantize_rows_fp8(orc.quantize_rows_fp8(d)), d)


def test_quantisation_decides_in_float32():
    """The codes are taken from the float32 value, the kernels' precision: a
    value just above a tie in fp64 that float32 rounds onto the tie gets the
    tie's even code."""
    x = np.zeros((1, 512))
    x[0, :64] = 1.0                                   # block maximum 1 -> k = -8 (0.875 < 1 <= 1.75)
    assert orc.fp8_block_exp(np.array([1.0]))[0] == -8
    tie = 1.0625 / 256                                # 1.0625 after scaling: between codes 0x38 and 0x39
    x[0, 1] = tie * (1 + 2.0 ** -40)
    assert float(np.float32(x[0, 1])) == tie
    assert orc.quantize_rows_fp8(x)[0, 1] == 0x38
    assert orc.quantize_rows_fp8(x, decide_in_float32=False)[0, 1] == 0x39
