"""GPU parity of the FP8 KV row format against the oracle, bit for bit:
csa_dequantize_rows on rows holding every E4M3 code under many block
exponents, and csa_quantize_rows on bf16 rows whose blocks span zero,
subnormal-range, tie and boundary values."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_dequantize_every_code_and_exponent(orc):
    rng = np.random.default_rng(21)
    R = 64
    rows = np.zeros((R, 640), dtype=np.uint8)
    rows[:, :448] = np.tile(np.arange(256, dtype=np.uint8), 112)[: R * 448].reshape(R, 448)
    rng.shuffle(rows[:, :448], axis=1)
    rows[:, 448:576] = W.bf16_bits(rng.standard_normal((R, 64)).astype(np.float32)).view(np.uint8).reshape(R, 128)
    rows[:, 576:583] = rng.integers(-40, 41, size=(R, 7)).astype(np.int8).view(np.uint8)
    print(f"[fp8] dequantize {R} rows", flush=True)
    got = _bits(K.csa_dequantize_rows(torch.from_numpy(rows).cuda()))
    ref = orc.dequantize_rows_fp8(rows)
    nan = np.isnan(ref)
    got_f = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(np.isnan(got_f), nan)
    assert np.array_equal(got[~nan], orc.round_bf16(ref[~nan]))
    # every value is exact: the oracle's fp64 value is a bf16 value
    assert np.array_equal((got[~nan].astype(np.uint32) << 16).view(np.float32).astype(np.float64), ref[~nan])


def _hard_rows(rng, R):
    x = rng.standard_normal((R, 512)).astype(np.float32)
    scale = np.exp2(rng.integers(-30, 20, size=(R, 8))).astype(np.float32)
    x *= np.repeat(scale, 64, axis=1)
    x[0, :64] = 0.0                                             # all-zero block
    x[1, :64] = 1e-30                                           # tiny block
    x[2, 64:128] = 0.0
    x[2, 64] = 448.0 * 2.0 ** 3                                 # maximum exactly on a boundary
    x[3, :64] = rng.choice([-1.0, 1.0], 64) * np.float32(1.0)
    x[3, 1:9] = np.array([1.0625, 1.1875, 1.3125, 1.4375, 1.5625, 1.6875, 1.8125, 1.9375], np.float32) / 256
    x[4, :64] = np.float32(2.0 ** -20) * rng.standard_normal(64).astype(np.float32)
    x[4, 0] = 1.0                                               # wide block: most values in the subnormal range
    return W.bf16_bits(x)


def test_quantize_matches_oracle_bit_for_bit(orc):
    rng = np.random.default_rng(22)
    R = 1000
    bits = _hard_rows(rng, R)
    print(f"[fp8] quantize {R} rows", flush=True)
    dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    got = K.csa_quantize_rows(dev).cpu().numpy()
    ref = orc.quantize_rows_fp8(orc.widen(bits))
    assert np.array_equal(got, ref)
    back = _bits(K.csa_dequantize_rows(K.csa_quantize_rows(dev)))
    assert np.array_equal(back, orc.round_bf16(orc.dequantize_rows_fp8(ref)))


def test_quantize_empty_and_odd_counts(orc):
    rng = np.random.default_rng(23)
    for R in (0, 1, 5):
        bits = W.bf16_bits(rng.standard_normal((R, 512)).astype(np.float32))
        dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16).reshape(R, 512)
        got = K.csa_quantize_rows(dev).cpu().numpy()
        assert got.shape == (R, 640)
        if R:
            assert np.array_equal(got, orc.quantize_rows_fp8(orc.widen(bits)))
