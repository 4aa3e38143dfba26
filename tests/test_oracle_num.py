"""Pins for the storage decoding the oracle applies to every input (CPU only).

bf16 is the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent, 7 fraction
bits).  ``oracle.num.f64`` turns the stored bit patterns into exact fp64
values; these tests check it against torch's own bfloat16 type, which is an
independent decoder, over every one of the 65,536 patterns, and against
values worked out by hand from the format.  ``synth.to_bf16`` (the encoder
that makes the stored patterns) is checked against torch's float32 ->
bfloat16 cast, which rounds to nearest even.
"""
import numpy as np
import torch

import oracle
import synth


def _torch_bf16_decode(u16):
    return torch.from_numpy(u16.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def test_bf16_decode_all_patterns_match_torch():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        got = oracle.num.f64(u)
    ref = _torch_bf16_decode(u)
    assert got.dtype == np.float64 and got.shape == (1 << 16,)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # the sign of zero survives the decoding
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # 0x7f81..0x7fff and 0xff81..0xffff are NaN: 2 * 127 patterns
    assert int(nan.sum()) == 254


def test_bf16_decode_hand_values():
    cases = {
        0x0000: 0.0, 0x8000: -0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0,
        0x3F00: 0.5, 0x3FC0: 1.5, 0x4049: 3.140625,           # 1.5703125 * 2
        0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,                    # largest finite
        0x0080: 2.0 ** -126,                                   # smallest normal
        0x0001: 2.0 ** -133,                                   # smallest subnormal
        0x007F: (1 - 2 ** -7) * 2.0 ** -126,                   # largest subnormal
        0x7F80: np.inf, 0xFF80: -np.inf,
        0xC2F7: -123.5,                                        # -(1 + 119/128) * 64
    }
    u = np.array(list(cases), dtype=np.uint16)
    got = oracle.num.f64(u)
    np.testing.assert_array_equal(got, np.array(list(cases.values()), dtype=np.float64))
    assert np.signbit(oracle.num.f64(np.array([0x8000], np.uint16)))[0]
    with np.errstate(invalid="ignore"):
        assert np.isnan(oracle.num.f64(np.array([0x7FC0, 0xFFC1, 0x7F81], np.uint16))).all()


def test_f64_passes_other_types_through():
    x = np.array([1.5, -2.25, 3e-8], np.float32)
    np.testing.assert_array_equal(oracle.num.f64(x), x.astype(np.float64))
    h = np.array([1.5, -0.0009765625, 65504.0], np.float16)
    np.testing.assert_array_equal(oracle.num.f64(h), h.astype(np.float64))


def test_to_bf16_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(20_000) * 1e30).astype(np.float32),
        (rng.standard_normal(20_000) * 1e-38).astype(np.float32),   # subnormals of fp32
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38], np.float32),
    ])
    # exact ties between two bf16 neighbours (low 16 bits = 0x8000), both parities
    ties = (rng.integers(0x0080, 0x7F00, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = synth.to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    # ties go to the even neighbour
    t = np.array([0x3F808000, 0x3F818000], np.uint32).view(np.float32)
    np.testing.assert_array_equal(synth.to_bf16(t), np.array([0x3F80, 0x3F82], np.uint16))


def test_store_then_decode_is_within_half_ulp():
    x = np.random.default_rng(9).standard_normal(100_000).astype(np.float32)
    back = oracle.num.f64(synth.store(x, "bf16"))
    # bf16 keeps 8 significant bits: round to nearest stays within the unit
    # roundoff 2^-8 relative (truncation would reach 2^-7), and N(0,1)
    # samples come close to that bound
    err = np.abs(back - x.astype(np.float64)) / np.abs(x.astype(np.float64))
    assert err.max() <= 2.0 ** -8
    assert err.max() > 2.0 ** -9
