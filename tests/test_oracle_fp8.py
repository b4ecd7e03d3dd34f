"""Exhaustive pins of the oracle's OCP e4m3fn codec (CPU only)."""
import math

import numpy as np
import torch

import oracle


def _finite_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3fn_to_f64(codes)
    return codes, vals


def test_decode_spot_values_from_the_definition():
    v = oracle.e4m3fn_to_f64(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x7E, 0x80, 0x81, 0xFE],
                                      dtype=np.uint8))
    assert list(v) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 448.0, -0.0,
                       -(2.0 ** -9), -448.0]
    assert math.copysign(1.0, v[7]) < 0
    nan = oracle.e4m3fn_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan))


def test_decode_matches_torch_on_every_code():
    codes, vals = _finite_table()
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(vals) & np.isnan(ref)
    assert np.array_equal(vals[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(vals), np.isnan(ref))
    assert int(np.sum(np.isnan(vals))) == 2          # 254 finite codes, 253 distinct values


def test_every_finite_code_round_trips():
    codes, vals = _finite_table()
    fin = ~np.isnan(vals)
    enc = oracle.e4m3fn_encode(vals[fin].astype(np.float32), np.float32(1.0))
    # -0 and +0 keep their sign bit
    assert np.array_equal(enc, codes[fin])


def test_encode_all_fp16_inputs_brute_force_nearest():
    """Every fp16 bit pattern: the code is the nearest finite e4m3fn value to
    clamp(x, +-448), ties to the code with an even mantissa field."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    enc = oracle.e4m3fn_encode(x, np.float32(1.0))
    codes, vals = _finite_table()
    fin = ~np.isnan(vals)
    fcodes, fvals = codes[fin], vals[fin]
    for xi, ci in zip(x.tolist(), enc.tolist()):
        if xi != xi:
            assert ci & 0x7F == 0x7F
            continue
        y = max(-448.0, min(448.0, xi))
        d = np.abs(fvals - y)
        best = d.min()
        cands = [int(c) for c in fcodes[d == best]]
        # +-0 tie: the sign follows the input
        if best == 0.0 and y == 0.0:
            want = 0x80 if math.copysign(1.0, xi) < 0 else 0x00
        else:
            same_sign = [c for c in cands if (c & 0x80) == (0x80 if y < 0 else 0)] or cands
            even = [c for c in same_sign if c % 2 == 0]
            want = even[0] if len(same_sign) > 1 else same_sign[0]
        assert ci == want, (xi, ci, want)


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 50, 20000), rng.uniform(-448, 448, 20000),
                        rng.normal(0, 2.0 ** -8, 5000)]).astype(np.float32)
    enc = oracle.e4m3fn_encode(x, np.float32(1.0))
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, ref)


def test_encode_saturates():
    big = np.array([449.0, 463.9, 464.0, 1e6, np.inf, -1e30], dtype=np.float32)
    enc = oracle.e4m3fn_encode(big, np.float32(1.0))
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def _f32(bits: int) -> np.float32:
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def test_quantiser_takes_the_binary32_reciprocal_and_a_binary32_product():
    """Codes worked out by hand from the e4m3fn definition and binary32
    rounding.  The quantiser's reading (the feature list names only "FP8 KV
    cache"): code = e4m3fn(RNE(fp32(x * fp32(1 / fp32(scale))))).  Each case is
    chosen so that dividing x by the scale, or keeping the reciprocal or the
    product in fp64, lands on the other side of an e4m3fn rounding boundary.

    Case A, scale 0.1:
      fp32(0.1) = 0x3DCCCCCD = 0.100000001490116...; 1/that = 9.99999985098839,
      which is 1.49e-7 below 10 while binary32 spacing in [8, 16) is 2^-20 =
      9.5e-7, so fp32(1/scale) = 10 exactly.
      x = 0x3F466666 = 0.77499997615814208984375; x * 10 = 7.75 - 2^-22
      exactly, the midpoint between the binary32 neighbours 7.75 - 2^-21 and
      7.75 (spacing 2^-21 in [4, 8)); ties-to-even picks 7.75 (0x40F80000,
      even significand).  In e4m3fn, 7.75 is the midpoint of 7.5 (1.875 * 2^2,
      mantissa 7, code 0x4F) and 8 (exponent field 10, mantissa 0, code 0x50);
      ties-to-even gives 8: code 0x50.
      Division: x / 0x3DCCCCCD = 7.7499996461..., 3.5e-7 below 7.75 (more than
      half a spacing, 2^-22 = 2.4e-7), so binary32 keeps it below 7.75 (it
      becomes 7.75 - 2^-21) -> 7.5 -> 0x4F.  An fp64
      product x * 10 = 7.7499997615... is below 7.75 too -> 0x4F.

    Case B, scale 0.3:
      fp32(0.3) = 0x3E99999A = 0.300000011920928955078125; 1/that =
      3.33333320087857...; the binary32 neighbours are 0x40555554 =
      3.33333301544 and 0x40555555 = 3.33333325386, and the latter is nearer:
      fp32(1/scale) = 3.3333332538604736.
      x = 0x3F700001 = 0.9375 + 2^-24; x * 3.3333332538604736 = 3.12500023841...,
      which binary32 rounds to 3.125 + 2^-22 (0x40480001), above the e4m3fn
      midpoint 3.125 of 3.0 (code 0x44) and 3.25 (code 0x45): code 0x45.
      Division: x / 0.3000000119 = 3.1250000745..., within half a spacing
      (2^-23) of 3.125, so binary32 rounds it to the midpoint 3.125 itself and
      ties-to-even gives 3.0 (mantissa 4) over 3.25 (mantissa 5): code 0x44.
    """
    inv_a = oracle.inv_scale_f32(0.1)
    assert inv_a == np.float32(10.0)
    assert oracle.quantise_e4m3fn(np.array([_f32(0x3F466666)]), 0.1)[0] == 0x50
    assert oracle.quantise_e4m3fn(np.array([-_f32(0x3F466666)]), 0.1)[0] == 0xD0

    inv_b = oracle.inv_scale_f32(0.3)
    assert inv_b.view(np.uint32) == 0x40555555
    assert oracle.quantise_e4m3fn(np.array([_f32(0x3F700001)]), 0.3)[0] == 0x45
    # the same x with scale 1: 0.9375 + 2^-24 rounds to 0.9375 (code 0x37)
    assert oracle.quantise_e4m3fn(np.array([_f32(0x3F700001)]), 1.0)[0] == 0x37


def test_cache_write_fp8_code_of_a_bf16_value_at_a_rounding_boundary():
    """One bf16 value through the oracle's cache write, scale 0.3, code worked
    out by hand: x = bf16 0x3B90 = 1.125 * 2^-8 = 0.00439453125; times
    fp32(1/0.3) = 3.3333332538604736 it is 0.0146484371507..., 3.5e-10 below
    0.0146484375 = 15 * 2^-10 while binary32 spacing there is 2^-30 = 9.3e-10,
    so the binary32 product is 0.0146484375 exactly: the midpoint of the
    largest e4m3fn subnormal 7 * 2^-9 (code 0x07, odd mantissa) and the
    smallest normal 2^-6 (code 0x08, even mantissa): code 0x08.  Dividing by
    the scale gives 0.0146484369... < the midpoint, code 0x07."""
    k = np.full((1, 1, 64), 0x3B90, dtype=np.uint16)
    v = np.full((1, 1, 64), 0xBB90, dtype=np.uint16)                 # -x
    kc = np.zeros((2, 1, 16, 64), dtype=np.uint8)
    vc = np.zeros((2, 1, 4, 64, 4), dtype=np.uint8)
    kc2, vc2 = oracle.cache_write(k, v, kc, vc, np.array([21], dtype=np.int32), 16, "e4m3fn",
                                  k_scale=0.3, v_scale=0.3)
    assert np.all(kc2[1, 0, 5] == 0x08)
    assert np.all(vc2[1, 0, 1, :, 1] == 0x88)
    kc2[1, 0, 5] = 0
    vc2[1, 0, 1, :, 1] = 0
    assert not kc2.any() and not vc2.any()
