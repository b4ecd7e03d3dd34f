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


def test_encode_saturates_and_applies_the_scale_in_binary32():
    big = np.array([449.0, 463.9, 464.0, 1e6, np.inf, -1e30], dtype=np.float32)
    enc = oracle.e4m3fn_encode(big, np.float32(1.0))
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    # the product is rounded to binary32 before the code is chosen
    s = 0.1
    inv = oracle.inv_scale_f32(s)
    assert inv == np.float32(np.float32(1.0) / np.float32(0.1))
    x = np.array([0.013, -0.7, 3.3], dtype=np.float32)
    y = (x * inv).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(x, inv), oracle.e4m3fn_encode(y, np.float32(1.0)))
