"""Pins for per-row symmetric INT8/FP8 quantisation and the E4M3FN codec."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_handworked_int8():
    gold = json.load(open(os.path.join(GOLD, "handworked.json")))
    for case in gold["int8"]:
        codes, s = oracle.quant_rows(np.array([case["row"]], np.float32), "i8")
        assert codes[0].tolist() == case["codes"], case
        if "scale" in case:
            assert float(s[0]) == case["scale"]


def test_e4m3_table_facts():
    v = oracle.e4m3_values()
    assert len(v) == 127 and v[-1] == 448.0 and v[1] == 2.0 ** -9
    assert np.all(np.diff(v) > 0)
    assert oracle.e4m3_decode(np.array([0x38], np.uint8))[0] == 1.0  # exponent bias 7
    assert oracle.e4m3_decode(np.array([0xFE], np.uint8))[0] == -448.0


def test_e4m3_encode_matches_torch_everywhere_in_range():
    # every bf16 value with |x| <= 448, plus many float32 values between
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    rng = np.random.default_rng(5)
    y = rng.uniform(-448, 448, 200000).astype(np.float32)
    z = (rng.uniform(-1, 1, 100000) * 2.0 ** rng.integers(-12, 0, 100000)).astype(np.float32)
    allx = np.concatenate([x, y, z])
    ours = oracle.e4m3_encode(allx)
    ref = torch.from_numpy(allx).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates():
    big = np.array([448.0, 449.0, 470.0, 1e6, -1e6], np.float32)
    assert oracle.e4m3_encode(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (np.arange(1 << 16, dtype=np.uint32) << 15 | 0x8000).view(np.float32)])
    x = x[np.isfinite(x)]
    ours = oracle.f32_to_bf16_bits_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("q", ["i8", "fp8"])
def test_quant_rows_properties(q):
    rng = np.random.default_rng(7)
    v = rng.standard_normal((64, 1000)).astype(np.float32) * rng.uniform(0.01, 50, (64, 1))
    v[3] = 0
    codes, s = oracle.quant_rows(v, q)
    Q = 127 if q == "i8" else 448
    dec = codes.astype(np.float64) if q == "i8" else oracle.e4m3_decode(codes)
    a = np.abs(v).max(1)
    assert s[3] == 0 and np.all(dec[3] == 0)
    nz = a > 0
    # the row maximum maps to the largest code exactly
    am = np.argmax(np.abs(v), axis=1)
    assert np.all(np.abs(dec[np.arange(64), am])[nz] == Q)
    # reconstruction error: half a step (INT8) or half a ulp of E4M3 (relative 2^-4)
    err = np.abs(dec * s[:, None].astype(np.float64) - v)
    if q == "i8":
        assert np.all(err <= s[:, None] * (0.5 + 1e-5) + 1e-12)
    else:
        bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-5)
        assert np.all(err <= bound + 1e-12)
