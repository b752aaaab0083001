"""Pins of the oracle's number formats (CPU only)."""
import json
import math
import os

import numpy as np
import torch

from oracle import numerics
from workloads import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_table_matches_torch_all_codes():
    # library routine: torch's float8_e4m3fn decode, every one of the 256 codes
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    tab = numerics.e4m3fn_table()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    assert np.array_equal(np.signbit(tab[ok]), np.signbit(ref[ok]))


def test_e4m3_hand_decoded_codes():
    g = json.load(open(os.path.join(GOLD, "e4m3fn_codes.json")))
    for code, val, _why in g["codes"]:
        got = numerics.decode_e4m3(np.array([code], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)
    assert np.nanmax(numerics.e4m3fn_table()) == 448.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 10000)
    bits = gen.bf16_bits(x)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(numerics.decode_bf16(bits), ref)


def test_generator_quantizer_error_within_half_spacing():
    # The generator's per-block quantizer, checked with the oracle's decoder:
    # every code must be the nearest E4M3 value of x/scale (|error| <= half the
    # spacing of adjacent codes around it), and the block's largest magnitude
    # maps to exactly 448.
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 64, 32)).astype(np.float32)
    codes, scale = gen.quantize_e4m3_blocks(x)
    vals = numerics.decode_e4m3(codes)
    y = x.astype(np.float64) / scale.astype(np.float64)[:, None, None]
    tab = numerics.e4m3fn_table()
    finite = np.sort(np.unique(tab[~np.isnan(tab)]))
    idx = np.searchsorted(finite, y)
    lo = finite[np.clip(idx - 1, 0, len(finite) - 1)]
    hi = finite[np.clip(idx, 0, len(finite) - 1)]
    best = np.minimum(np.abs(y - lo), np.abs(y - hi))
    assert np.all(np.abs(vals - y) <= best + 1e-6 * np.abs(y))
    amax_code = np.abs(vals).reshape(64, -1).max(axis=1)
    assert np.all(amax_code == 448.0)
