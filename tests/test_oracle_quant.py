"""Pins of the oracle's E4M3 query quantization (CPU only).

The encoder is checked against torch's float8_e4m3fn cast (a library routine)
on every code value, every tie and random values; the quantization rule
against hand-worked heads (tests/golden/quant_tiny.json) and against
properties any correct implementation has (the largest magnitude of a head
lands on 448, the relative error is at most half a code step, the scale folds
into the head weight).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import indexer, numerics, quant
from workloads import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_encoder_matches_torch_on_codes_ties_and_random_values():
    tab = numerics.e4m3fn_table()
    pos = tab[:0x7F]                                  # 0 .. 448
    mids = (pos[:-1] + pos[1:]) / 2                   # every tie between neighbours
    rng = np.random.default_rng(0)
    rnd = np.exp2(rng.uniform(-14, np.log2(463.9), 200_000)) * rng.choice([-1, 1], 200_000)
    # codes and ties are exact binary32 values, so the ties really are ties
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)
    for vals in (pos, -pos, mids, -mids, rnd, np.array([448.5, 463.9, -460.0])):
        x = np.asarray(vals, dtype=np.float32)
        assert np.array_equal(quant.encode_e4m3_rne(x), _torch_codes(x))


def test_encoder_round_trip_and_range():
    tab = numerics.e4m3fn_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    assert np.array_equal(quant.encode_e4m3_rne(tab[codes].astype(np.float32)), codes)
    with pytest.raises(ValueError):
        quant.encode_e4m3_rne(np.array([464.0], dtype=np.float32))
    with pytest.raises(ValueError):
        quant.encode_e4m3_rne(np.array([np.nan], dtype=np.float32))


def test_quantize_hand_worked_heads():
    g = json.load(open(os.path.join(GOLD, "quant_tiny.json")))
    for head in g["heads"]:
        q = np.array(head["q"], dtype=np.float32)
        bits = gen.bf16_bits(q)
        assert np.array_equal(numerics.decode_bf16(bits), q.astype(np.float64))   # bf16-exact inputs
        codes, ws, s = quant.quantize_queries(bits[None, :], np.array([head["w"]], np.float32))
        assert codes[0].tolist() == head["codes"], head["derivation"]
        vals = numerics.decode_e4m3(codes[0])
        assert np.array_equal(vals, np.array(head["values"]))
        assert np.array_equal(np.signbit(vals), np.signbit(np.array(head["values"])))
        assert s[0] == np.float32(head["s"])
        assert ws[0] == np.float32(head["w_scaled"])


def test_quantize_properties_on_random_heads():
    rng = np.random.default_rng(1)
    B, P, H, D = 3, 2, 16, 128
    q = (rng.standard_normal((B, P, H, D)) * np.exp(rng.uniform(-6, 6, (B, P, H, 1)))).astype(np.float32)
    q[0, 0, 3] = 0.0                                   # one all-zero head
    bits = gen.bf16_bits(q)
    qv = numerics.decode_bf16(bits)
    w = rng.standard_normal((B, P, H)).astype(np.float32)
    codes, ws, s = quant.quantize_queries(bits, w)
    vals = numerics.decode_e4m3(codes)
    amax = np.abs(qv).max(axis=-1)
    nz = amax >= 2.0 ** -64
    # the head's largest magnitude becomes exactly 448
    assert np.all(np.abs(vals).max(axis=-1)[nz] == 448.0)
    assert np.all(codes[~nz] == 0) and np.all(s[~nz] == 0) and np.all(ws[~nz] == 0)
    # dequantized value within half a code step: 2^-4 relative for normal
    # codes, 2^-10 absolute (times s) in the subnormal range
    deq = vals * s[..., None].astype(np.float64)
    err = np.abs(deq - qv)
    bound = np.maximum(np.abs(qv) * 2.0 ** -4, s[..., None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    # sign preserved wherever the code is not zero
    assert np.all(np.sign(vals[vals != 0]) == np.sign(qv[vals != 0]))
    assert np.array_equal(ws, (w * s).astype(np.float32))


def test_quantized_scores_track_bf16_scores():
    # With non-negative queries, keys and weights every dot product is a sum
    # of non-negative terms, so the quantized score is within the queries'
    # relative rounding (2^-4, plus the subnormal floor) of the exact one.
    # A wrong fold of the scale (w / s, or s missing) fails by orders of
    # magnitude.
    rng = np.random.default_rng(2)
    B, P, H, D, T = 1, 1, 16, 128, 256
    q = np.abs(rng.standard_normal((B, P, H, D))).astype(np.float32) * 3.0
    bits = gen.bf16_bits(q)
    w = rng.uniform(0.1, 1.0, (B, P, H)).astype(np.float32)
    k = np.abs(rng.standard_normal((T // 64, 64, D))).astype(np.float32)
    bt = np.arange(T // 64, dtype=np.int32)[None, :]
    ctx = np.array([T], dtype=np.int32)
    ref = indexer.indexer_scores(bits, "bf16", w, k, "f32", None, bt, ctx)
    codes, ws, _ = quant.quantize_queries(bits, w)
    got = indexer.indexer_scores(codes, "e4m3", ws, k, "f32", None, bt, ctx)
    rel = np.abs(got - ref) / ref
    assert np.all(rel[0, 0, :T] <= 2.0 ** -4 + 1e-3)
    assert rel[0, 0, :T].mean() < 0.02
