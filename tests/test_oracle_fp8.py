"""Pins for the oracle's FP8 path (quantise before dispatch; the low-latency
section of the event-driven EP scheduling page: FP8 on the wire, combine in
BF16; the memory-layout section of the DeepEP study notes: scales travel in
the payload).

Pinned against: torch's CPU cast to float8_e4m3fn (OCP E4M3FN, nearest-even)
over a structured sweep of fp32 bit patterns that reaches every rounding
decision, the decode table of all 256 codes, numpy's IEEE fp32 division for
the scale and the per-element quotient, hand-worked codes, and the
round-trip error bound of a 3-bit-mantissa format.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example_r4_e8_k2.json")


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _structured_patterns() -> np.ndarray:
    """Every (sign, exponent, top-7-mantissa) prefix combined with low halves
    that select exact values, ties, just-above/below-tie and sticky cases."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000,
                     0x1234, 0xFEDC], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    return pats


def test_encoder_matches_torch_structured(orc):
    pats = _structured_patterns()
    v = pats.view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= 464.0)
    v = v[keep]
    ours = orc.e4m3_rne_array(v)
    theirs = _torch_e4m3(v)
    bad = np.flatnonzero(ours != theirs)
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {v[bad[:5]]} -> {ours[bad[:5]]} vs {theirs[bad[:5]]}"


def test_encoder_matches_torch_random(orc):
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = pats.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 464.0)]
    # also dense coverage of the useful range
    v = np.concatenate([v, (rng.standard_normal(2_000_000) * 100).astype(np.float32),
                        np.float32(2.0) ** rng.uniform(-12, -5, 1_000_000).astype(np.float32)])
    v = v[np.abs(v) <= 464.0]
    np.testing.assert_array_equal(orc.e4m3_rne_array(v), _torch_e4m3(v))


def test_saturation_and_specials(orc):
    assert orc.e4m3_rne(448.0) == 0x7E
    assert orc.e4m3_rne(464.0) == 0x7E          # tie between 448 and 480: even mantissa
    assert orc.e4m3_rne(1e9) == 0x7E            # saturates (unreachable for scaled inputs)
    assert orc.e4m3_rne(-1e9) == 0xFE
    assert orc.e4m3_rne(-0.0) == 0x80
    assert orc.e4m3_rne(float("nan")) == 0x7F


def test_decode_table_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.array([orc.e4m3_to_f32(int(c)) for c in codes], np.float32)
    finite = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    assert np.isnan(ours[~finite]).all()
    # decoding then re-encoding is the identity on every finite code
    np.testing.assert_array_equal(orc.e4m3_rne_array(ours[finite]), codes[finite])


def test_worked_codes(orc):
    with open(GOLD) as f:
        g = json.load(f)["fp8"]
    x = np.zeros(128, np.float32)
    x[:len(g["values"])] = g["values"]
    xb = synth.to_bf16_bits(x)[None, :]
    q, s = orc.quantize_rows(xb)
    assert s[0, 0] == np.float32(g["scale"])
    assert q[0, :len(g["codes"])].tolist() == g["codes"]
    assert (q[0, len(g["codes"]):] == 0).all()


def test_zero_group_uses_floor(orc):
    xb = np.zeros((1, 256), np.uint16)
    xb[0, 128:] = synth.to_bf16_bits(np.linspace(-2, 2, 128, dtype=np.float32))
    q, s = orc.quantize_rows(xb)
    assert s[0, 0] == np.float32(1e-4) / np.float32(448.0)
    assert (q[0, :128] == 0).all()
    assert s[0, 1] == np.float32(2.0) / np.float32(448.0)


def test_nonfinite_groups(orc):
    """Groups holding Inf or NaN follow IEEE fp32 arithmetic through the same
    formula: the maximum is taken over the values that compare (a NaN never
    wins), an Inf maximum gives an Inf scale and signed-zero codes for the
    finite values, and every NaN quotient is coded 0x7F."""
    rng = np.random.default_rng(9)
    xf = rng.standard_normal(512).astype(np.float32)
    xb = synth.to_bf16_bits(xf)[None, :].copy()
    xb[0, 5] = 0x7F80                      # group 0: +Inf
    xb[0, 128 + 7] = 0x7FC0                # group 1: a quiet NaN ...
    xb[0, 128 + 9] = 0xFF81                # ... and a negative signalling NaN
    xb[0, 256 + 1] = 0xFF80                # group 2: -Inf and +Inf
    xb[0, 256 + 2] = 0x7F80
    xb[0, 384:] = 0x7FC1                   # group 3: all NaN
    q, s = orc.quantize_rows(xb)
    assert np.isinf(s[0, 0]) and np.isinf(s[0, 2])
    finite0 = np.delete(np.arange(128), 5)
    signs0 = (xb[0, finite0] >> 15).astype(np.uint8) * 0x80
    np.testing.assert_array_equal(q[0, finite0], signs0)
    assert q[0, 5] == 0x7F
    g1 = (xb[0, 128:256].astype(np.uint32) << 16).view(np.float32)
    nan1 = np.isnan(g1)
    assert s[0, 1] == np.float32(np.abs(g1[~nan1]).max()) / np.float32(448.0)
    assert (q[0, 128:256][nan1] == 0x7F).all()
    v = (g1[~nan1] / s[0, 1]).astype(np.float32)
    np.testing.assert_array_equal(q[0, 128:256][~nan1], _torch_e4m3(v))
    assert q[0, 257] == 0x7F and q[0, 258] == 0x7F
    assert s[0, 3] == np.float32(1e-4) / np.float32(448.0)
    assert (q[0, 384:] == 0x7F).all()


def _numpy_quantize(xb: np.ndarray):
    """The quantiser written with numpy's IEEE fp32 arithmetic and torch's cast."""
    T, h = xb.shape
    xf = (xb.astype(np.uint32) << 16).view(np.float32).reshape(T, h // 128, 128)
    amax = np.abs(xf).max(axis=2)
    s = np.maximum(amax, np.float32(1e-4)).astype(np.float32) / np.float32(448.0)
    v = (xf / s[:, :, None]).astype(np.float32)
    return _torch_e4m3(v.reshape(T, h)), s.astype(np.float32)


@pytest.mark.parametrize("cfg", [2, 5])
def test_quantize_matches_numpy_and_torch(orc, cfg):
    inp = synth.make_inputs(cfg, T=64)
    q, s = orc.quantize_rows(inp["x"])
    q_ref, s_ref = _numpy_quantize(inp["x"])
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(q, q_ref)


def test_round_trip_bound_and_outliers(orc):
    inp = synth.make_inputs(5, T=32)
    x = inp["x"]
    q, s = orc.quantize_rows(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    deq = np.vectorize(orc.e4m3_to_f32, otypes=[np.float32])(q).astype(np.float64)
    deq *= np.repeat(s, 128, axis=1)
    err = np.abs(deq - xf)
    sfull = np.repeat(s, 128, axis=1).astype(np.float64)
    # half an ulp of a 3-bit mantissa (relative 2^-4) in the normal range, half
    # the subnormal spacing 2^-9 (times s) below it; slack for the fp32 divide
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sfull) * (1 + 2.0 ** -20)
    assert (err <= bound).all()
    # groups holding an x50 outlier channel have a much larger scale
    xg = np.abs(xf).reshape(32, -1, 128).max(axis=2)
    big = xg > 20
    assert big.any() and (~big).any()
    assert np.median(s[big]) > 10 * np.median(s[~big])
