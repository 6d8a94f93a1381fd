"""Pins for the oracle's combine (the combine section of the DeepEP study
notes: the handle routes expert outputs back to their source token, where
they are reduced; combine stays in BF16 per the low-latency section of the
event-driven EP scheduling page).

Pinned against: torch's fp32->bf16 cast over a structured sweep reaching
every rounding decision; exact rational arithmetic (fractions) for the fp32
fused-multiply-add chain; the closed form for unit weights and identity
experts; a float64 reference within one bf16 ulp; a hand-worked example.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example_r4_e8_k2.json")


def _torch_bf16(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f32(bits16: np.ndarray) -> np.ndarray:
    return (bits16.astype(np.uint32) << 16).view(np.float32)


def test_bf16_rne_matches_torch_structured(orc):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000,
                     0x00FF, 0xFF00], np.uint32)
    v = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    ours = orc.bf16_rne_array(v)
    theirs = _torch_bf16(v)
    nan = np.isnan(v)
    np.testing.assert_array_equal(ours[~nan], theirs[~nan])
    assert (ours[nan] == 0x7FC0).all()


# ---- exact rational reference for the fp32 fma chain -------------------------

def _round_to_format(q: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round a rational to nearest-even in a binary format with `mant_bits`
    fraction bits, minimum normal exponent emin (gradual underflow below it)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant_bits)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r > (2 - Fraction(2) ** -mant_bits) * Fraction(2) ** emax:
        return sign * Fraction(10) ** 400  # overflow marker (not reached here)
    return sign * r


def _exact_combine(ws, ys):
    acc = Fraction(0)
    for w, y in zip(ws, ys):
        acc = _round_to_format(Fraction(float(w)) * Fraction(float(y)) + acc, 23, -126, 127)
    return _round_to_format(acc, 7, -126, 127)


def test_fma_chain_exact_rational(orc):
    rng = np.random.default_rng(11)
    T, K, h, n = 12, 8, 16, 40
    y = synth.to_bf16_bits(rng.standard_normal((n, h)).astype(np.float32) *
                           np.float32(2.0) ** rng.integers(-8, 8, (n, 1)).astype(np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    pos = rng.integers(0, n, (T, K)).astype(np.int32)
    pos[rng.random((T, K)) < 0.15] = -1
    out = orc.combine(y, w, pos)
    yf = _f32(y)
    for t in range(T):
        for c in range(h):
            ks = [k for k in range(K) if pos[t, k] >= 0]
            ref = _exact_combine([w[t, k] for k in ks], [yf[pos[t, k], c] for k in ks])
            got = float(_f32(out[t:t + 1, c:c + 1])[0, 0])
            assert Fraction(got) == ref, (t, c, got, float(ref))


def test_worked_example(orc):
    with open(GOLD) as f:
        g = json.load(f)
    h = g["combine"]["h"]
    n = 8
    y = synth.to_bf16_bits(np.repeat(np.arange(1, n + 1, dtype=np.float32)[:, None], h, axis=1))
    pos = np.array(g["expected"]["pos_exp"], np.int32)
    w = np.array(g["combine"]["topk_w"], np.float32)
    out = _f32(orc.combine(y, w, pos))
    for t, val in enumerate(g["combine"]["expected_row_values"]):
        assert (out[t] == np.float32(val)).all()


@pytest.mark.parametrize("cfg,fp8", [(1, False), (3, False), (4, False), (5, True)])
def test_unit_weight_identity_closed_form(orc, cfg, fp8):
    """Unit weights and identity experts: combine(dispatch(x)) equals
    bf16(K_valid(t) * x[t]) exactly (j*x with j <= 8 is exact in fp32 for an
    8-bit significand). With FP8 the dispatched value is bf16(dequant(q))."""
    inp = synth.make_inputs(cfg, T=96)
    wl = inp["workload"]
    topk = inp["topk_idx"].copy()
    topk[np.random.default_rng(3).random(topk.shape) < 0.1] = -1
    d = orc.dispatch(inp["x"], topk, inp["topk_w"], wl.E, wl.R, fp8=fp8)
    if fp8:
        deq = np.vectorize(orc.e4m3_to_f32, otypes=[np.float32])(d["recv_x"])
        deq = deq * np.repeat(d["recv_scales"], 128, axis=1)
        y = _torch_bf16(deq.astype(np.float32))
        xs = _torch_bf16((np.vectorize(orc.e4m3_to_f32, otypes=[np.float32])(
            orc.quantize_rows(inp["x"])[0]) * np.repeat(orc.quantize_rows(inp["x"])[1], 128, axis=1)
        ).astype(np.float32))
    else:
        y = d["recv_x"]
        xs = inp["x"]
    w1 = np.ones_like(inp["topk_w"])
    out = orc.combine(y, w1, d["pos_exp"])
    kval = (topk >= 0).sum(axis=1).astype(np.float32)
    ref = _torch_bf16(_f32(xs) * kval[:, None])
    # the accumulator starts at +0.0, so a zero sum (nothing routed, or an FP8
    # code that decodes to -0) comes out as +0.0: (+0) + (-0) = +0 under RNE
    ref[(ref & 0x7FFF) == 0] = 0
    np.testing.assert_array_equal(out, ref)


def test_float64_reference_within_one_ulp(orc):
    rng = np.random.default_rng(5)
    T, K, h, n = 64, 8, 256, 512
    y = synth.to_bf16_bits(rng.standard_normal((n, h)).astype(np.float32))
    w = rng.random((T, K)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    pos = rng.integers(0, n, (T, K)).astype(np.int32)
    out = _f32(orc.combine(y, w, pos)).astype(np.float64)
    yf = _f32(y).astype(np.float64)
    prods = w.astype(np.float64)[:, :, None] * yf[pos]
    ref = prods.sum(axis=1)
    mag = np.abs(prods).sum(axis=1)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    ulp = np.maximum(ulp, 2.0 ** -133)
    # one bf16 ulp of the result, plus the fp32 accumulation bound K*2^-24*sum|w*y|
    tol = ulp + K * 2.0 ** -24 * mag
    assert (np.abs(out - ref) <= tol).all()
    away = np.abs(ref) > 0.05 * mag
    assert (np.abs(out - ref)[away] <= ulp[away] * (1 + 2.0 ** -8)).all()
