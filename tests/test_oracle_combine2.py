"""Pins for the oracle's two-stage combine (the DeepEP v2 section of the
DeepEP study notes: the destination rank reduces the outputs of its own
experts for a token into one partial result, sent back to the source, whose
epilogue reduces over the destination ranks).

Pinned against: the closed form for unit weights and identity experts;
exact rational arithmetic for both stages, rounded step by step; the
special case of a single rank, where stage 1 is the one-stage combine; and
an error bound derived from the two roundings against a float64 reference.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

from test_oracle_combine import _f32, _round_to_format, _torch_bf16


def _route(orc, x, topk, w, E, R):
    d = orc.dispatch(x, topk, w, E, R)
    lay = d["layout"]
    n_send = int(lay["totals"][0])
    return d, lay, n_send


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_unit_weight_identity_closed_form(orc, cfg):
    """Identity experts (the expert output is the dispatched row) and unit
    weights: partial(t, r) = bf16(n_r * x[t]) with n_r the entries of t on
    rank r, and out[t] = bf16(sum over r of those partials). Every product
    n*x (n <= 8, 8-bit significand) and every sum of at most 8 same-sign
    terms within a factor 8 of each other is exact in fp32."""
    inp = synth.make_inputs(cfg, T=80)
    wl = inp["workload"]
    topk = inp["topk_idx"].copy()
    topk[np.random.default_rng(8).random(topk.shape) < 0.1] = -1
    ones = np.ones_like(inp["topk_w"])
    d, lay, n_send = _route(orc, inp["x"], topk, ones, wl.E, wl.R)
    part = orc.combine_partial(d["recv_x"], d["send_src"][:n_send], d["send_topk_idx"][:n_send],
                               d["send_topk_w"][:n_send], d["pos_exp"])
    out = orc.combine_final(part, lay["rank_off"], lay["pos_in_rank"])
    xf = _f32(inp["x"])
    L = wl.E // wl.R
    n_tr = np.zeros((topk.shape[0], wl.R), np.float32)
    for t in range(topk.shape[0]):
        for e in topk[t]:
            if e >= 0:
                n_tr[t, e // L] += 1
    # stage 1
    for i in range(n_send):
        t = d["send_src"][i]
        r = int(np.searchsorted(lay["rank_off"], i, side="right") - 1)
        want = _torch_bf16(xf[t] * n_tr[t, r])
        np.testing.assert_array_equal(part[i], want)
    # stage 2
    parts = _f32(_torch_bf16(xf[:, None, :] * n_tr[:, :, None]))  # [T, R, h]
    ref = _torch_bf16(parts.sum(axis=1, dtype=np.float32))
    ref[(ref & 0x7FFF) == 0] = 0  # an all-zero sum from +0.0 is +0.0
    np.testing.assert_array_equal(out, ref)


def test_both_stages_exact_rational(orc):
    """Both stages against exact rationals rounded to fp32 after every fma
    or add and to bf16 at the end of each stage. Row scales spread over 2^+-24
    so that the fp32 sums round, and their order shows."""
    rng = np.random.default_rng(12)
    T, K, E, R, h = 24, 6, 12, 4, 8
    topk = synth.random_routing(T, K, E, seed=13, p_drop=0.1)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    d, lay, n_send = _route(orc, x, topk, w, E, R)
    n_exp = int(lay["totals"][1])
    y = synth.to_bf16_bits(rng.standard_normal((n_exp, h)).astype(np.float32) *
                           np.float32(2.0) ** rng.integers(-24, 24, (n_exp, 1)).astype(np.float32))
    part = orc.combine_partial(y, d["send_src"][:n_send], d["send_topk_idx"][:n_send],
                               d["send_topk_w"][:n_send], d["pos_exp"])
    out = orc.combine_final(part, lay["rank_off"], lay["pos_in_rank"])
    yf, pf, of = _f32(y), _f32(part), _f32(out)
    for i in range(n_send):
        t = d["send_src"][i]
        for c in range(h):
            acc = Fraction(0)
            for k in range(K):
                if d["send_topk_idx"][i, k] >= 0:
                    prod = Fraction(float(d["send_topk_w"][i, k])) * Fraction(
                        float(yf[d["pos_exp"][t, k], c]))
                    acc = _round_to_format(prod + acc, 23, -126, 127)
            assert Fraction(float(pf[i, c])) == _round_to_format(acc, 7, -126, 127), (i, c)
    for t in range(T):
        for c in range(h):
            acc = Fraction(0)
            for r in range(R):
                p = lay["pos_in_rank"][t, r]
                if p >= 0:
                    acc = _round_to_format(acc + Fraction(float(pf[lay["rank_off"][r] + p, c])),
                                           23, -126, 127)
            assert Fraction(float(of[t, c])) == _round_to_format(acc, 7, -126, 127), (t, c)


def test_single_rank_equals_one_stage(orc):
    """With one rank every entry lands on it: stage 1 is then the one-stage
    combine's fp32 chain and rounding, and stage 2 adds one partial to +0.0
    (which only turns -0 into +0)."""
    inp = synth.make_inputs(4, T=200)
    wl = inp["workload"]
    topk = inp["topk_idx"].copy()
    topk[np.random.default_rng(2).random(topk.shape) < 0.1] = -1
    d, lay, n_send = _route(orc, inp["x"], topk, inp["topk_w"], wl.E, 1)
    y = synth.to_bf16_bits(np.random.default_rng(4).standard_normal(
        (int(lay["totals"][1]), wl.h)).astype(np.float32))
    part = orc.combine_partial(y, d["send_src"][:n_send], d["send_topk_idx"][:n_send],
                               d["send_topk_w"][:n_send], d["pos_exp"])
    out = orc.combine_final(part, lay["rank_off"], lay["pos_in_rank"])
    one = orc.combine(y, inp["topk_w"], d["pos_exp"])
    routed = np.flatnonzero((topk >= 0).any(axis=1))
    np.testing.assert_array_equal(part, one[d["send_src"][:n_send]])
    one_pz = one.copy()
    one_pz[(one_pz & 0x7FFF) == 0] = 0
    np.testing.assert_array_equal(out[routed], one_pz[routed])
    assert (out[np.setdiff1d(np.arange(topk.shape[0]), routed)] == 0).all()


def test_error_bound_against_float64(orc):
    """|out - exact| <= half a bf16 ulp of out + half a bf16 ulp of each
    partial + the fp32 chain bounds (K and R roundings of 2^-24)."""
    rng = np.random.default_rng(21)
    T, K, E, R, h = 64, 8, 64, 8, 64
    topk = synth.random_routing(T, K, E, seed=22)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    w = rng.random((T, K)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    d, lay, n_send = _route(orc, x, topk, w, E, R)
    y = synth.to_bf16_bits(rng.standard_normal((int(lay["totals"][1]), h)).astype(np.float32))
    part = orc.combine_partial(y, d["send_src"][:n_send], d["send_topk_idx"][:n_send],
                               d["send_topk_w"][:n_send], d["pos_exp"])
    out = _f32(orc.combine_final(part, lay["rank_off"], lay["pos_in_rank"])).astype(np.float64)
    yf = _f32(y).astype(np.float64)
    pf = _f32(part).astype(np.float64)
    prods = w.astype(np.float64)[:, :, None] * yf[d["pos_exp"]]      # [T, K, h]
    exact = prods.sum(axis=1)
    mag = np.abs(prods).sum(axis=1)

    def half_ulp_bf16(v):
        return np.spacing(np.abs(v).astype(np.float32)).astype(np.float64) * 2.0 ** 15

    part_err = np.zeros((T, h))
    part_mag = np.zeros((T, h))
    for t in range(T):
        for r in range(R):
            p = lay["pos_in_rank"][t, r]
            if p >= 0:
                part_err[t] += np.maximum(half_ulp_bf16(pf[lay["rank_off"][r] + p]), 2.0 ** -134)
                part_mag[t] += np.abs(pf[lay["rank_off"][r] + p])
    tol = (np.maximum(half_ulp_bf16(out), 2.0 ** -134) + part_err
           + K * 2.0 ** -24 * mag + R * 2.0 ** -24 * part_mag)
    assert (np.abs(out - exact) <= tol).all()


def _bits(vals):
    return _torch_bf16(np.array(vals, np.float32))


def test_summation_order_hand_worked(orc):
    """The order of both sums, pinned where it decides a bf16 result. Terms
    1, 2^-8, 2^-24, 2^-24 added from the first: 1 + 2^-8 is exact, and each
    2^-24 is half an fp32 ulp at that value, a tie that rounds back to the even
    neighbour, so the fp32 sum stays 1 + 2^-8, a bf16 tie that rounds to 1.0.
    Added from the last: 2^-24 + 2^-24 = 2^-23, then 2^-8 and 1 are exact, and
    1 + 2^-8 + 2^-23 lies above the tie, giving 1 + 2^-7."""
    terms = [1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]
    one, up = _bits([1.0])[0], _bits([1.0 + 2.0 ** -7])[0]
    assert (one, up) == (0x3F80, 0x3F81)
    # stage 2: one token, one partial row per rank, ranks in the terms' order
    part = _bits(terms)[:, None]
    rank_off = np.arange(5, dtype=np.int32)
    pos_in_rank = np.zeros((1, 4), np.int32)
    assert orc.combine_final(part, rank_off, pos_in_rank)[0, 0] == one
    # the same rows in reverse rank order: the terms are now added from the last
    assert orc.combine_final(part[::-1].copy(), rank_off, pos_in_rank)[0, 0] == up
    # stage 1: one row of one rank, four entries with unit weights, k in the terms' order
    y = _bits(terms)[:, None]
    send_src = np.zeros(1, np.int32)
    idx = np.zeros((1, 4), np.int64)
    w = np.ones((1, 4), np.float32)
    pos_exp = np.arange(4, dtype=np.int32)[None, :]
    assert orc.combine_partial(y, send_src, idx, w, pos_exp)[0, 0] == one
    assert orc.combine_partial(y, send_src, idx, w, pos_exp[:, ::-1].copy())[0, 0] == up
