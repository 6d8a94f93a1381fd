"""Pins for the oracle's low-latency fixed-slot dispatch (low-latency section
of the event-driven EP scheduling page: a private region per (source rank,
expert) addressed as (expert * num_ranks + src_rank) * chunk + slot, and a
count slot written after the data whose empty value differs from every
count; the Buffer section of the DeepEP study notes: counters start at -1;
section 4.2 of the low-latency dispatch page: the count lives at
local_expert * num_ranks + src_rank).

Pinned against: the hand-worked example, a direct evaluation of the address
formula with stable-argsort slots, bincount for the counts, and untouched
canary bytes / -1 counts in every region the call does not own.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example_r4_e8_k2.json")


def test_worked_example(orc):
    with open(GOLD) as f:
        g = json.load(f)
    ll = g["ll"]
    topk = np.array(g["topk_idx"], np.int64)
    x = synth.to_bf16_bits(np.arange(4 * 128, dtype=np.float32).reshape(4, 128))
    d = orc.ll_dispatch(x, topk, g["E"], g["R"], ll["src_rank"], ll["cap"], ll["R_buf"], fp8=False)
    np.testing.assert_array_equal(d["pos_ll"], np.array(ll["pos_ll"]))
    expect = np.full(g["E"] * ll["R_buf"], -1)
    for k, v in ll["count_written"].items():
        expect[int(k)] = v
    np.testing.assert_array_equal(d["ll_count"], expect)


def _slots(topk, E):
    T, K = topk.shape
    flat = topk.ravel()
    valid = flat >= 0
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    cnt = np.bincount(flat[valid], minlength=E)
    starts = np.concatenate([[0], np.cumsum(cnt)])
    slot = np.full(T * K, -1, np.int64)
    for e in range(E):
        m = order[starts[e]:starts[e + 1]]
        slot[m] = np.arange(m.size)
    return slot.reshape(T, K), cnt


@pytest.mark.parametrize("cfg,T,R_buf_full,src,fp8", [
    (1, None, True, 0, True), (1, None, False, 3, False), (1, 40, True, 3, False),
    (2, 24, False, 0, True), (2, 24, False, 31, False),
])
def test_address_formula(orc, cfg, T, R_buf_full, src, fp8):
    inp = synth.make_inputs(cfg, T=T)
    wl = inp["workload"]
    cap = wl.T if cfg == 1 else 32
    topk = inp["topk_idx"].copy()
    topk[np.random.default_rng(1).random(topk.shape) < 0.05] = -1
    T, K = topk.shape
    R_buf = wl.R if R_buf_full else 1
    d = orc.ll_dispatch(inp["x"], topk, wl.E, wl.R, src, cap, R_buf, fp8=fp8)
    slot, cnt = _slots(topk, wl.E)
    region = topk * wl.R + src if R_buf_full else topk
    row = np.where(topk >= 0, region * cap + slot, -1)
    np.testing.assert_array_equal(d["pos_ll"], row)
    if fp8:
        q, s = orc.quantize_rows(inp["x"])
    written = np.zeros(wl.E * R_buf * cap, bool)
    for t in range(T):
        for k in range(K):
            if row[t, k] < 0:
                continue
            r = row[t, k]
            written[r] = True
            assert d["ll_src"][r] == t
            if fp8:
                np.testing.assert_array_equal(d["ll_x"][r], q[t])
                np.testing.assert_array_equal(d["ll_scales"][r], s[t])
            else:
                np.testing.assert_array_equal(d["ll_x"][r], inp["x"][t])
    # every other row keeps its canary bytes
    assert (d["ll_x"][~written].view(np.uint8) == 0xA5).all()
    assert (d["ll_src"][~written].view(np.uint8) == 0xA5).all()
    # counts: bincount in the owned regions (zeros included), -1 elsewhere
    expect = np.full(wl.E * R_buf, -1, np.int64)
    owned = np.arange(wl.E) * wl.R + src if R_buf_full else np.arange(wl.E)
    expect[owned] = cnt
    np.testing.assert_array_equal(d["ll_count"], expect)


def test_compact_equals_full_slice(orc):
    inp = synth.make_inputs(1)
    wl = inp["workload"]
    src = 2
    full = orc.ll_dispatch(inp["x"], inp["topk_idx"], wl.E, wl.R, src, 64, wl.R, fp8=True)
    comp = orc.ll_dispatch(inp["x"], inp["topk_idx"], wl.E, wl.R, src, 64, 1, fp8=True)
    fx = full["ll_x"].reshape(wl.E, wl.R, 64, -1)[:, src]
    np.testing.assert_array_equal(fx.reshape(wl.E * 64, -1), comp["ll_x"])
    np.testing.assert_array_equal(full["ll_count"].reshape(wl.E, wl.R)[:, src], comp["ll_count"])


def test_capacity_error(orc):
    inp = synth.make_inputs(1)
    wl = inp["workload"]
    with pytest.raises(orc.OracleError) as ei:
        orc.ll_dispatch(inp["x"], inp["topk_idx"], wl.E, wl.R, 0, wl.T - 1, 1)
    assert ei.value.code == orc.ECAPACITY
