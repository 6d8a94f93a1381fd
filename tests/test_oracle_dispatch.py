"""Pins for the oracle's high-throughput dispatch: the rank-deduplicated pack
(dispatch section of the DeepEP study notes: senders scan their token range
in order and enqueue a token for every rank is_token_in_rank marks; v2: one
copy per destination rank) and the local permute into expert-contiguous
blocks (high-throughput section of the event-driven EP scheduling page).

Pinned against: the hand-worked example, byte equality of every row with the
source token's row, numpy's flatnonzero (segment order) and stable argsort
(expert-major order), and the per-row top-k metadata rule.
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
    topk = np.array(g["topk_idx"], np.int64)
    T = topk.shape[0]
    x = synth.to_bf16_bits(np.arange(T * 128, dtype=np.float32).reshape(T, 128) / 64)
    w = np.full(topk.shape, 0.5, np.float32)
    d = orc.dispatch(x, topk, w, g["E"], g["R"])
    ex = g["expected"]
    for key in ["send_src", "send_topk_idx", "recv_src", "pos_exp"]:
        np.testing.assert_array_equal(d[key], np.array(ex[key]), err_msg=key)
    np.testing.assert_array_equal(d["send_x"], x[ex["send_src"]])
    np.testing.assert_array_equal(d["recv_x"], x[ex["recv_src"]])


def _check_dispatch(orc, x, topk, w, E, R, fp8):
    T, K = topk.shape
    L = E // R
    d = orc.dispatch(x, topk, w, E, R, fp8=fp8)
    lay = d["layout"]
    if fp8:
        q, s = orc.quantize_rows(x)
        rows, srows = q, s
    else:
        rows, srows = x, None
    # pack: segment r lists flatnonzero(in_rank[:, r]) in order, rows are copies
    in_rank = lay["is_token_in_rank"].astype(bool)
    for r in range(R):
        a, b = lay["rank_off"][r], lay["rank_off"][r + 1]
        np.testing.assert_array_equal(d["send_src"][a:b], np.flatnonzero(in_rank[:, r]))
    np.testing.assert_array_equal(d["send_x"], rows[d["send_src"]])
    if fp8:
        np.testing.assert_array_equal(d["send_scales"], srows[d["send_src"]])
    # metadata: local index and weight where the expert sits on the row's rank
    seg_rank = np.repeat(np.arange(R), np.diff(lay["rank_off"]))
    src_topk = topk[d["send_src"]]
    local = (src_topk >= 0) & (src_topk // L == seg_rank[:, None])
    np.testing.assert_array_equal(d["send_topk_idx"],
                                  np.where(local, src_topk - seg_rank[:, None] * L, -1))
    np.testing.assert_array_equal(d["send_topk_w"], np.where(local, w[d["send_src"]], 0.0))
    # permute: expert-major, token order inside an expert (stable argsort)
    flat = topk.ravel()
    valid = flat >= 0
    order = np.argsort(np.where(valid, flat, E), kind="stable")[:valid.sum()]
    np.testing.assert_array_equal(d["recv_src"], order // K)
    np.testing.assert_array_equal(d["recv_x"], rows[order // K])
    if fp8:
        np.testing.assert_array_equal(d["recv_scales"], srows[order // K])
    pos = np.full(T * K, -1, np.int64)
    pos[order] = np.arange(order.size)
    np.testing.assert_array_equal(d["pos_exp"].ravel(), pos)
    return d


@pytest.mark.parametrize("cfg,T,fp8", [(1, None, False), (1, 64, True), (3, 200, False),
                                       (4, 300, False), (5, 64, True), (2, 128, True)])
def test_dispatch_against_library_routines(orc, cfg, T, fp8):
    inp = synth.make_inputs(cfg, T=T)
    wl = inp["workload"]
    _check_dispatch(orc, inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, fp8)


def test_dispatch_with_dropped_entries_and_r1(orc):
    rng = np.random.default_rng(9)
    x = synth.to_bf16_bits(rng.standard_normal((77, 256)).astype(np.float32))
    topk = synth.random_routing(77, 4, 16, 9, p_drop=0.25)
    w = rng.random((77, 4)).astype(np.float32)
    for R in (1, 2, 16):
        _check_dispatch(orc, x, topk, w, 16, R, fp8=False)
        _check_dispatch(orc, x, topk, w, 16, R, fp8=True)


def test_capacity_and_shape_errors(orc):
    inp = synth.make_inputs(1)
    wl = inp["workload"]
    lay = orc.layout(inp["topk_idx"], wl.E, wl.R)
    lay_small = dict(lay)
    lay_small["totals"] = lay["totals"] - 1  # the wrapper sizes buffers one row short
    with pytest.raises(orc.OracleError) as ei:
        orc.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, lay=lay_small)
    assert ei.value.code == orc.ECAPACITY
    x_odd = np.zeros((wl.T, 72), np.uint16)
    with pytest.raises(orc.OracleError) as ei:
        orc.dispatch(x_odd, inp["topk_idx"], inp["topk_w"], wl.E, wl.R, fp8=True)
    assert ei.value.code == orc.EUNSUPPORTED


def _two_level(orc, x, topk, w, E, R, N, fp8):
    """Node-level pack (R = N: one row per (token, node)), then inside each
    node the pack of that node's received rows over its R/N ranks, with the
    node-local expert indices the first level wrote. Returns, per rank, the
    rows, source tokens, rank-local indices, weights (and FP8 scales)."""
    L_node = E // N
    d1 = orc.dispatch(x, topk, w, E, N, fp8=fp8)
    ro1 = d1["layout"]["rank_off"]
    per_rank = {}
    for n in range(N):
        a, b = int(ro1[n]), int(ro1[n + 1])
        rows = d1["send_x"][a:b]
        if fp8:  # codes travel as bit patterns, two per 16-bit element
            rows = np.ascontiguousarray(rows).view(np.uint16)
        d2 = orc.dispatch(rows, d1["send_topk_idx"][a:b], d1["send_topk_w"][a:b], L_node,
                          R // N)
        ro2 = d2["layout"]["rank_off"]
        for g in range(R // N):
            a2, b2 = int(ro2[g]), int(ro2[g + 1])
            sel = d2["send_src"][a2:b2]
            out = dict(x=d2["send_x"][a2:b2], src=d1["send_src"][a:b][sel],
                       idx=d2["send_topk_idx"][a2:b2], w=d2["send_topk_w"][a2:b2])
            if fp8:
                out["x"] = np.ascontiguousarray(out["x"]).view(np.uint8)
                out["scales"] = d1["send_scales"][a:b][sel]
            per_rank[n * (R // N) + g] = out
    return per_rank


@pytest.mark.parametrize("fp8", [False, True])
def test_two_level_pack_equals_rank_level_pack(orc, fp8):
    """Two-level dedup (the DeepEP study notes' hybrid section: one copy per
    node, then one per GPU inside the node) delivers to every rank exactly
    the rows of the one-level rank-deduplicated pack, in the same order, with
    the same rank-local top-k indices and weights: node n's rank g is rank
    n*(R/N) + g, and a node-local index minus g*L is the rank-local one."""
    T, h, E, R, N, K = 200, 256, 32, 8, 2, 4
    rng = np.random.default_rng(11)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=12, p_drop=0.1)
    w = rng.random((T, K)).astype(np.float32)
    flat = orc.dispatch(x, topk, w, E, R, fp8=fp8)
    ro = flat["layout"]["rank_off"]
    two = _two_level(orc, x, topk, w, E, R, N, fp8)
    for r in range(R):
        a, b = int(ro[r]), int(ro[r + 1])
        got = two[r]
        np.testing.assert_array_equal(got["src"], flat["send_src"][a:b], err_msg=f"rank {r} src")
        np.testing.assert_array_equal(got["x"], flat["send_x"][a:b], err_msg=f"rank {r} rows")
        np.testing.assert_array_equal(got["idx"], flat["send_topk_idx"][a:b],
                                      err_msg=f"rank {r} indices")
        np.testing.assert_array_equal(got["w"], flat["send_topk_w"][a:b],
                                      err_msg=f"rank {r} weights")
        if fp8:
            np.testing.assert_array_equal(got["scales"], flat["send_scales"][a:b],
                                          err_msg=f"rank {r} scales")
    # the node level moves fewer rows than the rank level whenever a token
    # has two ranks in one node
    n1 = int(orc.layout(topk, E, N)["totals"][0])
    assert n1 < int(flat["layout"]["totals"][0])


@pytest.mark.parametrize("fp8", [False, True])
def test_threaded_oracle_equals_sequential(orc, fp8):
    """The oracle run over token ranges side by side (the benchmark's
    threaded CPU timing) gives exactly the sequential run's outputs, for the
    dispatch and the combine, with ragged ranges."""
    T, h, E, R, K = 301, 256, 32, 8, 4
    rng = np.random.default_rng(12)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=13, p_drop=0.05)
    w = rng.random((T, K)).astype(np.float32)
    seq = orc.dispatch(x, topk, w, E, R, fp8=fp8)
    for threads in (2, 7):
        par = orc.dispatch(x, topk, w, E, R, fp8=fp8, threads=threads)
        for k in ("send_x", "send_src", "send_topk_idx", "send_topk_w", "recv_x", "recv_src",
                  "pos_exp") + (("send_scales", "recv_scales") if fp8 else ()):
            assert np.array_equal(np.asarray(par[k]).view(np.uint8),
                                  np.asarray(seq[k]).view(np.uint8)), (threads, k)
    y = synth.to_bf16_bits(rng.standard_normal((T * K, h)).astype(np.float32))
    c1 = orc.combine(y, w, seq["pos_exp"])
    for threads in (3, 16):
        assert np.array_equal(orc.combine(y, w, seq["pos_exp"], threads=threads), c1)
