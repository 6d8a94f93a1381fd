"""Pins for the oracle's layout and offsets (get_dispatch_layout + prefix sums).

Pinned against: the hand-worked example at the worked-example shape of the
DeepEP study notes (section on the layout before dispatch), numpy library
routines (bincount, any, cumsum, flatnonzero, stable argsort), the
invariants the method implies (one copy per rank, counts summing to the
number of routed entries) and a brute-force characterisation by sorting on
tiny inputs.
"""
import itertools
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example_r4_e8_k2.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def test_worked_example(orc):
    g = _gold()
    lay = orc.layout(np.array(g["topk_idx"]), g["E"], g["R"], g["C"])
    for key in ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank",
                "rank_off", "exp_off", "pos_in_rank", "slot_in_expert",
                "channel_prefix", "totals"]:
        np.testing.assert_array_equal(lay[key], np.array(g["expected"][key]), err_msg=key)


def _library_view(topk, E, R, C):
    """The layout expressed through numpy library routines only."""
    T, K = topk.shape
    L = E // R
    flat = topk.ravel()
    valid = flat >= 0
    cnt_e = np.bincount(flat[valid], minlength=E)
    # -1 // L == -1, so a dropped entry never matches a rank
    in_rank = np.stack([np.any(topk // L == r, axis=1) for r in range(R)], axis=1)
    cnt_r = in_rank.sum(axis=0)
    pos_in_rank = np.full((T, R), -1, np.int64)
    for r in range(R):
        toks = np.flatnonzero(in_rank[:, r])
        pos_in_rank[toks, r] = np.arange(toks.size)
    # stable argsort of the flat expert ids: within an expert, flat order (t*K+k)
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    slot = np.full(T * K, -1, np.int64)
    starts = np.concatenate([[0], np.cumsum(cnt_e)])
    for e in range(E):
        members = order[starts[e]:starts[e + 1]]
        slot[members] = np.arange(members.size)
    span = -(-T // C)
    ends = np.minimum((np.arange(C) + 1) * span, T)
    csum = np.concatenate([np.zeros((1, R), np.int64), np.cumsum(in_rank, axis=0)])
    chan = csum[ends].T
    return dict(num_tokens_per_expert=cnt_e, num_tokens_per_rank=cnt_r,
                is_token_in_rank=in_rank.astype(np.uint8),
                rank_off=np.concatenate([[0], np.cumsum(cnt_r)]),
                exp_off=starts, pos_in_rank=pos_in_rank,
                slot_in_expert=slot.reshape(T, K), channel_prefix=chan,
                totals=np.array([cnt_r.sum(), cnt_e.sum()]))


@pytest.mark.parametrize("T,K,E,R,C,p_drop,seed", [
    (64, 2, 8, 4, 3, 0.0, 1),
    (257, 8, 256, 32, 24, 0.0, 2),
    (300, 6, 64, 8, 7, 0.1, 3),
    (65, 4, 16, 16, 100, 0.3, 4),
    (33, 3, 12, 1, 1, 0.0, 5),
    (1, 8, 8, 2, 4, 0.0, 6),
])
def test_against_library_routines(orc, T, K, E, R, C, p_drop, seed):
    topk = synth.random_routing(T, K, E, seed, p_drop)
    lay = orc.layout(topk, E, R, C)
    ref = _library_view(topk, E, R, C)
    for key, val in ref.items():
        np.testing.assert_array_equal(lay[key], val, err_msg=key)


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_invariants_on_workloads(orc, cfg):
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    topk = inp["topk_idx"]
    lay = orc.layout(topk, wl.E, wl.R, 16)
    T, K, L = wl.T, wl.K, wl.L
    cnt_e, cnt_r = lay["num_tokens_per_expert"], lay["num_tokens_per_rank"]
    assert cnt_e.sum() == T * K                      # every entry counted once
    assert (cnt_r <= T).all()                        # one copy per rank
    assert T <= cnt_r.sum() <= T * min(K, wl.R)
    for r in range(wl.R):
        assert cnt_r[r] <= cnt_e[r * L:(r + 1) * L].sum()
    assert lay["totals"].tolist() == [cnt_r.sum(), cnt_e.sum()]
    np.testing.assert_array_equal(lay["channel_prefix"][:, -1], cnt_r)
    assert (np.diff(lay["channel_prefix"], axis=1) >= 0).all()
    # positions form permutations of 0..count-1 within every rank / expert
    for r in range(wl.R):
        p = lay["pos_in_rank"][:, r]
        assert sorted(p[p >= 0].tolist()) == list(range(cnt_r[r]))
    for e in range(wl.E):
        s = lay["slot_in_expert"][topk == e]
        assert sorted(s.tolist()) == list(range(cnt_e[e]))


def _brute(topk, E, R):
    """Characterise positions by sorting (key, t, k) tuples."""
    T, K = topk.shape
    L = E // R
    ent = sorted((int(topk[t, k]), t, k) for t in range(T) for k in range(K) if topk[t, k] >= 0)
    slot = -np.ones((T, K), np.int64)
    for e in range(E):
        mine = [(t, k) for (ee, t, k) in ent if ee == e]
        for i, (t, k) in enumerate(mine):
            slot[t, k] = i
    pairs = sorted({(int(topk[t, k]) // L, t) for t in range(T) for k in range(K) if topk[t, k] >= 0})
    pos = -np.ones((T, R), np.int64)
    for r in range(R):
        mine = [t for (rr, t) in pairs if rr == r]
        for i, t in enumerate(mine):
            pos[t, r] = i
    return slot, pos


@pytest.mark.parametrize("R", [1, 2, 4])
def test_brute_force_tiny(orc, R):
    """Every routing of 2 tokens with K=2 over E=4 (ordered pairs, -1 allowed,
    repeats allowed: one row per k) against the sort-based characterisation."""
    E, K = 4, 2
    choices = list(range(-1, E))
    for a in itertools.product(choices, repeat=K):
        for b in itertools.product(choices, repeat=K):
            topk = np.array([a, b], np.int64)
            lay = orc.layout(topk, E, R, 2)
            slot, pos = _brute(topk, E, R)
            np.testing.assert_array_equal(lay["slot_in_expert"], slot)
            np.testing.assert_array_equal(lay["pos_in_rank"], pos)


def test_empty_and_errors(orc):
    lay = orc.layout(np.zeros((0, 4), np.int64), 8, 2, 3)
    assert lay["totals"].tolist() == [0, 0]
    assert lay["channel_prefix"].tolist() == [[0, 0, 0], [0, 0, 0]]
    assert lay["exp_off"].tolist() == [0] * 9
    with pytest.raises(orc.OracleError) as ei:
        orc.layout(np.array([[0, 8]]), 8, 2)
    assert ei.value.code == orc.EROUTE
    with pytest.raises(orc.OracleError) as ei:
        orc.layout(np.array([[0, -2]]), 8, 2)
    assert ei.value.code == orc.EROUTE
    with pytest.raises(orc.OracleError) as ei:
        orc.layout(np.array([[0, 1]]), 8, 3)
    assert ei.value.code == orc.EINVAL


def test_two_level_dedup_by_logical_node(orc):
    """Two-level dedup (the DeepEP study notes' hybrid section: deduplicate by
    node first, then by GPU inside the node) with R ranks grouped into N
    logical nodes of R/N ranks: the layout at node granularity (R = N) is the
    rank-level layout with each node's ranks OR-ed together, and the
    node-level send rows are one per (token, node)."""
    inp = synth.make_inputs(3, T=300)
    E, R, N = 256, 32, 4
    topk = inp["topk_idx"].copy()
    topk[np.random.default_rng(1).random(topk.shape) < 0.05] = -1
    rank_lay = orc.layout(topk, E, R)
    node_lay = orc.layout(topk, E, N)
    in_node = rank_lay["is_token_in_rank"].reshape(-1, N, R // N).any(axis=2)
    np.testing.assert_array_equal(node_lay["is_token_in_rank"], in_node.astype(np.uint8))
    np.testing.assert_array_equal(node_lay["num_tokens_per_rank"], in_node.sum(axis=0))
    np.testing.assert_array_equal(node_lay["num_tokens_per_expert"],
                                  rank_lay["num_tokens_per_expert"])
    assert int(node_lay["totals"][0]) == int(in_node.sum()) <= int(rank_lay["totals"][0])
