"""GPU parity for the two-stage combine (rank-level partial reduce, then
the final reduce over ranks) against the oracle's two stages, bit for bit.
The oracle's inputs come from the oracle's own dispatch; the GPU's from the
GPU dispatch (their equality is the dispatch parity tests' business)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import CANARY, dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu


def _eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    bad = np.flatnonzero((a != b).ravel())
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}"


def _two_stage(x, topk, w, E, R, seed, worst_case=False):
    import combine_get_dispatch_counts_amd as epx

    T, h = x.shape
    K = topk.shape[1]
    dev = torch.device("cuda")
    tk = torch.from_numpy(topk).cuda()
    wt = torch.from_numpy(w).cuda()
    lay = epx.get_dispatch_layout(tk, E, R)
    n_send, n_recv = (int(v) for v in lay.totals.cpu())
    cap_s, cap_r = (T * min(K, R), T * K) if worst_case else (n_send, n_recv)
    bufs = epx.alloc_dispatch(T, h, K, cap_s, cap_r, False, dev)
    d = epx.dispatch(dev_bf16(x), tk, wt, E, R, layout=lay, out=bufs)
    y = synth.expert_outputs(max(n_recv, 1), h, seed=seed, device="cuda")
    part = torch.empty((cap_s, h), dtype=torch.bfloat16, device=dev)
    part.view(torch.uint8).fill_(CANARY)
    epx.combine_partial(y, d, out=part)
    out = epx.combine_final(part, lay)
    flags = epx.get_error()
    assert flags == 0, f"device flags {flags:#x}"
    yh = host_bits(y)[:n_recv]
    return host_bits(part), host_bits(out), yh, n_send


def _oracle_two_stage(x, topk, w, E, R, y):
    o = oracle.dispatch(x, topk, w, E, R)
    lay = o["layout"]
    n_send = int(lay["totals"][0])
    part = oracle.combine_partial(y, o["send_src"][:n_send], o["send_topk_idx"][:n_send],
                                  o["send_topk_w"][:n_send], o["pos_exp"])
    out = oracle.combine_final(part, lay["rank_off"], lay["pos_in_rank"])
    return part, out


def _check(x, topk, w, E, R, seed, worst_case=False):
    gp, go, y, n_send = _two_stage(x, topk, w, E, R, seed, worst_case)
    op, oo = _oracle_two_stage(x, topk, w, E, R, y)
    _eq(gp[:n_send], op, "partial")
    _eq(go, oo, "out")
    assert (gp[n_send:].view(np.uint8) == CANARY).all(), "rows past the send total were written"


@pytest.mark.parametrize("cfg,T", [(1, None), (3, None), (4, None), (5, 2048)])
def test_two_stage_workloads(cfg, T):
    inp = synth.make_inputs(cfg, T=T)
    wl = inp["workload"]
    say(f"two-stage combine {wl.describe()} (worst-case capacity)")
    _check(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, seed=31 + cfg, worst_case=True)


@pytest.mark.parametrize("T,K,E,R,h,p_drop", [
    (1, 8, 256, 32, 7168, 0.0), (63, 2, 8, 4, 128, 0.0), (257, 8, 64, 8, 1024, 0.3),
    (100, 32, 64, 64, 256, 0.0), (300, 6, 24, 1, 512, 0.1), (130, 8, 128, 32, 136, 0.0),
])
def test_two_stage_edge_cases(T, K, E, R, h, p_drop):
    say(f"two-stage combine T={T} K={K} E={E} R={R} h={h} drop={p_drop}")
    rng = np.random.default_rng(T * 7 + K)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=T + 1, p_drop=p_drop)
    w = rng.random((T, K)).astype(np.float32)
    _check(x, topk, w, E, R, seed=T)


def test_two_stage_empty():
    import combine_get_dispatch_counts_amd as epx

    say("two-stage combine T=0")
    dev = torch.device("cuda")
    tk = torch.empty((0, 4), dtype=torch.int64, device=dev)
    lay = epx.get_dispatch_layout(tk, 16, 4)
    d = epx.dispatch(torch.empty((0, 128), dtype=torch.bfloat16, device=dev), tk,
                     torch.empty((0, 4), dtype=torch.float32, device=dev), 16, 4, layout=lay)
    part = epx.combine_partial(torch.empty((0, 128), dtype=torch.bfloat16, device=dev), d)
    out = epx.combine_final(part, lay)
    assert part.shape == (0, 128) and out.shape == (0, 128)
    assert epx.get_error() == 0


def test_two_stage_bad_handle_flags():
    """A send row naming a token outside [0, T) is flagged (its partial is
    +0) and a partial row index past the buffer is flagged and skipped."""
    import combine_get_dispatch_counts_amd as epx

    say("two-stage combine error paths")
    inp = synth.make_inputs(1)
    wl = inp["workload"]
    tk = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = epx.get_dispatch_layout(tk, wl.E, wl.R)
    d = epx.dispatch(dev_bf16(inp["x"]), tk, torch.from_numpy(inp["topk_w"]).cuda(), wl.E, wl.R,
                     layout=lay)
    y = synth.expert_outputs(d.recv_x.shape[0], wl.h, seed=5, device="cuda")
    d.send_src[0] = wl.T + 3
    part = epx.combine_partial(y, d)
    assert epx.get_error() == epx._lib.DEV_BAD_HANDLE
    assert (host_bits(part[0]) == 0).all()
    epx.combine_final(part[:1], lay)
    assert epx.get_error() == epx._lib.DEV_BAD_HANDLE
