"""The fused layout + dispatch launch against the oracle: every layout
output and every dispatch output bit for bit, at full size in the bench's
launch configuration and on edge shapes; its workspace shared with the
two-launch layout call; and the step replayed from a HIP graph."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import CANARY, dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank", "rank_off",
               "exp_off", "pos_in_rank", "slot_in_expert", "totals"]


def _eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if a.dtype.kind == "f":
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.flatnonzero((a != b).ravel())
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}"


def _fused_check(x, topk, w, E, R, fp8, C=None, ws=None):
    import combine_get_dispatch_counts_amd as epx

    T, h = x.shape
    K = topk.shape[1]
    dev = torch.device("cuda")
    cap_s, cap_r = T * min(K, R), T * K
    bufs = epx.alloc_dispatch(T, h, K, cap_s, cap_r, fp8, dev)
    for v in bufs.values():
        if v is not None:
            v.view(torch.uint8).fill_(CANARY)
    d = epx.dispatch_fused(dev_bf16(x), torch.from_numpy(topk).cuda(), torch.from_numpy(w).cuda(),
                           E, R, fp8=fp8, num_channels=C, out=bufs, workspace=ws)
    flags = epx.get_error()
    assert flags == 0, f"device flags {flags:#x}"
    o = oracle.dispatch(x, topk, w, E, R, fp8=fp8)
    ol = oracle.layout(topk, E, R, C)
    for k in LAYOUT_KEYS + (["channel_prefix"] if C else []):
        _eq(host_bits(getattr(d.layout, k)), ol[k], k)
    n_send, n_recv = (int(v) for v in ol["totals"])
    keys = ["send_x", "send_src", "send_topk_idx", "send_topk_w", "recv_x", "recv_src"]
    for k in keys:
        n = n_send if k.startswith("send") else n_recv
        _eq(host_bits(getattr(d, k))[:n], o[k], k)
        rest = host_bits(getattr(d, k))[n:]
        assert (rest.view(np.uint8) == CANARY).all(), f"rows of {k} past the total were written"
    _eq(host_bits(d.pos_exp), o["pos_exp"], "pos_exp")
    if fp8:
        ngrp = h // 128
        _eq(host_bits(d.send_scales)[:n_send, :ngrp], o["send_scales"], "send_scales")
        _eq(host_bits(d.recv_scales)[:n_recv, :ngrp], o["recv_scales"], "recv_scales")
        for k, n in (("send_scales", n_send), ("recv_scales", n_recv)):
            pad = host_bits(getattr(d, k))[:n, ngrp:]
            assert (pad.view(np.uint32) == 0).all(), f"{k} padding is not +0"
    return d


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_fused_workloads_full_size(cfg):
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    fp8 = wl.fp8 or cfg == 1
    say(f"fused layout+dispatch {wl.describe()} fp8={fp8}")
    _fused_check(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, fp8, C=24)


@pytest.mark.parametrize("T,K,E,R,h,fp8,kind", [
    (1, 8, 256, 32, 7168, False, "uniform"), (63, 2, 8, 4, 128, True, "uniform"),
    (65, 6, 64, 8, 4096, True, "uniform"), (257, 8, 256, 64, 256, True, "dropped"),
    (200, 4, 16, 1, 1024, False, "dropped"), (300, 32, 64, 8, 136, False, "uniform"),
    (300, 4, 16, 4, 128, False, "repeats"), (0, 4, 16, 4, 128, False, "uniform"),
    (513, 4, 128, 8, 512, False, "uniform"), (400, 6, 96, 12, 256, True, "dropped"),
    (999, 8, 96, 48, 128, False, "uniform"), (77, 3, 96, 6, 128, False, "repeats"),
    (130, 8, 256, 32, 7168, True, "dropped"), (600, 32, 512, 64, 256, True, "dropped"),
    (1500, 32, 512, 64, 128, False, "uniform"), (70, 8, 64, 8, 16384, True, "uniform"),
    (2100, 8, 64, 8, 9216, False, "dropped"), (90, 6, 64, 8, 8200, False, "uniform"),
])
def test_fused_edge_cases(T, K, E, R, h, fp8, kind):
    say(f"fused T={T} K={K} E={E} R={R} h={h} fp8={fp8} {kind}")
    rng = np.random.default_rng(T + K)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    if kind == "repeats":
        topk = rng.integers(-1, E, (T, K)).astype(np.int64)
    else:
        topk = synth.random_routing(T, K, E, seed=T + 3, p_drop=0.2 if kind == "dropped" else 0.0)
    w = rng.random((T, K)).astype(np.float32)
    _fused_check(x, topk, w, E, R, fp8, C=5 if T else None)


def _one_launch_runs(h, K, E, R, fp8, top=1 << 15):
    """The runs of T in [1, top) that epx_dispatch_fused does in one launch:
    small batches (every block computing the whole layout), then the tiled
    layout with one token per wave while its grid covers every compute unit
    and fits at once."""
    import combine_get_dispatch_counts_amd as epx

    runs, start = [], None
    for T in range(1, top):
        one = epx.fused_launches(T, h, K, E, R, fp8) == 1
        if one and start is None:
            start = T
        if not one and start is not None:
            runs.append((start, T - 1))
            start = None
    assert start is None, "one launch up to the end of the scan"
    return runs


def _one_launch_window(h, K, E, R, fp8):
    """The one-token-per-wave run (the last run of one-launch shapes)."""
    return _one_launch_runs(h, K, E, R, fp8)[-1]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("edge", ["one", "small_last", "gap", "first", "last", "above"])
def test_fused_one_and_two_launches(fp8, edge):
    """Where epx_dispatch_fused is one launch and where two: T = 1, the
    largest small batch, a shape between the two runs, both ends of the
    one-token-per-wave run and the shape past it, each against the oracle."""
    import combine_get_dispatch_counts_amd as epx

    h, K, E, R = 128, 4, 16, 4
    runs = _one_launch_runs(h, K, E, R, fp8)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert len(runs) == 2 and runs[0][0] == 1, runs
    assert runs[1][0] <= 8 * cus <= runs[1][1], runs
    assert epx.fused_launches(0, h, K, E, R, fp8) == 1
    T, want = {"one": (1, 1), "small_last": (runs[0][1], 1), "gap": (runs[0][1] + 1, 2),
               "first": (runs[1][0], 1), "last": (runs[1][1], 1),
               "above": (runs[1][1] + 1, 2)}[edge]
    assert epx.fused_launches(T, h, K, E, R, fp8) == want
    say(f"fused T={T} h={h} K={K} fp8={fp8} (one-launch runs {runs}, {want} launch(es))")
    rng = np.random.default_rng(T + h)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=T + 1, p_drop=0.1)
    w = rng.random((T, K)).astype(np.float32)
    _fused_check(x, topk, w, E, R, fp8)


@pytest.mark.parametrize("K,E,R,h,fp8,kind", [
    (8, 256, 64, 256, True, "dropped"), (32, 64, 8, 136, False, "uniform"),
    (4, 16, 4, 128, False, "repeats"), (6, 64, 8, 4096, True, "uniform"),
    (8, 128, 32, 512, False, "uniform"), (2, 8, 1, 128, True, "dropped"),
    (6, 96, 12, 256, False, "dropped"), (8, 96, 48, 128, True, "uniform"),
    (32, 512, 64, 128, False, "uniform"), (8, 64, 8, 9216, True, "dropped"),
    (8, 64, 8, 16384, False, "uniform"),
])
def test_fused_kernel_edge_cases(K, E, R, h, fp8, kind):
    """The one-launch kernel itself on edge shapes: T inside its window,
    with a ragged last tile (T % 256 != 0), K = 32, R = 1 and 64, repeated
    experts in a row, dropped routes, FP8."""
    import combine_get_dispatch_counts_amd as epx

    first, last = _one_launch_window(h, K, E, R, fp8)
    T = min(first + 37, last)
    assert epx.fused_launches(T, h, K, E, R, fp8) == 1
    say(f"fused kernel T={T} K={K} E={E} R={R} h={h} fp8={fp8} {kind}")
    rng = np.random.default_rng(T + K)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    if kind == "repeats":
        topk = rng.integers(-1, E, (T, K)).astype(np.int64)
    else:
        topk = synth.random_routing(T, K, E, seed=T + 3, p_drop=0.2 if kind == "dropped" else 0.0)
    w = rng.random((T, K)).astype(np.float32)
    _fused_check(x, topk, w, E, R, fp8, C=5)


@pytest.mark.parametrize("C_kind", ["dense", "past_T"])
def test_fused_kernel_many_channels(C_kind):
    """channel_prefix from the one-launch kernel when channels are shorter
    than a block's 8 tokens (several columns end in one block) and when
    there are more channels than tokens (every column past the last token
    ends at T), against the oracle."""
    import combine_get_dispatch_counts_amd as epx

    K, E, R, h, fp8 = 8, 64, 8, 256, False
    first, last = _one_launch_window(h, K, E, R, fp8)
    T = min(first + 101, last)
    assert epx.fused_launches(T, h, K, E, R, fp8) == 1
    C = 1000 if C_kind == "dense" else T + 7
    say(f"fused kernel T={T} C={C}")
    rng = np.random.default_rng(T + C)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=T + 5, p_drop=0.1)
    w = rng.random((T, K)).astype(np.float32)
    _fused_check(x, topk, w, E, R, fp8, C=C)


def test_fused_shares_workspace_with_layout():
    """One workspace for fused calls (small batches, which do not touch it,
    and one-launch / two-launch ones, which do) and two-launch layout calls
    in turn (the fused launch counts its blocks out as they finish, the
    layout kernel counts them in as they read the call number). After every
    call the counters are ready: no arrival pending, the second counter back
    at zero, the call number never going back."""
    import combine_get_dispatch_counts_amd as epx

    E, R, K, h = 64, 8, 6, 512
    ws = torch.zeros(epx.fused_workspace_size(4096, K, E, R), dtype=torch.uint8, device="cuda")
    last = 0

    def counters(what):
        nonlocal last
        head = ws[:128].cpu().numpy()  # calls << 32 | arrivals at byte 0; second counter at 64
        calls = int(head[:8].view(np.uint64)[0])
        assert calls & 0xFFFFFFFF == 0, f"arrivals pending after {what}: {calls:#x}"
        assert int(head[64:68].view(np.uint32)[0]) == 0, f"block count left by {what}"
        assert calls >> 32 >= last, f"call number went back after {what}"
        last = calls >> 32

    for i, T in enumerate([2048, 700, 4096, 1, 2048, 3000]):
        rng = np.random.default_rng(40 + i)
        x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
        topk = synth.random_routing(T, K, E, seed=50 + i)
        w = rng.random((T, K)).astype(np.float32)
        say(f"fused call {i} T={T} ({epx.fused_launches(T, h, K, E, R)} launch(es)) on a shared "
            "workspace")
        _fused_check(x, topk, w, E, R, False, ws=ws)
        counters(f"fused call {i}")
        lay = epx.get_dispatch_layout(torch.from_numpy(topk).cuda(), E, R, workspace=ws)
        assert epx.get_error() == 0
        counters(f"layout call {i}")
        ol = oracle.layout(topk, E, R)
        for k in LAYOUT_KEYS:
            _eq(host_bits(getattr(lay, k)), ol[k], f"layout call {i} {k}")


@pytest.mark.parametrize("T", [256, 1536, 2048])
def test_fused_step_in_graph(T):
    """A captured fused step (layout + dispatch, then combine) replayed three
    times equals the eager step bit for bit: the small-batch kernel (T =
    256), the two launches (T = 1536 at h = 4096: the tiled grid would not
    cover the device) and the tiled kernel (T = 2048)."""
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(4, T=T)
    wl = inp["workload"]
    h, E, R, K = wl.h, wl.E, wl.R, wl.K
    launches = epx.fused_launches(T, h, K, E, R)
    if T != 1536:
        assert launches == 1
    say(f"fused step in a graph T={T} ({launches} launch(es))")
    dev = torch.device("cuda")
    x, tk, w = dev_bf16(inp["x"]), torch.from_numpy(inp["topk_idx"]).cuda(), \
        torch.from_numpy(inp["topk_w"]).cuda()
    ws = torch.zeros(epx.fused_workspace_size(T, K, E, R), dtype=torch.uint8, device=dev)
    lay = epx.alloc_layout(T, K, E, R, None, dev)
    bufs = epx.alloc_dispatch(T, h, K, T * min(K, R), T * K, False, dev)
    y = synth.expert_outputs(T * K, h, seed=3, device="cuda")
    out = torch.empty((T, h), dtype=torch.bfloat16, device=dev)

    def step():
        d = epx.dispatch_fused(x, tk, w, E, R, layout=lay, out=bufs, workspace=ws)
        epx.combine(y, d.pos_exp, w, out=out)

    step()
    torch.cuda.synchronize()
    ref = [out.clone(), bufs["recv_x"].clone(), lay.pos_in_rank.clone()]
    if T == 256:  # the eager step itself against the oracle (larger T: other tests)
        o = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], E, R)
        n_recv = int(o["layout"]["totals"][1])
        _eq(host_bits(ref[1])[:n_recv], o["recv_x"], "eager recv_x")
        _eq(host_bits(ref[2]), o["layout"]["pos_in_rank"], "eager pos_in_rank")
        _eq(host_bits(ref[0]), oracle.combine(host_bits(y), inp["topk_w"],
                                              o["pos_exp"]), "eager combine")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(3):
        out.fill_(0)
        bufs["recv_x"].fill_(0)
        lay.pos_in_rank.fill_(-7)
        torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert epx.get_error() == 0
        for a, b in zip([out, bufs["recv_x"], lay.pos_in_rank], ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {replay} differs"


def test_fused_workspace_recovery():
    """A workspace in a state no call leaves (a layout call's arrivals left
    pending) is flagged by the fused call with no wait at all, and once it is
    zero-filled again the next call is correct."""
    import combine_get_dispatch_counts_amd as epx

    T, E, R, K, h = 2048, 64, 8, 6, 512
    ws = torch.zeros(epx.fused_workspace_size(T, K, E, R), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(61)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=62)
    w = rng.random((T, K)).astype(np.float32)
    say("fused call on a workspace with pending arrivals")
    _fused_check(x, topk, w, E, R, False, ws=ws)
    ws[:4].view(torch.int32).fill_(3)
    epx.dispatch_fused(dev_bf16(x), torch.from_numpy(topk).cuda(), torch.from_numpy(w).cuda(), E,
                       R, workspace=ws)
    flags = epx.get_error()
    assert flags == epx._lib.DEV_WORKSPACE, f"expected EPX_DEV_WORKSPACE, got {flags:#x}"
    ws.zero_()
    say("fused call after the workspace was zeroed")
    _fused_check(x, topk, w, E, R, False, ws=ws)


@pytest.mark.parametrize("T", [100, 4096, 9000])
def test_fused_flags_bad_route(T):
    """A top-k entry outside [-1, E) sets EPX_DEV_BAD_ROUTE in every regime
    of the fused call (small batch, tiled one launch, two launches); the
    entry is skipped, so no row lands outside the buffers."""
    import combine_get_dispatch_counts_amd as epx

    E, R, K, h = 64, 8, 4, 256
    rng = np.random.default_rng(T)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=T)
    topk[T // 2, 1] = E + 5
    topk[T - 1, 0] = -7
    w = rng.random((T, K)).astype(np.float32)
    say(f"fused call with bad routes T={T} ({epx.fused_launches(T, h, K, E, R)} launch(es))")
    d = epx.dispatch_fused(dev_bf16(x), torch.from_numpy(topk).cuda(), torch.from_numpy(w).cuda(),
                           E, R)
    flags = epx.get_error()
    assert flags == epx._lib.DEV_BAD_ROUTE, f"expected EPX_DEV_BAD_ROUTE, got {flags:#x}"
    pos = host_bits(d.pos_exp)
    assert pos[T // 2, 1] == -1 and pos[T - 1, 0] == -1
    assert int(d.layout.totals[1]) == T * K - 2
