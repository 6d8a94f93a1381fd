"""The paced store sweep changes when the dispatch stores its rows, never what
it stores: on the prefill (T=4096, h=7168, E=256, R=32, topk=8), the skewed
workload (T=8192: every wave slot of the device) and the FP8 prefill at
T=16384 (more tokens than one round of waves: launched in paced chunks) the
dispatch and the fused call give the same bytes with pacing off, at the default
rates, far below what the memory sustains and far above it, and the default
run matches the oracle; so do dispatches just below and just above the size
under which pacing is skipped. Also the setter's argument checks."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import host_bits, say

pytestmark = pytest.mark.gpu

DEFAULTS = (6450, 6400)  # the rates a new context starts with (include/epx.h)


def _run(epx, inp, fused, fp8, bufs, lay_buf, ws):
    wl = inp["workload"]
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda().view(torch.bfloat16)
    tk = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    for v in bufs.values():
        if v is not None:
            v.view(torch.uint8).fill_(0xA5)
    if fused:
        d = epx.dispatch_fused(x, tk, w, wl.E, wl.R, fp8=fp8, layout=lay_buf, out=bufs,
                               workspace=ws)
    else:
        lay = epx.get_dispatch_layout(tk, wl.E, wl.R, out=lay_buf)
        d = epx.dispatch(x, tk, w, wl.E, wl.R, fp8=fp8, layout=lay, out=bufs)
    flags = epx.get_error()
    assert flags == 0, f"device flags {flags:#x}"
    out = {k: host_bits(v) for k, v in bufs.items() if v is not None}
    out["totals"] = host_bits(d.layout.totals)
    return out


@pytest.mark.parametrize("cfg,fused,fp8", [
    (3, False, False), (3, False, True), (3, True, False), (3, True, True),
    (4, False, False),   # skewed routing
    (5, False, True),    # T = 16384: more tokens than one round, launched in paced chunks
])
def test_sweep_rate_does_not_change_outputs(cfg, fused, fp8):
    _check_rates(cfg, fused, fp8)


@pytest.mark.parametrize("T,fp8", [
    (1280, False), (1536, False),   # row bound 294 MB (left unpaced) / 352 MB (paced)
    (1024, True), (1152, True),     # FP8: 122 MB (left unpaced) / 137 MB (paced)
])
def test_sweep_size_threshold_edges(T, fp8):
    """Dispatches on either side of the size below which pacing is skipped
    (prefill shapes with fewer tokens): the same bytes at every rate, and the
    oracle's."""
    _check_rates(3, False, fp8, T)


@pytest.mark.parametrize("cfg,fp8,T", [
    (5, True, 10000),   # FP8, 64 ranks: three chunks of 3334, 3334 and 3332 tokens
    (3, False, 6001),   # bf16, h = 7168: two chunks of 3001 and 3000 tokens
])
def test_sweep_ragged_chunks(cfg, fp8, T):
    """Dispatches launched in chunks of unequal size (T not a multiple of
    the chunk count, so the last chunk's rows are placed by the estimate
    with its own token count): the same bytes at every rate, and the
    oracle's."""
    _check_rates(cfg, False, fp8, T)


def _check_rates(cfg, fused, fp8, T_override=None):
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(cfg, T=T_override)
    wl = inp["workload"]
    T, h, E, R, K = wl.T, wl.h, wl.E, wl.R, wl.K
    if fused:
        assert epx.fused_launches(T, h, K, E, R, fp8) == 1
    dev = torch.device("cuda")
    bufs = epx.alloc_dispatch(T, h, K, T * min(K, R), T * K, fp8, dev)
    lay_buf = epx.alloc_layout(T, K, E, R, None, dev)
    ws = torch.zeros(epx.fused_workspace_size(T, K, E, R), dtype=torch.uint8, device=dev)
    runs = {}
    prior = epx.get_sweep_rate()
    try:
        for rate in (DEFAULTS, (0, 0), (1500, 1500), (60000, 60000)):
            say(f"config {cfg} T={T} {'fused' if fused else 'dispatch'} fp8={fp8} sweep rate {rate}")
            epx.set_sweep_rate(*rate)
            runs[rate] = _run(epx, inp, fused, fp8, bufs, lay_buf, ws)
    finally:
        epx.set_sweep_rate(*prior)
    ref = runs[(0, 0)]
    for rate, got in runs.items():
        for k in ref:
            assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), \
                f"{k} differs at sweep rate {rate}"
    # the default run against the oracle (rows up to the totals)
    o = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], E, R, fp8=fp8)
    n_send, n_recv = (int(v) for v in ref["totals"])
    got = runs[DEFAULTS]
    for k in ["send_x", "send_src", "send_topk_idx", "send_topk_w", "recv_x", "recv_src",
              "pos_exp"]:
        g = got[k] if k == "pos_exp" else got[k][:n_send if k.startswith("send") else n_recv]
        assert np.array_equal(g.view(np.uint8), np.asarray(o[k]).view(np.uint8)), k
    if fp8:
        ngrp = h // 128
        for k, n in (("send_scales", n_send), ("recv_scales", n_recv)):
            assert np.array_equal(got[k][:n, :ngrp].view(np.uint32),
                                  np.asarray(o[k]).view(np.uint32)), k


def test_sweep_rate_receive_permute():
    """The receiver's permute of the prefill's 29 811 rank-major rows into 8
    local experts (the permute alone, which is left unpaced) stores the same
    bytes whatever the sweep rate."""
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(3)
    wl = inp["workload"]
    T, h, E, R, K = wl.T, wl.h, wl.E, wl.R, wl.K
    d = epx.dispatch(torch.from_numpy(inp["x"].view(np.int16)).cuda().view(torch.bfloat16),
                     torch.from_numpy(inp["topk_idx"]).cuda(),
                     torch.from_numpy(inp["topk_w"]).cuda(), E, R)
    rows, idx = d.send_x, d.send_topk_idx
    got = {}
    prior = epx.get_sweep_rate()
    try:
        for rate in (DEFAULTS, (0, 0)):
            say(f"receive permute of {rows.shape[0]} rows, sweep rate {rate}")
            epx.set_sweep_rate(*rate)
            rec = epx.recv_permute(rows, idx, E // R)
            assert epx.get_error() == 0
            n = int(rec.layout.totals[1].item())  # rows past the total are not written
            got[rate] = (host_bits(rec.x)[:n], host_bits(rec.src_row)[:n], host_bits(rec.pos))
    finally:
        epx.set_sweep_rate(*prior)
    for a, b in zip(got[DEFAULTS], got[(0, 0)]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_chunked_dispatch_in_graph():
    """The FP8 prefill dispatch (T = 16384: several paced chunk launches)
    captured in a HIP graph and replayed three times, with the outputs
    scribbled over and unrelated work run between replays: every replay
    stores what the eager call stored."""
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(5)
    wl = inp["workload"]
    T, h, E, R, K = wl.T, wl.h, wl.E, wl.R, wl.K
    dev = torch.device("cuda")
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda().view(torch.bfloat16)
    tk = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    ws = torch.zeros(epx.workspace_size(T, K, E, R), dtype=torch.uint8, device=dev)
    lay = epx.get_dispatch_layout(tk, E, R, workspace=ws, out=epx.alloc_layout(T, K, E, R, None, dev))
    bufs = epx.alloc_dispatch(T, h, K, T * min(K, R), T * K, True, dev)
    say(f"chunked FP8 dispatch T={T} in a graph")
    epx.dispatch(x, tk, w, E, R, fp8=True, layout=lay, out=bufs)
    torch.cuda.synchronize()
    n_send, n_recv = (int(v) for v in lay.totals.cpu())
    keys = ["send_x", "send_scales", "recv_x", "recv_scales", "recv_src", "pos_exp"]
    def used(k):
        v = bufs[k]
        return v[:n_send] if k.startswith("send") else v[:n_recv] if k.startswith("recv") else v
    ref = {k: used(k).clone() for k in keys}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        epx.dispatch(x, tk, w, E, R, fp8=True, layout=lay, out=bufs)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        epx.dispatch(x, tk, w, E, R, fp8=True, layout=lay, out=bufs)
    for replay in range(3):
        for k in keys:
            used(k).view(torch.uint8).fill_(0x5A)
        torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert epx.get_error() == 0
        for k in keys:
            assert torch.equal(used(k).view(torch.uint8), ref[k].view(torch.uint8)), \
                f"replay {replay}: {k} differs"


def test_sweep_rate_argument_checks():
    import combine_get_dispatch_counts_amd as epx

    prior = epx.get_sweep_rate()
    try:
        with pytest.raises(epx.EpxError):
            epx.set_sweep_rate(-1, 6000)
        with pytest.raises(epx.EpxError):
            epx.set_sweep_rate(6200, 100001)
        assert epx.get_sweep_rate() == prior  # a rejected call changes nothing
        epx.set_sweep_rate(100000, 0)
        assert epx.get_sweep_rate() == (100000, 0)
    finally:
        epx.set_sweep_rate(*prior)
    assert epx.get_sweep_rate() == prior


def test_calibrated_sweep_rate():
    """The calibration times a fill of a 1 GiB scratch and sets both rates
    to their fixed fractions of it; a scratch smaller than the memory-side
    cache is refused and leaves the rates alone. Outputs at the calibrated
    rates are those at the defaults (checked for the prefill dispatch)."""
    import combine_get_dispatch_counts_amd as epx

    prior = epx.get_sweep_rate()
    try:
        small = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        with pytest.raises(epx.EpxError):
            epx.calibrate_sweep_rate(small)
        assert epx.get_sweep_rate() == prior
        del small
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fill = epx.calibrate_sweep_rate(scratch)
        del scratch
        b, f = epx.get_sweep_rate()
        say(f"calibration: fill {fill} GB/s -> sweep rates {b} (bf16), {f} (FP8)")
        assert 2000 < fill < 20000, fill
        assert abs(b - fill * 0.956) <= 2, (b, fill)
        assert abs(f - fill * 0.948) <= 2, (f, fill)
    finally:
        epx.set_sweep_rate(*prior)


@pytest.mark.parametrize("fused,fp8", [(False, False), (False, True), (True, False), (True, True)])
def test_sweep_widest_one_pass_rows(fused, fp8):
    """Paced rows of 8192 channels, the widest one register pass holds (the
    largest row shape of each kernel), on the prefill routing at T = 2048:
    the same bytes at every rate, and the oracle's."""
    from dataclasses import replace

    _check_rates(replace(synth.WORKLOADS[3], h=8192), fused, fp8, 2048)
