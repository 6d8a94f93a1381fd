"""Multi-source receive on one GPU: R logical source ranks, each holding a
consecutive slice of the tokens, run layout and dispatch on their own
tokens; each destination receives its segment from every source, in source
order (the transport itself is a copy here), and arranges the received rows
into per-local-expert blocks (the receiver's permute of the high-throughput
mode). Because the sources hold consecutive token ranges, the receiver's
(source, token) order is global token order, so destination d's blocks must
equal the oracle's expert-major buffer over d's experts for all tokens.
The low-latency buffer is filled by every source, region (e, s) by source
s, and checked against the oracle source by source."""
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


@pytest.mark.parametrize("fp8", [False, True])
def test_multi_source_receive_permute(fp8):
    T, h, E, R, K = 512, 1024, 64, 8, 6
    rng = np.random.default_rng(77)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=78, p_drop=0.05)
    w = rng.random((T, K)).astype(np.float32)
    _check_receive(x, topk, w, E, R, fp8)


@pytest.mark.parametrize("fp8", [False, True])
def test_multi_source_receive_prefill_shape(fp8):
    """The prefill shape: 32 logical sources of 128 tokens each (T = 4096,
    h = 7168, E = 256, top-8 on the prefill routing), every one of the 32
    destinations' permuted blocks -- rows, FP8 scales and source rows --
    against the oracle's expert-major buffer over that destination's experts."""
    inp = synth.make_inputs(3)
    wl = inp["workload"]
    _check_receive(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, fp8)


def _check_receive(x, topk, w, E, R, fp8):
    import combine_get_dispatch_counts_amd as epx

    T, h = x.shape
    K = topk.shape[1]
    L, per = E // R, T // R
    say(f"multi-source receive T={T} h={h} E={E} R={R} K={K} fp8={fp8}")

    # every source: layout + dispatch over its own tokens
    sent = []
    for s in range(R):
        sl = slice(s * per, (s + 1) * per)
        tk = torch.from_numpy(np.ascontiguousarray(topk[sl])).cuda()
        lay = epx.get_dispatch_layout(tk, E, R)
        d = epx.dispatch(dev_bf16(np.ascontiguousarray(x[sl])), tk,
                         torch.from_numpy(np.ascontiguousarray(w[sl])).cuda(), E, R, fp8=fp8,
                         layout=lay)
        sent.append((lay.rank_off.cpu().numpy(), d))
    assert epx.get_error() == 0

    o = oracle.dispatch(x, topk, w, E, R, fp8=fp8)
    exp_off = o["layout"]["exp_off"]
    ngrp = h // 128
    for dst in range(R):
        seg = [(ro[dst], ro[dst + 1], d) for ro, d in sent]
        rows = torch.cat([d.send_x[a:b] for a, b, d in seg])
        idx = torch.cat([d.send_topk_idx[a:b] for a, b, d in seg])
        sc = torch.cat([d.send_scales[a:b] for a, b, d in seg]) if fp8 else None
        rec = epx.recv_permute(rows, idx, L, scales=sc)
        assert epx.get_error() == 0
        lo, hi = exp_off[dst * L], exp_off[(dst + 1) * L]
        n = hi - lo
        _eq(host_bits(rec.layout.num_tokens_per_expert),
            o["layout"]["num_tokens_per_expert"][dst * L:(dst + 1) * L], f"dst {dst} counts")
        _eq(host_bits(rec.x)[:n], o["recv_x"][lo:hi], f"dst {dst} rows")
        if fp8:
            _eq(host_bits(rec.scales)[:n, :ngrp], o["recv_scales"][lo:hi], f"dst {dst} scales")
        # each output row came from the received row holding the same token
        src_tok = np.concatenate([d.send_src[a:b].cpu().numpy() + s * per
                                  for s, (a, b, d) in enumerate(seg)])
        _eq(src_tok[host_bits(rec.src_row)[:n]], o["recv_src"][lo:hi], f"dst {dst} sources")


def test_low_latency_buffer_filled_by_every_source():
    import combine_get_dispatch_counts_amd as epx

    T, h, E, R, K, cap = 256, 1024, 64, 8, 6, 64
    per = T // R
    rng = np.random.default_rng(91)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=92)
    say(f"low-latency buffer from all {R} sources, T={T} h={h} E={E} cap={cap}")
    dev = torch.device("cuda")
    buf = epx.alloc_ll(E, R, cap, h, per, K, True, dev)
    buf.ll_x.view(torch.uint8).fill_(CANARY)
    buf.ll_src.view(torch.uint8).fill_(CANARY)
    pos = []
    for s in range(R):
        sl = slice(s * per, (s + 1) * per)
        epx.ll_dispatch(dev_bf16(np.ascontiguousarray(x[sl])),
                        torch.from_numpy(np.ascontiguousarray(topk[sl])).cuda(), E, R, s, cap, R,
                        True, buf)
        pos.append(host_bits(buf.pos_ll).copy())
    assert epx.get_error() == 0
    counts = host_bits(buf.ll_count).reshape(E, R)
    assert (counts >= 0).all(), "a region count was left empty"
    x4 = host_bits(buf.ll_x).reshape(E, R, cap, h)
    src4 = host_bits(buf.ll_src).reshape(E, R, cap)
    for s in range(R):
        sl = slice(s * per, (s + 1) * per)
        o = oracle.ll_dispatch(np.ascontiguousarray(x[sl]), np.ascontiguousarray(topk[sl]), E, R,
                               s, cap, 1, fp8=True)
        _eq(counts[:, s], o["ll_count"], f"source {s} counts")
        _eq(src4[:, s].reshape(-1), o["ll_src"], f"source {s} sources")
        written = o["ll_src"] >= 0
        _eq(x4[:, s].reshape(E * cap, h)[written], o["ll_x"][written], f"source {s} rows")
        # the handle addresses the full layout: region e*R + s
        p = o["pos_ll"]
        full = np.where(p >= 0, ((p // cap) * R + s) * cap + p % cap, -1)
        _eq(pos[s], full, f"source {s} handle")


@pytest.mark.parametrize("fp8", [False, True])
def test_two_level_dedup_node_then_rank(fp8):
    """Two-level dedup on the GPU: the pack at node granularity (R = N
    logical nodes, one row per (token, node)), then inside every node the
    pack of the node's received rows over its R/N ranks, using the
    node-local indices and weights the first pack wrote (FP8 codes move as
    bit patterns, their scales travel with the source row). Every rank must
    receive exactly the oracle's one-level rank-major rows, in order."""
    import combine_get_dispatch_counts_amd as epx

    T, h, E, R, N, K = 512, 1024, 64, 8, 2, 6
    L_node, per_node = E // N, R // N
    rng = np.random.default_rng(55)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=56, p_drop=0.05)
    w = rng.random((T, K)).astype(np.float32)
    say(f"two-level dedup T={T} h={h} E={E} R={R} nodes={N} K={K} fp8={fp8}")

    tk = torch.from_numpy(topk).cuda()
    lay1 = epx.get_dispatch_layout(tk, E, N)
    d1 = epx.dispatch(dev_bf16(x), tk, torch.from_numpy(w).cuda(), E, N, fp8=fp8, layout=lay1)
    assert epx.get_error() == 0
    o = oracle.dispatch(x, topk, w, E, R, fp8=fp8)
    ro = o["layout"]["rank_off"]
    assert int(lay1.totals[0]) < int(o["layout"]["totals"][0]), "no token shared a node"
    ro1 = lay1.rank_off.cpu().numpy()
    ngrp = h // 128
    for n in range(N):
        a, b = int(ro1[n]), int(ro1[n + 1])
        rows = d1.send_x[a:b]
        if fp8:
            rows = rows.view(torch.bfloat16)  # codes as bit patterns, h/2 wide
        idx, wn = d1.send_topk_idx[a:b], d1.send_topk_w[a:b]
        lay2 = epx.get_dispatch_layout(idx, L_node, per_node)
        d2 = epx.dispatch(rows, idx, wn, L_node, per_node, layout=lay2)
        assert epx.get_error() == 0
        ro2 = lay2.rank_off.cpu().numpy()
        src1 = host_bits(d1.send_src)[a:b]
        for g in range(per_node):
            r = n * per_node + g
            a2, b2 = int(ro2[g]), int(ro2[g + 1])
            fa, fb = int(ro[r]), int(ro[r + 1])
            sel = host_bits(d2.send_src)[a2:b2]
            _eq(src1[sel], o["send_src"][fa:fb], f"rank {r} sources")
            got = host_bits(d2.send_x)[a2:b2]
            if fp8:
                got = np.ascontiguousarray(got).view(np.uint8)
                _eq(host_bits(d1.send_scales)[a:b][sel, :ngrp], o["send_scales"][fa:fb],
                    f"rank {r} scales")
            _eq(got, o["send_x"][fa:fb], f"rank {r} rows")
            _eq(host_bits(d2.send_topk_idx)[a2:b2], o["send_topk_idx"][fa:fb], f"rank {r} indices")
            _eq(host_bits(d2.send_topk_w)[a2:b2], o["send_topk_w"][fa:fb], f"rank {r} weights")


def test_permute_side_rows_and_errors():
    """epx_permute on its own: rows of an odd width (48 bytes) with 64-byte
    side rows, every entry to its local-expert block in received order, the
    side row with it; an entry outside [-1, L) sets EPX_DEV_BAD_ROUTE and is
    skipped, and a capacity one row short sets EPX_DEV_OVERFLOW and writes
    nothing past it."""
    import ctypes

    import combine_get_dispatch_counts_amd as epx
    from combine_get_dispatch_counts_amd import _lib

    N, K, L = 300, 3, 5
    rng = np.random.default_rng(5)
    idx = rng.integers(-1, L, (N, K)).astype(np.int64)
    rows = rng.integers(0, 256, (N, 48), dtype=np.uint8)
    side = rng.integers(0, 256, (N, 64), dtype=np.uint8)
    o = oracle.layout(idx, L, 1)
    n_out = int(o["totals"][1])
    dev = torch.device("cuda")
    lib = _lib.load()

    def run(idx_np, cap):
        tk = torch.from_numpy(idx_np).to(dev)
        lay = epx.get_dispatch_layout(tk, L, 1)
        out = torch.full((cap + 2, 48), CANARY, dtype=torch.uint8, device=dev)
        out_side = torch.full((cap + 2, 64), CANARY, dtype=torch.uint8, device=dev)
        src = torch.full((cap + 2,), -9, dtype=torch.int32, device=dev)
        pos = torch.empty((N, K), dtype=torch.int32, device=dev)
        r = torch.from_numpy(rows).to(dev)
        sd = torch.from_numpy(side).to(dev)
        rc = lib.epx_permute(epx.api._ctx(dev), ctypes.c_void_p(r.data_ptr()), 48,
                             ctypes.c_void_p(sd.data_ptr()), 64, ctypes.c_void_p(tk.data_ptr()),
                             N, K, L, ctypes.c_void_p(lay.exp_off.data_ptr()),
                             ctypes.c_void_p(lay.slot_in_expert.data_ptr()),
                             ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(out_side.data_ptr()),
                             ctypes.c_void_p(src.data_ptr()), cap, ctypes.c_void_p(pos.data_ptr()),
                             epx.api._stream(dev))
        assert rc == 0
        return epx.get_error(), host_bits(out), host_bits(out_side), host_bits(src), host_bits(pos)

    say(f"epx_permute N={N} K={K} L={L}, 48-byte rows, 64-byte side rows")
    flags, out, out_side, src, pos = run(idx, n_out)
    assert flags == 0
    order = np.argsort(np.where(idx >= 0, idx, L).ravel(), kind="stable")[:n_out]
    want_src = (order // K).astype(np.int32)
    _eq(src[:n_out], want_src, "src_row")
    _eq(out[:n_out], rows[want_src], "rows")
    _eq(out_side[:n_out], side[want_src], "side rows")
    assert (out[n_out:] == CANARY).all() and (src[n_out:] == -9).all()
    want_pos = np.full(N * K, -1, np.int32)
    want_pos[order] = np.arange(n_out, dtype=np.int32)
    _eq(pos.ravel(), want_pos, "pos")

    bad = idx.copy()
    bad[7, 1] = L  # outside [-1, L): skipped and flagged by the layout and the permute
    flags, *_ = run(bad, n_out)
    assert flags & _lib.DEV_BAD_ROUTE
    flags, out, _, src, _ = run(idx, n_out - 1)
    assert flags & _lib.DEV_OVERFLOW
    assert (out[n_out - 1:] == CANARY).all() and (src[n_out - 1:] == -9).all()


@pytest.mark.parametrize("width", [8192, 14336, 16400, 32768])
def test_permute_row_widths(width):
    """epx_permute on rows with no side rows at the widths that pick each
    row register shape (up to 512 vectors, up to 896, more, and rows that
    take two register passes, one of them ragged): every row to each of its
    local-expert blocks in received order, bit for bit, with its handle."""
    import ctypes

    import combine_get_dispatch_counts_amd as epx
    from combine_get_dispatch_counts_amd import _lib

    N, K, L = 700, 4, 6
    rng = np.random.default_rng(width)
    idx = rng.integers(-1, L, (N, K)).astype(np.int64)
    rows = rng.integers(0, 256, (N, width), dtype=np.uint8)
    o = oracle.layout(idx, L, 1)
    n_out = int(o["totals"][1])
    dev = torch.device("cuda")
    say(f"epx_permute N={N} K={K} L={L}, {width}-byte rows")
    tk = torch.from_numpy(idx).to(dev)
    lay = epx.get_dispatch_layout(tk, L, 1)
    out = torch.full((n_out + 2, width), CANARY, dtype=torch.uint8, device=dev)
    src = torch.full((n_out + 2,), -9, dtype=torch.int32, device=dev)
    pos = torch.empty((N, K), dtype=torch.int32, device=dev)
    r = torch.from_numpy(rows).to(dev)
    rc = _lib.load().epx_permute(epx.api._ctx(dev), ctypes.c_void_p(r.data_ptr()), width, None, 0,
                                 ctypes.c_void_p(tk.data_ptr()), N, K, L,
                                 ctypes.c_void_p(lay.exp_off.data_ptr()),
                                 ctypes.c_void_p(lay.slot_in_expert.data_ptr()),
                                 ctypes.c_void_p(out.data_ptr()), None,
                                 ctypes.c_void_p(src.data_ptr()), n_out,
                                 ctypes.c_void_p(pos.data_ptr()), epx.api._stream(dev))
    assert rc == 0
    assert epx.get_error() == 0
    out, src, pos = host_bits(out), host_bits(src), host_bits(pos)
    order = np.argsort(np.where(idx >= 0, idx, L).ravel(), kind="stable")[:n_out]
    want_src = (order // K).astype(np.int32)
    _eq(src[:n_out], want_src, "src_row")
    _eq(out[:n_out], rows[want_src], "rows")
    assert (out[n_out:] == CANARY).all() and (src[n_out:] == -9).all()
    want_pos = np.full(N * K, -1, np.int32)
    want_pos[order] = np.arange(n_out, dtype=np.int32)
    _eq(pos.ravel(), want_pos, "pos")
