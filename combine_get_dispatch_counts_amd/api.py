"""Thin torch binding over libepx: tensors in, tensors out.

Every step of the path runs in the HIP kernels behind the C ABI; this module
only allocates output tensors with torch (device memory), takes the current
HIP stream, and marshals pointers and sizes. Names follow the C ABI
(epx_get_dispatch_layout -> get_dispatch_layout, and so on).

Shapes: x [T,h] bf16; topk_idx [T,K] int64 (-1 = no route); topk_weights
[T,K] fp32. Destination ranks are logical partitions of the experts:
rank r holds experts [r*L, (r+1)*L), L = num_experts // num_ranks.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import EpxError, check

_contexts: dict[int, ctypes.c_void_p] = {}


def _ctx(device: torch.device) -> ctypes.c_void_p:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _contexts:
        h = ctypes.c_void_p()
        check(_lib.load().epx_create(ctypes.byref(h), idx), "epx_create")
        _contexts[idx] = h
    return _contexts[idx]


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _p(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor | None, dtype: torch.dtype, name: str, ndim: int | None = None,
          shape: tuple | None = None, device: torch.device | None = None):
    """Reject what the kernels cannot take: the C ABI sees bare pointers and
    row counts, so every buffer's dtype, shape and device is checked here."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _nbytes(ws: torch.Tensor, dev: torch.device) -> int:
    if not ws.is_cuda or ws.device != dev or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return ws.numel() * ws.element_size()


def _check_layout(lay: "Layout", T: int, K: int, E: int, R: int, C: int | None,
                  dev: torch.device) -> None:
    i32 = torch.int32
    _need(lay.num_tokens_per_expert, i32, "num_tokens_per_expert", shape=(E,), device=dev)
    _need(lay.num_tokens_per_rank, i32, "num_tokens_per_rank", shape=(R,), device=dev)
    _need(lay.is_token_in_rank, torch.uint8, "is_token_in_rank", shape=(T, R), device=dev)
    _need(lay.rank_off, i32, "rank_off", shape=(R + 1,), device=dev)
    _need(lay.exp_off, i32, "exp_off", shape=(E + 1,), device=dev)
    _need(lay.pos_in_rank, i32, "pos_in_rank", shape=(T, R), device=dev)
    _need(lay.slot_in_expert, i32, "slot_in_expert", shape=(T, K), device=dev)
    _need(lay.totals, i32, "totals", shape=(2,), device=dev)
    if C:
        _need(lay.channel_prefix, i32, "channel_prefix", shape=(R, C), device=dev)


def _check_dispatch_out(out: dict, T: int, h: int, K: int, fp8: bool,
                        dev: torch.device) -> None:
    """``out`` as alloc_dispatch makes it (row slices of those tensors
    included): the send arrays share send_x's row count, the receive
    arrays recv_x's."""
    dt = torch.uint8 if fp8 else torch.bfloat16
    _need(out.get("send_x"), dt, "send_x", ndim=2, device=dev)
    _need(out.get("recv_x"), dt, "recv_x", ndim=2, device=dev)
    ns, nr = out["send_x"].shape[0], out["recv_x"].shape[0]
    _need(out["send_x"], dt, "send_x", shape=(ns, h))
    _need(out["recv_x"], dt, "recv_x", shape=(nr, h))
    _need(out.get("send_src"), torch.int32, "send_src", shape=(ns,), device=dev)
    _need(out.get("send_topk_idx"), torch.int64, "send_topk_idx", shape=(ns, K), device=dev)
    _need(out.get("send_topk_w"), torch.float32, "send_topk_w", shape=(ns, K), device=dev)
    _need(out.get("recv_src"), torch.int32, "recv_src", shape=(nr,), device=dev)
    _need(out.get("pos_exp"), torch.int32, "pos_exp", shape=(T, K), device=dev)
    if fp8:
        st = scale_stride(h)
        _need(out.get("send_scales"), torch.float32, "send_scales", shape=(ns, st), device=dev)
        _need(out.get("recv_scales"), torch.float32, "recv_scales", shape=(nr, st), device=dev)


_workspaces: dict[tuple[int, int], torch.Tensor] = {}


def _layout_workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    """A zero-filled layout workspace of >= nbytes for this device and
    stream, kept for later calls (the layout call leaves it reusable)."""
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def workspace_size(T: int, K: int, E: int, R: int) -> int:
    n = ctypes.c_size_t()
    check(_lib.load().epx_workspace_size(T, K, E, R, ctypes.byref(n)), "epx_workspace_size")
    return n.value


def ll_size_hint(max_tokens_per_rank: int, h: int, R: int, E: int, fp8: bool) -> int:
    return int(_lib.load().epx_ll_size_hint(max_tokens_per_rank, h, R, E, int(fp8)))


def set_sweep_rate(bf16_gbps: int, fp8_gbps: int, device: torch.device | None = None) -> None:
    """Rate (GB/s of destination rows) of the high-throughput dispatch's
    paced store sweep for bf16 and FP8 rows; 0 turns pacing off. Outputs do
    not depend on it (see epx_set_sweep_rate in include/epx.h)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    check(_lib.load().epx_set_sweep_rate(_ctx(device), int(bf16_gbps), int(fp8_gbps)),
          "epx_set_sweep_rate")


def get_sweep_rate(device: torch.device | None = None) -> tuple[int, int]:
    """The context's current sweep rates (bf16, FP8) in GB/s."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    b, f = ctypes.c_int(), ctypes.c_int()
    check(_lib.load().epx_get_sweep_rate(_ctx(device), ctypes.byref(b), ctypes.byref(f)),
          "epx_get_sweep_rate")
    return b.value, f.value


def calibrate_sweep_rate(scratch: torch.Tensor) -> int:
    """Set the sweep rates from a fill of ``scratch`` (a contiguous GPU tensor
    of at least 512 MiB, overwritten) timed on the current stream; waits for
    the stream. Returns the measured fill rate in GB/s."""
    if not scratch.is_cuda or not scratch.is_contiguous():
        raise ValueError("scratch must be a contiguous GPU tensor")
    dev = scratch.device
    fill = ctypes.c_int()
    check(_lib.load().epx_calibrate_sweep_rate(_ctx(dev), _p(scratch),
                                               scratch.numel() * scratch.element_size(),
                                               ctypes.byref(fill), _stream(dev)),
          "epx_calibrate_sweep_rate")
    return fill.value


def get_error(device: torch.device | None = None) -> int:
    """Synchronise the current stream, return and clear the device error bits."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    flags = ctypes.c_int()
    rc = _lib.load().epx_get_error(_ctx(device), ctypes.byref(flags), _stream(device))
    if rc not in (_lib.EPX_OK, _lib.EPX_EDEVICE):
        check(rc, "epx_get_error")
    return flags.value


@dataclass
class Layout:
    num_tokens_per_expert: torch.Tensor  # [E] int32
    num_tokens_per_rank: torch.Tensor    # [R] int32
    is_token_in_rank: torch.Tensor       # [T,R] uint8
    rank_off: torch.Tensor               # [R+1] int32
    exp_off: torch.Tensor                # [E+1] int32
    pos_in_rank: torch.Tensor            # [T,R] int32
    slot_in_expert: torch.Tensor         # [T,K] int32
    channel_prefix: torch.Tensor | None  # [R,C] int32
    totals: torch.Tensor                 # [2] int32 (send rows, recv rows)
    num_experts: int
    num_ranks: int


def alloc_layout(T: int, K: int, E: int, R: int, num_channels: int | None,
                 device: torch.device) -> Layout:
    """Output tensors for get_dispatch_layout (reusable across calls)."""
    i32 = dict(dtype=torch.int32, device=device)
    return Layout(
        num_tokens_per_expert=torch.empty(E, **i32),
        num_tokens_per_rank=torch.empty(R, **i32),
        is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=device),
        rank_off=torch.empty(R + 1, **i32),
        exp_off=torch.empty(E + 1, **i32),
        pos_in_rank=torch.empty((T, R), **i32),
        slot_in_expert=torch.empty((T, K), **i32),
        channel_prefix=torch.empty((R, num_channels), **i32) if num_channels else None,
        totals=torch.empty(2, **i32),
        num_experts=E, num_ranks=R)


def get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                        num_channels: int | None = None, workspace: torch.Tensor | None = None,
                        totals_host: torch.Tensor | None = None,
                        out: Layout | None = None) -> Layout:
    """Counts, is_token_in_rank and receive offsets for topk_idx. ``out``
    (from alloc_layout with the same shapes) avoids allocating; ``workspace``
    must hold workspace_size(T, K, E, R) bytes and be zero-filled before its
    first use (each call leaves it ready for the next; without one, a cached
    workspace per device and stream is used); ``totals_host`` (pinned int32
    [2]) also receives the totals, readable after a stream synchronisation."""
    _need(topk_idx, torch.int64, "topk_idx", 2)
    dev = topk_idx.device
    T, K = topk_idx.shape
    E, R = num_experts, num_ranks
    lay = out if out is not None else alloc_layout(T, K, E, R, num_channels, dev)
    _check_layout(lay, T, K, E, R, num_channels, dev)
    if workspace is None:
        workspace = _layout_workspace(dev, workspace_size(T, K, E, R))
    ws_bytes = _nbytes(workspace, dev)
    if totals_host is not None and not (totals_host.is_pinned() and totals_host.numel() >= 2
                                        and totals_host.dtype == torch.int32):
        raise ValueError("totals_host must be a pinned int32 tensor of >= 2 elements")
    cp = lay.channel_prefix if num_channels else None
    rc = _lib.load().epx_get_dispatch_layout(
        _ctx(dev), _p(topk_idx), T, K, E, R, num_channels or 0,
        _p(lay.num_tokens_per_expert), _p(lay.num_tokens_per_rank), _p(lay.is_token_in_rank),
        _p(lay.rank_off), _p(lay.exp_off), _p(lay.pos_in_rank), _p(lay.slot_in_expert),
        _p(cp), _p(lay.totals), _p(totals_host), _p(workspace),
        ws_bytes, _stream(dev))
    check(rc, "epx_get_dispatch_layout")
    return lay


def get_dispatch_layout_noalloc(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                                num_channels: int | None = None,
                                totals_host: torch.Tensor | None = None,
                                out: Layout | None = None) -> Layout:
    """get_dispatch_layout with the library's own fixed device scratch as
    the workspace (no allocation by the library; with ``out`` given, none
    here either). Calls on one GPU share that scratch and must not overlap."""
    _need(topk_idx, torch.int64, "topk_idx", 2)
    dev = topk_idx.device
    T, K = topk_idx.shape
    E, R = num_experts, num_ranks
    lay = out if out is not None else alloc_layout(T, K, E, R, num_channels, dev)
    _check_layout(lay, T, K, E, R, num_channels, dev)
    if totals_host is not None and not (totals_host.is_pinned() and totals_host.numel() >= 2
                                        and totals_host.dtype == torch.int32):
        raise ValueError("totals_host must be a pinned int32 tensor of >= 2 elements")
    cp = lay.channel_prefix if num_channels else None
    rc = _lib.load().epx_get_dispatch_layout_noalloc(
        _ctx(dev), _p(topk_idx), T, K, E, R, num_channels or 0,
        _p(lay.num_tokens_per_expert), _p(lay.num_tokens_per_rank), _p(lay.is_token_in_rank),
        _p(lay.rank_off), _p(lay.exp_off), _p(lay.pos_in_rank), _p(lay.slot_in_expert),
        _p(cp), _p(lay.totals), _p(totals_host), _stream(dev))
    check(rc, "epx_get_dispatch_layout_noalloc")
    return lay


def scale_stride(h: int) -> int:
    """fp32 entries per FP8 scale row: h/128 rounded up to whole 128-byte
    lines; the entries past h/128 are written as +0.0."""
    n = _lib.load().epx_scale_stride(h)
    if n <= 0:  # the code epx_dispatch gives for such an h with fp8
        bad_h = h < 8 or h % 8 != 0
        raise EpxError(_lib.EPX_EINVAL if bad_h else _lib.EPX_EUNSUPPORTED,
                       f"FP8 rows need h % 128 == 0 (h = {h})")
    return n


@dataclass
class Dispatched:
    """Dispatch outputs. FP8 scales are [rows, scale_stride(h)]: the group
    scales of row i are ``send_scales[i, :h // 128]``."""
    send_x: torch.Tensor          # [rows, h] bf16, or uint8 codes with fp8
    send_scales: torch.Tensor | None
    send_src: torch.Tensor        # [rows] int32
    send_topk_idx: torch.Tensor   # [rows, K] int64
    send_topk_w: torch.Tensor     # [rows, K] fp32
    recv_x: torch.Tensor          # [rows, h] expert-major
    recv_scales: torch.Tensor | None
    recv_src: torch.Tensor        # [rows] int32
    pos_exp: torch.Tensor         # [T, K] int32 -- the handle for combine
    layout: Layout


def alloc_dispatch(T: int, h: int, K: int, send_rows: int, recv_rows: int, fp8: bool,
                   device: torch.device) -> dict:
    """Output buffers for dispatch with the given row capacities."""
    dt = torch.uint8 if fp8 else torch.bfloat16
    f32 = dict(dtype=torch.float32, device=device)
    return dict(
        send_x=torch.empty((send_rows, h), dtype=dt, device=device),
        send_scales=torch.empty((send_rows, scale_stride(h)), **f32) if fp8 else None,
        send_src=torch.empty(send_rows, dtype=torch.int32, device=device),
        send_topk_idx=torch.empty((send_rows, K), dtype=torch.int64, device=device),
        send_topk_w=torch.empty((send_rows, K), **f32),
        recv_x=torch.empty((recv_rows, h), dtype=dt, device=device),
        recv_scales=torch.empty((recv_rows, scale_stride(h)), **f32) if fp8 else None,
        recv_src=torch.empty(recv_rows, dtype=torch.int32, device=device),
        pos_exp=torch.empty((T, K), dtype=torch.int32, device=device))


def dispatch(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
             num_experts: int, num_ranks: int, fp8: bool = False, layout: Layout | None = None,
             out: dict | None = None, exact: bool = True) -> Dispatched:
    """Rank-deduplicated pack + expert-major permute (+ FP8).

    Buffers: ``out`` (from alloc_dispatch) if given; else, with ``exact``,
    one host wait on the layout totals sizes them exactly (the pages' CPU
    wait before allocating the receive tensor); otherwise worst-case sizes
    T*min(K,R) and T*K rows are used and no wait happens."""
    _need(x, torch.bfloat16, "x", 2)
    dev = x.device
    T, h = x.shape
    _need(topk_idx, torch.int64, "topk_idx", 2, device=dev)
    K = topk_idx.shape[1]
    _need(topk_idx, torch.int64, "topk_idx", shape=(T, K))
    _need(topk_weights, torch.float32, "topk_weights", shape=(T, K), device=dev)
    if layout is None:
        layout = get_dispatch_layout(topk_idx, num_experts, num_ranks)
    _check_layout(layout, T, K, num_experts, num_ranks, None, dev)
    if out is None:
        if exact:
            n_send, n_recv = (int(v) for v in layout.totals.cpu())
        else:
            n_send, n_recv = T * min(K, num_ranks), T * K
        out = alloc_dispatch(T, h, K, n_send, n_recv, fp8, dev)
    _check_dispatch_out(out, T, h, K, fp8, dev)
    rc = _lib.load().epx_dispatch(
        _ctx(dev), _p(x), h, _p(topk_idx), _p(topk_weights), T, K, num_experts, num_ranks,
        _p(layout.rank_off), _p(layout.exp_off), _p(layout.pos_in_rank),
        _p(layout.slot_in_expert), int(fp8),
        _p(out["send_x"]), _p(out["send_scales"]), _p(out["send_src"]),
        _p(out["send_topk_idx"]), _p(out["send_topk_w"]), out["send_x"].shape[0],
        _p(out["recv_x"]), _p(out["recv_scales"]), _p(out["recv_src"]), out["recv_x"].shape[0],
        _p(out["pos_exp"]), _stream(dev))
    check(rc, "epx_dispatch")
    return Dispatched(layout=layout, **out)


@dataclass
class Received:
    """A receiver's rows arranged into per-local-expert blocks."""
    x: torch.Tensor                # [N*K cap, h'] rows, expert-major (row order inside a block)
    scales: torch.Tensor | None    # FP8 scale rows, arranged alike
    src_row: torch.Tensor          # [rows] the received row each output row came from
    pos: torch.Tensor              # [N, K] output row of (received row, k), or -1
    layout: Layout                 # counts / offsets over the local experts


def recv_permute(rows: torch.Tensor, local_topk_idx: torch.Tensor, num_local_experts: int,
                 scales: torch.Tensor | None = None) -> Received:
    """The receiver's side of the high-throughput mode: its received rows
    (one per source token, in source then token order) into contiguous
    per-local-expert blocks, row order kept inside each block. ``rows`` are
    bf16 [N, h], or FP8 codes uint8 [N, h] with ``scales`` [N, stride] fp32;
    ``local_topk_idx`` [N, K] int64 holds each row's local expert indices
    (-1 for entries of other ranks), as dispatch's send_topk_idx does. The
    layout of those indices, then one epx_permute launch that moves each row
    and its scale row, bit for bit."""
    dev = rows.device
    _need(local_topk_idx, torch.int64, "local_topk_idx", 2, device=dev)
    N, K = local_topk_idx.shape
    L = num_local_experts
    for name, pl in (("rows", rows), ("scales", scales)):
        if pl is None:
            continue
        if not pl.is_cuda or pl.device != dev or not pl.is_contiguous() or pl.dim() != 2 \
                or pl.shape[0] != N:
            raise ValueError(f"{name} must be a contiguous 2-d tensor on {dev} with one row "
                             "per received row")
    lay = get_dispatch_layout(local_topk_idx, L, 1)
    cap = N * K
    row_bytes = rows.shape[1] * rows.element_size()
    side_bytes = scales.shape[1] * scales.element_size() if scales is not None else 0
    out = torch.empty((cap, rows.shape[1]), dtype=rows.dtype, device=dev)
    out_side = (torch.empty((cap, scales.shape[1]), dtype=scales.dtype, device=dev)
                if scales is not None else None)
    pos = torch.empty((N, K), dtype=torch.int32, device=dev)
    src_row = torch.empty(cap, dtype=torch.int32, device=dev)
    rc = _lib.load().epx_permute(
        _ctx(dev), _p(rows), row_bytes, _p(scales), side_bytes, _p(local_topk_idx), N, K, L,
        _p(lay.exp_off), _p(lay.slot_in_expert), _p(out), _p(out_side), _p(src_row), cap,
        _p(pos), _stream(dev))
    check(rc, "epx_permute")
    return Received(x=out, scales=out_side, src_row=src_row, pos=pos, layout=lay)


def fused_workspace_size(T: int, K: int, E: int, R: int) -> int:
    n = ctypes.c_size_t()
    check(_lib.load().epx_fused_workspace_size(T, K, E, R, ctypes.byref(n)),
          "epx_fused_workspace_size")
    return n.value


def fused_launches(T: int, h: int, K: int, E: int, R: int, fp8: bool = False,
                   device: torch.device | None = None) -> int:
    """How many launches dispatch_fused takes for this shape: 1 for small
    batches (T <= 1024) and while the tiled grid covers every compute unit
    and fits on the device at once, else 2."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    n = ctypes.c_int()
    check(_lib.load().epx_fused_launches(_ctx(device), T, h, K, E, R, int(fp8), ctypes.byref(n)),
          "epx_fused_launches")
    return n.value


def dispatch_fused(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                   num_experts: int, num_ranks: int, fp8: bool = False,
                   num_channels: int | None = None, layout: Layout | None = None,
                   out: dict | None = None, workspace: torch.Tensor | None = None,
                   totals_host: torch.Tensor | None = None) -> Dispatched:
    """get_dispatch_layout and dispatch in one launch (two outside the
    shapes fused_launches reports as one; no host wait either way): the same
    outputs as the two calls. ``layout`` (from alloc_layout) and
    ``out`` (from alloc_dispatch) avoid allocating; without ``out`` the
    buffers get the worst-case capacities T*min(K,R) and T*K rows.
    ``workspace`` must hold fused_workspace_size(T, K, E, R) bytes and be
    zero-filled before its first use (without one, a cached workspace per
    device and stream is used)."""
    _need(x, torch.bfloat16, "x", 2)
    dev = x.device
    T, h = x.shape
    _need(topk_idx, torch.int64, "topk_idx", 2, device=dev)
    K = topk_idx.shape[1]
    _need(topk_idx, torch.int64, "topk_idx", shape=(T, K))
    _need(topk_weights, torch.float32, "topk_weights", shape=(T, K), device=dev)
    E, R = num_experts, num_ranks
    lay = layout if layout is not None else alloc_layout(T, K, E, R, num_channels, dev)
    _check_layout(lay, T, K, E, R, num_channels, dev)
    if out is None:
        out = alloc_dispatch(T, h, K, T * min(K, R), T * K, fp8, dev)
    _check_dispatch_out(out, T, h, K, fp8, dev)
    if workspace is None:
        workspace = _layout_workspace(dev, fused_workspace_size(T, K, E, R))
    ws_bytes = _nbytes(workspace, dev)
    if totals_host is not None and not (totals_host.is_pinned() and totals_host.numel() >= 2
                                        and totals_host.dtype == torch.int32):
        raise ValueError("totals_host must be a pinned int32 tensor of >= 2 elements")
    cp = lay.channel_prefix if num_channels else None
    rc = _lib.load().epx_dispatch_fused(
        _ctx(dev), _p(x), h, _p(topk_idx), _p(topk_weights), T, K, E, R, num_channels or 0,
        _p(lay.num_tokens_per_expert), _p(lay.num_tokens_per_rank), _p(lay.is_token_in_rank),
        _p(lay.rank_off), _p(lay.exp_off), _p(lay.pos_in_rank), _p(lay.slot_in_expert),
        _p(cp), _p(lay.totals), _p(totals_host), _p(workspace), ws_bytes, int(fp8),
        _p(out["send_x"]), _p(out["send_scales"]), _p(out["send_src"]),
        _p(out["send_topk_idx"]), _p(out["send_topk_w"]), out["send_x"].shape[0],
        _p(out["recv_x"]), _p(out["recv_scales"]), _p(out["recv_src"]), out["recv_x"].shape[0],
        _p(out["pos_exp"]), _stream(dev))
    check(rc, "epx_dispatch_fused")
    return Dispatched(layout=lay, **out)


def combine(expert_out: torch.Tensor, pos: torch.Tensor, topk_weights: torch.Tensor,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """out[t] = bf16(sum over valid k, in k order, of w[t,k] * expert_out[pos[t,k]])."""
    _need(expert_out, torch.bfloat16, "expert_out", 2)
    dev = expert_out.device
    _need(pos, torch.int32, "pos", 2, device=dev)
    T, K = pos.shape
    h = expert_out.shape[1]
    _need(topk_weights, torch.float32, "topk_weights", shape=(T, K), device=dev)
    if out is None:
        out = torch.empty((T, h), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", shape=(T, h), device=dev)
    rc = _lib.load().epx_combine(_ctx(dev), _p(expert_out), expert_out.shape[0], h,
                                 _p(topk_weights), _p(pos), T, K, _p(out), _stream(dev))
    check(rc, "epx_combine")
    return out


def combine_partial(expert_out: torch.Tensor, dispatched: Dispatched,
                    out: torch.Tensor | None = None,
                    num_rows: torch.Tensor | None = None) -> torch.Tensor:
    """Stage 1 of the two-stage combine: one bf16 partial row per rank-major
    row of ``dispatched`` (its rank's experts reduced with the token's
    weights). Rows past the layout's send-row total are not written."""
    _need(expert_out, torch.bfloat16, "expert_out", 2)
    dev = expert_out.device
    d = dispatched
    _need(d.send_topk_idx, torch.int64, "send_topk_idx", 2, device=dev)
    cap, K = d.send_topk_idx.shape
    _need(d.pos_exp, torch.int32, "pos_exp", 2, device=dev)
    T = d.pos_exp.shape[0]
    h = expert_out.shape[1]
    _need(d.pos_exp, torch.int32, "pos_exp", shape=(T, K))
    _need(d.send_src, torch.int32, "send_src", shape=(cap,), device=dev)
    _need(d.send_topk_w, torch.float32, "send_topk_w", shape=(cap, K), device=dev)
    if out is None:
        out = torch.empty((cap, h), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", shape=(cap, h), device=dev)
    if num_rows is None:
        num_rows = d.layout.totals[:1]
    _need(num_rows, torch.int32, "num_rows", shape=(1,), device=dev)
    rc = _lib.load().epx_combine_partial(
        _ctx(dev), _p(expert_out), expert_out.shape[0], h, _p(d.send_src), _p(d.send_topk_idx),
        _p(d.send_topk_w), _p(d.pos_exp), T, K, cap, _p(num_rows), _p(out), _stream(dev))
    check(rc, "epx_combine_partial")
    return out


def combine_final(partial: torch.Tensor, layout: Layout,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Stage 2: each token's partial rows summed in rank order (fp32) into bf16."""
    _need(partial, torch.bfloat16, "partial", 2)
    dev = partial.device
    _need(layout.pos_in_rank, torch.int32, "pos_in_rank", 2, device=dev)
    T, R = layout.pos_in_rank.shape
    _need(layout.rank_off, torch.int32, "rank_off", shape=(R + 1,), device=dev)
    h = partial.shape[1]
    if out is None:
        out = torch.empty((T, h), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", shape=(T, h), device=dev)
    rc = _lib.load().epx_combine_final(_ctx(dev), _p(partial), partial.shape[0], h,
                                       _p(layout.rank_off), _p(layout.pos_in_rank), T, R, _p(out),
                                       _stream(dev))
    check(rc, "epx_combine_final")
    return out


def ll_reset(ll_count: torch.Tensor) -> None:
    _need(ll_count, torch.int32, "ll_count")
    dev = ll_count.device
    check(_lib.load().epx_ll_reset(_ctx(dev), _p(ll_count), ll_count.numel(), _stream(dev)),
          "epx_ll_reset")


@dataclass
class LowLatency:
    ll_x: torch.Tensor              # [E*R_buf*cap, h] bf16 or uint8
    ll_scales: torch.Tensor | None  # [E*R_buf*cap, scale_stride(h)] fp32
    ll_src: torch.Tensor            # [E*R_buf*cap] int32
    ll_count: torch.Tensor          # [E*R_buf] int32
    pos_ll: torch.Tensor            # [T,K] int32 -- the handle for combine


def alloc_ll(E: int, R_buf: int, cap: int, h: int, T: int, K: int, fp8: bool,
             device: torch.device) -> LowLatency:
    rows = E * R_buf * cap
    buf = LowLatency(
        ll_x=torch.empty((rows, h), dtype=torch.uint8 if fp8 else torch.bfloat16, device=device),
        ll_scales=torch.empty((rows, scale_stride(h)), dtype=torch.float32,
                              device=device) if fp8 else None,
        ll_src=torch.empty(rows, dtype=torch.int32, device=device),
        ll_count=torch.empty(E * R_buf, dtype=torch.int32, device=device),
        pos_ll=torch.empty((T, K), dtype=torch.int32, device=device))
    ll_reset(buf.ll_count)
    return buf


def ll_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                src_rank: int, cap: int, R_buf: int | None = None, fp8: bool = True,
                buf: LowLatency | None = None, next_buf: LowLatency | None = None,
                stats: torch.Tensor | None = None) -> LowLatency:
    """Fixed-slot low-latency dispatch (one launch, no host wait). ``buf``
    must come from alloc_ll (its counts start at -1). ``next_buf``, the
    other buffer of a ping-pong pair, gets its counts reset to -1 by the same
    launch; ``stats`` (int32 [2] on the device) receives the entries routed
    and the fullest region's count."""
    _need(x, torch.bfloat16, "x", 2)
    dev = x.device
    T, h = x.shape
    _need(topk_idx, torch.int64, "topk_idx", 2, device=dev)
    K = topk_idx.shape[1]
    _need(topk_idx, torch.int64, "topk_idx", shape=(T, K))
    R_buf = num_ranks if R_buf is None else R_buf
    if buf is None:
        buf = alloc_ll(num_experts, R_buf, cap, h, T, K, fp8, dev)
    rows = num_experts * R_buf * cap
    _need(buf.ll_x, torch.uint8 if fp8 else torch.bfloat16, "ll_x", shape=(rows, h), device=dev)
    if fp8:
        _need(buf.ll_scales, torch.float32, "ll_scales", shape=(rows, scale_stride(h)),
              device=dev)
    _need(buf.ll_src, torch.int32, "ll_src", shape=(rows,), device=dev)
    _need(buf.ll_count, torch.int32, "ll_count", shape=(num_experts * R_buf,), device=dev)
    _need(buf.pos_ll, torch.int32, "pos_ll", shape=(T, K), device=dev)
    if stats is not None:
        _need(stats, torch.int32, "stats", device=dev)
        if stats.numel() < 2:
            raise ValueError("stats needs 2 int32 entries")
    nxt = next_buf.ll_count if next_buf is not None else None
    if nxt is not None:
        _need(nxt, torch.int32, "next_buf.ll_count", device=dev)
    rc = _lib.load().epx_ll_dispatch(
        _ctx(dev), _p(x), h, _p(topk_idx), T, K, num_experts, num_ranks, src_rank, cap, R_buf,
        int(fp8), _p(buf.ll_x), _p(buf.ll_scales), _p(buf.ll_src), _p(buf.ll_count),
        _p(buf.pos_ll), _p(nxt), nxt.numel() if nxt is not None else 0, _p(stats), _stream(dev))
    check(rc, "epx_ll_dispatch")
    return buf


__all__ = ["EpxError", "Layout", "Dispatched", "LowLatency", "workspace_size", "ll_size_hint",
           "scale_stride", "get_error", "alloc_layout", "get_dispatch_layout", "alloc_dispatch",
           "get_dispatch_layout_noalloc", "dispatch", "combine", "combine_partial",
           "combine_final", "ll_reset", "alloc_ll",
           "ll_dispatch", "Received", "recv_permute", "fused_workspace_size",
           "fused_launches", "dispatch_fused", "set_sweep_rate", "get_sweep_rate",
           "calibrate_sweep_rate"]
