"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, on the same seeded inputs.

Bar: layout, offsets, permutations, metadata, FP8 codes and scales
bit-exact; combine bit-exact against the oracle's fp32 fma chain (which is
itself within one bf16 ulp of the exact sum away from cancellation, see
test_oracle_combine). Full-size workload cases use the benchmark's launch
configuration (worst-case preallocated capacities, no host wait).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

from _gpu import CANARY, dev_bf16, dispatch, host_bits, layout, say

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank", "rank_off",
               "exp_off", "pos_in_rank", "slot_in_expert", "totals"]


def _eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if a.dtype.kind == "f":
        a, b = a.view(np.uint32 if a.itemsize == 4 else np.uint64), b.view(
            np.uint32 if b.itemsize == 4 else np.uint64)
    bad = np.flatnonzero((a != b).ravel())
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at flat {bad[:5]}: " \
                          f"{a.ravel()[bad[:5]]} vs {b.ravel()[bad[:5]]}"


def _check_layout(topk, E, R, C):
    g = layout(topk, E, R, C)
    o = oracle.layout(topk, E, R, C)
    for k in LAYOUT_KEYS + (["channel_prefix"] if C else []):
        _eq(g[k], o[k], k)
    return o


def _edge_cases():
    cases = []
    for T in (0, 1, 63, 64, 65, 257):
        cases.append(("uniform", T, 8, 256, 32, 16, 0.0))
    for K in (1, 2, 6, 8, 32):
        cases.append(("uniform", 300, K, 64, 8, 7, 0.0))
    for R in (1, 4, 8, 32, 64):
        cases.append(("uniform", 513, 4, 128, R, 33, 0.0))
    # ranks that are not powers of two: multiples of 4 (12, 24, 48; 48 also a
    # multiple of 16) and others (2, 3, 6) take the layout's other row paths
    for R in (2, 3, 6, 12, 24, 48):
        cases.append(("uniform", 777, 6, 96, R, 9, 0.05))
    cases.append(("dropped", 700, 8, 256, 32, 5, 0.3))
    cases.append(("one_expert", 1000, 1, 64, 8, 10, 0.0))
    cases.append(("max_experts", 600, 8, 512, 64, 3, 0.0))
    cases.append(("repeats", 300, 4, 16, 4, 4, 0.0))
    # 512-token tiles (T > 4096) with eight counting waves each, every row
    # likely to repeat an expert
    cases.append(("repeats", 5000, 8, 32, 8, 7, 0.0))
    cases.append(("many_channels", 100, 2, 8, 4, 1000, 0.0))
    return cases


@pytest.mark.parametrize("kind,T,K,E,R,C,p_drop", _edge_cases())
def test_layout_edge_cases(kind, T, K, E, R, C, p_drop):
    say(f"layout {kind} T={T} K={K} E={E} R={R} C={C}")
    if kind == "one_expert":
        topk = np.full((T, K), 5, np.int64)
    elif kind == "repeats":
        topk = np.random.default_rng(T).integers(-1, E, (T, K)).astype(np.int64)
    else:
        topk = synth.random_routing(T, K, E, seed=T * 31 + K, p_drop=p_drop)
    _check_layout(topk, E, R, C)


def test_layout_workspace_reuse_and_recovery():
    """One workspace across calls of different sizes (each call leaves it
    ready for the next); then a workspace in a state no call leaves (its
    arrival count past the tiles) is flagged without any wait, and once it
    is zero-filled again the next call is correct."""
    import combine_get_dispatch_counts_amd as epx

    E, R, K, C = 256, 32, 8, 7
    ws = torch.zeros(epx.workspace_size(4096, K, E, R), dtype=torch.uint8, device="cuda")

    def run_and_check(T, seed):
        topk = synth.random_routing(T, K, E, seed=seed)
        lay = epx.get_dispatch_layout(torch.from_numpy(topk).cuda(), E, R, C, workspace=ws)
        flags = epx.get_error()
        return topk, lay, flags

    for i, T in enumerate([4096, 1000, 4096, 257, 3000, 1]):
        say(f"layout workspace reuse call {i} T={T}")
        topk, lay, flags = run_and_check(T, 100 + i)
        assert flags == 0
        o = oracle.layout(topk, E, R, C)
        for k in LAYOUT_KEYS + ["channel_prefix"]:
            _eq(host_bits(getattr(lay, k)), o[k], f"call {i} {k}")
    say("layout workspace with its arrival count past the tiles")
    ws[:4].view(torch.int32).fill_(1 << 20)
    _, _, flags = run_and_check(2000, 7)
    assert flags == 8, f"expected EPX_DEV_WORKSPACE, got {flags:#x}"
    ws.zero_()
    topk, lay, flags = run_and_check(2000, 8)
    assert flags == 0
    o = oracle.layout(topk, E, R, C)
    for k in LAYOUT_KEYS + ["channel_prefix"]:
        _eq(host_bits(getattr(lay, k)), o[k], f"after recovery {k}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_layout_workloads(cfg):
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    say(f"layout {wl.describe()}")
    _check_layout(inp["topk_idx"], wl.E, wl.R, 24)


def _check_dispatch(x, topk, w, E, R, fp8, worst_case=False, guard=0):
    g = dispatch(x, topk, w, E, R, fp8, worst_case=worst_case, guard=guard)
    assert g["flags"] == 0, f"device flags {g['flags']:#x}"
    o = oracle.dispatch(x, topk, w, E, R, fp8=fp8)
    keys = ["send_x", "send_src", "send_topk_idx", "send_topk_w", "recv_x", "recv_src", "pos_exp"]
    if fp8:
        keys += ["send_scales", "recv_scales"]
        for k in ("send_scales_pad", "recv_scales_pad"):
            assert (g[k].view(np.uint32) == 0).all(), f"{k}: scale row padding is not +0"
    for k in keys:
        _eq(g[k], o[k], k)
    for region in ("guard", "unused"):
        for k, v in g.get(region, {}).items():
            assert (v.view(np.uint8) == CANARY).all(), f"{region} rows of {k} were written"
    return g, o


@pytest.mark.parametrize("T,K,E,R,h,fp8,p_drop", [
    (1, 8, 256, 32, 7168, False, 0.0), (63, 2, 8, 4, 128, False, 0.0),
    (65, 6, 64, 8, 4096, True, 0.0), (257, 8, 256, 64, 256, True, 0.2),
    (200, 4, 16, 1, 1024, False, 0.1), (130, 8, 128, 32, 7168, True, 0.0),
    (300, 32, 512, 64, 256, True, 0.1), (600, 32, 512, 64, 1024, False, 0.0),
    # rows longer than one register pass: two full passes, partial second passes
    (40, 8, 64, 8, 16384, True, 0.1), (40, 8, 64, 8, 16384, False, 0.1),
    (33, 6, 64, 8, 9216, False, 0.0), (45, 8, 64, 8, 9216, True, 0.0),
    (50, 4, 32, 4, 8200, False, 0.0),
    (96, 3, 24, 4, 136, False, 0.0), (0, 4, 16, 4, 128, True, 0.0),
])
def test_dispatch_edge_cases(T, K, E, R, h, fp8, p_drop):
    say(f"dispatch T={T} K={K} E={E} R={R} h={h} fp8={fp8} drop={p_drop}")
    rng = np.random.default_rng(T + h)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32) * 3)
    topk = synth.random_routing(T, K, E, seed=T + 7, p_drop=p_drop)
    w = rng.random((T, K)).astype(np.float32)
    _check_dispatch(x, topk, w, E, R, fp8, guard=3)


def test_dispatch_special_values():
    """Zeros, signed zeros, tiny and huge bf16 values, an all-zero FP8 group,
    subnormal e4m3 results and values at rounding ties."""
    say("dispatch special values")
    T, h = 16, 512
    rng = np.random.default_rng(4)
    xf = rng.standard_normal((T, h)).astype(np.float32)
    xf[0] = 0.0
    xf[1] = -0.0
    xf[2, :128] = 0.0
    xf[3, :128] = np.float32(2.0) ** rng.integers(-40, -20, 128).astype(np.float32)
    xf[4] *= np.float32(1e30)
    xf[5, :128] = np.linspace(-448, 448, 128, dtype=np.float32)
    xf[6, :128] = np.float32(448.0) * np.float32(2.0) ** -np.arange(128, dtype=np.float32) / 4
    x = synth.to_bf16_bits(xf)
    topk = synth.random_routing(T, 4, 16, seed=5)
    w = rng.random((T, 4)).astype(np.float32)
    for fp8 in (False, True):
        _check_dispatch(x, topk, w, 16, 4, fp8)


def test_dispatch_fp8_nonfinite_groups():
    """FP8 groups holding +-Inf or NaN (quiet, signalling, either sign) take
    the exact-division branch; so do the finite groups of the same tokens
    (the branch is taken per token), while other tokens keep the fast one."""
    say("dispatch fp8 non-finite groups")
    T, h = 12, 1024
    rng = np.random.default_rng(12)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    x[0, 5] = 0x7F80
    x[0, 3 * 128 + 1] = 0xFF80
    x[0, 3 * 128 + 2] = 0x7FC0
    x[1, 128 + 7] = 0x7FC0
    x[1, 128 + 9] = 0xFF81
    x[2, 256:384] = 0x7FC1
    x[3, :] = 0x7F80
    x[4, 640 + 3] = 0xFF80
    x[4, 640 + 4] = 0x7F80
    x[5, 1023] = 0xFFC0
    topk = synth.random_routing(T, 3, 8, seed=13)
    w = rng.random((T, 3)).astype(np.float32)
    _check_dispatch(x, topk, w, 8, 4, True)


def _patterns_below(rng, top: np.ndarray, n: int) -> np.ndarray:
    """n bf16 patterns per entry of `top`, uniform over the magnitude patterns
    0..top, random sign."""
    mag = (rng.random((top.size, n)) * (top[:, None].astype(np.float64) + 1)).astype(np.uint32)
    sign = rng.integers(0, 2, (top.size, n)).astype(np.uint32) << 15
    return (mag | sign).astype(np.uint16)


@pytest.mark.parametrize("arrangement", ["sorted", "shuffled", "group_max_planted"])
def test_dispatch_fp8_every_bf16_pattern(arrangement):
    """Every one of the 65536 bf16 patterns (NaNs and infinities included)
    through the FP8 dispatch, against the oracle's IEEE division and
    format-definition encoder; the planted arrangement sweeps group maxima
    over the whole finite range, each with values spread below it."""
    say(f"dispatch fp8 every bf16 pattern, {arrangement}")
    rng = np.random.default_rng(65536)
    h = 4096
    if arrangement == "sorted":
        x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    elif arrangement == "shuffled":
        x = rng.permutation(65536).astype(np.uint16)
    else:
        top = rng.integers(0, 0x7F80, 2048).astype(np.uint32)
        groups = _patterns_below(rng, top, 128)
        groups[np.arange(top.size), rng.integers(0, 128, top.size)] = top
        x = groups.ravel()
    x = x.reshape(-1, h)
    T = x.shape[0]
    topk = synth.random_routing(T, 4, 16, seed=T)
    w = rng.random((T, 4)).astype(np.float32)
    _check_dispatch(x, topk, w, 16, 4, True)


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_dispatch_workloads_full_size(cfg):
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    say(f"dispatch {wl.describe()} (worst-case capacities, as benchmarked)")
    _check_dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, wl.fp8 or cfg == 1,
                    worst_case=True)


def test_dispatch_config1_bf16_and_fp8():
    inp = synth.make_inputs(1)
    wl = inp["workload"]
    for fp8 in (False, True):
        say(f"dispatch {wl.describe()} fp8={fp8}")
        _check_dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, fp8, guard=2)


def test_dispatch_deterministic():
    inp = synth.make_inputs(4, T=2048)
    wl = inp["workload"]
    say("dispatch twice, bitwise")
    a = dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, False)
    b = dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, False)
    for k in ["send_x", "recv_x", "send_src", "recv_src", "pos_exp", "send_topk_idx"]:
        _eq(a[k], b[k], k)


# ------------------------------------------------------------------ combine

def _gpu_combine(y: torch.Tensor, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    import combine_get_dispatch_counts_amd as epx

    out = epx.combine(y, torch.from_numpy(pos).cuda(), torch.from_numpy(w).cuda())
    assert epx.get_error() == 0
    return host_bits(out)


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_combine_workloads(cfg):
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    say(f"combine {wl.describe()}")
    o = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R)
    n_exp = int(o["layout"]["totals"][1])
    y = synth.expert_outputs(n_exp, wl.h, seed=77 + cfg, device="cuda")
    g = dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, False)
    _eq(g["pos_exp"], o["pos_exp"], "pos_exp")
    out = _gpu_combine(y, g["pos_exp"], inp["topk_w"])          # GPU handle
    ref = oracle.combine(host_bits(y), inp["topk_w"], o["pos_exp"])  # oracle handle
    _eq(out, ref, "combined_x")


def test_combine_edge_cases():
    rng = np.random.default_rng(12)
    for T, K, h, n in [(1, 1, 8, 1), (37, 8, 7168, 300), (64, 32, 256, 2000), (5, 3, 64, 0),
                       (21, 8, 16384, 100), (9, 4, 8200, 30)]:
        say(f"combine T={T} K={K} h={h} rows={n}")
        y = synth.expert_outputs(max(n, 1), h, seed=T, device="cuda")[:n]
        pos = rng.integers(-1, max(n, 1), (T, K)).astype(np.int32) if n else np.full((T, K), -1, np.int32)
        w = rng.standard_normal((T, K)).astype(np.float32)
        out = _gpu_combine(y.contiguous() if n else torch.empty((0, h), dtype=torch.bfloat16,
                                                                   device="cuda"), pos, w)
        ref = oracle.combine(host_bits(y) if n else np.zeros((0, h), np.uint16), w, pos)
        _eq(out, ref, "combined_x")


@pytest.mark.parametrize("cfg,fp8", [(1, False), (3, False), (5, True)])
def test_identity_experts_closed_form(cfg, fp8):
    """combine(dispatch(x)) with unit weights and identity experts equals
    bf16(K_valid * x) exactly (with FP8: x replaced by bf16(dequant(q)))."""
    inp = synth.make_inputs(cfg, T=512 if cfg != 1 else None)
    wl = inp["workload"]
    say(f"identity-expert closed form {wl.describe()} fp8={fp8}")
    g = dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], wl.E, wl.R, fp8)
    recv = g["_dispatched"].recv_x
    if fp8:
        def deq(q, s):
            return (q.view(torch.float8_e4m3fn).float() * s.repeat_interleave(128, 1)).to(torch.bfloat16)

        y = deq(recv, g["_dispatched"].recv_scales[:, :wl.h // 128])  # the GPU's rows
        q, sc = oracle.quantize_rows(inp["x"])             # the expected rows: the oracle's codes
        xs = deq(torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda())
    else:
        y = recv
        xs = dev_bf16(inp["x"])
    ones = np.ones_like(inp["topk_w"])
    out = _gpu_combine(y.contiguous(), g["pos_exp"], ones)
    kval = torch.from_numpy((inp["topk_idx"] >= 0).sum(1).astype(np.float32)).cuda()
    ref = host_bits((xs.float() * kval[:, None]).to(torch.bfloat16)).copy()
    ref[(ref & 0x7FFF) == 0] = 0
    _eq(out, ref, "unit-weight combine")


# ------------------------------------------------------------------ low latency

def _check_ll_scales(got: np.ndarray, want: np.ndarray, want_src: np.ndarray, what: str):
    """Scale rows [rows, stride] against the oracle's [rows, h/128]: the
    used columns bit-exact, the padding +0 on written rows and untouched
    (canary) on the others."""
    ngrp = want.shape[1]
    _eq(got[:, :ngrp], want, what)
    pad = got[:, ngrp:].view(np.uint32)
    written = want_src >= 0
    assert (pad[written] == 0).all(), f"{what}: padding of written rows is not +0"
    assert (pad[~written] == np.uint32(0x01010101 * CANARY)).all(), \
        f"{what}: padding of untouched rows was written"


def _ll_gpu(x, topk, E, R, src, cap, R_buf, fp8):
    import combine_get_dispatch_counts_amd as epx

    T, h = x.shape
    K = topk.shape[1]
    buf = epx.alloc_ll(E, R_buf, cap, h, T, K, fp8, torch.device("cuda"))
    buf.ll_x.view(torch.uint8).fill_(CANARY)
    if buf.ll_scales is not None:
        buf.ll_scales.view(torch.uint8).fill_(CANARY)
    buf.ll_src.view(torch.uint8).fill_(CANARY)
    epx.ll_dispatch(dev_bf16(x), torch.from_numpy(topk).cuda(), E, R, src, cap, R_buf, fp8, buf)
    assert epx.get_error() == 0
    return buf


@pytest.mark.parametrize("cfg,T,src,R_buf_full,fp8,cap", [
    (1, None, 0, True, True, 64), (1, None, 3, True, False, 64), (1, None, 2, False, True, 80),
    (2, 24, 31, False, False, 32), (2, None, 0, False, True, 128), (2, 1, 5, False, True, 1),
    # larger decode batches: several tokens per block (2, 4 and 8), the last
    # block ragged at T = 600
    (2, 300, 31, False, False, 300), (2, 600, 0, False, True, 600), (2, 1024, 7, False, True, 1024),
])
def test_ll_dispatch_small(cfg, T, src, R_buf_full, fp8, cap):
    inp = synth.make_inputs(cfg, T=T)
    wl = inp["workload"]
    topk = inp["topk_idx"].copy()
    topk[np.random.default_rng(2).random(topk.shape) < 0.05] = -1
    R_buf = wl.R if R_buf_full else 1
    say(f"ll_dispatch {wl.describe()} T={topk.shape[0]} src={src} R_buf={R_buf} fp8={fp8} cap={cap}")
    buf = _ll_gpu(inp["x"], topk, wl.E, wl.R, src, cap, R_buf, fp8)
    o = oracle.ll_dispatch(inp["x"], topk, wl.E, wl.R, src, cap, R_buf, fp8=fp8)
    _eq(host_bits(buf.pos_ll), o["pos_ll"], "pos_ll")
    _eq(host_bits(buf.ll_count), o["ll_count"], "ll_count")
    _eq(host_bits(buf.ll_src), o["ll_src"], "ll_src")
    _eq(host_bits(buf.ll_x), o["ll_x"], "ll_x")
    if fp8:
        _check_ll_scales(host_bits(buf.ll_scales), o["ll_scales"], o["ll_src"], "ll_scales")


def test_ll_dispatch_eight_tokens_per_block():
    """A decode batch of 2000 tokens (eight tokens per block, one wave each,
    the last block ragged) on the decode routing at a narrower hidden size."""
    inp = synth.make_inputs(2, T=2000)
    wl = inp["workload"]
    x = np.ascontiguousarray(inp["x"][:, :1024])
    topk = inp["topk_idx"]
    say(f"ll_dispatch T=2000 h=1024 E={wl.E} R={wl.R} cap=2000")
    buf = _ll_gpu(x, topk, wl.E, wl.R, 3, 2000, 1, True)
    o = oracle.ll_dispatch(x, topk, wl.E, wl.R, 3, 2000, 1, fp8=True)
    _eq(host_bits(buf.pos_ll), o["pos_ll"], "pos_ll")
    _eq(host_bits(buf.ll_count), o["ll_count"], "ll_count")
    _eq(host_bits(buf.ll_src), o["ll_src"], "ll_src")
    _eq(host_bits(buf.ll_x), o["ll_x"], "ll_x")
    _check_ll_scales(host_bits(buf.ll_scales), o["ll_scales"], o["ll_src"], "ll_scales")


@pytest.mark.parametrize("h,fp8,K", [(1152, True, 4), (1152, False, 4), (9216, True, 8),
                                      (10368, True, 32), (10368, False, 6), (136, False, 3)])
def test_ll_dispatch_row_slices(h, fp8, K):
    """Rows cut into 1024-channel slices over the block's waves: a partial
    last slice, more slices than waves (each wave then takes several), and
    K above the wave count."""
    T, E, R, src, cap = 40, 32, 8, 5, 40
    rng = np.random.default_rng(h + K)
    x = synth.to_bf16_bits((rng.standard_normal((T, h)) *
                            np.exp(rng.normal(0, 3, (T, 1)))).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=h, p_drop=0.1)
    say(f"ll_dispatch slices T={T} h={h} E={E} R={R} K={K} fp8={fp8}")
    buf = _ll_gpu(x, topk, E, R, src, cap, 1, fp8)
    o = oracle.ll_dispatch(x, topk, E, R, src, cap, 1, fp8=fp8)
    _eq(host_bits(buf.pos_ll), o["pos_ll"], "pos_ll")
    _eq(host_bits(buf.ll_count), o["ll_count"], "ll_count")
    _eq(host_bits(buf.ll_src), o["ll_src"], "ll_src")
    _eq(host_bits(buf.ll_x), o["ll_x"], "ll_x")
    if fp8:
        _check_ll_scales(host_bits(buf.ll_scales), o["ll_scales"], o["ll_src"], "ll_scales")


@pytest.mark.parametrize("fp8", [False, True])
def test_ll_dispatch_largest_shapes(fp8):
    """The low-latency kernel at the largest supported routing shape: E =
    512 experts, R = 64 ranks (the last source rank), K = 32 entries per
    token, every region's count and row against the oracle."""
    T, h, E, R, K, src, cap = 100, 256, 512, 64, 32, 63, 100
    rng = np.random.default_rng(64)
    x = synth.to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    topk = synth.random_routing(T, K, E, seed=65, p_drop=0.1)
    say(f"ll_dispatch T={T} h={h} E={E} R={R} K={K} src={src} fp8={fp8}")
    buf = _ll_gpu(x, topk, E, R, src, cap, 1, fp8)
    o = oracle.ll_dispatch(x, topk, E, R, src, cap, 1, fp8=fp8)
    _eq(host_bits(buf.pos_ll), o["pos_ll"], "pos_ll")
    _eq(host_bits(buf.ll_count), o["ll_count"], "ll_count")
    _eq(host_bits(buf.ll_src), o["ll_src"], "ll_src")
    _eq(host_bits(buf.ll_x), o["ll_x"], "ll_x")
    if fp8:
        _check_ll_scales(host_bits(buf.ll_scales), o["ll_scales"], o["ll_src"], "ll_scales")


def test_ll_dispatch_decode_full_buffer():
    """Decode workload at full size: T=128, E=256, R=32, cap=128, FP8, the
    full logical buffer of all 32 destinations (1,048,576 rows, 7.75 GB).
    The owned regions (src_rank's slice) are compared with the oracle's
    compact layout; every other region must keep its canary and count -1."""
    inp = synth.make_inputs(2)
    wl = inp["workload"]
    for src in (0, wl.R - 1):
        say(f"ll_dispatch full buffer {wl.describe()} src={src}")
        buf = _ll_gpu(inp["x"], inp["topk_idx"], wl.E, wl.R, src, wl.cap, wl.R, True)
        o = oracle.ll_dispatch(inp["x"], inp["topk_idx"], wl.E, wl.R, src, wl.cap, 1, fp8=True)
        E, R, cap, h = wl.E, wl.R, wl.cap, wl.h
        x4 = buf.ll_x.view(E, R, cap, h)
        s4 = buf.ll_scales.view(E, R, cap, -1)
        _eq(host_bits(x4[:, src]).reshape(E * cap, h), o["ll_x"], "owned ll_x")
        _check_ll_scales(host_bits(s4[:, src]).reshape(E * cap, -1), o["ll_scales"], o["ll_src"],
                         "owned ll_scales")
        _eq(host_bits(buf.ll_src.view(E, R, cap)[:, src]).reshape(-1), o["ll_src"], "owned ll_src")
        cnt = host_bits(buf.ll_count).reshape(E, R)
        _eq(cnt[:, src], o["ll_count"], "owned counts")
        assert (np.delete(cnt, src, axis=1) == -1).all()
        for name, t in (("ll_x", buf.ll_x), ("ll_scales", buf.ll_scales), ("ll_src", buf.ll_src)):
            touched = (t.view(torch.uint8).view(E, R, -1) != CANARY).any(dim=2)
            touched[:, src] = False
            assert not bool(touched.any()), f"a foreign region of {name} was written"
            del touched
        # handle rows follow the address formula of the full layout
        slot_rows = o["pos_ll"]
        e = inp["topk_idx"]
        full = np.where(slot_rows >= 0, (e * R + src) * cap + (slot_rows - e * cap), -1)
        _eq(host_bits(buf.pos_ll), full, "pos_ll")
        del buf, x4, s4
        torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [1, 2])
def test_ll_combine(cfg):
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    say(f"ll combine {wl.describe()}")
    cap = max(wl.cap, wl.T)
    buf = _ll_gpu(inp["x"], inp["topk_idx"], wl.E, wl.R, 0, cap, 1, True)
    o = oracle.ll_dispatch(inp["x"], inp["topk_idx"], wl.E, wl.R, 0, cap, 1, fp8=True)
    _eq(host_bits(buf.pos_ll), o["pos_ll"], "pos_ll")
    y = synth.expert_outputs(buf.ll_x.shape[0], wl.h, seed=5 + cfg, device="cuda")
    out = _gpu_combine(y, host_bits(buf.pos_ll), inp["topk_w"])
    _eq(out, oracle.combine(host_bits(y), inp["topk_w"], o["pos_ll"]), "ll combined_x")


@pytest.mark.parametrize("cfg,src", [(1, 0), (1, 3), (2, 17)])
def test_ll_combine_full_layout(cfg, src):
    """Combine through the handle of a low-latency dispatch into the full
    layout (R_buf = R: region e*R + src of every destination's buffer side by
    side), over expert outputs covering all E*R*cap rows: the rows of other
    sources' regions are never read, so the result equals the oracle's
    combine through its own full-layout handle."""
    inp = synth.make_inputs(cfg)
    wl = inp["workload"]
    T = wl.T if cfg == 1 else 8   # the decode shape's full layout at cap 8: 65 536 rows
    x, topk, w = (np.ascontiguousarray(inp[k][:T]) for k in ("x", "topk_idx", "topk_w"))
    cap = max(wl.cap, T) if cfg == 1 else 8
    say(f"ll combine, full layout: {wl.describe()} T={T} src={src} cap={cap}")
    buf = _ll_gpu(x, topk, wl.E, wl.R, src, cap, wl.R, True)
    o = oracle.ll_dispatch(x, topk, wl.E, wl.R, src, cap, wl.R, fp8=True)
    _eq(host_bits(buf.pos_ll), o["pos_ll"], "pos_ll")
    assert buf.ll_x.shape[0] == wl.E * wl.R * cap
    y = synth.expert_outputs(buf.ll_x.shape[0], wl.h, seed=40 + cfg, device="cuda")
    out = _gpu_combine(y, host_bits(buf.pos_ll), w)
    # the oracle gets only the rows the handle names (a relabelling of row
    # indices, no arithmetic), not the whole E*R*cap buffer
    p = o["pos_ll"]
    used = np.unique(p[p >= 0])
    relabel = np.where(p >= 0, np.searchsorted(used, np.maximum(p, 0)), -1).astype(np.int32)
    y_used = host_bits(y[torch.from_numpy(used).cuda()])
    _eq(out, oracle.combine(y_used, w, relabel), "full-layout ll combined_x")


def test_totals_host_mapped():
    """The totals also land in a caller's pinned host int32[2] (the CPU-
    mapped receive counter the host polls before allocating, [P2] "Buffer
    与内存视角"): after a stream synchronisation they equal the oracle's, from
    the layout call and from the fused call (one launch, and two)."""
    import combine_get_dispatch_counts_amd as epx

    for cfg, T in ((3, None), (1, None), (4, None), (3, 2048)):
        inp = synth.make_inputs(cfg, T=T)
        wl = inp["workload"]
        o = oracle.layout(inp["topk_idx"], wl.E, wl.R)
        tk = torch.from_numpy(inp["topk_idx"]).cuda()
        host = torch.full((2,), -7, dtype=torch.int32).pin_memory()
        say(f"host-mapped totals, layout call: {wl.describe()}")
        epx.get_dispatch_layout(tk, wl.E, wl.R, totals_host=host)
        torch.cuda.synchronize()
        _eq(host.numpy(), o["totals"], "host totals (layout)")
        host.fill_(-7)
        say(f"host-mapped totals, fused call ({epx.fused_launches(wl.T, wl.h, wl.K, wl.E, wl.R)} "
            "launch(es))")
        x = torch.from_numpy(inp["x"].view(np.int16)).cuda().view(torch.bfloat16)
        epx.dispatch_fused(x, tk, torch.from_numpy(inp["topk_w"]).cuda(), wl.E, wl.R,
                           totals_host=host)
        torch.cuda.synchronize()
        _eq(host.numpy(), o["totals"], "host totals (fused)")
        assert epx.get_error() == 0


# ------------------------------------------------------------------ errors

def test_error_paths():
    """Every error is forced from the host; each kernel still bounds-checks
    and exits normally."""
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(1)
    wl = inp["workload"]
    x, tk, w = dev_bf16(inp["x"]), torch.from_numpy(inp["topk_idx"]).cuda(), \
        torch.from_numpy(inp["topk_w"]).cuda()
    say("errors: T > cap")
    with pytest.raises(epx.EpxError) as ei:
        epx.ll_dispatch(x, tk, wl.E, wl.R, 0, wl.T - 1, 1, True)
    assert ei.value.code == -2
    say("errors: fp8 with h % 128 != 0")
    x136 = torch.zeros((wl.T, 136), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(epx.EpxError) as ei:
        epx.dispatch(x136, tk, w, wl.E, wl.R, fp8=True, exact=False)
    assert ei.value.code == -3
    say("errors: misaligned x")
    big = torch.zeros(wl.T * wl.h + 1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(epx.EpxError) as ei:
        epx.dispatch(big[1:].view(wl.T, wl.h), tk, w, wl.E, wl.R, exact=False)
    assert ei.value.code == -1
    say("errors: E % R != 0")
    with pytest.raises(epx.EpxError) as ei:
        epx.get_dispatch_layout(tk, wl.E, 3)
    assert ei.value.code == -1
    assert epx.get_error() == 0
    say("errors: top-k entry out of range")
    bad = inp["topk_idx"].copy()
    bad[5, 1] = wl.E + 3
    bad[9, 0] = -7
    epx.get_dispatch_layout(torch.from_numpy(bad).cuda(), wl.E, wl.R, 4)
    assert epx.get_error() == 1
    say("errors: capacity one row short, guard rows stay untouched")
    lay = epx.get_dispatch_layout(tk, wl.E, wl.R)
    n_send, n_recv = (int(v) for v in lay.totals.cpu())
    buf = epx.alloc_dispatch(wl.T, wl.h, wl.K, n_send + 4, n_recv + 4, False, x.device)
    for v in buf.values():
        if v is not None:
            v.view(torch.uint8).fill_(CANARY)
    view = dict(buf)
    for k in list(view):
        if view[k] is None:
            continue
        if k.startswith("send"):
            view[k] = buf[k][:n_send - 1]
        elif k.startswith("recv"):
            view[k] = buf[k][:n_recv - 1]
    epx.dispatch(x, tk, w, wl.E, wl.R, layout=lay, out=view)
    assert epx.get_error() == 2
    for k, v in buf.items():
        if k == "pos_exp" or v is None:
            continue
        n = n_send if k.startswith("send") else n_recv
        assert bool((v[n - 1:].view(torch.uint8) == CANARY).all()), f"{k} written past capacity"
    say("errors: combine handle beyond the expert-output rows")
    y = synth.expert_outputs(10, wl.h, seed=1, device="cuda")
    pos = torch.full((wl.T, wl.K), -1, dtype=torch.int32, device="cuda")
    pos[3, 0] = 10
    pos[4, 1] = 2
    out = epx.combine(y, pos, w)
    assert epx.get_error() == 4
    ref = oracle.combine(host_bits(y), inp["topk_w"], np.where(host_bits(pos) >= 10, -1, host_bits(pos)))
    _eq(host_bits(out), ref, "combine skipping the bad handle row")
    say("errors: LL row repeating an expert past the capacity")
    rep = np.zeros((4, 2), np.int64)  # every entry to expert 0: 8 rows, cap 4
    buf = epx.alloc_ll(wl.E, 1, 4, wl.h, 4, 2, False, x.device)
    buf.ll_x.view(torch.uint8).fill_(CANARY)
    epx.ll_dispatch(x[:4].contiguous(), torch.from_numpy(rep).cuda(), wl.E, wl.R, 0, 4, 1, False, buf)
    assert epx.get_error() == 2
    assert bool((buf.ll_x[4:].view(torch.uint8) == CANARY).all())


def test_binding_rejects_mismatched_buffers():
    """The C ABI takes bare pointers and row counts, so the binding checks
    every caller-supplied buffer's dtype, shape and device first: each bad
    buffer below raises before anything is launched, and the device flags
    stay clear."""
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(1)
    wl = inp["workload"]
    T, h, K, E, R = wl.T, wl.h, wl.K, wl.E, wl.R
    dev = torch.device("cuda", torch.cuda.current_device())
    x, tk, w = dev_bf16(inp["x"]), torch.from_numpy(inp["topk_idx"]).cuda(), \
        torch.from_numpy(inp["topk_w"]).cuda()
    lay = epx.get_dispatch_layout(tk, E, R)
    cap_s, cap_r = T * min(K, R), T * K

    def bad_out(fp8=False, **repl):
        out = epx.alloc_dispatch(T, h, K, cap_s, cap_r, fp8, dev)
        out.update(repl)
        return out

    say("binding: mismatched dispatch buffers")
    cases = [
        (ValueError, dict(send_src=torch.empty(cap_s - 1, dtype=torch.int32, device=dev))),
        (ValueError, dict(send_topk_idx=torch.empty((cap_s, K + 1), dtype=torch.int64,
                                                    device=dev))),
        (TypeError, dict(recv_src=torch.empty(cap_r, dtype=torch.int64, device=dev))),
        (ValueError, dict(pos_exp=torch.empty((T - 1, K), dtype=torch.int32, device=dev))),
        (ValueError, dict(recv_x=torch.empty((cap_r, h), dtype=torch.bfloat16,
                                             device=dev)[:, :h - 8])),
        (ValueError, dict(send_topk_w=torch.empty((cap_s, K), dtype=torch.float32))),
    ]
    for exc, repl in cases:
        with pytest.raises(exc):
            epx.dispatch(x, tk, w, E, R, layout=lay, out=bad_out(**repl))
        with pytest.raises(exc):
            epx.dispatch_fused(x, tk, w, E, R, out=bad_out(**repl))
    with pytest.raises(TypeError):  # bf16 rows where FP8 codes belong
        epx.dispatch(x, tk, w, E, R, fp8=True, layout=lay, out=bad_out(False))
    with pytest.raises(ValueError):
        epx.dispatch(x, tk, w, E, R, fp8=True, layout=lay,
                     out=bad_out(True, recv_scales=torch.empty((cap_r, 1), device=dev)))
    with pytest.raises(ValueError):
        epx.dispatch(x, tk, w.cpu(), E, R, layout=lay, out=bad_out())
    with pytest.raises(ValueError):
        epx.dispatch(x, tk[:, :K - 1].contiguous(), w, E, R, layout=lay, out=bad_out())

    say("binding: mismatched layout buffers and workspaces")
    with pytest.raises(ValueError):
        epx.get_dispatch_layout(tk, E, R, out=epx.alloc_layout(T + 1, K, E, R, None, dev))
    with pytest.raises(ValueError):
        epx.get_dispatch_layout(tk, E, R, 4, out=epx.alloc_layout(T, K, E, R, None, dev))
    with pytest.raises(ValueError):
        epx.get_dispatch_layout(tk, E, R, workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        epx.dispatch(x, tk, w, E, R, layout=epx.alloc_layout(T, K, 2 * E, R, None, dev),
                     out=bad_out())

    say("binding: mismatched combine buffers")
    d = epx.dispatch(x, tk, w, E, R, layout=lay)
    y = synth.expert_outputs(d.recv_x.shape[0], h, seed=3, device="cuda")
    with pytest.raises(ValueError):
        epx.combine(y, d.pos_exp, w, out=torch.empty((T - 1, h), dtype=torch.bfloat16,
                                                     device=dev))
    with pytest.raises(ValueError):
        epx.combine(y, d.pos_exp, w[:, :K - 1].contiguous())
    with pytest.raises(ValueError):
        epx.combine_partial(y, d, out=torch.empty((d.send_x.shape[0] - 1, h),
                                                  dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        epx.combine_final(torch.empty((d.send_x.shape[0], h), dtype=torch.bfloat16, device=dev),
                          lay, out=torch.empty((T, h + 8), dtype=torch.bfloat16, device=dev))

    say("binding: low-latency buffer of another capacity")
    buf = epx.alloc_ll(E, 1, T + 1, h, T, K, True, dev)
    with pytest.raises(ValueError):
        epx.ll_dispatch(x, tk, E, R, 0, T, 1, True, buf)
    assert epx.get_error() == 0


def test_ll_ping_pong_and_fill_stats():
    """Four decode steps over a ping-pong pair: each step dispatches into one
    buffer and resets the other's counts in the same launch (garbage written
    there first must read -1 afterwards); the rows, handles and counts of the
    step match the oracle, and the fill stats equal the oracle's count sum
    and largest count."""
    import combine_get_dispatch_counts_amd as epx

    wl = synth.WORKLOADS[2]
    E, R, K, h, cap, src = wl.E, wl.R, wl.K, wl.h, wl.cap, 5
    dev = torch.device("cuda")
    bufs = [epx.alloc_ll(E, 1, cap, h, wl.T, K, True, dev) for _ in range(2)]
    stats = torch.zeros(2, dtype=torch.int32, device=dev)
    for step in range(4):
        cur, nxt = bufs[step % 2], bufs[(step + 1) % 2]
        inp = synth.make_inputs(2, seed=500 + step)
        topk = inp["topk_idx"].copy()
        topk[np.random.default_rng(step).random(topk.shape) < 0.1 * step] = -1
        say(f"ll ping-pong step {step}")
        nxt.ll_count.fill_(7)
        cur.ll_src.view(torch.uint8).fill_(CANARY)
        epx.ll_dispatch(dev_bf16(inp["x"]), torch.from_numpy(topk).cuda(), E, R, src, cap, 1,
                        True, cur, next_buf=nxt, stats=stats)
        assert epx.get_error() == 0
        assert bool((nxt.ll_count == -1).all()), "the other buffer's counts were not reset"
        o = oracle.ll_dispatch(inp["x"], topk, E, R, src, cap, 1, fp8=True)
        _eq(host_bits(cur.pos_ll), o["pos_ll"], "pos_ll")
        _eq(host_bits(cur.ll_count), o["ll_count"], "ll_count")
        _eq(host_bits(cur.ll_src), o["ll_src"], "ll_src")
        written = o["ll_src"] >= 0
        _eq(host_bits(cur.ll_x)[written], o["ll_x"][written], "ll_x rows")
        counts = o["ll_count"]
        assert host_bits(stats).tolist() == [int(counts.sum()), int(counts.max())]
    with pytest.raises(epx.EpxError) as ei:
        epx.ll_dispatch(dev_bf16(inp["x"]), torch.from_numpy(topk).cuda(), E, R, src, cap, 1,
                        True, bufs[0], next_buf=bufs[0])
    assert ei.value.code == -1
