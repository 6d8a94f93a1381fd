"""CPU oracle for the single-GPU DeepEP-style dispatch/combine path.

TEST INFRASTRUCTURE. This package wraps ``liboracle.so`` (built from
``oracle.c`` with gcc) with numpy in/out. Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the HIP path and never imports the product package.

Every function follows the plain definitions written in ``oracle.c`` (see the
citations there). All arrays are numpy; bf16 data is carried as uint16 bit
patterns, e4m3 as uint8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

OK, EINVAL, ECAPACITY, EUNSUPPORTED, EROUTE = 0, -1, -2, -3, -5


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} returned {code}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (always, unless force=False and it exists)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.orc_bf16_rne.argtypes, L.orc_bf16_rne.restype = [f32], ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes, L.orc_bf16_to_f32.restype = [ctypes.c_uint16], f32
        L.orc_e4m3_rne.argtypes, L.orc_e4m3_rne.restype = [f32], ctypes.c_uint8
        L.orc_e4m3_to_f32.argtypes, L.orc_e4m3_to_f32.restype = [ctypes.c_uint8], f32
        L.orc_bf16_rne_n.argtypes, L.orc_bf16_rne_n.restype = [P, P, ctypes.c_size_t], None
        L.orc_e4m3_rne_n.argtypes, L.orc_e4m3_rne_n.restype = [P, P, ctypes.c_size_t], None
        L.orc_quantize_row.argtypes, L.orc_quantize_row.restype = [P, i32, P, P], None
        L.orc_layout.argtypes = [P, i32, i32, i32, i32, i32] + [P] * 9
        L.orc_layout.restype = i32
        L.orc_dispatch.argtypes = ([P, i32, P, P, i32, i32, i32, i32] + [P] * 5 + [i32]
                                   + [P] * 5 + [i64] + [P] * 3 + [i64, P])
        L.orc_dispatch.restype = i32
        L.orc_dispatch_tokens.argtypes = L.orc_dispatch.argtypes + [i32, i32]
        L.orc_dispatch_tokens.restype = i32
        L.orc_ll_dispatch.argtypes = [P, i32, P] + [i32] * 8 + [P] * 5
        L.orc_ll_dispatch.restype = i32
        L.orc_combine.argtypes = [P, i64, i32, P, P, i32, i32, P]
        L.orc_combine.restype = i32
        L.orc_combine_partial.argtypes = [P, i64, i32, P, P, P, i64, P, i32, i32, P]
        L.orc_combine_partial.restype = i32
        L.orc_combine_final.argtypes = [P, i64, i32, P, P, i32, i32, P]
        L.orc_combine_final.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(rc, what)


# ---------------------------------------------------------------- scalars

def bf16_rne(v: float) -> int:
    return int(lib().orc_bf16_rne(float(v)))


def e4m3_rne(v: float) -> int:
    return int(lib().orc_e4m3_rne(float(v)))


def e4m3_to_f32(q: int) -> float:
    return float(lib().orc_e4m3_to_f32(int(q)))


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    """Array form of bf16_rne (a C loop over the scalar definition)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_rne_n(_p(v), _p(out), v.size)
    return out


def e4m3_rne_array(v: np.ndarray) -> np.ndarray:
    """Array form of e4m3_rne (a C loop over the scalar definition)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e4m3_rne_n(_p(v), _p(out), v.size)
    return out


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """FP8-quantise each bf16 row of x [T,h] -> (q uint8 [T,h], scales f32 [T,h/128])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, h = x.shape
    q = np.empty((T, h), np.uint8)
    s = np.empty((T, h // 128), np.float32)
    for t in range(T):
        lib().orc_quantize_row(_p(x[t]), h, _p(q[t]), _p(s[t]))
    return q, s


# ---------------------------------------------------------------- layout

def layout(topk_idx: np.ndarray, E: int, R: int, C: int | None = None) -> dict:
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = topk_idx.shape
    out = dict(
        num_tokens_per_expert=np.empty(E, np.int32),
        num_tokens_per_rank=np.empty(R, np.int32),
        is_token_in_rank=np.empty((T, R), np.uint8),
        rank_off=np.empty(R + 1, np.int32),
        exp_off=np.empty(E + 1, np.int32),
        pos_in_rank=np.empty((T, R), np.int32),
        slot_in_expert=np.empty((T, K), np.int32),
        channel_prefix=np.empty((R, C), np.int32) if C else None,
        totals=np.empty(2, np.int32),
    )
    rc = lib().orc_layout(_p(topk_idx), T, K, E, R, C or 0,
                          _p(out["num_tokens_per_expert"]), _p(out["num_tokens_per_rank"]),
                          _p(out["is_token_in_rank"]), _p(out["rank_off"]), _p(out["exp_off"]),
                          _p(out["pos_in_rank"]), _p(out["slot_in_expert"]),
                          _p(out["channel_prefix"]), _p(out["totals"]))
    _check(rc, "layout")
    if out["channel_prefix"] is None:
        del out["channel_prefix"]
    return out


# ---------------------------------------------------------------- dispatch

def _slices(T: int, threads: int) -> list[tuple[int, int]]:
    """[0, T) cut into `threads` contiguous token ranges."""
    n = max(1, min(threads, T))
    step = -(-T // n) if T else 0
    return [(a, min(a + step, T)) for a in range(0, T, step)] if T else [(0, 0)]


def _run_threads(fn, ranges, threads: int) -> list:
    """fn over the token ranges, side by side when threads > 1 (ctypes drops
    the interpreter lock during each call)."""
    if threads <= 1 or len(ranges) == 1:
        return [fn(a, b) for a, b in ranges]
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def dispatch(x: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, E: int, R: int,
             fp8: bool = False, lay: dict | None = None, threads: int = 1) -> dict:
    """Layout (if not given), then the rank-deduplicated pack and the
    expert-major permute. threads > 1 runs the pack and permute of disjoint
    token ranges side by side (same outputs; the layout stays sequential)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, h = x.shape
    K = topk_idx.shape[1]
    if lay is None:
        lay = layout(topk_idx, E, R)
    n_rank, n_exp = int(lay["totals"][0]), int(lay["totals"][1])
    if fp8:
        send_x = np.empty((n_rank, h), np.uint8)
        recv_x = np.empty((n_exp, h), np.uint8)
        send_scales = np.empty((n_rank, h // 128), np.float32)
        recv_scales = np.empty((n_exp, h // 128), np.float32)
    else:
        send_x = np.empty((n_rank, h), np.uint16)
        recv_x = np.empty((n_exp, h), np.uint16)
        send_scales = recv_scales = None
    out = dict(
        send_x=send_x, send_scales=send_scales,
        send_src=np.empty(n_rank, np.int32),
        send_topk_idx=np.empty((n_rank, K), np.int64),
        send_topk_w=np.empty((n_rank, K), np.float32),
        recv_x=recv_x, recv_scales=recv_scales,
        recv_src=np.empty(n_exp, np.int32),
        pos_exp=np.empty((T, K), np.int32),
    )
    def run(t0: int, t1: int) -> int:
        return lib().orc_dispatch_tokens(
            _p(x), h, _p(topk_idx), _p(topk_w), T, K, E, R,
            _p(lay["is_token_in_rank"]), _p(lay["rank_off"]), _p(lay["exp_off"]),
            _p(lay["pos_in_rank"]), _p(lay["slot_in_expert"]), int(bool(fp8)),
            _p(send_x), _p(send_scales), _p(out["send_src"]), _p(out["send_topk_idx"]),
            _p(out["send_topk_w"]), n_rank,
            _p(recv_x), _p(recv_scales), _p(out["recv_src"]), n_exp, _p(out["pos_exp"]),
            t0, t1)

    for rc in _run_threads(run, _slices(T, threads), threads):
        _check(rc, "dispatch")
    out["layout"] = lay
    return out


def ll_dispatch(x: np.ndarray, topk_idx: np.ndarray, E: int, R: int, src_rank: int,
                cap: int, R_buf: int, fp8: bool = True, canary: int = 0xA5,
                ll_x: np.ndarray | None = None) -> dict:
    """Low-latency fixed-slot dispatch into a buffer pre-filled with `canary`
    bytes (scales and src too) and count = -1 (the caller's initial state)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, h = x.shape
    K = topk_idx.shape[1]
    rows = E * R_buf * cap
    if ll_x is None:
        ll_x = np.empty((rows, h), np.uint8 if fp8 else np.uint16)
        ll_x.view(np.uint8).fill(canary)
    ll_scales = np.empty((rows, h // 128), np.float32) if fp8 else None
    if ll_scales is not None:
        ll_scales.view(np.uint8).fill(canary)
    ll_src = np.empty(rows, np.int32)
    ll_src.view(np.uint8).fill(canary)
    ll_count = np.full(E * R_buf, -1, np.int32)
    pos_ll = np.empty((T, K), np.int32)
    rc = lib().orc_ll_dispatch(_p(x), h, _p(topk_idx), T, K, E, R, src_rank, cap, R_buf,
                               int(bool(fp8)), _p(ll_x), _p(ll_scales), _p(ll_src),
                               _p(ll_count), _p(pos_ll))
    _check(rc, "ll_dispatch")
    return dict(ll_x=ll_x, ll_scales=ll_scales, ll_src=ll_src, ll_count=ll_count,
                pos_ll=pos_ll)


def combine(expert_out: np.ndarray, topk_w: np.ndarray, pos: np.ndarray,
            threads: int = 1) -> np.ndarray:
    """threads > 1 reduces disjoint token ranges side by side (same outputs:
    every token is reduced on its own)."""
    expert_out = np.ascontiguousarray(expert_out, dtype=np.uint16)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    n_rows, h = expert_out.shape
    T, K = pos.shape
    out = np.empty((T, h), np.uint16)

    def run(t0: int, t1: int) -> int:
        return lib().orc_combine(_p(expert_out), n_rows, h, _p(topk_w[t0:t1]), _p(pos[t0:t1]),
                                 t1 - t0, K, _p(out[t0:t1]))

    for rc in _run_threads(run, _slices(T, threads), threads):
        _check(rc, "combine")
    return out


def combine_partial(expert_out: np.ndarray, send_src: np.ndarray, send_topk_idx: np.ndarray,
                    send_topk_w: np.ndarray, pos_exp: np.ndarray) -> np.ndarray:
    """Stage 1 of the two-stage combine: one bf16 partial row per rank-major
    row (the rows of send_src)."""
    expert_out = np.ascontiguousarray(expert_out, dtype=np.uint16)
    send_src = np.ascontiguousarray(send_src, dtype=np.int32)
    send_topk_idx = np.ascontiguousarray(send_topk_idx, dtype=np.int64)
    send_topk_w = np.ascontiguousarray(send_topk_w, dtype=np.float32)
    pos_exp = np.ascontiguousarray(pos_exp, dtype=np.int32)
    n_rows, h = expert_out.shape
    T, K = pos_exp.shape
    n_send = send_src.shape[0]
    out = np.empty((n_send, h), np.uint16)
    rc = lib().orc_combine_partial(_p(expert_out), n_rows, h, _p(send_src), _p(send_topk_idx),
                                   _p(send_topk_w), n_send, _p(pos_exp), T, K, _p(out))
    _check(rc, "combine_partial")
    return out


def combine_final(partial: np.ndarray, rank_off: np.ndarray, pos_in_rank: np.ndarray) -> np.ndarray:
    """Stage 2: each token's partial rows summed over ranks ascending."""
    partial = np.ascontiguousarray(partial, dtype=np.uint16)
    rank_off = np.ascontiguousarray(rank_off, dtype=np.int32)
    pos_in_rank = np.ascontiguousarray(pos_in_rank, dtype=np.int32)
    n_send, h = partial.shape
    T, R = pos_in_rank.shape
    out = np.empty((T, h), np.uint16)
    rc = lib().orc_combine_final(_p(partial), n_send, h, _p(rank_off), _p(pos_in_rank), T, R,
                                 _p(out))
    _check(rc, "combine_final")
    return out

