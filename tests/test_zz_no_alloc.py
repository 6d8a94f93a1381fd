"""The layout entry point that allocates nothing (its workspace is the
library's fixed device scratch array) against epx_get_dispatch_layout with a
caller workspace: every output bit-identical, on two calls in a row -- the
prefill routing, then a smaller batch, so the second call finds the
first call's state in the array -- and on a one-tile batch (no hand-over)
after them. A shape whose workspace exceeds the array is refused with
nothing launched. Runs last: it shares the array with nothing else."""
import numpy as np
import pytest
import torch

import synth
from _gpu import host_bits, say

pytestmark = pytest.mark.gpu

KEYS = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank", "rank_off",
        "exp_off", "pos_in_rank", "slot_in_expert", "channel_prefix", "totals"]


def _both(epx, topk: np.ndarray, E: int, R: int, C: int):
    tk = torch.from_numpy(topk).cuda()
    T, K = topk.shape
    ref = epx.get_dispatch_layout(tk, E, R, C)
    got = epx.alloc_layout(T, K, E, R, C, tk.device)
    for k in KEYS:  # scribble every output first
        getattr(got, k).view(torch.uint8).fill_(0x5A)
    epx.get_dispatch_layout_noalloc(tk, E, R, C, out=got)
    assert epx.get_error() == 0
    for k in KEYS:
        a, b = host_bits(getattr(got, k)), host_bits(getattr(ref, k))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{k} differs"


def test_noalloc_layout_matches_layout():
    import combine_get_dispatch_counts_amd as epx

    inp = synth.make_inputs(3)   # T=4096, E=256, R=32, topk=8: 16 tiles
    wl = inp["workload"]
    say(f"no-alloc layout T={wl.T} E={wl.E} R={wl.R}")
    _both(epx, inp["topk_idx"], wl.E, wl.R, 24)
    small = synth.random_routing(1000, 6, 64, seed=5, p_drop=0.05)   # 4 tiles
    say("no-alloc layout T=1000 E=64 R=8 (smaller, after the first)")
    _both(epx, small, 64, 8, 7)
    say("no-alloc layout T=200 (one tile)")
    _both(epx, synth.random_routing(200, 8, 256, seed=6), 256, 32, 3)


def test_noalloc_layout_refuses_oversize():
    import combine_get_dispatch_counts_amd as epx

    # E + R = 576 words per 256-token tile: 1 MiB holds 227 tiles
    T = 228 * 256
    tk = torch.full((T, 1), 0, dtype=torch.int64, device="cuda")
    with pytest.raises(epx.EpxError) as ex:
        epx.get_dispatch_layout_noalloc(tk, 512, 64)
    assert ex.value.code == -2
    assert epx.get_error() == 0
