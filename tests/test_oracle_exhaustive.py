"""Exhaustive pins for the oracle's two rounding encoders, written from the
format definitions (OCP E4M3FN for the FP8 dispatch of the low-latency
section of the event-driven EP scheduling page; bf16 for the combine output
of the DeepEP study notes' combine section), against torch's CPU casts:

- e4m3: every fp32 bit pattern with |v| <= 464 (both signs, about 2.28e9
  patterns; above 464 the quotient x / s never goes, and torch maps it to
  NaN where the format saturates);
- bf16: all 2^32 fp32 bit patterns (NaNs: the oracle's quiet 0x7FC0).

Chunks of 2^24 patterns run on a thread pool (the C encoder and torch's
cast both release the GIL)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

CHUNK = 1 << 24
WORKERS = max(1, min(8, os.cpu_count() or 1))


def _patterns(lo: int, hi: int) -> np.ndarray:
    return np.arange(lo, hi, dtype=np.uint64).astype(np.uint32)


def _run(fn, ranges):
    with ThreadPoolExecutor(WORKERS) as ex:
        bad = [b for b in ex.map(fn, ranges) if b]
    assert not bad, f"mismatches: {bad[:3]}"


def _ranges(lo: int, hi: int):
    return [(a, min(a + CHUNK, hi)) for a in range(lo, hi, CHUNK)]


def test_e4m3_encoder_exhaustive(orc):
    top = int(np.array([464.0], np.float32).view(np.uint32)[0])  # 0x43E80000

    def check(r):
        v = _patterns(*r).view(np.float32)
        ours = orc.e4m3_rne_array(v)
        theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.flatnonzero(ours != theirs)
        return None if bad.size == 0 else (r, v[bad[:4]].tolist(), ours[bad[:4]].tolist(),
                                           theirs[bad[:4]].tolist())

    _run(check, _ranges(0, top + 1) + _ranges(0x80000000, 0x80000000 + top + 1))


def test_bf16_rne_exhaustive(orc):
    def check(r):
        v = _patterns(*r).view(np.float32)
        ours = orc.bf16_rne_array(v)
        theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(v)
        bad = np.flatnonzero((ours != theirs) & ~nan)
        bad_nan = np.count_nonzero(ours[nan] != 0x7FC0)
        if bad.size == 0 and bad_nan == 0:
            return None
        return (r, v[bad[:4]].tolist(), ours[bad[:4]].tolist(), theirs[bad[:4]].tolist(), bad_nan)

    _run(check, _ranges(0, 1 << 32))
