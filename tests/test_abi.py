"""The C-ABI library loads and exports every function include/epx.h declares;
host-only helpers behave as documented. No GPU work is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "epx.h")


def _declared() -> list[str]:
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(epx_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from combine_get_dispatch_counts_amd import _lib

    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    from combine_get_dispatch_counts_amd import _lib

    names = _declared()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in epx.h but not exported"
    assert sorted(_lib.SIGNATURES) == names, "ctypes table and header disagree"


def test_library_is_gfx950_hip():
    from combine_get_dispatch_counts_amd import _lib

    with open(_lib.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob
    assert b"gfx942" not in blob  # built for gfx950 only


def test_workspace_size(lib):
    n = ctypes.c_size_t()
    assert lib.epx_workspace_size(4096, 8, 256, 32, ctypes.byref(n)) == 0
    assert n.value == 128 + 16 * (256 + 32) * 8     # head + 16 tiles of 256 tokens
    assert lib.epx_workspace_size(0, 8, 256, 32, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.epx_workspace_size(10, 8, 256, 30, ctypes.byref(n)) == -1   # E % R
    assert lib.epx_workspace_size(10, 33, 256, 32, ctypes.byref(n)) == -1  # K > 32
    assert lib.epx_workspace_size(10, 8, 1024, 32, ctypes.byref(n)) == -1  # E > 512
    assert lib.epx_workspace_size(10, 8, 256, 128, ctypes.byref(n)) == -1  # R > 64


def _up(n):
    return (n + 127) // 128 * 128


@pytest.mark.parametrize("cap,h,R,E,fp8", [(128, 7168, 32, 256, 1), (128, 7168, 32, 256, 0),
                                          (6, 128, 4, 8, 1), (1, 8, 1, 1, 0)])
def test_ll_size_hint(lib, cap, h, R, E, fp8):
    rows = E * R * cap
    data = rows * (h if fp8 else 2 * h)
    stride = -(-(h // 128) // 32) * 32
    want = _up(data) + (_up(rows * stride * 4) if fp8 else 0) + _up(rows * 4) + _up(E * R * 4)
    assert lib.epx_ll_size_hint(cap, h, R, E, fp8) == want


@pytest.mark.parametrize("h,stride", [(128, 32), (4096, 32), (4224, 64), (7168, 64),
                                      (8192, 64), (9216, 96), (16384, 128)])
def test_scale_stride(lib, h, stride):
    """Scale rows: h/128 entries rounded up to whole 128-byte lines."""
    assert lib.epx_scale_stride(h) == stride
    assert stride >= h // 128 and (stride * 4) % 128 == 0 and stride - h // 128 < 32


def test_scale_stride_rejects(lib):
    for h in (0, -128, 100, 7000):
        assert lib.epx_scale_stride(h) == 0


def test_ll_size_hint_rejects(lib):
    assert lib.epx_ll_size_hint(0, 7168, 32, 256, 1) == 0
    assert lib.epx_ll_size_hint(128, 7000, 32, 256, 1) == 0   # fp8 needs h % 128
    assert lib.epx_ll_size_hint(128, 7168, 30, 256, 1) == 0


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.epx_strerror(code)
    assert b"unknown" in lib.epx_strerror(7)


def test_binding_scale_stride():
    import combine_get_dispatch_counts_amd as epx

    assert epx.scale_stride(7168) == 64
    with pytest.raises(epx.EpxError) as ei:
        epx.scale_stride(136)
    assert ei.value.code == -3
    with pytest.raises(epx.EpxError) as ei:
        epx.scale_stride(4)
    assert ei.value.code == -1


def test_fused_launches_rejects(lib):
    """Argument checks come before any device call: no context, no output."""
    n = ctypes.c_int(-5)
    assert lib.epx_fused_launches(None, 4096, 7168, 8, 256, 32, 0, ctypes.byref(n)) == -1
    assert lib.epx_fused_launches(None, 4096, 7168, 8, 256, 32, 0, None) == -1
    assert n.value == -5


def test_fused_workspace_size(lib):
    n = ctypes.c_size_t()
    assert lib.epx_fused_workspace_size(4096, 8, 256, 32, ctypes.byref(n)) == 0
    # the layout's workspace: a 128-byte head and one 8-byte word per (tile, expert or rank)
    assert n.value == 128 + 16 * 288 * 8
    m = ctypes.c_size_t()
    assert lib.epx_workspace_size(4096, 8, 256, 32, ctypes.byref(m)) == 0
    assert m.value == n.value
    assert lib.epx_fused_workspace_size(0, 8, 256, 32, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.epx_fused_workspace_size(10, 8, 256, 30, ctypes.byref(n)) == -1


def test_set_sweep_rate_needs_a_context(lib):
    """Argument checks come first: no context, no setting."""
    assert lib.epx_set_sweep_rate(None, 6200, 6000) == -1
    assert lib.epx_set_sweep_rate(None, 0, 0) == -1


def test_sweep_rate_calls_need_a_context(lib):
    b, f = ctypes.c_int(), ctypes.c_int()
    assert lib.epx_get_sweep_rate(None, ctypes.byref(b), ctypes.byref(f)) == -1
    fill = ctypes.c_int()
    assert lib.epx_calibrate_sweep_rate(None, None, 1 << 30, ctypes.byref(fill), None) == -1
