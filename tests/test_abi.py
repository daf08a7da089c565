"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments before any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import structured_sparse_attention_amd as svg
from structured_sparse_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svg_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return svg.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), f"{n} declared in svg_attn.h but not exported"
    assert sorted(svg.EXPORTED) == names


def test_abi_version(lib):
    assert svg.abi_version() == 1


def _spec(kinds, frames=4, gh=8, gw=8, wf=1, ws=8, sink=1, rnd=0):
    arr = np.asarray(kinds, dtype=np.int32)
    s = _lib.MaskSpec(frames, gh, gw, len(arr), arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                      wf, ws, sink, rnd)
    return s, arr


def _build(lib, spec, bq=32, bk=32):
    out = ctypes.c_void_p()
    st = lib.svg_build_tile_map(ctypes.byref(spec) if spec is not None else None, bq, bk,
                                None, ctypes.byref(out))
    return st, out


@pytest.mark.parametrize("mutate,status", [
    (dict(frames=0), svg.ERR_INVALID_ARG),
    (dict(gh=0), svg.ERR_INVALID_ARG),
    (dict(wf=-1), svg.ERR_INVALID_ARG),
    (dict(ws=-3), svg.ERR_INVALID_ARG),
    (dict(rnd=7), svg.ERR_INVALID_ARG),
    (dict(kinds=[0, 5]), svg.ERR_INVALID_ARG),
    (dict(kinds=[]), svg.ERR_INVALID_ARG),
    (dict(frames=1 << 16, gh=1 << 8, gw=1 << 8), svg.ERR_INVALID_ARG),
])
def test_build_rejects_bad_spec(lib, mutate, status):
    args = dict(kinds=[0, 1])
    args.update(mutate)
    spec, keep = _spec(**args)
    st, out = _build(lib, spec)
    assert st == status
    assert not out.value
    assert lib.svg_last_error().decode()


@pytest.mark.parametrize("bq,bk", [(48, 32), (96, 64), (300, 128), (256, 48), (256, 16),
                                   (256, 2048), (0, 128), (-256, 128)])
def test_build_rejects_unsupported_tiles(lib, bq, bk):
    spec, keep = _spec([0, 1])
    st, out = _build(lib, spec, bq, bk)
    assert st == svg.ERR_UNSUPPORTED
    assert not out.value


def test_build_null_arguments(lib):
    assert _build(lib, None)[0] == svg.ERR_INVALID_ARG
    spec, keep = _spec([0, 1])
    assert lib.svg_build_tile_map(ctypes.byref(spec), 32, 32, None, None) == svg.ERR_INVALID_ARG
    spec.head_kind = None
    assert _build(lib, spec)[0] == svg.ERR_INVALID_ARG


def test_map_calls_reject_null(lib):
    assert lib.svg_tile_map_destroy(None) == svg.OK
    info = _lib.TileMapInfo()
    assert lib.svg_tile_map_info_get(None, ctypes.byref(info)) == svg.ERR_INVALID_ARG
    assert lib.svg_tile_map_rebuild(None, None) == svg.ERR_INVALID_ARG
    assert lib.svg_tile_map_stats(None, None, 1) == svg.ERR_INVALID_ARG
    assert lib.svg_tile_map_copy_classes(None, None, 0) == svg.ERR_INVALID_ARG
    assert lib.svg_tile_map_copy_schedule(None, None, None, None, None, 0) == svg.ERR_INVALID_ARG


def test_attn_rejects_bad_arguments_before_hip(lib):
    kinds = np.array([0, 1], dtype=np.int32)
    kp = kinds.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p = 1 << 20  # never dereferenced: validation fails first
    f = lib.svg_attn_fwd
    assert f(None, p, p, p, 256, 2, 64, 0.125, kp, p, 0, None) == svg.ERR_INVALID_ARG
    assert f(p, p, p, p, 256, 2, 64, 0.125, kp, None, 0, None) == svg.ERR_INVALID_ARG
    assert f(p, p, p, p, 256, 2, 64, 0.125, None, p, 0, None) == svg.ERR_INVALID_ARG
    assert f(p, p, p, p, 256, 2, 64, -1.0, kp, p, 0, None) == svg.ERR_INVALID_ARG
    assert f(p, p, p, p, 256, 2, 64, float("inf"), kp, p, 0, None) == svg.ERR_INVALID_ARG
    assert f(p, p, p, p, 256, 2, 64, 0.125, kp, p, 8, None) == svg.ERR_INVALID_ARG
    assert "flags" in lib.svg_last_error().decode()


def test_autotune_rejects_bad_arguments_before_hip(lib):
    kinds = np.array([0, 1], dtype=np.int32)
    kp = kinds.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    spec = _lib.MaskSpec(4, 8, 8, 2, kp, 1, 8, 1, 0)
    p = 1 << 20  # never dereferenced: validation fails first
    tq = np.array([256, 100], dtype=np.int32)
    tk = np.array([128, 128], dtype=np.int32)
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    ms = (ctypes.c_float * 2)()
    best = ctypes.c_int32()
    f = lib.svg_autotune_tiles
    args = lambda **kw: dict(dict(spec=ctypes.byref(spec), q=p, k=p, v=p, o=p, d=64, sc=0.125,
                                  tq=ip(tq), tk=ip(tk), n=1, reps=3, st=None, ms=ms,
                                  best=ctypes.byref(best)), **kw).values()
    assert f(*args(spec=None)) == svg.ERR_INVALID_ARG
    assert f(*args(q=None)) == svg.ERR_INVALID_ARG
    assert f(*args(n=0)) == svg.ERR_INVALID_ARG
    assert f(*args(reps=0)) == svg.ERR_INVALID_ARG
    assert f(*args(best=None)) == svg.ERR_INVALID_ARG
    assert f(*args(n=2)) == svg.ERR_UNSUPPORTED        # tile_q 100 has no kernel
    assert "candidate 1" in lib.svg_last_error().decode()
    assert f(*args(d=96)) == svg.ERR_UNSUPPORTED       # head_dim 96 has no kernel


@pytest.mark.parametrize("name", ["svg_route_heads", "svg_route_heads_noalloc"])
def test_route_rejects_bad_arguments_before_hip(lib, name):
    spec = _lib.MaskSpec(4, 8, 8, 2, None, 1, 8, 1, 0)
    p = 1 << 20  # never dereferenced: validation fails first
    rows = np.array([0, 5, 255], dtype=np.int32)
    bad = np.array([0, 256], dtype=np.int32)
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    kinds = np.zeros(2, dtype=np.int32)
    f = getattr(lib, name)
    assert f(None, p, p, p, 64, 0.125, ip(rows), 3, None, None, ip(kinds)) == svg.ERR_INVALID_ARG
    assert f(ctypes.byref(spec), None, p, p, 64, 0.125, ip(rows), 3, None, None,
             ip(kinds)) == svg.ERR_INVALID_ARG
    assert f(ctypes.byref(spec), p, p, p, 64, 0.125, ip(bad), 2, None, None,
             ip(kinds)) == svg.ERR_INVALID_ARG
    assert "rows[1]" in lib.svg_last_error().decode()
    assert f(ctypes.byref(spec), p, p, p, 64, 0.125, ip(rows), 0, None, None,
             ip(kinds)) == svg.ERR_INVALID_ARG
    assert f(ctypes.byref(spec), p, p, p, 64, -1.0, ip(rows), 3, None, None,
             ip(kinds)) == svg.ERR_INVALID_ARG
    assert f(ctypes.byref(spec), p, p, p, 96, 0.125, ip(rows), 3, None, None,
             ip(kinds)) == svg.ERR_UNSUPPORTED
    assert f(ctypes.byref(spec), p + 8, p, p, 64, 0.125, ip(rows), 3, None, None,
             ip(kinds)) == svg.ERR_ALIGNMENT


def test_permute_rejects_bad_arguments_before_hip(lib):
    kinds = np.array([0, 1], dtype=np.int32)
    kp = kinds.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = lib.svg_permute_tokens
    a, b = 1 << 20, 1 << 30
    assert f(None, b, 4, 64, 2, 64, kp, 0, None) == svg.ERR_INVALID_ARG
    assert f(a, b, 0, 64, 2, 64, kp, 0, None) == svg.ERR_INVALID_ARG
    assert f(a, b, 4, 64, 2, 60, kp, 0, None) == svg.ERR_UNSUPPORTED
    assert f(a, b, 1 << 12, 1 << 12, 2, 64, kp, 0, None) == svg.ERR_UNSUPPORTED  # head >= 2 GiB
    assert f(a, b, 4, 64, 2, 64, kp, 2, None) == svg.ERR_INVALID_ARG
    assert f(a + 8, b, 4, 64, 2, 64, kp, 0, None) == svg.ERR_ALIGNMENT
    assert f(a, a + 16, 4, 64, 2, 64, kp, 0, None) == svg.ERR_INVALID_ARG  # overlap
    bad = np.array([0, 3], dtype=np.int32)
    assert f(a, b, 4, 64, 2, 64, bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 0,
             None) == svg.ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = _lib._lib
    _lib._lib = None
    try:
        return _lib.load(path)
    finally:
        _lib._lib = saved


class _FakeDeviceTensor:
    """Stands in for a CUDA bf16 tensor: the wrappers' checks run before any
    pointer reaches the library, so nothing is dereferenced."""

    def __init__(self, shape):
        import torch
        self.shape = shape
        self.dtype = torch.bfloat16
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 1 << 20


def test_wrappers_reject_a_head_kind_list_of_the_wrong_length():
    t = _FakeDeviceTensor((2, 256, 64))
    with pytest.raises(ValueError, match="head_kind has 1 entries"):
        svg.svg_attn_fwd(t, t, t, t, ["spatial"], None)
    with pytest.raises(ValueError, match="head_kind has 3 entries"):
        svg.svg_attn_fwd(t, t, t, t, ["spatial", "temporal", "dense"], None)
    with pytest.raises(ValueError, match="head_kind has 1 entries"):
        svg.svg_permute_tokens(t, t, 4, 64, ["temporal"], svg.TO_KERNEL_LAYOUT)
