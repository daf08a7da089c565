"""ctypes binding of libsvgattn (argument marshalling only).

Every computation runs in the HIP library. PyTorch is used for device memory
and the current stream; tensors are passed by pointer. When the library is
missing this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Union

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvgattn.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_SHAPE_MISMATCH = -3
ERR_ALIGNMENT = -4
ERR_HIP = -5
ERR_OOM = -6

HEAD_SPATIAL, HEAD_TEMPORAL, HEAD_DENSE = 0, 1, 2
ROUND_EXACT, ROUND_TILE = 0, 1
TILE_SKIP, TILE_FULL, TILE_BOUNDARY = 0, 1, 2
TO_KERNEL_LAYOUT, TO_ORIGINAL_LAYOUT = 0, 1
ATTN_MASK_ALL_TILES = 1

_KIND_NAMES = {"spatial": HEAD_SPATIAL, "temporal": HEAD_TEMPORAL, "dense": HEAD_DENSE}

# Every symbol the public header declares (checked by the tests).
EXPORTED = (
    "svg_build_tile_map", "svg_tile_map_rebuild", "svg_tile_map_info_get",
    "svg_tile_map_stats", "svg_tile_map_copy_classes", "svg_tile_map_copy_schedule",
    "svg_tile_map_plan_info", "svg_tile_map_destroy", "svg_attn_fwd", "svg_autotune_tiles",
    "svg_route_heads", "svg_route_heads_noalloc", "svg_permute_tokens", "svg_last_error",
    "svg_abi_version",
)


class SvgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"svg status {status}: {message}")
        self.status = status


class MaskSpec(ctypes.Structure):
    _fields_ = [
        ("frames", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("head_kind", ctypes.POINTER(ctypes.c_int32)),
        ("frame_window", ctypes.c_int32), ("temporal_band", ctypes.c_int32),
        ("sink_first_frame", ctypes.c_int32), ("round_mode", ctypes.c_int32),
    ]


class TileMapInfo(ctypes.Structure):
    _fields_ = [
        ("seq_len", ctypes.c_int64), ("num_heads", ctypes.c_int32),
        ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("num_q_tiles", ctypes.c_int32), ("num_k_tiles", ctypes.c_int32),
        ("frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
        ("entry_capacity", ctypes.c_int64),
    ]


class HeadStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "tiles", "skip", "full", "boundary", "exec_full", "exec_boundary",
        "exec_sink", "retained_pairs")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("workgroups", ctypes.c_int32), ("xcds", ctypes.c_int32)] + [
        (n, ctypes.c_int64) for n in ("work_items", "split_rows", "partial_slots", "max_load",
                                      "total_load")]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsvgattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m structured_sparse_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    pI32 = ctypes.POINTER(ctypes.c_int32)
    sigs = {
        "svg_build_tile_map": (I32, [ctypes.POINTER(MaskSpec), I32, I32, P, ctypes.POINTER(P)]),
        "svg_tile_map_rebuild": (I32, [P, P]),
        "svg_tile_map_info_get": (I32, [P, ctypes.POINTER(TileMapInfo)]),
        "svg_tile_map_stats": (I32, [P, ctypes.POINTER(HeadStats), I32]),
        "svg_tile_map_copy_classes": (I32, [P, ctypes.POINTER(ctypes.c_uint8), SZ]),
        "svg_tile_map_copy_schedule": (I32, [P, pI32, pI32, pI32, pI32, SZ]),
        "svg_tile_map_plan_info": (I32, [P, ctypes.POINTER(PlanInfo)]),
        "svg_tile_map_destroy": (I32, [P]),
        "svg_attn_fwd": (I32, [P, P, P, P, I64, I32, I32, ctypes.c_float, pI32, P, U32, P]),
        "svg_autotune_tiles": (I32, [ctypes.POINTER(MaskSpec), P, P, P, P, I32, ctypes.c_float,
                                     pI32, pI32, I32, I32, P, ctypes.POINTER(ctypes.c_float),
                                     pI32]),
        "svg_route_heads": (I32, [ctypes.POINTER(MaskSpec), P, P, P, I32, ctypes.c_float, pI32,
                                  I32, P, ctypes.POINTER(ctypes.c_float), pI32]),
        "svg_route_heads_noalloc": (I32, [ctypes.POINTER(MaskSpec), P, P, P, I32, ctypes.c_float,
                                          pI32, I32, P, ctypes.POINTER(ctypes.c_float), pI32]),
        "svg_permute_tokens": (I32, [P, P, I32, I32, I32, I32, pI32, I32, P]),
        "svg_last_error": (ctypes.c_char_p, []),
        "svg_abi_version": (I32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        msg = load().svg_last_error().decode(errors="replace")
        raise SvgError(status, msg)


def _kinds(head_kind: Sequence[Union[str, int]]) -> np.ndarray:
    return np.ascontiguousarray(
        [_KIND_NAMES[k] if isinstance(k, str) else int(k) for k in head_kind], dtype=np.int32)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


class TileMap:
    """Owner of a device tile map built by ``svg_build_tile_map``."""

    def __init__(self, handle: ctypes.c_void_p, head_kind: np.ndarray):
        self._h = handle
        self.head_kind = head_kind
        info = TileMapInfo()
        _check(load().svg_tile_map_info_get(self._h, ctypes.byref(info)))
        self.info = info

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("tile map already destroyed")
        return self._h

    def rebuild(self, stream=None) -> None:
        _check(load().svg_tile_map_rebuild(self.handle, _stream(stream)))

    def stats(self) -> list:
        n = self.info.num_heads
        arr = (HeadStats * n)()
        _check(load().svg_tile_map_stats(self.handle, arr, n))
        return [{f: getattr(s, f) for f, _ in HeadStats._fields_} for s in arr]

    def classes(self) -> np.ndarray:
        i = self.info
        out = np.empty((i.num_heads, i.num_q_tiles, i.num_k_tiles), dtype=np.uint8)
        _check(load().svg_tile_map_copy_classes(
            self.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), out.size))
        return out

    def schedule(self):
        """(row_ptr [R+1], n_full [R], sink_ab [R,2], entries) with R = H*nQ."""
        i = self.info
        R = i.num_heads * i.num_q_tiles
        row_ptr = np.empty(R + 1, dtype=np.int32)
        _check(load().svg_tile_map_copy_schedule(self.handle, _i32p(row_ptr), None, None, None, 0))
        n_full = np.empty(R, dtype=np.int32)
        sink_ab = np.empty((R, 2), dtype=np.int32)
        entries = np.empty(max(1, int(row_ptr[-1])), dtype=np.int32)
        _check(load().svg_tile_map_copy_schedule(self.handle, _i32p(row_ptr), _i32p(n_full),
                                                 _i32p(sink_ab), _i32p(entries), entries.size))
        return row_ptr, n_full, sink_ab, entries[: int(row_ptr[-1])]

    def plan_info(self) -> dict:
        pi = PlanInfo()
        _check(load().svg_tile_map_plan_info(self.handle, ctypes.byref(pi)))
        return {f: getattr(pi, f) for f, _ in PlanInfo._fields_}

    def destroy(self) -> None:
        if self._h:
            _check(load().svg_tile_map_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def svg_build_tile_map(frames: int, grid_h: int, grid_w: int,
                       head_kind: Sequence[Union[str, int]], frame_window: int,
                       temporal_band: int, sink_first_frame: bool = True,
                       round_mode: int = ROUND_EXACT, tile_q: int = 256,
                       tile_k: int = 128, stream=None) -> TileMap:
    kinds = _kinds(head_kind)
    spec = MaskSpec(frames, grid_h, grid_w, len(kinds), _i32p(kinds), frame_window,
                    temporal_band, 1 if sink_first_frame else 0, round_mode)
    h = ctypes.c_void_p()
    _check(load().svg_build_tile_map(ctypes.byref(spec), tile_q, tile_k, _stream(stream),
                                     ctypes.byref(h)))
    return TileMap(h, kinds)


def _bf16_tensor(t, name):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA bfloat16 tensor")
    return t


def svg_attn_fwd(q, k, v, o, head_kind: Sequence[Union[str, int]], tile_map: TileMap,
                 scale: Optional[float] = None, flags: int = 0, stream=None) -> None:
    """O = masked softmax(scale Q K^T) V; q, k, v, o: bf16 [H, N, d] (kernel layout)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _bf16_tensor(t, n)
    H, N, d = q.shape
    for t, n in ((k, "k"), (v, "v"), (o, "o")):
        if tuple(t.shape) != (H, N, d):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {(H, N, d)}")
    kinds = _kinds(head_kind)
    if len(kinds) != H:
        raise ValueError(f"head_kind has {len(kinds)} entries, q has {H} heads")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load().svg_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), N, H, d,
                               float(scale), _i32p(kinds), tile_map.handle, flags,
                               _stream(stream)))


def svg_autotune_tiles(q, k, v, o, frames: int, grid_h: int, grid_w: int,
                       head_kind: Sequence[Union[str, int]], frame_window: int,
                       temporal_band: int, candidates: Sequence[tuple],
                       sink_first_frame: bool = True, round_mode: int = ROUND_EXACT,
                       reps: int = 3, scale: Optional[float] = None, stream=None):
    """Time the attention forward for each (tile_q, tile_k) candidate.

    Returns (index of the fastest candidate, list of mean ms per call)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _bf16_tensor(t, n)
    H, N, d = q.shape
    kinds = _kinds(head_kind)
    if len(kinds) != H or N != frames * grid_h * grid_w:
        raise ValueError("q's shape disagrees with the mask specification")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    spec = MaskSpec(frames, grid_h, grid_w, H, _i32p(kinds), frame_window, temporal_band,
                    1 if sink_first_frame else 0, round_mode)
    tq = np.ascontiguousarray([c[0] for c in candidates], dtype=np.int32)
    tk = np.ascontiguousarray([c[1] for c in candidates], dtype=np.int32)
    ms = (ctypes.c_float * max(1, len(candidates)))()
    best = ctypes.c_int32(-1)
    _check(load().svg_autotune_tiles(ctypes.byref(spec), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), o.data_ptr(), d, float(scale), _i32p(tq),
                                     _i32p(tk), len(candidates), reps, _stream(stream), ms,
                                     ctypes.byref(best)))
    return int(best.value), [float(ms[i]) for i in range(len(candidates))]


def svg_route_heads(q, k, v, frames: int, grid_h: int, grid_w: int, frame_window: int,
                    temporal_band: int, rows, sink_first_frame: bool = True,
                    scale: Optional[float] = None, stream=None, no_alloc: bool = False):
    """Route each head to the spatial or temporal mask from sampled query rows.

    q, k, v: bf16 [H, N, d] in the original frame-major order; rows: original
    query indices. Returns (kinds: list of "spatial"/"temporal", err: float32
    [H, 2] numpy array of the spatial and temporal mean squared errors).
    no_alloc: use svg_route_heads_noalloc (the library's static scratch)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16_tensor(t, n)
    H, N, d = q.shape
    for t, n in ((k, "k"), (v, "v")):
        if tuple(t.shape) != (H, N, d):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {(H, N, d)}")
    if N != frames * grid_h * grid_w:
        raise ValueError("q's shape disagrees with frames * grid_h * grid_w")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r = np.ascontiguousarray(rows, dtype=np.int32)
    spec = MaskSpec(frames, grid_h, grid_w, H, None, frame_window, temporal_band,
                    1 if sink_first_frame else 0, ROUND_EXACT)
    err = np.zeros((H, 2), dtype=np.float32)
    kinds = np.zeros(H, dtype=np.int32)
    fn = load().svg_route_heads_noalloc if no_alloc else load().svg_route_heads
    _check(fn(ctypes.byref(spec), q.data_ptr(), k.data_ptr(), v.data_ptr(), d, float(scale),
              _i32p(r), len(r), _stream(stream),
              err.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _i32p(kinds)))
    names = {HEAD_SPATIAL: "spatial", HEAD_TEMPORAL: "temporal"}
    return [names[int(x)] for x in kinds], err


def svg_permute_tokens(src, dst, frames: int, tokens_per_frame: int,
                       head_kind: Sequence[Union[str, int]], direction: int,
                       stream=None) -> None:
    """Re-order rows of bf16 [H, N, d] between original and kernel layouts."""
    _bf16_tensor(src, "src")
    _bf16_tensor(dst, "dst")
    H, N, d = src.shape
    if tuple(dst.shape) != (H, N, d) or N != frames * tokens_per_frame:
        raise ValueError("src/dst shapes disagree with frames * tokens_per_frame")
    kinds = _kinds(head_kind)
    if len(kinds) != H:
        raise ValueError(f"head_kind has {len(kinds)} entries, src has {H} heads")
    _check(load().svg_permute_tokens(src.data_ptr(), dst.data_ptr(), frames, tokens_per_frame,
                                     H, d, _i32p(kinds), direction, _stream(stream)))


def abi_version() -> int:
    return int(load().svg_abi_version())
