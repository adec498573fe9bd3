"""CPU oracle for the collective data plane -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's ``cpu_baseline`` leg may
import this package.  The product library never does, and the two share no
code: this wrapper drives ``liboracle.so`` built from ``ccl_oracle.c`` (plain
scalar C, ``-O2 -fno-fast-math -ffp-contract=off``).

What each call computes, with the passages it follows, is documented in
``ccl_oracle.c``.  Arrays are numpy: ``f32`` -> float32, ``i32`` -> int32,
``bf16`` / ``f16`` -> uint16 holding the bit pattern.

Layouts for reshard are ``(mesh_dims, start_rank, placements)`` where each
placement is ``"R"`` (Replicate) or ``("S", d)`` (Shard along tensor dim d),
one per mesh axis, as the M2N/T-CCL digest (lqnn.cn news 207677) s1.3
describes them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ccl_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": (0, np.float32), "bf16": (1, np.uint16), "i32": (2, np.int32),
          "f16": (3, np.uint16)}
OPS = {"sum": 0, "min": 1, "max": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall",
             "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
        pp = ctypes.POINTER(ctypes.c_void_p)
        p64 = ctypes.POINTER(ctypes.c_int64)
        pu64 = ctypes.POINTER(ctypes.c_uint64)
        pint = ctypes.POINTER(ctypes.c_int)
        lib.orc_all_reduce.argtypes = [pp, pp, i32, sz, i32, i32]
        lib.orc_reduce_scatter.argtypes = [pp, pp, i32, sz, i32, i32]
        lib.orc_all_gather.argtypes = [pp, pp, i32, sz, i32]
        lib.orc_fold_at.argtypes = [pp, i32, i32, i32, pu64, sz, vp]
        lib.orc_reduce.argtypes = [pp, vp, i32, sz, i32, i32]
        lib.orc_broadcast.argtypes = [vp, pp, i32, sz, i32]
        lib.orc_all_reduce_rmsnorm.argtypes = [pp, pp, i32, sz, sz, vp, ctypes.c_double, i32]
        lib.orc_quantize_e4m3.argtypes = [vp, i32, sz, sz, vp, vp]
        lib.orc_quantize_e4m3.restype = i32
        lib.orc_e4m3_value.argtypes = [ctypes.c_uint]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_nearest_sat.argtypes = [ctypes.c_float]
        lib.orc_e4m3_nearest_sat.restype = ctypes.c_uint
        lay = [i32, p64, i64, pint, pint]
        lib.orc_reshard.argtypes = [i32, p64, i32] + lay + lay + [pp, pp]
        lib.orc_reshard_at.argtypes = [i32, p64, i32] + lay + lay + [pp, i64, pu64, sz, vp]
        lib.orc_local_numel.argtypes = [i32, p64, i32, p64, pint, pint, i64]
        lib.orc_local_numel.restype = i64
        lib.orc_narrow_bf16.argtypes = [ctypes.c_float]
        lib.orc_narrow_bf16.restype = ctypes.c_uint16
        lib.orc_widen_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_widen_bf16.restype = ctypes.c_float
        lib.orc_narrow_f16.argtypes = [ctypes.c_float]
        lib.orc_narrow_f16.restype = ctypes.c_uint16
        lib.orc_widen_f16.argtypes = [ctypes.c_uint16]
        lib.orc_widen_f16.restype = ctypes.c_float
        for f in ("orc_all_reduce", "orc_reduce_scatter", "orc_all_gather", "orc_fold_at",
                  "orc_reshard", "orc_reshard_at", "orc_reduce", "orc_broadcast",
                  "orc_all_reduce_rmsnorm"):
            getattr(lib, f).restype = i32
        _lib = lib
    return _lib


def _ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))


def _check_bufs(xs, dtype):
    code, npdt = DTYPES[dtype]
    out = []
    for x in xs:
        x = np.ascontiguousarray(x)
        if x.dtype != npdt:
            raise TypeError(f"oracle: {dtype} buffers must be {np.dtype(npdt)}, got {x.dtype}")
        out.append(x)
    if len({x.size for x in out}) > 1:
        raise ValueError("oracle: rank buffers differ in size")
    return code, npdt, out


def _rc(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments (code {rc})")


def all_reduce(xs, dtype: str, op: str = "sum"):
    code, npdt, xs = _check_bufs(xs, dtype)
    P, n = len(xs), xs[0].size
    ys = [np.empty(n, npdt) for _ in range(P)]
    _rc(_load().orc_all_reduce(_ptrs(xs), _ptrs(ys), P, n, code, OPS[op]), "all_reduce")
    return ys


def reduce_scatter(xs, dtype: str, op: str = "sum"):
    code, npdt, xs = _check_bufs(xs, dtype)
    P, n = len(xs), xs[0].size
    if n % P:
        raise ValueError("oracle: reduce_scatter needs P to divide the buffer length")
    m = n // P
    ys = [np.empty(m, npdt) for _ in range(P)]
    _rc(_load().orc_reduce_scatter(_ptrs(xs), _ptrs(ys), P, m, code, OPS[op]), "reduce_scatter")
    return ys


def all_gather(xs, dtype: str):
    code, npdt, xs = _check_bufs(xs, dtype)
    P, m = len(xs), xs[0].size
    ys = [np.empty(P * m, npdt) for _ in range(P)]
    _rc(_load().orc_all_gather(_ptrs(xs), _ptrs(ys), P, m, code), "all_gather")
    return ys


def reduce(xs, dtype: str, op: str = "sum"):
    """The root's output of a reduce: the fold of all P inputs."""
    code, npdt, xs = _check_bufs(xs, dtype)
    y = np.empty(xs[0].size, npdt)
    _rc(_load().orc_reduce(_ptrs(xs), y.ctypes.data, len(xs), xs[0].size, code, OPS[op]), "reduce")
    return y


def broadcast(x, P: int, dtype: str):
    """Every rank's output of a broadcast from one root buffer."""
    code, npdt, (x,) = _check_bufs([x], dtype)
    ys = [np.empty(x.size, npdt) for _ in range(P)]
    _rc(_load().orc_broadcast(x.ctypes.data, _ptrs(ys), P, x.size, code), "broadcast")
    return ys


def all_reduce_rmsnorm(xs, rows: int, hidden: int, gamma, eps: float, dtype: str):
    """All-reduce (sum) with a row-wise RMSNorm between the two halves."""
    code, npdt, xs = _check_bufs(xs, dtype)
    gamma = np.ascontiguousarray(gamma, dtype=npdt)
    if xs[0].size != rows * hidden or gamma.size != hidden:
        raise ValueError("oracle: shapes do not match rows x hidden")
    P = len(xs)
    ys = [np.empty(rows * hidden, npdt) for _ in range(P)]
    _rc(_load().orc_all_reduce_rmsnorm(_ptrs(xs), _ptrs(ys), P, rows, hidden, gamma.ctypes.data,
                                       float(eps), code), "all_reduce_rmsnorm")
    return ys


def fold_at(xs, dtype: str, op: str, idx):
    """The reduction over ranks at the given element indices only."""
    code, npdt, xs = _check_bufs(xs, dtype)
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.size, npdt)
    _rc(_load().orc_fold_at(_ptrs(xs), len(xs), code, OPS[op],
                            idx.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), idx.size,
                            out.ctypes.data), "fold_at")
    return out


def _layout_args(layout):
    dims, start, placements = layout
    dims = list(dims)
    if len(placements) != len(dims):
        raise ValueError("oracle: one placement per mesh axis")
    kind, sdim = [], []
    for p in placements:
        if p == "R":
            kind.append(0)
            sdim.append(0)
        else:
            tag, d = p
            if tag != "S":
                raise ValueError(f"oracle: bad placement {p!r}")
            kind.append(1)
            sdim.append(int(d))
    keep = (np.array(dims, np.int64), np.array(kind, np.intc), np.array(sdim, np.intc))
    args = [len(dims), keep[0].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(start),
            keep[1].ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
            keep[2].ctypes.data_as(ctypes.POINTER(ctypes.c_int))]
    return args, keep


def mesh_size(layout) -> int:
    return int(np.prod(layout[0]))


def local_numel(shape, layout, rank_index: int = 0) -> int:
    """Elements held by the rank at position ``rank_index`` of the layout's mesh."""
    shp = np.array(shape, np.int64)
    args, _keep = _layout_args(layout)
    n = _load().orc_local_numel(len(shape), shp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                args[0], args[1], args[3], args[4], int(rank_index))
    if n < 0:
        raise ValueError("oracle: invalid layout")
    return int(n)


def reshard(shape, src_layout, dst_layout, src_bufs, fill=0):
    """Brute-force reshard.  ``src_bufs[l]`` is the l-th rank of the source mesh;
    returns one buffer per destination-mesh rank (pre-filled with ``fill`` so a
    test can see any element left unwritten)."""
    src_bufs = [np.ascontiguousarray(b) for b in src_bufs]
    dt = src_bufs[0].dtype
    shp = np.array(shape, np.int64)
    sa, k1 = _layout_args(src_layout)
    da, k2 = _layout_args(dst_layout)
    nd = mesh_size(dst_layout)
    dst = [np.full(local_numel(shape, dst_layout, l), fill, dt) for l in range(nd)]
    rc = _load().orc_reshard(len(shape), shp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             dt.itemsize, *sa, *da, _ptrs(src_bufs), _ptrs(dst))
    del k1, k2
    _rc(rc, "reshard")
    return dst


def reshard_at(shape, src_layout, dst_layout, src_bufs, dst_rank_index, local_idx):
    """Values destination rank ``dst_rank_index`` must hold at the given local
    element offsets."""
    src_bufs = [np.ascontiguousarray(b) for b in src_bufs]
    dt = src_bufs[0].dtype
    shp = np.array(shape, np.int64)
    sa, k1 = _layout_args(src_layout)
    da, k2 = _layout_args(dst_layout)
    idx = np.ascontiguousarray(local_idx, dtype=np.uint64)
    out = np.empty(idx.size, dt)
    rc = _load().orc_reshard_at(len(shape), shp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                dt.itemsize, *sa, *da, _ptrs(src_bufs), int(dst_rank_index),
                                idx.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), idx.size,
                                out.ctypes.data)
    del k1, k2
    _rc(rc, "reshard_at")
    return out


def narrow_bf16(x: float) -> int:
    return int(_load().orc_narrow_bf16(float(x)))


def widen_bf16(h: int) -> float:
    return float(_load().orc_widen_bf16(int(h)))


def quantize_e4m3(x, dtype: str, block: int = 128):
    """Blockwise FP8 E4M3 quantization: (codes uint8, scales float32)."""
    code, npdt, (x,) = _check_bufs([x], dtype)
    codes = np.empty(x.size, np.uint8)
    scales = np.empty((x.size + block - 1) // block, np.float32)
    _rc(_load().orc_quantize_e4m3(x.ctypes.data, code, x.size, block, codes.ctypes.data,
                                  scales.ctypes.data), "quantize_e4m3")
    return codes, scales


def reshard_fp8(shape, src_layout, dst_layout, src_bufs, dtype: str, block: int = 128):
    """Reshard, then quantize every destination buffer blockwise to E4M3."""
    dst = reshard(shape, src_layout, dst_layout, src_bufs)
    return [quantize_e4m3(d, dtype, block) for d in dst]


def e4m3_value(code: int) -> float:
    return float(_load().orc_e4m3_value(int(code)))


def e4m3_nearest_sat(y: float) -> int:
    return int(_load().orc_e4m3_nearest_sat(float(y)))


def narrow_f16(x: float) -> int:
    return int(_load().orc_narrow_f16(float(x)))


def widen_f16(h: int) -> float:
    return float(_load().orc_widen_f16(int(h)))
