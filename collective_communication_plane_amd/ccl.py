"""Thin ctypes binding of libccl's C ABI (include/ccl.h), same names as the C calls.

Argument marshalling only: every call goes straight to the native library,
which runs all of its work in its own HIP kernels.  Buffers may be passed as
integers (device addresses) or as objects with ``data_ptr()`` (e.g. torch
tensors); streams as integers (hipStream_t), objects with ``cuda_stream``, or
None for the null stream.  Calls return the C status code (0 = CCL_OK);
``check()`` turns a non-zero code into ``CclError``.

If libccl.so has not been built the first call raises ``RuntimeError``; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libccl.so")

CCL_OK = 0
CCL_ERR_INVALID_ARG = 1
CCL_ERR_UNSUPPORTED = 2
CCL_ERR_ALIASING = 3
CCL_ERR_LAYOUT = 4
CCL_ERR_HIP = 5
CCL_ERR_NOMEM = 6
CCL_ERR_SCRATCH_LIMIT = 7

CCL_FLOAT32 = 0
CCL_BFLOAT16 = 1
CCL_INT32 = 2
CCL_FLOAT16 = 3

CCL_SUM = 0
CCL_MIN = 1
CCL_MAX = 2

CCL_REPLICATE = 0
CCL_SHARD = 1

CCL_MAX_RANKS = 16
CCL_MAX_MESH_DIMS = 4
CCL_MAX_TENSOR_DIMS = 8
CCL_MAX_MESH_RANKS = 64
CCL_NOALLOC_SCRATCH_BYTES = 2 << 20

DTYPES = {"f32": CCL_FLOAT32, "bf16": CCL_BFLOAT16, "i32": CCL_INT32, "f16": CCL_FLOAT16}
OPS = {"sum": CCL_SUM, "min": CCL_MIN, "max": CCL_MAX}


class LaunchConfig(ctypes.Structure):
    _fields_ = [("chunk_bytes", ctypes.c_uint64), ("workgroups", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("nontemporal", ctypes.c_int32), ("occupancy", ctypes.c_int32),
                ("store_policy", ctypes.c_int32)]


class Placement(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dim", ctypes.c_int32)]


class Mesh(ctypes.Structure):
    _fields_ = [("ndims", ctypes.c_int32), ("start_rank", ctypes.c_int32),
                ("dims", ctypes.c_int64 * CCL_MAX_MESH_DIMS)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("shape", ctypes.c_int64 * CCL_MAX_TENSOR_DIMS)]


class Interval(ctypes.Structure):
    _fields_ = [("src_rank", ctypes.c_int32), ("dst_shard", ctypes.c_int32),
                ("leader", ctypes.c_int32), ("num_replicas", ctypes.c_int32),
                ("src_offset", ctypes.c_uint64), ("dst_offset", ctypes.c_uint64),
                ("length", ctypes.c_uint64)]


class CclError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {ccl_get_error_string(status)} ({status})")


_lib = None

EXPORTS = [
    "ccl_all_reduce", "ccl_reduce_scatter", "ccl_all_gather", "ccl_reduce", "ccl_broadcast",
    "ccl_all_reduce_rmsnorm", "ccl_all_reduce_rmsnorm_noalloc",
    "ccl_reshard_plan",
    "ccl_reshard_copy", "ccl_reshard_copy_fp8", "ccl_plan_destroy", "ccl_plan_num_intervals", "ccl_plan_get_interval",
    "ccl_plan_local_bytes", "ccl_plan_num_dst_shards", "ccl_plan_shard_replicas",
    "ccl_get_error_string", "ccl_version",
]


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libccl.so not found at {_LIB_PATH}: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    pp = ctypes.POINTER(ctypes.c_void_p)
    pcfg = ctypes.POINTER(LaunchConfig)
    lib.ccl_all_reduce.argtypes = [pp, pp, i32, sz, i32, i32, vp, pcfg]
    lib.ccl_reduce_scatter.argtypes = [pp, pp, i32, sz, i32, i32, vp, pcfg]
    lib.ccl_all_gather.argtypes = [pp, pp, i32, sz, i32, vp, pcfg]
    lib.ccl_reduce.argtypes = [pp, vp, i32, sz, i32, i32, i32, vp, pcfg]
    lib.ccl_all_reduce_rmsnorm.argtypes = [pp, pp, i32, sz, sz, vp, ctypes.c_float, i32, vp, pcfg]
    lib.ccl_all_reduce_rmsnorm_noalloc.argtypes = [pp, pp, i32, sz, sz, vp, ctypes.c_float, i32, vp,
                                                   pcfg]
    lib.ccl_broadcast.argtypes = [vp, pp, i32, sz, i32, i32, vp, pcfg]
    lib.ccl_reshard_plan.argtypes = [ctypes.POINTER(TensorDesc), ctypes.POINTER(Mesh),
                                     ctypes.POINTER(Placement), ctypes.POINTER(Mesh),
                                     ctypes.POINTER(Placement), ctypes.POINTER(vp)]
    lib.ccl_reshard_copy.argtypes = [vp, pp, pp, vp, pcfg]
    lib.ccl_reshard_copy_fp8.argtypes = [vp, pp, pp, pp, vp, pcfg]
    lib.ccl_plan_destroy.argtypes = [vp]
    lib.ccl_plan_num_intervals.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64)]
    lib.ccl_plan_get_interval.argtypes = [vp, ctypes.c_uint64, ctypes.POINTER(Interval)]
    lib.ccl_plan_local_bytes.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_uint64)]
    lib.ccl_plan_num_dst_shards.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    lib.ccl_plan_shard_replicas.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                            ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.ccl_get_error_string.argtypes = [i32]
    lib.ccl_get_error_string.restype = ctypes.c_char_p
    lib.ccl_version.argtypes = []
    for name in EXPORTS:
        if name != "ccl_get_error_string":
            getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _ptr_array(bufs: Sequence) -> ctypes.Array:
    return (ctypes.c_void_p * max(1, len(bufs)))(*[_addr(b) for b in bufs])


def _stream(stream) -> int:
    if stream is None:
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _cfg(cfg):
    if cfg is None:
        return None
    if isinstance(cfg, dict):
        cfg = LaunchConfig(**cfg)
    return ctypes.byref(cfg)


def _pp(arr):
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))


def check(status: int, what: str = "ccl") -> None:
    if status != CCL_OK:
        raise CclError(status, what)


# ------------------------------------------------------------------ calls

def ccl_all_reduce(send, recv, nranks: int, count: int, dtype: int, op: int, stream=None,
                   cfg=None) -> int:
    s, r = _ptr_array(send), _ptr_array(recv)
    return _load().ccl_all_reduce(_pp(s), _pp(r), nranks, count, dtype, op, _stream(stream),
                                  _cfg(cfg))


def ccl_reduce_scatter(send, recv, nranks: int, recvcount: int, dtype: int, op: int,
                       stream=None, cfg=None) -> int:
    s, r = _ptr_array(send), _ptr_array(recv)
    return _load().ccl_reduce_scatter(_pp(s), _pp(r), nranks, recvcount, dtype, op,
                                      _stream(stream), _cfg(cfg))


def ccl_all_gather(send, recv, nranks: int, sendcount: int, dtype: int, stream=None,
                   cfg=None) -> int:
    s, r = _ptr_array(send), _ptr_array(recv)
    return _load().ccl_all_gather(_pp(s), _pp(r), nranks, sendcount, dtype, _stream(stream),
                                  _cfg(cfg))


def ccl_all_reduce_rmsnorm(send, recv, nranks: int, rows: int, hidden: int, gamma, eps: float,
                           dtype: int, stream=None, cfg=None) -> int:
    s, r = _ptr_array(send), _ptr_array(recv)
    return _load().ccl_all_reduce_rmsnorm(_pp(s), _pp(r), nranks, rows, hidden, _addr(gamma),
                                          float(eps), dtype, _stream(stream), _cfg(cfg))


def ccl_all_reduce_rmsnorm_noalloc(send, recv, nranks: int, rows: int, hidden: int, gamma,
                                   eps: float, dtype: int, stream=None, cfg=None) -> int:
    s, r = _ptr_array(send), _ptr_array(recv)
    return _load().ccl_all_reduce_rmsnorm_noalloc(_pp(s), _pp(r), nranks, rows, hidden,
                                                  _addr(gamma), float(eps), dtype, _stream(stream),
                                                  _cfg(cfg))


def ccl_reduce(send, recv, nranks: int, count: int, dtype: int, op: int, root: int = 0,
               stream=None, cfg=None) -> int:
    s = _ptr_array(send)
    return _load().ccl_reduce(_pp(s), _addr(recv), nranks, count, dtype, op, root,
                              _stream(stream), _cfg(cfg))


def ccl_broadcast(send, recv, nranks: int, count: int, dtype: int, root: int = 0, stream=None,
                  cfg=None) -> int:
    r = _ptr_array(recv)
    return _load().ccl_broadcast(_addr(send), _pp(r), nranks, count, dtype, root,
                                 _stream(stream), _cfg(cfg))


def make_mesh(dims: Sequence[int], start_rank: int) -> Mesh:
    m = Mesh()
    m.ndims = len(dims)
    m.start_rank = start_rank
    for k, d in enumerate(dims):
        m.dims[k] = d
    return m


def make_placements(placements) -> ctypes.Array:
    """["R", ("S", d), ...] -> ccl_placement_t array."""
    arr = (Placement * max(1, len(placements)))()
    for k, p in enumerate(placements):
        if p == "R":
            arr[k].kind, arr[k].dim = CCL_REPLICATE, 0
        else:
            arr[k].kind, arr[k].dim = CCL_SHARD, int(p[1])
    return arr


def make_tensor_desc(shape: Sequence[int], dtype: int) -> TensorDesc:
    t = TensorDesc()
    t.ndim = len(shape)
    t.dtype = dtype
    for d, n in enumerate(shape):
        t.shape[d] = n
    return t


def ccl_reshard_plan(tensor: TensorDesc, src_mesh: Mesh, src_placements, dst_mesh: Mesh,
                     dst_placements):
    """Returns (status, plan handle or None)."""
    out = ctypes.c_void_p()
    st = _load().ccl_reshard_plan(ctypes.byref(tensor), ctypes.byref(src_mesh), src_placements,
                                  ctypes.byref(dst_mesh), dst_placements, ctypes.byref(out))
    return st, (out.value if st == CCL_OK else None)


def ccl_reshard_copy(plan, src_bufs, dst_bufs, stream=None, cfg=None) -> int:
    s, d = _ptr_array(src_bufs), _ptr_array(dst_bufs)
    return _load().ccl_reshard_copy(plan, _pp(s), _pp(d), _stream(stream), _cfg(cfg))


def ccl_reshard_copy_fp8(plan, src_bufs, dst_codes, dst_scales, stream=None, cfg=None) -> int:
    s, c, f = _ptr_array(src_bufs), _ptr_array(dst_codes), _ptr_array(dst_scales)
    return _load().ccl_reshard_copy_fp8(plan, _pp(s), _pp(c), _pp(f), _stream(stream), _cfg(cfg))


def ccl_plan_destroy(plan) -> int:
    return _load().ccl_plan_destroy(plan)


def ccl_plan_num_intervals(plan):
    n = ctypes.c_uint64()
    st = _load().ccl_plan_num_intervals(plan, ctypes.byref(n))
    return st, n.value


def ccl_plan_get_interval(plan, i: int):
    iv = Interval()
    st = _load().ccl_plan_get_interval(plan, i, ctypes.byref(iv))
    return st, iv


def ccl_plan_local_bytes(plan, side: int, index: int):
    n = ctypes.c_uint64()
    st = _load().ccl_plan_local_bytes(plan, side, index, ctypes.byref(n))
    return st, n.value


def ccl_plan_num_dst_shards(plan):
    n = ctypes.c_int32()
    st = _load().ccl_plan_num_dst_shards(plan, ctypes.byref(n))
    return st, n.value


def ccl_plan_shard_replicas(plan, dst_shard: int):
    cap = CCL_MAX_MESH_RANKS
    ranks = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32()
    st = _load().ccl_plan_shard_replicas(plan, dst_shard, ranks, cap, ctypes.byref(n))
    return st, list(ranks[: n.value])


def ccl_get_error_string(status: int) -> str:
    return _load().ccl_get_error_string(status).decode()


def ccl_version() -> int:
    return _load().ccl_version()


def plan_intervals(plan) -> list[Interval]:
    """All intervals of a plan (convenience over the two inspection calls)."""
    st, n = ccl_plan_num_intervals(plan)
    check(st, "ccl_plan_num_intervals")
    out = []
    for i in range(n):
        st, iv = ccl_plan_get_interval(plan, i)
        check(st, "ccl_plan_get_interval")
        out.append(iv)
    return out
