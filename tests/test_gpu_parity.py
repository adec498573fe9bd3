"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small and medium sizes (several chunks plus a ragged tail) are compared with
the full oracle element by element; ragged counts, unaligned pointers, in-place
forms, every launch-config knob and the guard bands around every buffer are
covered.  Full-size configurations live in test_gpu_configs.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from _parity import DevBuf, assert_parity, upload_all
from collective_communication_plane_amd import ccl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NP = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "f16": np.uint16}
ESZ = {"f32": 4, "bf16": 2, "i32": 4, "f16": 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def stream():
    return torch.cuda.current_stream()


def dist_of(dtype):
    return "int20" if dtype == "i32" else "uniform"


def run_ar(xs, dtype, op, offset=0, cfg=None, out_offset=None):
    P, n = len(xs), xs[0].size
    dx = upload_all(xs, DEV, offset)
    dy = [DevBuf(n * ESZ[dtype], DEV, offset if out_offset is None else out_offset)
          for _ in range(P)]
    st = ccl.ccl_all_reduce([b.ptr for b in dx], [b.ptr for b in dy], P, n, ccl.DTYPES[dtype],
                            ccl.OPS[op], stream(), cfg)
    ccl.check(st, "all_reduce")
    torch.cuda.synchronize()
    for b in dx + dy:
        assert b.guards_intact()
    return [b.download(NP[dtype]) for b in dy]


# ------------------------------------------------------------- all-reduce

@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32", "f16"])
@pytest.mark.parametrize("op", ["sum", "min", "max"])
def test_all_reduce_matches_oracle(P, dtype, op):
    n = 3 * 16384 + 5  # several 64 KiB chunks plus a ragged tail
    xs = si.rank_buffers(P, n, dtype, dist_of(dtype), seed=P * 7 + len(op))
    got = run_ar(xs, dtype, op)
    want = oracle.all_reduce(xs, dtype, op)
    for q in range(P):
        assert_parity(got[q], want[q], dtype, op, f"AR P={P} {dtype} {op} q={q}")
        np.testing.assert_array_equal(got[q].view(np.uint8), got[0].view(np.uint8))


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 4095, 4096, 4097, 65537])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_reduce_ragged_counts(n, dtype):
    xs = si.rank_buffers(4, n, dtype, "uniform", seed=n)
    got = run_ar(xs, dtype, "sum")
    want = oracle.all_reduce(xs, dtype, "sum")
    for q in range(4):
        assert_parity(got[q], want[q], dtype, "sum", f"AR n={n}")


# every buffer at the same element-aligned offset from a 16-byte boundary
@pytest.mark.parametrize("dtype,offset", [("f32", 4), ("f32", 8), ("f32", 12),
                                          ("bf16", 2), ("bf16", 4), ("bf16", 8), ("bf16", 12)])
def test_all_reduce_unaligned_alike(offset, dtype):
    xs = si.rank_buffers(3, 10001, dtype, "uniform", seed=offset)
    got = run_ar(xs, dtype, "sum", offset=offset)
    want = oracle.all_reduce(xs, dtype, "sum")
    for q in range(3):
        assert_parity(got[q], want[q], dtype, "sum", f"AR offset={offset}")


def test_all_reduce_misaligned_relative_to_each_other():
    """Inputs at offset 0, outputs at offset 4: inputs are realigned in VGPRs."""
    xs = si.rank_buffers(4, 5003, "f32", "uniform", seed=3)
    got = run_ar(xs, "f32", "max", offset=0, out_offset=4)
    want = oracle.all_reduce(xs, "f32", "max")
    for q in range(4):
        assert_parity(got[q], want[q], "f32", "max", "AR mixed alignment")


def test_all_reduce_in_place():
    P, n = 8, 20000
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=12)
    bufs = upload_all(xs, DEV)
    ptrs = [b.ptr for b in bufs]
    ccl.check(ccl.ccl_all_reduce(ptrs, ptrs, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM, stream()))
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs, "bf16", "sum")
    for q in range(P):
        assert bufs[q].guards_intact()
        assert_parity(bufs[q].download(np.uint16), want[q], "bf16", "sum", "AR in place")


def test_all_reduce_denormals_and_signed_zero():
    tiny = np.array([1e-45, -1e-45, 1.1754942e-38, -0.0, 0.0, 3e-39, -2e-39, 5e-40],
                    np.float32)
    xs = [np.tile(tiny, 600), np.tile(tiny[::-1], 600), np.tile(tiny * np.float32(0.5), 600)]
    for op in ("sum", "min", "max"):
        got = run_ar(xs, "f32", op)
        want = oracle.all_reduce(xs, "f32", op)
        np.testing.assert_array_equal(got[0].view(np.uint32), want[0].view(np.uint32))
    xb = [si.to_bf16_bits(x) for x in xs]
    for op in ("sum", "min", "max"):
        got = run_ar(xb, "bf16", op)
        want = oracle.all_reduce(xb, "bf16", op)
        np.testing.assert_array_equal(got[0], want[0])


def test_bf16_rounding_ties_exercised():
    """Pairs whose fp32 sum lands exactly halfway between bf16 values."""
    base = si.rank_buffers(1, 8192, "bf16", "uniform", seed=77)[0]
    f = si.bf16_bits_to_f32(base)
    # x + x*2^-8 has a 1 in the first dropped bit: a tie for many x
    half = si.to_bf16_bits(f * np.float32(2.0 ** -8))
    xs = [base, half]
    got = run_ar(xs, "bf16", "sum")
    want = oracle.all_reduce(xs, "bf16", "sum")
    np.testing.assert_array_equal(got[0], want[0])


@pytest.mark.parametrize("cfg", [
    dict(chunk_bytes=1024), dict(chunk_bytes=16384), dict(chunk_bytes=1 << 20),
    dict(workgroups=1), dict(workgroups=7), dict(workgroups=1000),
    dict(unroll=1), dict(unroll=2), dict(unroll=4), dict(stages=2), dict(stages=4),
    dict(nontemporal=1), dict(nontemporal=2), dict(nontemporal=3), dict(nontemporal=4),
    dict(chunk_bytes=4096, workgroups=3, unroll=1, nontemporal=4),
    dict(store_policy=1), dict(store_policy=2), dict(store_policy=1, occupancy=2),
    dict(store_policy=1, stages=2), dict(store_policy=1, stages=3, chunk_bytes=8192),
    dict(store_policy=1, chunk_bytes=1 << 20, workgroups=7), dict(store_policy=1, unroll=4),
    dict(store_policy=1, nontemporal=1), dict(store_policy=2, stages=2),
])
def test_launch_config_does_not_change_results(cfg):
    P, n = 8, 50001
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=5)
    want = oracle.all_reduce(xs, "bf16", "sum")
    got = run_ar(xs, "bf16", "sum", cfg=ccl.LaunchConfig(**cfg))
    for q in range(P):
        np.testing.assert_array_equal(got[q], want[q])
    # fp32 normal draws, whose sums change bits under any other fold order
    xf = si.rank_buffers(P, n, "f32", "normal", seed=8)
    want = oracle.all_reduce(xf, "f32", "sum")
    got = run_ar(xf, "f32", "sum", cfg=ccl.LaunchConfig(**cfg))
    for q in range(P):
        np.testing.assert_array_equal(got[q].view(np.uint32), want[q].view(np.uint32))
    # fp16, max (its own kernel instantiations)
    xh = si.rank_buffers(P, n, "f16", "normal", seed=9)
    want = oracle.all_reduce(xh, "f16", "max")
    got = run_ar(xh, "f16", "max", cfg=ccl.LaunchConfig(**cfg))
    for q in range(P):
        np.testing.assert_array_equal(got[q], want[q])
    # reduce-scatter and all-gather under the same config
    m = n // P + 3
    xr = si.rank_buffers(P, P * m, "f32", "uniform", seed=6)
    np.testing.assert_array_equal(np.concatenate(run_rs(xr, "f32", "min", cfg=ccl.LaunchConfig(**cfg))),
                                  np.concatenate(oracle.reduce_scatter(xr, "f32", "min")))
    xg = si.rank_buffers(P, m, "bf16", "normal", seed=7)
    got = run_ag(xg, "bf16", cfg=ccl.LaunchConfig(**cfg))
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xg))


@pytest.mark.parametrize("P", [2, 3, 4, 5, 6, 7, 9, 12, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unroll2_all_reduce_folds_in_rank_order(P, dtype):
    """With two vectors per lane in flight and nontemporal stores, the
    all-reduce kernel loads the last rank into its first slot and puts the
    slots back in rank order before the fold; a fold in any other order would
    still land within the parity bar, so the result must be bit-equal.  With
    these fp32 normal draws, starting the fold at rank P - 1 instead changes
    16,000-33,000 of the 50,001 sums at every P from 3 (two-term sums are
    order-free)."""
    n = 50001
    xs = si.rank_buffers(P, n, dtype, "normal", seed=40 + P)
    want = oracle.all_reduce(xs, dtype, "sum")
    got = run_ar(xs, dtype, "sum", cfg=ccl.LaunchConfig(unroll=2, store_policy=2))
    for q in range(P):
        np.testing.assert_array_equal(got[q], want[q])


# -------------------------------------------------------- reduce-scatter

def run_rs(xs, dtype, op, offset=0, cfg=None, out_offset=None):
    P = len(xs)
    m = xs[0].size // P
    dx = upload_all(xs, DEV, offset)
    dy = [DevBuf(m * ESZ[dtype], DEV, offset if out_offset is None else out_offset)
          for _ in range(P)]
    ccl.check(ccl.ccl_reduce_scatter([b.ptr for b in dx], [b.ptr for b in dy], P, m,
                                     ccl.DTYPES[dtype], ccl.OPS[op], stream(), cfg),
              "reduce_scatter")
    torch.cuda.synchronize()
    for b in dx + dy:
        assert b.guards_intact()
    return [b.download(NP[dtype]) for b in dy]


@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32", "f16"])
@pytest.mark.parametrize("op", ["sum", "min", "max"])
@pytest.mark.parametrize("m", [1, 13, 3 * 8192 + 3])
def test_reduce_scatter_matches_oracle(P, dtype, op, m):
    xs = si.rank_buffers(P, P * m, dtype, dist_of(dtype), seed=P + m)
    got = run_rs(xs, dtype, op)
    want = oracle.reduce_scatter(xs, dtype, op)
    for s in range(P):
        assert_parity(got[s], want[s], dtype, op, f"RS P={P} m={m} s={s}")


def test_reduce_scatter_unaligned_and_mixed():
    xs = si.rank_buffers(4, 4 * 3001, "bf16", "uniform", seed=8)
    want = oracle.reduce_scatter(xs, "bf16", "sum")
    for off, ooff in [(2, 2), (6, 6), (0, 2), (4, 0)]:
        got = run_rs(xs, "bf16", "sum", offset=off, out_offset=ooff)
        for s in range(4):
            assert_parity(got[s], want[s], "bf16", "sum", f"RS offsets {off}/{ooff}")


@pytest.mark.parametrize("m", [4099, 4096])
def test_reduce_scatter_in_place_nccl_form(m):
    P = 8
    xs = si.rank_buffers(P, P * m, "f32", "uniform", seed=9)
    bufs = upload_all(xs, DEV)
    send = [b.ptr for b in bufs]
    recv = [b.ptr + s * m * 4 for s, b in enumerate(bufs)]
    ccl.check(ccl.ccl_reduce_scatter(send, recv, P, m, ccl.CCL_FLOAT32, ccl.CCL_SUM, stream()))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, "f32", "sum")
    for s in range(P):
        got = bufs[s].download(np.float32)[s * m:(s + 1) * m]
        assert_parity(got, want[s], "f32", "sum", "RS in place")


# ------------------------------------------------------------ all-gather

def run_ag(xs, dtype, offset=0, cfg=None, out_offset=None):
    P, m = len(xs), xs[0].size
    dx = upload_all(xs, DEV, offset)
    dy = [DevBuf(P * m * ESZ[dtype], DEV, offset if out_offset is None else out_offset)
          for _ in range(P)]
    ccl.check(ccl.ccl_all_gather([b.ptr for b in dx], [b.ptr for b in dy], P, m,
                                 ccl.DTYPES[dtype], stream(), cfg), "all_gather")
    torch.cuda.synchronize()
    for b in dx + dy:
        assert b.guards_intact()
    return [b.download(NP[dtype]) for b in dy]


@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32", "f16"])
@pytest.mark.parametrize("m", [1, 9, 3 * 8192 + 1])
def test_all_gather_matches_oracle(P, dtype, m):
    xs = si.rank_buffers(P, m, dtype, dist_of(dtype), seed=P * m)
    got = run_ag(xs, dtype)
    want = oracle.all_gather(xs, dtype)
    for q in range(P):
        np.testing.assert_array_equal(got[q], want[q])


def test_all_gather_unaligned_and_mixed():
    xs = si.rank_buffers(3, 2047, "bf16", "normal", seed=10)
    want = oracle.all_gather(xs, "bf16")
    for off, ooff in [(2, 2), (14, 14), (0, 6), (2, 0)]:
        got = run_ag(xs, "bf16", offset=off, out_offset=ooff)
        for q in range(3):
            np.testing.assert_array_equal(got[q], want[q])


# m = 4096 makes every shard a whole number of 256-byte lines, so the default
# launch takes write-through stores; m = 5000 does not
@pytest.mark.parametrize("m", [5000, 4096])
def test_all_gather_in_place_nccl_form(m):
    P = 8
    xs = si.rank_buffers(P, m, "bf16", "normal", seed=11)
    outs = [DevBuf(P * m * 2, DEV) for _ in range(P)]
    for r in range(P):  # rank r's contribution sits in its own slot of its output
        outs[r].base[outs[r].pad + r * m * 2: outs[r].pad + (r + 1) * m * 2].copy_(
            torch.from_numpy(xs[r].view(np.uint8).copy()))
    send = [o.ptr + r * m * 2 for r, o in enumerate(outs)]
    ccl.check(ccl.ccl_all_gather(send, [o.ptr for o in outs], P, m, ccl.CCL_BFLOAT16, stream()))
    torch.cuda.synchronize()
    want = oracle.all_gather(xs, "bf16")
    for q in range(P):
        assert outs[q].guards_intact()
        np.testing.assert_array_equal(outs[q].download(np.uint16), want[q])


def test_rs_then_ag_equals_ar_on_gpu():
    P, m = 8, 6151
    xs = si.rank_buffers(P, P * m, "bf16", "uniform", seed=13)
    rs = run_rs(xs, "bf16", "sum")
    ag = run_ag(rs, "bf16")
    ar = run_ar(xs, "bf16", "sum")
    for q in range(P):
        np.testing.assert_array_equal(ag[q], ar[q])


# ------------------------------------------------------------- rejections

def test_rejected_calls_touch_nothing():
    P, n = 4, 1000
    xs = si.rank_buffers(P, n, "f32", "uniform", seed=14)
    dx = upload_all(xs, DEV)
    dy = [DevBuf(n * 4, DEV) for _ in range(P)]
    send = [b.ptr for b in dx]
    recv = [b.ptr for b in dy]
    bad_recv = recv[:1] + [recv[0] + 8] + recv[2:]  # two outputs overlap
    assert ccl.ccl_all_reduce(send, bad_recv, P, n, ccl.CCL_FLOAT32, ccl.CCL_SUM,
                              stream()) == ccl.CCL_ERR_ALIASING
    assert ccl.ccl_all_reduce(send, recv, P, n, ccl.CCL_FLOAT32, 9, stream()) == ccl.CCL_ERR_INVALID_ARG
    assert ccl.ccl_all_reduce(send, recv, P, n, ccl.CCL_FLOAT32, ccl.CCL_SUM, stream(),
                              ccl.LaunchConfig(chunk_bytes=100)) == ccl.CCL_ERR_INVALID_ARG
    torch.cuda.synchronize()
    for b in dy:
        assert (b.base == b.fill).all().item()


# --------------------------------------------------------- LDS pipeline

@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("P", [1, 3, 8, 16])
@pytest.mark.parametrize("chunk", [4096, 16384, 65536])
def test_lds_pipeline_all_reduce(stages, P, chunk):
    n = 5 * 8192 + 7  # several tiles and chunks plus a ragged tail
    cfg = ccl.LaunchConfig(stages=stages, chunk_bytes=chunk)
    for dtype, op in [("bf16", "sum"), ("f32", "max"), ("i32", "sum")]:
        xs = si.rank_buffers(P, n, dtype, dist_of(dtype), seed=stages + P)
        got = run_ar(xs, dtype, op, cfg=cfg)
        want = oracle.all_reduce(xs, dtype, op)
        for q in range(P):
            assert_parity(got[q], want[q], dtype, op, f"LDS AR S={stages} P={P} {dtype}")


@pytest.mark.parametrize("stages", [2, 4])
@pytest.mark.parametrize("P", [2, 8, 16])
def test_lds_pipeline_reduce_scatter_and_all_gather(stages, P):
    cfg = ccl.LaunchConfig(stages=stages, chunk_bytes=8192)
    m = 3 * 4096 + 5
    xs = si.rank_buffers(P, P * m, "bf16", "uniform", seed=P)
    got = run_rs(xs, "bf16", "sum", cfg=cfg)
    want = oracle.reduce_scatter(xs, "bf16", "sum")
    for s in range(P):
        assert_parity(got[s], want[s], "bf16", "sum", f"LDS RS S={stages} P={P}")
    xg = si.rank_buffers(P, m, "f32", "normal", seed=P + 1)
    got = run_ag(xg, "f32", cfg=cfg)
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xg))


@pytest.mark.parametrize("cfg", [dict(stages=2, workgroups=1), dict(stages=3, workgroups=5),
                                 dict(stages=4, workgroups=300, nontemporal=4)])
def test_lds_pipeline_few_workgroups_and_offsets(cfg):
    P, n = 8, 70001
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=21)
    want = oracle.all_reduce(xs, "bf16", "sum")
    for off in (0, 6):
        got = run_ar(xs, "bf16", "sum", offset=off, cfg=ccl.LaunchConfig(chunk_bytes=16384, **cfg))
        for q in range(P):
            np.testing.assert_array_equal(got[q], want[q])


@pytest.mark.parametrize("P", [2, 4, 5, 8, 9, 12, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "i32"])
def test_default_write_through_on_line_aligned_shards(P, dtype):
    """Shards of whole 256-byte lines take the write-through stores by default
    (reduce-scatter up to P = 8, all-gather at P = 2 and 4..12); results equal
    the oracle and the nontemporal-only launch bit for bit."""
    m = 3 * 4096 // ESZ[dtype]
    xr = si.rank_buffers(P, P * m, dtype, dist_of(dtype), seed=P + 60)
    want = oracle.reduce_scatter(xr, dtype, "sum")
    got = run_rs(xr, dtype, "sum")
    nt = run_rs(xr, dtype, "sum", cfg=ccl.LaunchConfig(store_policy=2))
    for s in range(P):
        assert_parity(got[s], want[s], dtype, "sum", f"RS write-through P={P}")
        np.testing.assert_array_equal(got[s], nt[s])
    xg = si.rank_buffers(P, m, dtype, dist_of(dtype), seed=P + 61)
    got = run_ag(xg, dtype)
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xg))


@pytest.mark.parametrize("pol", [1, 2])
@pytest.mark.parametrize("P", [3, 8, 12])
def test_store_policies_on_realigned_and_offset_buffers(P, pol):
    """Write-through and nontemporal-only stores on the realigning kernel
    (ragged shards, inputs at another offset than outputs) and on buffers
    whose common offset leaves a scalar head."""
    cfg = ccl.LaunchConfig(store_policy=pol)
    m = 1237
    xr = si.rank_buffers(P, P * m, "bf16", "uniform", seed=P + 40)
    got = run_rs(xr, "bf16", "sum", offset=2, out_offset=0, cfg=cfg)
    want = oracle.reduce_scatter(xr, "bf16", "sum")
    for s in range(P):
        assert_parity(got[s], want[s], "bf16", "sum", f"RS realigned pol={pol}")
    xg = si.rank_buffers(P, m, "bf16", "normal", seed=P + 41)
    got = run_ag(xg, "bf16", offset=6, out_offset=0, cfg=cfg)
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xg))
    xa = si.rank_buffers(P, 5 * m, "f32", "uniform", seed=P + 42)
    want = oracle.all_reduce(xa, "f32", "max")
    for off, out_off in ((4, 0), (8, 8)):
        got = run_ar(xa, "f32", "max", offset=off, out_offset=out_off, cfg=cfg)
        for q in range(P):
            np.testing.assert_array_equal(got[q], want[q])


@pytest.mark.parametrize("stages", [1, 2, 3])
@pytest.mark.parametrize("P,m", [(1, 1), (2, 1), (3, 3), (4, 5), (8, 7), (16, 2)])
def test_segments_without_whole_vectors(stages, P, m):
    """Shards shorter than one 16-byte vector are all scalar head/tail."""
    cfg = ccl.LaunchConfig(stages=stages, chunk_bytes=4096)
    xs = si.rank_buffers(P, P * m, "f32", "uniform", seed=m)
    got = run_rs(xs, "f32", "sum", cfg=cfg)
    want = oracle.reduce_scatter(xs, "f32", "sum")
    for s in range(P):
        assert_parity(got[s], want[s], "f32", "sum", f"RS tiny S={stages}")
    xb = si.rank_buffers(P, m, "bf16", "normal", seed=m)
    got = run_ag(xb, "bf16", cfg=cfg)
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xb))
    got = run_ar(xb, "bf16", "max", cfg=cfg)
    want = oracle.all_reduce(xb, "bf16", "max")
    for q in range(P):
        np.testing.assert_array_equal(got[q], want[q])


# ------------------------------------------------- realigned and element-wise paths

def run_offsets(kind, xs, dtype, op, in_offs, out_offs, cfg=None):
    """Run one collective with a separate byte offset per input and output buffer."""
    P = len(xs)
    e = ESZ[dtype]
    if kind == "ar":
        n_in, n_out, cnt = xs[0].size, xs[0].size, xs[0].size
    elif kind == "rs":
        n_in, n_out, cnt = xs[0].size, xs[0].size // P, xs[0].size // P
    else:
        n_in, n_out, cnt = xs[0].size, P * xs[0].size, xs[0].size
    dx = [DevBuf(n_in * e, DEV, o).upload(x) for x, o in zip(xs, in_offs)]
    dy = [DevBuf(n_out * e, DEV, o) for o in out_offs]
    fn = {"ar": lambda: ccl.ccl_all_reduce([b.ptr for b in dx], [b.ptr for b in dy], P, cnt,
                                           ccl.DTYPES[dtype], ccl.OPS[op], stream(), cfg),
          "rs": lambda: ccl.ccl_reduce_scatter([b.ptr for b in dx], [b.ptr for b in dy], P, cnt,
                                               ccl.DTYPES[dtype], ccl.OPS[op], stream(), cfg),
          "ag": lambda: ccl.ccl_all_gather([b.ptr for b in dx], [b.ptr for b in dy], P, cnt,
                                           ccl.DTYPES[dtype], stream(), cfg)}[kind]
    ccl.check(fn(), kind)
    torch.cuda.synchronize()
    for b in dx + dy:
        assert b.guards_intact()
    return [b.download(NP[dtype]) for b in dy]


@pytest.mark.parametrize("P", [2, 3, 5, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m", [4097, 12289 * 3 + 1])
def test_ragged_shards_take_the_realigned_path(P, dtype, m):
    """Shard sizes that are not a multiple of 16 bytes put each segment's inputs
    and outputs at different offsets mod 16."""
    xs = si.rank_buffers(P, P * m, dtype, "uniform", seed=P + m)
    got = run_offsets("rs", xs, dtype, "sum", [0] * P, [0] * P)
    want = oracle.reduce_scatter(xs, dtype, "sum")
    for s_ in range(P):
        assert_parity(got[s_], want[s_], dtype, "sum", f"RS ragged P={P} m={m}")
    xg = si.rank_buffers(P, m, dtype, "normal", seed=m)
    got = run_offsets("ag", xg, dtype, "sum", [0] * P, [0] * P)
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xg))


@pytest.mark.parametrize("dtype", ["bf16", "f32", "i32"])
def test_inputs_at_assorted_offsets(dtype):
    """Every input at its own offset; outputs aligned alike (realigned path)."""
    P, n = 6, 30011
    step = ESZ[dtype]
    offs = [(k * step * 3) % 16 for k in range(P)]
    xs = si.rank_buffers(P, n, dtype, dist_of(dtype), seed=31)
    for op in ("sum", "max"):
        got = run_offsets("ar", xs, dtype, op, offs, [4 % 16 if step == 4 else 2] * P)
        want = oracle.all_reduce(xs, dtype, op)
        for q in range(P):
            assert_parity(got[q], want[q], dtype, op, f"AR assorted offsets {op}")


def test_outputs_misaligned_to_each_other_use_elementwise_kernel():
    P, n = 4, 20003
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=41)
    outs = [0, 2, 4, 6]
    got = run_offsets("ar", xs, "bf16", "sum", [0] * P, outs)
    want = oracle.all_reduce(xs, "bf16", "sum")
    for q in range(P):
        assert_parity(got[q], want[q], "bf16", "sum", "AR outputs misaligned")
    xr = si.rank_buffers(P, P * 1001, "f32", "uniform", seed=42)
    got = run_offsets("rs", xr, "f32", "min", [0, 4, 8, 12], [4, 0, 12, 8])
    want = oracle.reduce_scatter(xr, "f32", "min")
    for s_ in range(P):
        np.testing.assert_array_equal(got[s_], want[s_])
    xg = si.rank_buffers(P, 777, "bf16", "normal", seed=43)
    got = run_offsets("ag", xg, "bf16", "sum", [2, 0, 6, 4], [0, 2, 4, 8])
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xg))


@pytest.mark.parametrize("in_offs, out_offs, path", [
    ([4] * 6, [4] * 6, "scalar head and tail around the vector body"),
    ([0] * 6, [4] * 6, "inputs realigned in VGPRs"),
    ([0, 4, 8, 12, 0, 4], [8] * 6, "inputs at assorted offsets, realigned"),
    ([0] * 6, [0, 4, 8, 12, 0, 4], "outputs misaligned to each other: element-wise kernel"),
])
def test_misaligned_paths_fold_in_rank_order(in_offs, out_offs, path):
    """Every kernel family folds in rank order: fp32 normal sums, whose bits
    change under any other order, equal the oracle's bit for bit on the paths
    that misaligned buffers take (all-reduce and reduce-scatter)."""
    P = 6
    xs = si.rank_buffers(P, 30011, "f32", "normal", seed=51)
    got = run_offsets("ar", xs, "f32", "sum", in_offs, out_offs)
    want = oracle.all_reduce(xs, "f32", "sum")
    for q in range(P):
        np.testing.assert_array_equal(got[q].view(np.uint32), want[q].view(np.uint32), path)
    xr = si.rank_buffers(P, P * 5003, "f32", "normal", seed=52)
    got = run_offsets("rs", xr, "f32", "sum", in_offs, out_offs)
    want = oracle.reduce_scatter(xr, "f32", "sum")
    for s_ in range(P):
        np.testing.assert_array_equal(got[s_].view(np.uint32), want[s_].view(np.uint32), path)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 6, 8, 12, 16])
def test_default_launch_for_every_rank_count(P):
    """The defaults change with P (chunk sizes, unroll, residency caps, store policy)."""
    m = 3 * 4096 + 8
    xs = si.rank_buffers(P, P * m, "bf16", "uniform", seed=P)
    got = run_rs(xs, "bf16", "sum")
    want = oracle.reduce_scatter(xs, "bf16", "sum")
    for s_ in range(P):
        assert_parity(got[s_], want[s_], "bf16", "sum", f"RS default P={P}")
    got = run_ag(xs[:P], "bf16")
    for q in range(P):
        np.testing.assert_array_equal(got[q], np.concatenate(xs))
    got = run_ar(xs, "bf16", "sum")
    want = oracle.all_reduce(xs, "bf16", "sum")
    for q in range(P):
        assert_parity(got[q], want[q], "bf16", "sum", f"AR default P={P}")


# ---------------------------------------------------------- reduce / broadcast

@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "i32"])
@pytest.mark.parametrize("op", ["sum", "min", "max"])
def test_reduce_matches_oracle(P, dtype, op):
    n = 2 * 8192 + 11
    xs = si.rank_buffers(P, n, dtype, dist_of(dtype), seed=P + 3)
    dx = upload_all(xs, DEV)
    dy = DevBuf(n * ESZ[dtype], DEV)
    root = P - 1
    ccl.check(ccl.ccl_reduce([b.ptr for b in dx], dy.ptr, P, n, ccl.DTYPES[dtype], ccl.OPS[op],
                             root, stream()), "reduce")
    torch.cuda.synchronize()
    assert dy.guards_intact()
    assert_parity(dy.download(NP[dtype]), oracle.reduce(xs, dtype, op), dtype, op, f"reduce P={P}")


@pytest.mark.parametrize("P", [1, 2, 5, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [1, 7, 3 * 8192 + 5])
def test_broadcast_matches_oracle(P, dtype, n):
    x = si.rank_buffers(1, n, dtype, "normal", seed=n)[0]
    dx = DevBuf(x.nbytes, DEV).upload(x)
    dy = [DevBuf(x.nbytes, DEV) for _ in range(P)]
    ccl.check(ccl.ccl_broadcast(dx.ptr, [b.ptr for b in dy], P, n, ccl.DTYPES[dtype], 0, stream()),
              "broadcast")
    torch.cuda.synchronize()
    want = oracle.broadcast(x, P, dtype)
    for q in range(P):
        assert dy[q].guards_intact()
        np.testing.assert_array_equal(dy[q].download(NP[dtype]), want[q])


def test_reduce_and_broadcast_in_place_and_offsets():
    P, n = 8, 40003
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=50)
    want = oracle.reduce(xs, "bf16", "sum")
    # in place on the root's send buffer
    dx = upload_all(xs, DEV)
    ccl.check(ccl.ccl_reduce([b.ptr for b in dx], dx[3].ptr, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM,
                             3, stream()))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dx[3].download(np.uint16), want)
    # inputs at offset 2, output aligned: realigned path
    dx = [DevBuf(x.nbytes, DEV, 2).upload(x) for x in xs]
    dy = DevBuf(n * 2, DEV)
    ccl.check(ccl.ccl_reduce([b.ptr for b in dx], dy.ptr, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM,
                             0, stream()))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dy.download(np.uint16), want)
    # broadcast in place at the root, the others at assorted offsets
    x = xs[0]
    outs = [DevBuf(x.nbytes, DEV, o) for o in (0, 2, 4, 6, 8, 10, 12, 14)]
    outs[5].upload(x)
    st = ccl.ccl_broadcast(outs[5].ptr, [b.ptr for b in outs], P, n, ccl.CCL_BFLOAT16, 5, stream())
    ccl.check(st)
    torch.cuda.synchronize()
    for b in outs:
        np.testing.assert_array_equal(b.download(np.uint16), x)


def test_reduce_and_broadcast_reject_bad_arguments():
    P, n = 4, 100
    bufs = [DevBuf(n * 4, DEV) for _ in range(P)]
    ptrs = [b.ptr for b in bufs]
    assert ccl.ccl_reduce(ptrs, ptrs[0], P, n, ccl.CCL_FLOAT32, ccl.CCL_SUM, P, stream()) == \
        ccl.CCL_ERR_INVALID_ARG  # root out of range
    assert ccl.ccl_reduce(ptrs, ptrs[0] + 4, P, n, ccl.CCL_FLOAT32, ccl.CCL_SUM, 0, stream()) == \
        ccl.CCL_ERR_ALIASING
    assert ccl.ccl_broadcast(ptrs[0], ptrs, P, n, ccl.CCL_FLOAT32, -1, stream()) == \
        ccl.CCL_ERR_INVALID_ARG
    assert ccl.ccl_broadcast(ptrs[0] + 8, ptrs, P, n, ccl.CCL_FLOAT32, 0, stream()) == \
        ccl.CCL_ERR_ALIASING
    torch.cuda.synchronize()
    for b in bufs:
        assert (b.base == b.fill).all().item()


def test_zero_length_calls_touch_nothing():
    """count 0 / rows 0 / an empty tensor: every entry point returns CCL_OK and
    leaves the (canary-filled) buffers as they were."""
    P = 4
    bufs = [DevBuf(256, DEV) for _ in range(2 * P)]
    send, recv = [b.ptr for b in bufs[:P]], [b.ptr for b in bufs[P:]]
    gamma = DevBuf(64, DEV)
    stream = torch.cuda.current_stream()
    for dt in (ccl.CCL_FLOAT32, ccl.CCL_BFLOAT16, ccl.CCL_INT32, ccl.CCL_FLOAT16):
        assert ccl.ccl_all_reduce(send, recv, P, 0, dt, ccl.CCL_SUM, stream) == ccl.CCL_OK
        assert ccl.ccl_reduce_scatter(send, recv, P, 0, dt, ccl.CCL_MAX, stream) == ccl.CCL_OK
        assert ccl.ccl_all_gather(send, recv, P, 0, dt, stream) == ccl.CCL_OK
        assert ccl.ccl_reduce(send, recv[0], P, 0, dt, ccl.CCL_MIN, 1, stream) == ccl.CCL_OK
        assert ccl.ccl_broadcast(send[0], recv, P, 0, dt, 2, stream) == ccl.CCL_OK
    assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, 0, 64, gamma.ptr, 1e-6, ccl.CCL_BFLOAT16,
                                      stream) == ccl.CCL_OK
    desc = ccl.make_tensor_desc((0, 64), ccl.CCL_BFLOAT16)
    st, plan = ccl.ccl_reshard_plan(desc, ccl.make_mesh([2], 0), ccl.make_placements([("S", 1)]),
                                    ccl.make_mesh([2], 2), ccl.make_placements(["R"]))
    ccl.check(st, "reshard_plan")
    try:
        assert ccl.ccl_reshard_copy(plan, send[:2], recv[:2], stream) == ccl.CCL_OK
        assert ccl.ccl_reshard_copy_fp8(plan, send[:2], recv[:2], [gamma.ptr, gamma.ptr + 32],
                                        stream) == ccl.CCL_OK
    finally:
        ccl.check(ccl.ccl_plan_destroy(plan))
    torch.cuda.synchronize()
    for b in bufs + [gamma]:
        assert b.guards_intact()
        assert bool((b.base == b.fill).all().item()), "a zero-length call wrote"
