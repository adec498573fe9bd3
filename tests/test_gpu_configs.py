"""GPU parity at the full sizes of the benchmark workloads, default launch config.

Workloads (seed 0, numpy PCG64, rank r = r-th draw):
  AR-1   all-reduce sum, P=4 x 1,048,576 fp32 uniform[-1,1)    -> full oracle
  RS-bf  reduce-scatter sum, P=8 x 67,108,864 bf16 normal(0,1) -> full oracle
  RS-i   the same with int32 uniform in [-2^20, 2^20]           -> full oracle
  AG     all-gather, P=8 x 16,777,216 bf16 normal(0,1)         -> oracle samples
                                                                 + exact slot checks
  AR-256 all-reduce sum, P=8 x 256 MiB bf16 uniform (the headline workload)
                                                               -> oracle samples
                                                                 + replica identity
  sweep  all-reduce P=8, fp32/bf16, 4 KiB .. 1 GiB per rank in powers of 4,
         sum/min/max, chunk 16 KiB .. 1 MiB                    -> full oracle up to
                                                                 16 MiB per rank,
                                                                 samples above
  LDS    the same sweep's chunk axis through the LDS pipeline (2, 3 and 4
         stages; 16 KiB, 128 KiB and 1 MiB chunks) on 64 MiB (+ a ragged
         tail) and 256 MiB per rank, bf16 and fp32     -> bit-equal to the
                                                          register-direct
                                                          kernel + samples
  rules  the all-reduce's default launch inside each branch of its size- and
         P-dependent rules (P = 2-16, 16-512 MiB per rank) -> oracle samples
                                                             + replica identity
  AG-wt  all-gather at P = 13 and 16, 256 MiB of input in all (write-through
         by default)                                   -> exact slot checks
The 1 GiB points draw their inputs on the GPU (PyTorch's seeded generator) and
copy back only the sampled inputs for the oracle.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from _parity import assert_parity
from collective_communication_plane_amd import ccl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NP = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}
TORCH_BITS = {"f32": torch.int32, "bf16": torch.int16, "i32": torch.int32}


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).to(DEV)


def down(t: torch.Tensor, dt) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy().view(dt)


def gather_at(ts, idx: np.ndarray, dt) -> list[np.ndarray]:
    """Values of each device buffer at the sampled element indices."""
    it = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    return [t.view(torch.uint8).view(TORCH_BITS[dt])[it].cpu().numpy().view(NP[dt]) for t in ts]


def test_ar1_p4_1mi_fp32_full_oracle():
    P, n = 4, 1_048_576
    xs = si.rank_buffers(P, n, "f32", "uniform", seed=0)
    dx = [up(x) for x in xs]
    dy = [torch.empty_like(t) for t in dx]
    ccl.check(ccl.ccl_all_reduce(dx, dy, P, n, ccl.CCL_FLOAT32, ccl.CCL_SUM,
                                 torch.cuda.current_stream()))
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs, "f32", "sum")
    for q in range(P):
        n_neq = assert_parity(down(dy[q], np.float32), want[q], "f32", "sum", f"AR-1 q={q}")
        print(f"AR-1 q={q}: non-bit-equal {n_neq}")


@pytest.mark.parametrize("dtype,dist", [("bf16", "normal"), ("i32", "int20")])
def test_rs_p8_64mi_full_oracle(dtype, dist):
    P, N = 8, 67_108_864
    M = N // P
    xs = si.rank_buffers(P, N, dtype, dist, seed=0)
    dx = [up(x) for x in xs]
    dy = [torch.empty(M * xs[0].itemsize, dtype=torch.uint8, device=DEV) for _ in range(P)]
    ccl.check(ccl.ccl_reduce_scatter(dx, dy, P, M, ccl.DTYPES[dtype], ccl.CCL_SUM,
                                     torch.cuda.current_stream()))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, dtype, "sum")
    for s in range(P):
        n_neq = assert_parity(down(dy[s], NP[dtype]), want[s], dtype, "sum", f"RS {dtype} s={s}")
        print(f"RS {dtype} s={s}: non-bit-equal {n_neq}")


def test_ag_p8_16mi_bf16():
    P, M = 8, 16_777_216
    xs = si.rank_buffers(P, M, "bf16", "normal", seed=0)
    dx = [up(x) for x in xs]
    dy = [torch.empty(P * M * 2, dtype=torch.uint8, device=DEV) for _ in range(P)]
    ccl.check(ccl.ccl_all_gather(dx, dy, P, M, ccl.CCL_BFLOAT16, torch.cuda.current_stream()))
    torch.cuda.synchronize()
    # every slot of every output is byte-identical to the owner's input
    for q in range(P):
        for r in range(P):
            assert torch.equal(dy[q][r * M * 2:(r + 1) * M * 2], dx[r]), (q, r)
    # and sampled positions agree with the oracle's concatenation
    idx = si.sample_indices(P * M, 100_000)
    want = np.concatenate(xs)[idx.astype(np.int64)]
    got = gather_at(dy, idx, "bf16")
    for q in range(P):
        np.testing.assert_array_equal(got[q], want)


def _ar_sampled(ts_in, P, n, dtype, op, cfg=None, k=200_000, host_inputs=None):
    outs = [torch.empty_like(t) for t in ts_in]
    ccl.check(ccl.ccl_all_reduce(ts_in, outs, P, n, ccl.DTYPES[dtype], ccl.OPS[op],
                                 torch.cuda.current_stream(), cfg))
    torch.cuda.synchronize()
    for q in range(1, P):
        assert torch.equal(outs[q].view(torch.uint8), outs[0].view(torch.uint8)), q
    idx = si.sample_indices(n, k)
    if host_inputs is not None:
        want = oracle.fold_at(host_inputs, dtype, op, idx)
    else:
        xin = gather_at(ts_in, idx, dtype)
        want = oracle.fold_at(xin, dtype, op, np.arange(idx.size, dtype=np.uint64))
    got = gather_at([outs[0]], idx, dtype)[0]
    n_neq = assert_parity(got, want, dtype, op, f"AR n={n} {dtype} {op}")
    del outs
    return n_neq


def test_ar_p8_256mib_bf16_headline():
    P, n = 8, 134_217_728
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=0)
    dx = [up(x) for x in xs]
    print("non-bit-equal:", _ar_sampled(dx, P, n, "bf16", "sum", host_inputs=xs))


def test_ar_p8_256mib_bf16_headline_in_bench_layout():
    """The headline workload in the buffer layout the benchmark times: inputs and
    outputs as byte views into one allocation each, 2 MiB + 4 KiB apart."""
    import bench

    P, n = 8, 134_217_728
    xs = si.rank_buffers(P, n, "bf16", "uniform", seed=0)
    dx, stride = bench.rank_slab(P, 2 * n, DEV)
    dy, _ = bench.rank_slab(P, 2 * n, DEV)
    assert stride % 256 == 0 and stride >= 2 * n + bench.RANK_GAP
    for d, x in zip(dx, xs):
        d.copy_(torch.from_numpy(np.ascontiguousarray(x).view(np.uint8)))
    ccl.check(ccl.ccl_all_reduce(dx, dy, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM,
                                 torch.cuda.current_stream()))
    torch.cuda.synchronize()
    for q in range(1, P):
        assert torch.equal(dy[q], dy[0]), q
    idx = si.sample_indices(n, 200_000, seed=11)
    want = oracle.fold_at(xs, "bf16", "sum", idx)
    got = gather_at([dy[0]], idx, "bf16")[0]
    assert_parity(got, want, "bf16", "sum", "AR headline, bench layout")
    # the inputs were not written
    for d, x in zip(dx, xs):
        assert torch.equal(d[:1 << 20].cpu(), torch.from_numpy(x.view(np.uint8)[:1 << 20].copy()))


SWEEP_BYTES = [4096 * 4 ** k for k in range(10)]  # 4 KiB .. 1 GiB per rank


@pytest.mark.parametrize("nbytes", SWEEP_BYTES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ar_sweep_sizes(nbytes, dtype):
    P = 8
    esz = 4 if dtype == "f32" else 2
    n = nbytes // esz
    ops = ["sum", "min", "max"]
    if nbytes <= 16 << 20:
        xs = si.rank_buffers(P, n, dtype, "uniform", seed=0)
        dx = [up(x) for x in xs]
        for op in ops:
            dy = [torch.empty_like(t) for t in dx]
            ccl.check(ccl.ccl_all_reduce(dx, dy, P, n, ccl.DTYPES[dtype], ccl.OPS[op],
                                         torch.cuda.current_stream()))
            torch.cuda.synchronize()
            want = oracle.all_reduce(xs, dtype, op)[0]
            for q in range(P):
                assert_parity(down(dy[q], NP[dtype]), want, dtype, op, f"{nbytes}B {op} q={q}")
    else:
        dx = si.device_rank_buffers(P, n, dtype, "uniform", seed=0, device=DEV)
        for op in ops:
            _ar_sampled(dx, P, n, dtype, op)


@pytest.mark.parametrize("chunk", [16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10,
                                   512 << 10, 1 << 20])
@pytest.mark.parametrize("op", ["sum", "min", "max"])
def test_ar_sweep_chunks(chunk, op):
    P, n = 8, (64 << 20) // 2 + 3  # 64 MiB bf16 per rank plus a ragged tail
    dx = si.device_rank_buffers(P, n, "bf16", "uniform", seed=1, device=DEV)
    _ar_sampled(dx, P, n, "bf16", op, cfg=ccl.LaunchConfig(chunk_bytes=chunk), k=50_000)


_DEV_CACHE: dict = {}


def _cached_inputs(P, n, dtype, seed):
    """Device inputs drawn once per (P, n, dtype, seed) and reused by the
    parametrizations that follow; only the latest set is kept."""
    key = (P, n, dtype, seed)
    if key not in _DEV_CACHE:
        _DEV_CACHE.clear()
        torch.cuda.empty_cache()
        _DEV_CACHE[key] = si.device_rank_buffers(P, n, dtype, "uniform", seed=seed, device=DEV)
    return _DEV_CACHE[key]


# bytes per rank: 64 MiB plus a ragged tail (3 bf16 or 1 fp32 element), and 256 MiB
LDS_SIZES = [(64 << 20) + 6, 256 << 20]


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("chunk", [16 << 10, 128 << 10, 1 << 20])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nbytes", LDS_SIZES)
def test_lds_pipeline_sweep_chunks(nbytes, dtype, chunk, stages):
    """The LDS pipeline at the sweep's chunk sizes on large buffers: up to 256
    tiles per chunk walk its tile cursor and vmcnt bookkeeping.  The outputs
    must equal the register-direct kernel's bit for bit (same fold, same
    order) and the oracle at sampled indices; every replica is identical."""
    P = 8
    esz = 4 if dtype == "f32" else 2
    n = nbytes // esz
    print(f"LDS sweep: {dtype} n={n} chunk={chunk} stages={stages}", flush=True)
    dx = _cached_inputs(P, n, dtype, 3)
    ops = ["sum", "min", "max"] if nbytes < (256 << 20) or chunk == (128 << 10) else ["sum"]
    st = torch.cuda.current_stream()
    for op in ops:
        ref = [torch.empty_like(t) for t in dx]
        ccl.check(ccl.ccl_all_reduce(dx, ref, P, n, ccl.DTYPES[dtype], ccl.OPS[op], st,
                                     ccl.LaunchConfig(chunk_bytes=chunk, stages=1)))
        outs = [torch.empty_like(t) for t in dx]
        ccl.check(ccl.ccl_all_reduce(dx, outs, P, n, ccl.DTYPES[dtype], ccl.OPS[op], st,
                                     ccl.LaunchConfig(chunk_bytes=chunk, stages=stages)))
        torch.cuda.synchronize()
        for q in range(P):
            assert torch.equal(outs[q], ref[q]), (op, q)
        idx = si.sample_indices(n, 50_000, seed=stages)
        xin = gather_at(dx, idx, dtype)
        want = oracle.fold_at(xin, dtype, op, np.arange(idx.size, dtype=np.uint64))
        got = gather_at([outs[P - 1]], idx, dtype)[0]
        assert_parity(got, want, dtype, op, f"LDS S={stages} chunk={chunk} {dtype} {op}")
        del ref, outs


# Every branch of the all-reduce's size- and P-dependent launch rules, at a
# size where the branch applies, through the default launch (no config):
# (P, MiB per rank, dtype, op, branch)
RULE_CASES = [
    (2, 192, "bf16", "sum", "P = 2, 129-256 MiB: unroll 1"),
    (2, 320, "bf16", "max", "P = 2 above 256 MiB: write-through, 4 KiB chunks, unroll 1"),
    (4, 256, "f32", "min", "P = 3, 4 from 256 MiB: write-through, 8 KiB chunks"),
    (3, 64, "f32", "min", "3 <= P <= 8 up to 128 MiB: 8 KiB chunks, unroll 2"),
    (5, 128, "bf16", "sum", "the same at its upper bound"),
    (7, 160, "bf16", "sum", "P = 7 above 128 MiB: write-through"),
    (4, 144, "bf16", "min", "P = 4 above 128 MiB: write-through, 8 KiB chunks"),
    (6, 160, "f32", "sum", "P = 6 above 128 MiB: write-through"),
    (8, 136, "bf16", "min", "P = 8 above 128 MiB: write-through"),
    (9, 16, "f32", "sum", "P >= 9 from 16 MiB: write-through"),
    (12, 32, "bf16", "max", "the same at P = 12"),
    (16, 64, "bf16", "sum", "the same at P = 16"),
    (6, 512, "bf16", "sum", "congruent inputs from 512 MiB: 16 KiB chunks, write-through"),
    (5, 512, "f32", "max", "the same at P = 5: 8 KiB chunks, write-through"),
]


@pytest.mark.parametrize("P, mib, dtype, op, branch", RULE_CASES,
                         ids=[f"P{c[0]}-{c[1]}MiB-{c[2]}-{c[3]}" for c in RULE_CASES])
def test_ar_default_rule_branches(P, mib, dtype, op, branch):
    esz = 4 if dtype == "f32" else 2
    n = (mib << 20) // esz
    print(f"AR default launch, P={P}, {mib} MiB per rank, {dtype} {op}: {branch}", flush=True)
    dx = si.device_rank_buffers(P, n, dtype, "uniform", seed=P, device=DEV)
    _ar_sampled(dx, P, n, dtype, op)


@pytest.mark.parametrize("P, mib", [(2, 288), (4, 144), (4, 256), (8, 136), (12, 20), (16, 17)])
def test_ar_write_through_shapes_with_a_ragged_tail(P, mib):
    """The all-reduce's write-through shapes (P = 2: 4 KiB chunks, unroll 1;
    P = 4: 8 KiB chunks; P >= 5: 4 KiB chunks) on a count 5 elements past whole
    vectors, so the last chunk is partial and a scalar tail follows it.  Every
    output equals the nontemporal-only launch (store_policy = 2) byte for byte,
    and sampled points, the last 4096 elements among them, equal the oracle."""
    n = (mib << 20) // 2 + 5
    print(f"AR write-through shape, P={P}, n={n} bf16", flush=True)
    dx = si.device_rank_buffers(P, n, "bf16", "normal", seed=40 + P, device=DEV)
    wt = [torch.empty_like(t) for t in dx]
    nt = [torch.empty_like(t) for t in dx]
    stream = torch.cuda.current_stream()
    ccl.check(ccl.ccl_all_reduce(dx, wt, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM, stream))
    ccl.check(ccl.ccl_all_reduce(dx, nt, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM, stream,
                                 ccl.LaunchConfig(store_policy=2)))
    torch.cuda.synchronize()
    for q in range(P):
        assert torch.equal(wt[q].view(torch.int16), nt[q].view(torch.int16)), q
    idx = np.unique(np.concatenate([si.sample_indices(n, 50_000, seed=P),
                                    np.arange(n - 4096, n, dtype=np.uint64)]))
    xin = gather_at(dx, idx, "bf16")
    want = oracle.fold_at(xin, "bf16", "sum", np.arange(idx.size, dtype=np.uint64))
    for q in (0, P - 1):
        got = gather_at([wt[q]], idx, "bf16")[0]
        assert_parity(got, want, "bf16", "sum", f"AR WT P={P} rank {q}")
    del dx, wt, nt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P, mib", [(4, 512), (5, 512)])
def test_ar_staggered_inputs_from_512mib(P, mib):
    """Inputs staggered against each other (one allocation, 2 MiB + 4 KiB
    apart), where the congruence test picks other chunk sizes than for
    separate allocations: 4 KiB chunks at P = 4 (instead of 8 KiB) and at
    P = 5 (instead of 8 KiB for congruent inputs).  The default launch equals
    both forced shapes byte for byte, and sampled points equal the oracle."""
    import bench

    n = (mib << 20) // 4 + 3  # fp32, a count 3 past whole vectors
    print(f"AR staggered, P={P}, n={n} f32", flush=True)
    dx, _ = bench.rank_slab(P, 4 * n, DEV)
    src = si.device_rank_buffers(P, n, "f32", "normal", seed=60 + P, device=DEV)
    for d, t in zip(dx, src):
        d.copy_(t.view(torch.uint8))
    del src
    xs = [d.view(torch.float32) for d in dx]
    outs = {}
    stream = torch.cuda.current_stream()
    for name, cfg in (("default", None),
                      ("4K", ccl.LaunchConfig(chunk_bytes=4096, unroll=1, occupancy=3)),
                      ("8K", ccl.LaunchConfig(chunk_bytes=8192, unroll=1, occupancy=3))):
        ys, _ = bench.rank_slab(P, 4 * n, DEV)
        outs[name] = [y.view(torch.float32) for y in ys]
        ccl.check(ccl.ccl_all_reduce(xs, outs[name], P, n, ccl.CCL_FLOAT32, ccl.CCL_SUM, stream,
                                     cfg))
    torch.cuda.synchronize()
    for name in ("4K", "8K"):
        for q in range(P):
            assert torch.equal(outs[name][q].view(torch.int32),
                               outs["default"][q].view(torch.int32)), (name, q)
    idx = si.sample_indices(n, 50_000, seed=P)
    xin = gather_at(xs, idx, "f32")
    want = oracle.fold_at(xin, "f32", "sum", np.arange(idx.size, dtype=np.uint64))
    got = gather_at([outs["default"][P - 1]], idx, "f32")[0]
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    del dx, xs, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P", [13, 16])
def test_ag_write_through_up_to_p16(P):
    """All-gather at P = 13 and 16 with 256 MiB of input in all (write-through
    by default): every output slot equals its owner's input, byte for byte."""
    M = (256 << 20) // P // 2 // 128 * 128
    print(f"AG default launch, P={P}, M={M} bf16", flush=True)
    dx = si.device_rank_buffers(P, M, "bf16", "normal", seed=P, device=DEV)
    dy = [torch.empty(P * M, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    ccl.check(ccl.ccl_all_gather(dx, dy, P, M, ccl.CCL_BFLOAT16, torch.cuda.current_stream()))
    torch.cuda.synchronize()
    for q in range(P):
        for s in range(P):
            assert torch.equal(dy[q][s * M:(s + 1) * M].view(torch.int16), dx[s].view(torch.int16)), (q, s)
