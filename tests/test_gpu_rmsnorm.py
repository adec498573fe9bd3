"""GPU parity of the all-reduce with RMSNorm fused between its halves."""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from _parity import DevBuf, assert_rmsnorm_parity, upload_all
from collective_communication_plane_amd import ccl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NP = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}
ESZ = {"f32": 4, "bf16": 2, "f16": 2}


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def run(xs, rows, hidden, gamma, eps, dtype, in_place=False, cfg=None):
    P = len(xs)
    dx = upload_all(xs, DEV)
    dg = DevBuf(gamma.nbytes, DEV).upload(gamma)
    dy = dx if in_place else [DevBuf(rows * hidden * ESZ[dtype], DEV) for _ in range(P)]
    ccl.check(ccl.ccl_all_reduce_rmsnorm([b.ptr for b in dx], [b.ptr for b in dy], P, rows,
                                         hidden, dg.ptr, eps, ccl.DTYPES[dtype],
                                         torch.cuda.current_stream(), cfg), "ar_rmsnorm")
    torch.cuda.synchronize()
    for b in dx + dy + [dg]:
        assert b.guards_intact()
    return [b.download(NP[dtype]) for b in dy]


@pytest.mark.parametrize("stages", [1, 2])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("hidden", [64, 1024, 7168, 8192])
def test_matches_oracle(P, dtype, hidden, stages):
    if dtype == "f32" and hidden > 8192:
        pytest.skip("fp32 rows are limited to 8192 elements")
    rows, eps = 19, 1e-6
    xs = si.rank_buffers(P, rows * hidden, dtype, "normal", seed=P + hidden)
    gamma = si.rank_buffers(1, hidden, dtype, "uniform", seed=7)[0]
    # stages=2 on a grid of 5 workgroups: every workgroup pipelines 3-4 rows
    cfg = ccl.LaunchConfig(stages=2, workgroups=5) if stages == 2 else ccl.LaunchConfig(stages=1)
    got = run(xs, rows, hidden, gamma, eps, dtype, cfg=cfg)
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, eps, dtype)
    for q in range(P):
        assert_rmsnorm_parity(got[q], want[q], dtype, hidden, f"P={P} {dtype} H={hidden}")
        np.testing.assert_array_equal(got[q], got[0])


@pytest.mark.parametrize("cfg", [None, dict(stages=1), dict(stages=2, workgroups=2)])
def test_bf16_hidden_16384_and_in_place(cfg):
    P, rows, hidden = 4, 9, 16384
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=3)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=4)[0]
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, 1e-5, "bf16")
    got = run(xs, rows, hidden, gamma, 1e-5, "bf16", in_place=True,
              cfg=ccl.LaunchConfig(**cfg) if cfg else None)
    for q in range(P):
        assert_rmsnorm_parity(got[q], want[q], "bf16", hidden, "in place")


@pytest.mark.parametrize("cfg", [dict(workgroups=1), dict(workgroups=7), dict(occupancy=1),
                                 dict(occupancy=32), dict(nontemporal=1), dict(nontemporal=2),
                                 dict(nontemporal=4), dict(stages=1), dict(stages=2),
                                 dict(stages=2, workgroups=1), dict(stages=2, workgroups=39),
                                 dict(stages=2, workgroups=40), dict(stages=2, workgroups=41),
                                 dict(stages=2, occupancy=1), dict(stages=2, occupancy=3),
                                 dict(stages=2, nontemporal=4), dict(store_policy=1),
                                 dict(store_policy=2), dict(stages=2, store_policy=2),
                                 dict(stages=2, store_policy=1, nontemporal=2)])
def test_launch_config_does_not_change_results(cfg):
    P, rows, hidden = 8, 40, 4096
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=9)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=10)[0]
    base = run(xs, rows, hidden, gamma, 1e-6, "bf16")
    got = run(xs, rows, hidden, gamma, 1e-6, "bf16", cfg=ccl.LaunchConfig(**cfg))
    for q in range(P):
        np.testing.assert_array_equal(got[q], base[q])


def test_rejections():
    P, rows, hidden = 2, 4, 64
    bufs = [DevBuf(rows * hidden * 2, DEV) for _ in range(2 * P)]
    g = DevBuf(hidden * 2, DEV)
    send, recv = [b.ptr for b in bufs[:P]], [b.ptr for b in bufs[P:]]
    st = torch.cuda.current_stream()
    assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, rows, 60, g.ptr, 1e-6, ccl.CCL_BFLOAT16,
                                      st) == ccl.CCL_ERR_UNSUPPORTED  # 120-byte rows
    assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, rows, 32768, g.ptr, 1e-6, ccl.CCL_BFLOAT16,
                                      st) == ccl.CCL_ERR_UNSUPPORTED  # row too long
    assert ccl.ccl_all_reduce_rmsnorm([send[0] + 2, send[1]], recv, P, rows, hidden, g.ptr, 1e-6,
                                      ccl.CCL_BFLOAT16, st) == ccl.CCL_ERR_UNSUPPORTED
    assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, rows, hidden, g.ptr, -1.0, ccl.CCL_BFLOAT16,
                                      st) == ccl.CCL_ERR_INVALID_ARG
    assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, rows, hidden, g.ptr, 1e-6, ccl.CCL_INT32,
                                      st) == ccl.CCL_ERR_INVALID_ARG
    assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, rows, hidden, g.ptr, 1e-6, ccl.CCL_BFLOAT16,
                                      st, ccl.LaunchConfig(stages=3)) == ccl.CCL_ERR_UNSUPPORTED
    assert ccl.ccl_all_reduce_rmsnorm(send, [recv[0], recv[0] + 16], P, rows, hidden, g.ptr, 1e-6,
                                      ccl.CCL_BFLOAT16, st) == ccl.CCL_ERR_ALIASING
    torch.cuda.synchronize()
    for b in bufs[P:]:
        assert (b.base == b.fill).all().item()


@pytest.mark.parametrize("stages", [1, 2, "split", "default"])
def test_full_size_sampled_rows(stages):
    """P=8, 16384 tokens x 8192 hidden bf16 (256 MiB per rank): exact replica
    identity on the GPU and sampled rows against the oracle, one workgroup per
    row, row-pipelined, and split into 4 KiB pieces."""
    P, rows, hidden = 8, 16384, 8192
    dx = si.device_rank_buffers(P, rows * hidden, "bf16", "normal", seed=0, device=DEV)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=1)[0]
    dg = torch.from_numpy(gamma.view(np.int16).copy()).to(DEV)
    dy = [torch.empty_like(t) for t in dx]
    ccl.check(ccl.ccl_all_reduce_rmsnorm(dx, dy, P, rows, hidden, dg, 1e-6, ccl.CCL_BFLOAT16,
                                         torch.cuda.current_stream(),
                                         None if stages == "default"
                                         else ccl.LaunchConfig(chunk_bytes=4096) if stages == "split"
                                         else ccl.LaunchConfig(stages=stages)))
    torch.cuda.synchronize()
    for q in range(1, P):
        assert torch.equal(dy[q].view(torch.int16), dy[0].view(torch.int16))
    sample = si.sample_indices(rows, 64, seed=2).astype(np.int64)
    xs = [t.view(rows, hidden)[torch.from_numpy(sample).to(DEV)].view(torch.int16).cpu().numpy()
          .view(np.uint16).ravel() for t in dx]
    want = oracle.all_reduce_rmsnorm(xs, sample.size, hidden, gamma, 1e-6, "bf16")[0]
    got = dy[0].view(rows, hidden)[torch.from_numpy(sample).to(DEV)].view(torch.int16).cpu().numpy()
    assert_rmsnorm_parity(got.view(np.uint16).ravel(), want, "bf16", hidden, "full size")


# ------------------------------------------------------------ split rows
# chunk_bytes = 4096 cuts every row into 4 KiB pieces (one vector per lane):
# a fold pass (one workgroup per piece) parks the folded row in the first
# output and writes per-piece sums of squares, a norm pass scales and stores.

SPLIT = dict(chunk_bytes=4096)


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 9, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("row_bytes", [4112, 8192, 12304, 16384, 20496, 32768])
def test_split_rows_match_oracle(P, dtype, row_bytes):
    """Rows of 2..8 pieces, the last one full or holding a single vector."""
    hidden = row_bytes // ESZ[dtype]
    rows, eps = 37, 1e-6
    xs = si.rank_buffers(P, rows * hidden, dtype, "normal", seed=P + row_bytes)
    gamma = si.rank_buffers(1, hidden, dtype, "uniform", seed=8)[0]
    print(f"split: P={P} {dtype} hidden={hidden}", flush=True)
    got = run(xs, rows, hidden, gamma, eps, dtype, cfg=ccl.LaunchConfig(**SPLIT))
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, eps, dtype)
    for q in range(P):
        assert_rmsnorm_parity(got[q], want[q], dtype, hidden, f"split P={P} {dtype} H={hidden}")
        np.testing.assert_array_equal(got[q], got[0])


@pytest.mark.parametrize("cfg", [dict(), dict(occupancy=1), dict(occupancy=2), dict(nontemporal=4),
                                 dict(store_policy=1), dict(nontemporal=1), dict(workgroups=3)])
def test_split_launch_fields_do_not_change_results(cfg):
    """Residency caps (both passes) and the cache hints leave the split
    kernels' bits unchanged."""
    P, rows, hidden = 8, 300, 16384
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=12)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=13)[0]
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, 1e-6, "bf16")
    base = run(xs, rows, hidden, gamma, 1e-6, "bf16", cfg=ccl.LaunchConfig(**SPLIT))
    got = run(xs, rows, hidden, gamma, 1e-6, "bf16", cfg=ccl.LaunchConfig(**SPLIT, **cfg))
    for q in range(P):
        assert_rmsnorm_parity(base[q], want[q], "bf16", hidden, "split base")
        np.testing.assert_array_equal(got[q], base[q])


def test_split_in_place_repeated_calls_and_streams():
    """In place; then calls back to back with new inputs, alternating between
    the current stream and a second one (each stream has its own partial-sum
    scratch)."""
    P, rows, hidden = 4, 65, 8192
    st = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=21)[0]
    dg = DevBuf(gamma.nbytes, DEV).upload(gamma)
    cfg = ccl.LaunchConfig(**SPLIT)
    # in place
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=20)
    got = run(xs, rows, hidden, gamma, 1e-6, "bf16", in_place=True, cfg=cfg)
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, 1e-6, "bf16")
    for q in range(P):
        assert_rmsnorm_parity(got[q], want[q], "bf16", hidden, "split in place")
    # five calls queued back to back, alternating streams, then checked
    sets = [si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=30 + k) for k in range(5)]
    dxs = [upload_all(x, DEV) for x in sets]
    dys = [[DevBuf(rows * hidden * 2, DEV) for _ in range(P)] for _ in sets]
    torch.cuda.synchronize()
    for k, (dx, dy) in enumerate(zip(dxs, dys)):
        s = side if k % 2 else st
        ccl.check(ccl.ccl_all_reduce_rmsnorm([b.ptr for b in dx], [b.ptr for b in dy], P, rows,
                                             hidden, dg.ptr, 1e-6, ccl.CCL_BFLOAT16, s, cfg))
    torch.cuda.synchronize()
    for k, (x, dy) in enumerate(zip(sets, dys)):
        want = oracle.all_reduce_rmsnorm(x, rows, hidden, gamma, 1e-6, "bf16")
        for q in range(P):
            assert_rmsnorm_parity(dy[q].download(np.uint16), want[q], "bf16", hidden, f"call {k}")


def test_split_many_pieces_in_flight():
    """200,000 rows of 2 pieces (400,000 workgroups) in one call."""
    P, rows, hidden = 2, 200_000, 4096
    dx = si.device_rank_buffers(P, rows * hidden, "bf16", "normal", seed=5, device=DEV)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=6)[0]
    dg = torch.from_numpy(gamma.view(np.int16).copy()).to(DEV)
    dy = [torch.empty_like(t) for t in dx]
    ccl.check(ccl.ccl_all_reduce_rmsnorm(dx, dy, P, rows, hidden, dg, 1e-6, ccl.CCL_BFLOAT16,
                                         torch.cuda.current_stream(), ccl.LaunchConfig(**SPLIT)))
    torch.cuda.synchronize()
    assert torch.equal(dy[1].view(torch.int16), dy[0].view(torch.int16))
    sample = si.sample_indices(rows, 96, seed=3).astype(np.int64)
    it = torch.from_numpy(sample).to(DEV)
    xs = [t.view(rows, hidden)[it].view(torch.int16).cpu().numpy().view(np.uint16).ravel()
          for t in dx]
    want = oracle.all_reduce_rmsnorm(xs, sample.size, hidden, gamma, 1e-6, "bf16")[0]
    got = dy[0].view(rows, hidden)[it].view(torch.int16).cpu().numpy().view(np.uint16).ravel()
    assert_rmsnorm_parity(got, want, "bf16", hidden, "many pieces")


def test_split_rejections():
    P, rows, hidden = 2, 4, 4096
    bufs = [DevBuf(rows * hidden * 2, DEV) for _ in range(2 * P)]
    g = DevBuf(hidden * 2, DEV)
    send, recv = [b.ptr for b in bufs[:P]], [b.ptr for b in bufs[P:]]
    st = torch.cuda.current_stream()
    for cfg in (dict(chunk_bytes=2048), dict(chunk_bytes=4096, stages=2)):
        assert ccl.ccl_all_reduce_rmsnorm(send, recv, P, rows, hidden, g.ptr, 1e-6,
                                          ccl.CCL_BFLOAT16, st,
                                          ccl.LaunchConfig(**cfg)) == ccl.CCL_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    for b in bufs[P:]:
        assert (b.base == b.fill).all().item()


def test_default_split_writes_through_past_256mib_per_rank():
    """P = 8 x 24576 x 8192 bf16 (384 MiB per rank): the default split form
    writes through in its norm pass; the outputs equal the nontemporal-only
    launch's bit for bit and the oracle on sampled rows."""
    P, rows, hidden = 8, 24576, 8192
    dx = si.device_rank_buffers(P, rows * hidden, "bf16", "normal", seed=4, device=DEV)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=5)[0]
    dg = torch.from_numpy(gamma.view(np.int16).copy()).to(DEV)
    st = torch.cuda.current_stream()
    dy = [torch.empty_like(t) for t in dx]
    ccl.check(ccl.ccl_all_reduce_rmsnorm(dx, dy, P, rows, hidden, dg, 1e-6, ccl.CCL_BFLOAT16, st))
    dz = [torch.empty_like(t) for t in dx]
    ccl.check(ccl.ccl_all_reduce_rmsnorm(dx, dz, P, rows, hidden, dg, 1e-6, ccl.CCL_BFLOAT16, st,
                                         ccl.LaunchConfig(chunk_bytes=4096, store_policy=2)))
    torch.cuda.synchronize()
    for q in range(P):
        assert torch.equal(dy[q].view(torch.int16), dz[q].view(torch.int16)), q
        assert torch.equal(dy[q].view(torch.int16), dy[0].view(torch.int16)), q
    del dz
    sample = si.sample_indices(rows, 64, seed=9).astype(np.int64)
    it = torch.from_numpy(sample).to(DEV)
    xs = [t.view(rows, hidden)[it].view(torch.int16).cpu().numpy().view(np.uint16).ravel()
          for t in dx]
    want = oracle.all_reduce_rmsnorm(xs, sample.size, hidden, gamma, 1e-6, "bf16")[0]
    got = dy[0].view(rows, hidden)[it].view(torch.int16).cpu().numpy().view(np.uint16).ravel()
    assert_rmsnorm_parity(got, want, "bf16", hidden, "default split, write-through")


@pytest.mark.parametrize("P, hidden, split", [(8, 4096, True), (6, 8192, False), (4, 16384, False),
                                              (12, 8192, True), (6, 12288, False)])
def test_default_form_by_rank_count_and_row_length(P, hidden, split):
    """The default launch picks the split-row form at P >= 8 for rows of at
    least 8 KiB and a one-pass form otherwise: its bits equal those of the
    explicitly requested form (the two forms add the sum of squares in
    different orders), and the oracle's within the bar."""
    rows = 23
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=P + hidden)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=3)[0]
    got = run(xs, rows, hidden, gamma, 1e-6, "bf16")
    one_pass = ccl.LaunchConfig(stages=2 if hidden * 2 > 16384 and P >= 6 else 1)
    ref = run(xs, rows, hidden, gamma, 1e-6, "bf16",
              cfg=ccl.LaunchConfig(chunk_bytes=4096) if split else one_pass)
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, 1e-6, "bf16")
    for q in range(P):
        np.testing.assert_array_equal(got[q], ref[q])
        assert_rmsnorm_parity(got[q], want[q], "bf16", hidden, f"default P={P} H={hidden}")
