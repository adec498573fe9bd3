"""ccl_all_reduce_rmsnorm_noalloc, the entry point that allocates nothing.

It runs the same kernels as ccl_all_reduce_rmsnorm, with the split-row
form's partial sums in a fixed device array instead of a library-allocated
per-stream buffer, so its outputs must equal that entry point's bit for bit:
checked on two calls in a row, the second with fewer rows (the array keeps
the first call's sums), for the split form and the one-pass form, and
against the oracle on the split form.  Device memory in use must not change
across a first call on a fresh stream (ccl_all_reduce_rmsnorm would allocate
its stream's buffer there).  A call needing more scratch than the array holds
is rejected before anything is launched.
"""
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


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def _both(P, rows, hidden, seed, stream, cfg=None):
    """Run both entry points on the same inputs; returns (noalloc, regular, inputs, gamma)."""
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=seed)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=seed + 1)[0]
    dx = upload_all(xs, DEV)
    dg = DevBuf(gamma.nbytes, DEV).upload(gamma)
    ya = [DevBuf(rows * hidden * 2, DEV) for _ in range(P)]
    yb = [DevBuf(rows * hidden * 2, DEV) for _ in range(P)]
    send = [b.ptr for b in dx]
    torch.cuda.synchronize()
    ccl.check(ccl.ccl_all_reduce_rmsnorm_noalloc(send, [b.ptr for b in ya], P, rows, hidden,
                                                 dg.ptr, 1e-6, ccl.CCL_BFLOAT16, stream, cfg),
              "noalloc")
    ccl.check(ccl.ccl_all_reduce_rmsnorm(send, [b.ptr for b in yb], P, rows, hidden, dg.ptr, 1e-6,
                                         ccl.CCL_BFLOAT16, stream, cfg), "regular")
    torch.cuda.synchronize()
    for b in dx + ya + yb + [dg]:
        assert b.guards_intact()
    return ([b.download(np.uint16) for b in ya], [b.download(np.uint16) for b in yb], xs, gamma)


@pytest.mark.parametrize("P, hidden, cfg", [
    (8, 8192, None),                          # default split form (P >= 6, 16 KiB rows)
    (4, 8192, dict(chunk_bytes=4096)),        # split form by request
    (8, 16384, dict(occupancy=1)),            # split form, 32 KiB rows, one workgroup per CU
    (4, 8192, None),                          # one-pass form (needs no scratch)
])
def test_noalloc_equals_regular_on_two_calls_in_a_row(P, hidden, cfg):
    st = torch.cuda.current_stream()
    c = ccl.LaunchConfig(**cfg) if cfg else None
    for rows, seed in [(300, 1), (37, 2)]:  # the second call is smaller
        print(f"noalloc: P={P} rows={rows} hidden={hidden} cfg={cfg}", flush=True)
        got, ref, xs, gamma = _both(P, rows, hidden, seed, st, c)
        for q in range(P):
            np.testing.assert_array_equal(got[q], ref[q])
        if P == 8:
            want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, 1e-6, "bf16")
            for q in range(P):
                assert_rmsnorm_parity(got[q], want[q], "bf16", hidden, f"noalloc rows={rows}")


def test_noalloc_in_place_and_no_device_allocation():
    P, rows, hidden = 8, 64, 8192
    xs = si.rank_buffers(P, rows * hidden, "bf16", "normal", seed=7)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=8)[0]
    want = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, 1e-6, "bf16")
    dx = upload_all(xs, DEV)
    dg = DevBuf(gamma.nbytes, DEV).upload(gamma)
    fresh = torch.cuda.Stream()
    # load the library's kernels and give the new stream its first launch
    # before measuring, so that only this call sits between the two readings
    y = [DevBuf(rows * hidden * 2, DEV) for _ in range(P)]
    ccl.check(ccl.ccl_all_reduce_rmsnorm_noalloc([b.ptr for b in dx], [b.ptr for b in y], P, rows,
                                                 hidden, dg.ptr, 1e-6, ccl.CCL_BFLOAT16,
                                                 torch.cuda.current_stream()), "warm-up")
    with torch.cuda.stream(fresh):
        torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    ccl.check(ccl.ccl_all_reduce_rmsnorm_noalloc([b.ptr for b in dx], [b.ptr for b in dx], P,
                                                 rows, hidden, dg.ptr, 1e-6, ccl.CCL_BFLOAT16,
                                                 fresh), "noalloc in place")
    fresh.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)
    for q in range(P):
        assert_rmsnorm_parity(dx[q].download(np.uint16), want[q], "bf16", hidden, "in place")


def test_noalloc_rejects_requests_beyond_its_scratch():
    """16 KiB rows take 4 pieces, i.e. 16 bytes of sums per row: 131,072 rows
    fill the 2 MiB array and one more row is refused before any launch (the
    pointers are never dereferenced)."""
    P, hidden = 8, 8192
    base, stride = 1 << 44, 1 << 40
    send = [base + r * stride for r in range(P)]
    recv = [base + (P + r) * stride for r in range(P)]
    gamma = base + 2 * P * stride
    rows = ccl.CCL_NOALLOC_SCRATCH_BYTES // 16 + 1
    st = torch.cuda.current_stream()
    assert ccl.ccl_all_reduce_rmsnorm_noalloc(send, recv, P, rows, hidden, gamma, 1e-6,
                                              ccl.CCL_BFLOAT16, st) == ccl.CCL_ERR_SCRATCH_LIMIT
    assert ccl.ccl_get_error_string(ccl.CCL_ERR_SCRATCH_LIMIT) != "unknown status"
