"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library launches only kernels on the caller's stream (a
reshard plan's one-time table upload happens in an eager call first), so a
replay must equal an eager call on the same inputs.  Each replay follows
eager work that rewrites the inputs in place, and is checked on its own.
"""
from __future__ import annotations

import gc

import pytest
import torch

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


def _refill(ts, gen, scale=1.0):
    for t in ts:
        if t.dtype == torch.int32:
            t.copy_(torch.randint(-(2 ** 20), 2 ** 20, t.shape, generator=gen, device=DEV,
                                  dtype=torch.int32))
        else:
            t.copy_(torch.randn(t.shape, generator=gen, device=DEV).mul_(scale).to(t.dtype))


def _check_replays(calls, inputs, outputs, replays=3):
    """calls(stream) enqueues the library calls; inputs are rewritten eagerly
    before every replay, then the replay's outputs are compared with an eager
    run of the same calls on the same inputs."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(0)
    _refill(inputs, gen)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on a side stream, as capture wants
        calls(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):  # capture on the warmed-up stream
        calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for k in range(replays):
        _refill(inputs, gen, scale=1.0 + k)
        for o in outputs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        for o in outputs:
            o.zero_()
        calls(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outputs)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {k} output {i}"
    del g


def test_collectives_in_a_graph():
    P, n, m = 4, 65537, 8195
    x_ar = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    y_ar = [torch.empty_like(t) for t in x_ar]
    y_ar2 = [torch.empty_like(t) for t in x_ar]
    x_rs = [torch.empty(P * m, dtype=torch.float32, device=DEV) for _ in range(P)]
    y_rs = [torch.empty(m, dtype=torch.float32, device=DEV) for _ in range(P)]
    x_ag = [torch.empty(m, dtype=torch.int32, device=DEV) for _ in range(P)]
    y_ag = [torch.empty(P * m, dtype=torch.int32, device=DEV) for _ in range(P)]
    y_red = torch.empty(P * m, dtype=torch.float32, device=DEV)
    y_bc = [torch.empty(m, dtype=torch.int32, device=DEV) for _ in range(P)]
    lds = ccl.LaunchConfig(stages=2, chunk_bytes=4096)

    def calls(stream):
        ccl.check(ccl.ccl_all_reduce(x_ar, y_ar, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM, stream))
        ccl.check(ccl.ccl_all_reduce(x_ar, y_ar2, P, n, ccl.CCL_BFLOAT16, ccl.CCL_MAX, stream,
                                     lds))
        ccl.check(ccl.ccl_reduce_scatter(x_rs, y_rs, P, m, ccl.CCL_FLOAT32, ccl.CCL_SUM, stream))
        ccl.check(ccl.ccl_all_gather(x_ag, y_ag, P, m, ccl.CCL_INT32, stream))
        ccl.check(ccl.ccl_reduce(x_rs, y_red, P, P * m, ccl.CCL_FLOAT32, ccl.CCL_MIN, 1, stream))
        ccl.check(ccl.ccl_broadcast(x_ag[2], y_bc, P, m, ccl.CCL_INT32, 2, stream))

    _check_replays(calls, x_ar + x_rs + x_ag, y_ar + y_ar2 + y_rs + y_ag + [y_red] + y_bc)


def test_fused_and_reshard_calls_in_a_graph():
    P, rows, hidden = 4, 37, 2048
    x = [torch.empty(rows * hidden, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    y = [torch.empty_like(t) for t in x]
    gamma = torch.empty(hidden, dtype=torch.bfloat16, device=DEV)
    shape = (64, 384)
    src = [torch.empty(16 * 384, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    dst = [torch.empty(32 * 384, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    codes = [torch.empty(32 * 384, dtype=torch.uint8, device=DEV) for _ in range(4)]
    scales = [torch.empty(32 * 384 // 128, dtype=torch.float32, device=DEV) for _ in range(4)]
    st, plan = ccl.ccl_reshard_plan(ccl.make_tensor_desc(shape, ccl.CCL_BFLOAT16),
                                    ccl.make_mesh([1, 4], 0), ccl.make_placements(["R", ("S", 0)]),
                                    ccl.make_mesh([2, 2], 4), ccl.make_placements(["R", ("S", 0)]))
    ccl.check(st, "reshard_plan")
    try:
        def calls(stream):
            ccl.check(ccl.ccl_all_reduce_rmsnorm(x, y, P, rows, hidden, gamma, 1e-6,
                                                 ccl.CCL_BFLOAT16, stream))
            ccl.check(ccl.ccl_reshard_copy(plan, src, dst, stream))
            ccl.check(ccl.ccl_reshard_copy_fp8(plan, src, codes, scales, stream))

        _check_replays(calls, x + [gamma] + src, y + dst + codes + scales)
    finally:
        torch.cuda.synchronize()
        ccl.check(ccl.ccl_plan_destroy(plan))


def test_write_through_calls_in_a_graph():
    """Write-through stores (buffer stores with the device-scope bit) replay
    bit-identically from a graph: the all-gather on line-aligned shards by
    default, the split-row RMSNorm, the all-reduce (register-direct at P = 8
    and 2, and the LDS pipeline), reshard copy and FP8 codes by request."""
    P, n, m = 8, 65536, 8192
    wt = ccl.LaunchConfig(store_policy=1)
    wt_lds = ccl.LaunchConfig(store_policy=1, stages=2, chunk_bytes=4096)
    x_ar = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    y_ar = [torch.empty_like(t) for t in x_ar]
    y_lds = [torch.empty_like(t) for t in x_ar]
    x_2 = [torch.empty(n + 3, dtype=torch.float32, device=DEV) for _ in range(2)]
    y_2 = [torch.empty_like(t) for t in x_2]
    x_ag = [torch.empty(m, dtype=torch.float32, device=DEV) for _ in range(P)]
    y_ag = [torch.empty(P * m, dtype=torch.float32, device=DEV) for _ in range(P)]
    rows, hidden = 9, 16384
    x_n = [torch.empty(rows * hidden, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    y_n = [torch.empty_like(t) for t in x_n]
    gamma = torch.empty(hidden, dtype=torch.bfloat16, device=DEV)
    shape = (64, 384)
    src = [torch.empty(16 * 384, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    dst = [torch.empty(32 * 384, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    codes = [torch.empty(32 * 384, dtype=torch.uint8, device=DEV) for _ in range(4)]
    scales = [torch.empty(32 * 384 // 128, dtype=torch.float32, device=DEV) for _ in range(4)]
    st, plan = ccl.ccl_reshard_plan(ccl.make_tensor_desc(shape, ccl.CCL_BFLOAT16),
                                    ccl.make_mesh([1, 4], 0), ccl.make_placements(["R", ("S", 0)]),
                                    ccl.make_mesh([2, 2], 4), ccl.make_placements(["R", ("S", 0)]))
    ccl.check(st, "reshard_plan")
    try:
        def calls(stream):
            ccl.check(ccl.ccl_all_reduce(x_ar, y_ar, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM, stream, wt))
            ccl.check(ccl.ccl_all_reduce(x_ar, y_lds, P, n, ccl.CCL_BFLOAT16, ccl.CCL_MIN, stream,
                                         wt_lds))
            ccl.check(ccl.ccl_all_reduce(x_2, y_2, 2, n + 3, ccl.CCL_FLOAT32, ccl.CCL_SUM, stream, wt))
            ccl.check(ccl.ccl_all_gather(x_ag, y_ag, P, m, ccl.CCL_FLOAT32, stream))
            ccl.check(ccl.ccl_all_reduce_rmsnorm(x_n, y_n, P, rows, hidden, gamma, 1e-6,
                                                 ccl.CCL_BFLOAT16, stream, wt))
            ccl.check(ccl.ccl_reshard_copy(plan, src, dst, stream, wt))
            ccl.check(ccl.ccl_reshard_copy_fp8(plan, src, codes, scales, stream, wt))

        _check_replays(calls, x_ar + x_2 + x_ag + x_n + [gamma] + src,
                       y_ar + y_lds + y_2 + y_ag + y_n + dst + codes + scales)
    finally:
        torch.cuda.synchronize()
        ccl.check(ccl.ccl_plan_destroy(plan))


def test_split_rmsnorm_in_a_graph_and_capture_fallback():
    """The split-row RMSNorm (P = 8, 16 KiB rows: the default form) replays
    bit-identically when captured on a stream that made an eager call first.
    Captured on a fresh stream, which has no partial-sum scratch yet and
    cannot allocate during capture, the call runs the one-pass form instead:
    the replay equals an eager call with stages = 1."""
    P, rows, hidden = 8, 40, 8192
    x = [torch.empty(rows * hidden, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    y = [torch.empty_like(t) for t in x]
    gamma = torch.empty(hidden, dtype=torch.bfloat16, device=DEV)

    def calls(stream):
        ccl.check(ccl.ccl_all_reduce_rmsnorm(x, y, P, rows, hidden, gamma, 1e-6,
                                             ccl.CCL_BFLOAT16, stream))

    _check_replays(calls, x + [gamma], y)

    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    _refill(x + [gamma], gen)
    fresh = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=fresh):
        calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for o in y:
        o.zero_()
    g.replay()
    torch.cuda.synchronize()
    got = [o.clone() for o in y]
    ccl.check(ccl.ccl_all_reduce_rmsnorm(x, y, P, rows, hidden, gamma, 1e-6, ccl.CCL_BFLOAT16,
                                         torch.cuda.current_stream(), ccl.LaunchConfig(stages=1)))
    torch.cuda.synchronize()
    for a, b in zip(got, y):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del g

    # the split form asked for explicitly, with a residency cap: captured on
    # another fresh stream it falls back the same way and keeps the cap
    cfg = ccl.LaunchConfig(chunk_bytes=4096, occupancy=1)
    fresh2 = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=fresh2):
        ccl.check(ccl.ccl_all_reduce_rmsnorm(x, y, P, rows, hidden, gamma, 1e-6,
                                             ccl.CCL_BFLOAT16, torch.cuda.current_stream(), cfg))
    torch.cuda.synchronize()
    for o in y:
        o.zero_()
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(got, y):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del g
