"""GPU parity with rank buffers past 4 GiB, where 32-bit element or byte
offsets would wrap (MI355X holds 288 GB, so such buffers are ordinary).

Inputs are drawn on the GPU with PyTorch's seeded generator; only sampled
values come back.  Sampled outputs are checked against the oracle applied to
the gathered inputs (the operations are element-wise, or row-wise for the
fused RMSNorm), the reshard against its copy property.  Every sample set
includes the indices around 2^31 elements (4 GiB of bf16) and the tail.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from _parity import assert_parity, assert_rmsnorm_parity
from collective_communication_plane_amd import ccl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TWO31 = 1 << 31


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def samples(n: int, k: int = 100_000, seed: int = 3) -> np.ndarray:
    """Random indices plus the ones next to 2^31 and 2^32 and the ends."""
    extra = [0, 1, n // 2, n - 2, n - 1]
    for b in (TWO31, 2 * TWO31):
        extra += [b - 2, b - 1, b, b + 1, b + 7, b + 8]
    extra = [e for e in extra if 0 <= e < n]
    idx = np.concatenate([si.sample_indices(n, k, seed).astype(np.int64), np.array(extra)])
    return np.unique(idx)


def gather(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of a device buffer at the given element indices."""
    it = torch.from_numpy(idx).to(DEV)
    return t.view(torch.int16)[it].cpu().numpy().view(np.uint16)


def test_all_reduce_past_4gib_per_rank():
    P, n = 2, TWO31 + 4099  # 4 GiB + 8 KiB of bf16 per rank
    dx = si.device_rank_buffers(P, n, "bf16", "uniform", seed=0, device=DEV)
    idx = samples(n)
    xin = [gather(t, idx) for t in dx]
    want = oracle.all_reduce(xin, "bf16", "sum")[0]
    for cfg in (None, ccl.LaunchConfig(stages=2, chunk_bytes=8192)):
        dy = [torch.empty_like(t) for t in dx]
        ccl.check(ccl.ccl_all_reduce(dx, dy, P, n, ccl.CCL_BFLOAT16, ccl.CCL_SUM,
                                     torch.cuda.current_stream(), cfg), "all_reduce")
        torch.cuda.synchronize()
        assert torch.equal(dy[0], dy[1])
        assert_parity(gather(dy[0], idx), want, "bf16", "sum", f"AR n={n} cfg={cfg}")
        del dy


def test_reduce_scatter_past_4gib_shards():
    # shards of 2^31 + 5 bf16: the second one starts 4 GiB + 10 B into each
    # input, at another offset mod 16 than its output (the realigning kernel)
    P, M = 2, TWO31 + 5
    dx = si.device_rank_buffers(P, P * M, "bf16", "normal", seed=1, device=DEV)
    dy = [torch.empty(M, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    ccl.check(ccl.ccl_reduce_scatter(dx, dy, P, M, ccl.CCL_BFLOAT16, ccl.CCL_SUM,
                                     torch.cuda.current_stream()), "reduce_scatter")
    torch.cuda.synchronize()
    idx = samples(M)
    for s in range(P):
        xin = [gather(t, idx + s * M) for t in dx]
        want = oracle.all_reduce(xin, "bf16", "sum")[0]
        assert_parity(gather(dy[s], idx), want, "bf16", "sum", f"RS shard {s}")


def test_all_gather_past_4gib_outputs():
    P, M = 2, TWO31 + 3
    dx = si.device_rank_buffers(P, M, "bf16", "normal", seed=2, device=DEV)
    dy = [torch.empty(P * M, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    ccl.check(ccl.ccl_all_gather(dx, dy, P, M, ccl.CCL_BFLOAT16, torch.cuda.current_stream()),
              "all_gather")
    torch.cuda.synchronize()
    idx = samples(M)
    for r in range(P):
        want = gather(dx[r], idx)
        for q in range(P):
            np.testing.assert_array_equal(gather(dy[q], idx + r * M), want)


def test_reshard_gather_past_4gib():
    # [2, 2^31 + 64] bf16: Shard(0) over 2 ranks -> Replicate on 1 rank; the
    # second source row lands 4 GiB + 128 B into the destination
    L = TWO31 + 64
    shape = (2, L)
    src = ([2], 0, [("S", 0)])
    dst = ([1], 2, ["R"])
    dx = si.device_rank_buffers(2, L, "bf16", "normal", seed=4, device=DEV)
    dy = torch.empty(2 * L, dtype=torch.bfloat16, device=DEV)
    st, plan = ccl.ccl_reshard_plan(ccl.make_tensor_desc(shape, ccl.CCL_BFLOAT16),
                                    ccl.make_mesh(*src[:2]), ccl.make_placements(src[2]),
                                    ccl.make_mesh(*dst[:2]), ccl.make_placements(dst[2]))
    ccl.check(st, "reshard_plan")
    try:
        ccl.check(ccl.ccl_reshard_copy(plan, dx, [dy], torch.cuda.current_stream()),
                  "reshard_copy")
        torch.cuda.synchronize()
    finally:
        ccl.check(ccl.ccl_plan_destroy(plan))
    idx = samples(L)
    for r in range(2):
        np.testing.assert_array_equal(gather(dy, idx + r * L), gather(dx[r], idx))


def test_all_reduce_rmsnorm_past_4gib_per_rank():
    P, hidden = 2, 8192
    rows = TWO31 // hidden + 3  # 4 GiB + 48 KiB of bf16 per rank
    n = rows * hidden
    dx = si.device_rank_buffers(P, n, "bf16", "normal", seed=5, device=DEV)
    gamma = si.rank_buffers(1, hidden, "bf16", "uniform", seed=6)[0]
    dg = torch.from_numpy(gamma.view(np.int16).copy()).to(DEV)
    dy = [torch.empty_like(t) for t in dx]
    ccl.check(ccl.ccl_all_reduce_rmsnorm(dx, dy, P, rows, hidden, dg, 1e-6, ccl.CCL_BFLOAT16,
                                         torch.cuda.current_stream()), "all_reduce_rmsnorm")
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([si.sample_indices(rows, 40, seed=7).astype(np.int64),
                                     [TWO31 // hidden - 1, TWO31 // hidden, rows - 1]]))
    idx = (pick[:, None] * hidden + np.arange(hidden)[None, :]).ravel()
    xin = [gather(t, idx) for t in dx]
    want = oracle.all_reduce_rmsnorm(xin, pick.size, hidden, gamma, 1e-6, "bf16")
    for q in range(P):
        assert_rmsnorm_parity(gather(dy[q], idx), want[q], "bf16", hidden, f"rank {q}")


@pytest.mark.parametrize("P", [7, 8, 12])
def test_reduce_scatter_and_reduce_launch_forms_around_160mib(P):
    """Reduce-scatter and reduce at P = 7, 8, 12 on both sides of 160 MiB per
    rank, where the LDS pipeline once took over from the register-direct
    kernel.  These torch tensors start on 256 bytes, so the default launch is
    register-direct with write-through stores at P <= 8.  It, the LDS pipeline
    forced with stages = 2 (writing through as the default would) and
    nontemporal-only stores (store_policy = 2) must all give the oracle's
    values (sum, sampled) and equal one another."""
    TORCH = {"bf16": torch.int16, "f32": torch.int32}
    for dtype, per_rank_mib in (("bf16", 144), ("bf16", 176), ("f32", 168)):
        esz = 2 if dtype == "bf16" else 4
        # shard lengths of whole 16-byte vectors keep every shard aligned, so
        # the aligned kernels (not the realigning one) run on both sides
        M = (per_rank_mib << 20) // esz // P // 8 * 8 + 8
        assert (P * M * esz > (160 << 20)) == (per_rank_mib > 160)
        dx = si.device_rank_buffers(P, P * M, dtype, "normal", seed=P, device=DEV)
        dy = [torch.empty(M, dtype=dx[0].dtype, device=DEV) for _ in range(P)]
        code = ccl.CCL_BFLOAT16 if dtype == "bf16" else ccl.CCL_FLOAT32
        ccl.check(ccl.ccl_reduce_scatter(dx, dy, P, M, code, ccl.CCL_SUM,
                                         torch.cuda.current_stream()), "reduce_scatter")
        forced = {}
        for name, cfg in (("lds", ccl.LaunchConfig(stages=2, chunk_bytes=8192)),
                          ("nt", ccl.LaunchConfig(store_policy=2))):
            forced[name] = [torch.empty(M, dtype=dx[0].dtype, device=DEV) for _ in range(P)]
            ccl.check(ccl.ccl_reduce_scatter(dx, forced[name], P, M, code, ccl.CCL_SUM,
                                             torch.cuda.current_stream(), cfg), "reduce_scatter")
        red = torch.empty(P * M, dtype=dx[0].dtype, device=DEV)
        ccl.check(ccl.ccl_reduce(dx, red, P, P * M, code, ccl.CCL_SUM, P - 1,
                                 torch.cuda.current_stream()), "reduce")
        torch.cuda.synchronize()
        idx = samples(M, k=20_000, seed=P)
        npdt = np.uint16 if dtype == "bf16" else np.uint32

        def at(t, i):
            it = torch.from_numpy(i).to(DEV)
            return t.view(TORCH[dtype])[it].cpu().numpy().view(npdt)

        for s in (0, P // 2, P - 1):
            xin = [at(t, idx + s * M) for t in dx]
            if dtype == "f32":
                xin = [x.view(np.float32) for x in xin]
            want = oracle.all_reduce(xin, dtype, "sum")[0]
            got = at(dy[s], idx)
            got_red = at(red, idx + s * M)
            if dtype == "f32":
                got, got_red = got.view(np.float32), got_red.view(np.float32)
            assert_parity(got, want, dtype, "sum", f"RS P={P} {dtype} {per_rank_mib} MiB shard {s}")
            assert_parity(got_red, want, dtype, "sum", f"reduce P={P} {dtype} {per_rank_mib} MiB")
            for name, ys in forced.items():
                assert torch.equal(ys[s], dy[s]), f"RS {name} P={P} {dtype} shard {s}"
        del dx, dy, red, forced
        torch.cuda.empty_cache()
