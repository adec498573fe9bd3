"""Concurrent calls from several host threads, each on its own stream with its
own buffers, sharing one reshard plan whose device table is first built by
all threads at once.  Every kernel is deterministic, so each thread's outputs
must equal, bit for bit, a single-threaded run of the same calls afterwards;
that serial run is anchored to the oracle (all-reduce and reshard).
"""
from __future__ import annotations

import gc
import threading

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from _parity import assert_parity
from collective_communication_plane_amd import ccl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS = 4
ITERS = 8
P, N, M = 4, (1 << 18) + 7, 4099
SHAPE = (64, 384)
SRC = ([1, 4], 0, ["R", ("S", 0)])
DST = ([2, 2], 4, ["R", ("S", 0)])


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def _up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).to(DEV)


class Work:
    """One thread's inputs, outputs and stream."""

    def __init__(self, k: int):
        self.x_ar = si.rank_buffers(P, N, "bf16", "uniform", seed=100 + k)
        self.x_rs = si.rank_buffers(P, P * M, "f32", "normal", seed=200 + k)
        self.x_ag = si.rank_buffers(P, M, "i32", "int20", seed=300 + k)
        g = si.tensor(SHAPE, "bf16", "w002", seed=400 + k)
        self.src_host = np.split(g, 4, axis=0)
        self.d_ar = [_up(x) for x in self.x_ar]
        self.d_rs = [_up(x) for x in self.x_rs]
        self.d_ag = [_up(x) for x in self.x_ag]
        self.d_src = [_up(b) for b in self.src_host]
        self.y_ar = [torch.empty(N * 2, dtype=torch.uint8, device=DEV) for _ in range(P)]
        self.y_rs = [torch.empty(M * 4, dtype=torch.uint8, device=DEV) for _ in range(P)]
        self.y_ag = [torch.empty(P * M * 4, dtype=torch.uint8, device=DEV) for _ in range(P)]
        self.y_dst = [torch.empty(SHAPE[0] // 2 * SHAPE[1] * 2, dtype=torch.uint8, device=DEV)
                      for _ in range(4)]
        self.stream = torch.cuda.Stream()

    def outputs(self):
        return self.y_ar + self.y_rs + self.y_ag + self.y_dst

    def run(self, plan, stream, iters: int):
        for _ in range(iters):
            ccl.check(ccl.ccl_all_reduce(self.d_ar, self.y_ar, P, N, ccl.CCL_BFLOAT16,
                                         ccl.CCL_SUM, stream), "all_reduce")
            ccl.check(ccl.ccl_reduce_scatter(self.d_rs, self.y_rs, P, M, ccl.CCL_FLOAT32,
                                             ccl.CCL_MAX, stream), "reduce_scatter")
            ccl.check(ccl.ccl_all_gather(self.d_ag, self.y_ag, P, M, ccl.CCL_INT32, stream),
                      "all_gather")
            ccl.check(ccl.ccl_reshard_copy(plan, self.d_src, self.y_dst, stream), "reshard")


def test_threads_on_separate_streams_share_a_plan():
    works = [Work(k) for k in range(THREADS)]
    st, plan = ccl.ccl_reshard_plan(ccl.make_tensor_desc(SHAPE, ccl.CCL_BFLOAT16),
                                    ccl.make_mesh(*SRC[:2]), ccl.make_placements(SRC[2]),
                                    ccl.make_mesh(*DST[:2]), ccl.make_placements(DST[2]))
    ccl.check(st, "reshard_plan")
    torch.cuda.synchronize()
    try:
        start = threading.Barrier(THREADS)
        errors = []

        def body(w: Work):
            try:
                start.wait()  # the plan's first use (its table upload) in every thread at once
                w.run(plan, w.stream, ITERS)
                w.stream.synchronize()
            except Exception as e:  # reported after join
                errors.append(e)

        threads = [threading.Thread(target=body, args=(w,)) for w in works]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a thread did not finish"
        assert not errors, errors
        torch.cuda.synchronize()
        got = [[o.clone() for o in w.outputs()] for w in works]

        # the same calls, one thread, one stream, one after another
        for w in works:
            for o in w.outputs():
                o.zero_()
            w.run(plan, torch.cuda.current_stream(), 1)
        torch.cuda.synchronize()
        for k, w in enumerate(works):
            for i, (a, b) in enumerate(zip(got[k], w.outputs())):
                assert torch.equal(a, b), f"thread {k} output {i}"
    finally:
        torch.cuda.synchronize()
        ccl.check(ccl.ccl_plan_destroy(plan))

    # anchor the serial run to the oracle
    for w in works:
        want = oracle.all_reduce(w.x_ar, "bf16", "sum")[0]
        got_ar = w.y_ar[P - 1].cpu().numpy().view(np.uint16)
        assert_parity(got_ar, want, "bf16", "sum", "all-reduce")
        want_dst = oracle.reshard(SHAPE, SRC, DST, w.src_host)
        for l, d in enumerate(w.y_dst):
            np.testing.assert_array_equal(d.cpu().numpy().view(np.uint16), want_dst[l])
