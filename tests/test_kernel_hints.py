"""The collective kernels' cache hints (register-direct, the LDS pipeline's
loads and stores, and the realigning kernel's stores), read from the gfx950
assembly that hipcc emits for them (code built here, from this repository's
sources).

Each stream of the register-direct kernel is meant to be nontemporal except
one (input 0's loads or output 0's stores, by collective), and a launch that
turns the hints off runs a separate all-plain path.  The compiler is free to
merge a nontemporal access with a plain one on the two sides of a branch,
which silently drops the hint; the kernel source guards against that.  These
tests count the hinted and plain vector accesses of a few instantiations, so
a compiler or source change that moves a hint fails here rather than as an
unexplained bandwidth change.  CPU only: hipcc cross-compiles for gfx950."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "collective_communication_plane_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SLICES = {
    "ar_bf16": ("KIND_AR", "CCL_BFLOAT16"),
    "rs_bf16": ("KIND_RS", "CCL_BFLOAT16"),
    "ag_b16": ("KIND_AG", "CCL_BFLOAT16"),
}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("hints")

    def build(name):
        kind, dt = SLICES[name]
        path = os.path.join(out, name + ".s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               f"-DCCL_INST_KIND={kind}", f"-DCCL_INST_DT={dt}", f"-DCCL_INST_NAME=dispatch_{name}",
               "--cuda-device-only", "-S", "-x", "hip", os.path.join(CSRC, "ccl_coll_inst.hip"),
               "-o", path]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(path) as f:
            return name, f.read()

    with ThreadPoolExecutor(max_workers=3) as ex:
        return dict(ex.map(build, SLICES))


def kernel_body(text: str, kind: int, dt: int, op: int, pmax: int, u: int, wt: bool) -> str:
    sym = (f"_ZN3ccl12_GLOBAL__N_115coll_vec_kernelILi{kind}ELi{dt}ELi{op}ELi{pmax}ELi{u}"
           f"ELb{int(wt)}EEEvNS_8CollArgsE")
    m = re.search(rf"^{re.escape(sym)}:.*?^\s*s_endpgm", text, re.S | re.M)
    assert m, sym
    return m.group(0)


def counts(body: str) -> dict:
    lines = body.splitlines()
    def n(pat):
        return sum(1 for l in lines if re.search(pat, l))
    return {
        "ld_nt": n(r"global_load_dwordx4 .* nt\s*$"),
        "ld_plain": n(r"global_load_dwordx4 .* off\s*$"),
        "st_nt": n(r"global_store_dwordx4 .* nt\s*$"),
        "st_plain": n(r"global_store_dwordx4 .* off\s*$"),
        "st_wt": n(r"buffer_store_dwordx4 .* nt sc1\s*$"),
    }


# (slice, kind, pmax, unroll, write-through) -> expected counts.  The
# nontemporal path holds pmax x u hinted loads (or stores) less the cacheable
# slot-0 stream's; the all-plain path holds pmax x u plain ones, plus the
# slot-0 stream's plain accesses of the nontemporal path (which the compiler
# may share between the two paths: both are plain).
CASES = [
    # all-reduce, nontemporal stores: output 0 cacheable, every load hinted
    ("ar_bf16", 0, 8, 1, False, dict(ld_nt=8, ld_plain=8, st_nt=7, st_plain=9, st_wt=0)),
    # all-reduce with two vectors per lane in flight: input 0 and output 0
    ("ar_bf16", 0, 8, 2, False, dict(ld_nt=14, ld_plain=18, st_nt=14, st_plain=18, st_wt=0)),
    # all-reduce writing through: input 0 cacheable, every store written through
    ("ar_bf16", 0, 4, 1, True, dict(ld_nt=3, ld_plain=5, st_nt=0, st_plain=0, st_wt=4)),
    # reduce-scatter writing through: input 0 cacheable
    ("rs_bf16", 1, 8, 2, True, dict(ld_nt=14, ld_plain=18, st_nt=0, st_plain=0, st_wt=2)),
    ("rs_bf16", 1, 16, 1, False, dict(ld_nt=15, ld_plain=17, st_nt=1, st_plain=1, st_wt=0)),
    # all-gather: the input cacheable (one plain load serves both paths), every
    # store hinted
    ("ag_b16", 2, 8, 1, True, dict(ld_nt=0, ld_plain=1, st_nt=0, st_plain=0, st_wt=8)),
    ("ag_b16", 2, 8, 1, False, dict(ld_nt=0, ld_plain=1, st_nt=8, st_plain=8, st_wt=0)),
]


@pytest.mark.parametrize("slice_, kind, pmax, u, wt, want", CASES)
def test_register_direct_hints(asm, slice_, kind, pmax, u, wt, want):
    got = counts(kernel_body(asm[slice_], kind, 1, 0, pmax, u, wt))
    assert got == want, got


def test_loads_of_a_lane_are_all_in_flight_before_the_fold(asm):
    """No wait for loaded data between the hinted loads of the all-reduce's
    nontemporal path: every rank's vector is requested before the first is
    used."""
    body = kernel_body(asm["ar_bf16"], 0, 1, 0, 8, 1, False)
    lines = [l.strip() for l in body.splitlines()]
    idx = [i for i, l in enumerate(lines) if re.match(r"global_load_dwordx4 .* nt$", l)]
    assert len(idx) == 8
    between = lines[idx[0]:idx[-1]]
    assert not any(l.startswith("s_waitcnt") and "vmcnt" in l for l in between)


# The LDS pipeline and the realigning kernel, P <= 8: (slice, kernel symbol
# stem, nontemporal stores, plain stores, written-through stores, hinted and
# plain direct-to-LDS loads).  LDS pipeline: output 0 cacheable for the
# all-reduce and all-gather (7 hinted stores and one plain, plus the all-plain
# path's 8), the reduce-scatter's one output hinted; its write-through path
# writes every output through.  Its producer issues the rank loads of a tile
# in three forms (all plain, all hinted, and the write-through path's input 0
# plain with the rest hinted), each twice (the pipeline's fill and its steady
# state): 8 + 8 + 8 per form for P = 8, 30 of the 48 hinted.  The
# all-gather's one input gives 2 + 2 + 2, the hinted path's 2 hinted.
# Realigning kernel: every store hinted (its loads go through the cache).
OTHER_CASES = [
    ("ar_bf16", "15coll_lds_kernelILi0ELi1ELi0ELi8ELi2E", 7, 9, 8, 30, 18),
    ("rs_bf16", "15coll_lds_kernelILi1ELi1ELi0ELi8ELi2E", 1, 1, 1, 30, 18),
    ("ag_b16", "15coll_lds_kernelILi2ELi1ELi0ELi8ELi2E", 7, 9, 8, 2, 4),
    ("ar_bf16", "19coll_realign_kernelILi0ELi1ELi0ELi8E", 8, 8, 0, 0, 0),
    ("rs_bf16", "19coll_realign_kernelILi1ELi1ELi0ELi8E", 1, 1, 0, 0, 0),
    ("ag_b16", "19coll_realign_kernelILi2ELi1ELi0ELi8E", 8, 8, 0, 0, 0),
]


@pytest.mark.parametrize("slice_, stem, st_nt, st_plain, st_wt, lds_nt, lds_plain", OTHER_CASES)
def test_lds_and_realign_hints(asm, slice_, stem, st_nt, st_plain, st_wt, lds_nt, lds_plain):
    sym = f"_ZN3ccl12_GLOBAL__N_1{stem}EEvNS_8CollArgsE"
    m = re.search(rf"^{re.escape(sym)}:.*?^\s*s_endpgm", asm[slice_], re.S | re.M)
    assert m, sym
    body = m.group(0)
    got = counts(body)
    lines = body.splitlines()
    got_lds_nt = sum(1 for l in lines if re.search(r"global_load_lds_dwordx4 .* nt\s*$", l))
    got_lds_plain = sum(1 for l in lines if re.search(r"global_load_lds_dwordx4 .* off\s*$", l))
    assert (got["st_nt"], got["st_plain"], got["st_wt"], got_lds_nt, got_lds_plain) == \
        (st_nt, st_plain, st_wt, lds_nt, lds_plain), (got, got_lds_nt, got_lds_plain)
