"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test ties an oracle function to something other than the oracle itself:
independent numpy / PyTorch library routines, closed forms, the textbook
error bound of recursive summation, invariants the pages state (all-reduce =
reduce-scatter then all-gather; every replica identical), and the worked
examples of the M2N/T-CCL digest (lqnn.cn news 207677) s1.4 kept under
tests/golden/.
"""
from __future__ import annotations

import itertools
import struct

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from _golden import load_example
from _layout import chunk_piece, local_blocks

PS = [1, 2, 3, 4, 8]


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u))[0]


# ------------------------------------------------------------- bf16 rounding

@pytest.mark.parametrize(
    "f32_pattern, bf16_pattern",
    [
        (0x3F800000, 0x3F80),  # 1.0 exact
        (0x3F808000, 0x3F80),  # halfway, even below -> stays
        (0x3F818000, 0x3F82),  # halfway, odd below -> rounds up to even
        (0x3F808001, 0x3F81),  # just above halfway -> up
        (0x3F807FFF, 0x3F80),  # just below halfway -> down
        (0xBF818000, 0xBF82),  # negative halfway, odd -> away from zero to even
        (0x7F7FFFFF, 0x7F80),  # largest finite fp32 rounds to +inf
        (0x7F800000, 0x7F80),  # +inf
        (0xFF800000, 0xFF80),  # -inf
        (0x00000001, 0x0000),  # smallest denormal rounds to +0
        (0x00008000, 0x0000),  # denormal halfway, even -> 0
        (0x00018000, 0x0002),  # denormal halfway, odd -> up
        (0x80000000, 0x8000),  # -0 keeps its sign
        (0x7FC00001, 0x7FC0),  # NaN -> canonical quiet NaN
    ],
)
def test_bf16_rne_hand_worked(f32_pattern, bf16_pattern):
    assert oracle.narrow_bf16(bits_f32(f32_pattern)) == bf16_pattern


def test_bf16_narrow_matches_torch_rne():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    want = si.to_bf16_bits(x)
    got = np.array([oracle.narrow_bf16(float(v)) for v in x[:20000]], np.uint16)
    np.testing.assert_array_equal(got, want[:20000])


def test_bf16_widen_is_exact():
    h = np.arange(0, 2**16, 257, dtype=np.uint16)
    h = h[~np.isnan(si.bf16_bits_to_f32(h))]
    want = si.bf16_bits_to_f32(h)
    got = np.array([oracle.widen_bf16(int(v)) for v in h], np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


# -------------------------------------------------------------- reductions

def seq_sum_f32(xs):
    """Independent fp32 reference: numpy elementwise IEEE adds in rank order."""
    acc = xs[0].astype(np.float32).copy()
    for x in xs[1:]:
        acc = np.add(acc, x.astype(np.float32), dtype=np.float32)
    return acc


@pytest.mark.parametrize("P", PS)
@pytest.mark.parametrize("n", [0, 1, 37, 4099])
@pytest.mark.parametrize("dist", ["uniform", "normal"])
def test_allreduce_f32_sum_equals_sequential_numpy(P, n, dist):
    """Bit-equal to numpy's adds in rank order.  The normal draws carry full
    24-bit mantissas, so a fold in another order changes bits from P = 3 on
    (the uniform draws' sums of a few ranks are exact in any order)."""
    xs = si.rank_buffers(P, n, "f32", dist, seed=P * 100 + n)
    ys = oracle.all_reduce(xs, "f32", "sum")
    want = seq_sum_f32(xs)
    for y in ys:
        np.testing.assert_array_equal(y.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("P", PS)
def test_allreduce_bf16_sum_equals_fp32_fold_then_torch_rne(P):
    xs = si.rank_buffers(P, 5000, "bf16", "normal", seed=P)
    ys = oracle.all_reduce(xs, "bf16", "sum")
    want = si.to_bf16_bits(seq_sum_f32([si.bf16_bits_to_f32(x) for x in xs]))
    for y in ys:
        np.testing.assert_array_equal(y, want)


@pytest.mark.parametrize("P", PS)
def test_allreduce_i32_sum_exact_and_wrapping(P):
    rng = np.random.default_rng(P)
    xs = si.rank_buffers(P, 3001, "i32", "int20", seed=P)
    # plus a block of huge values that must wrap in two's complement
    big = rng.integers(-(2**31), 2**31, size=(P, 64), dtype=np.int64).astype(np.int32)
    xs = [np.concatenate([x, b]) for x, b in zip(xs, big)]
    ys = oracle.all_reduce(xs, "i32", "sum")
    want = (np.sum(np.stack(xs).astype(np.int64), axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    for y in ys:
        np.testing.assert_array_equal(y, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("op", ["min", "max"])
@pytest.mark.parametrize("P", PS)
def test_allreduce_minmax_equals_numpy_reduce(dtype, op, P):
    dist = "int20" if dtype == "i32" else "uniform"
    xs = si.rank_buffers(P, 2049, dtype, dist, seed=11 * P)
    ys = oracle.all_reduce(xs, dtype, op)
    fn = np.minimum if op == "min" else np.maximum
    if dtype == "bf16":
        want = si.to_bf16_bits(fn.reduce([si.bf16_bits_to_f32(x) for x in xs]))
    else:
        want = fn.reduce(xs)
    for y in ys:
        np.testing.assert_array_equal(y, want)


def test_minmax_ties_keep_earlier_rank_signed_zero():
    pz, nz = np.float32(0.0), np.float32(-0.0)
    for op in ("min", "max"):
        y = oracle.all_reduce([np.array([pz, nz]), np.array([nz, pz])], "f32", op)[0]
        # rank 0's zero survives in both columns
        assert y.view(np.uint32).tolist() == [0x00000000, 0x80000000]


@pytest.mark.parametrize("P", [2, 3, 5, 8])
def test_fp32_fold_within_recursive_summation_bound(P):
    """|fl(sum) - sum| <= gamma_{P-1} * sum|x| (recursive summation, u = 2^-24)."""
    xs = si.rank_buffers(P, 20000, "f32", "normal", seed=3 * P)
    got = oracle.all_reduce(xs, "f32", "sum")[0].astype(np.float64)
    X = np.stack(xs).astype(np.float64)
    exact = np.sum(X, axis=0)
    u = 2.0 ** -24
    gamma = (P - 1) * u / (1 - (P - 1) * u)
    bound = gamma * np.sum(np.abs(X), axis=0)
    assert np.all(np.abs(got - exact) <= bound)
    # and a dropped term would be far outside it
    assert np.any(np.abs(got - (exact - X[-1])) > bound)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_equal_inputs_sum_to_P_times_x(P, dtype):
    """With 8-bit significands every partial sum r*x (r <= 8) is exact in fp32,
    so the fold of P equal buffers is exactly P*x; bf16 output of a power-of-two
    P is exact too."""
    h = si.rank_buffers(1, 1000, "bf16", "uniform", seed=5)[0]
    x = si.bf16_bits_to_f32(h)
    if dtype == "f32":
        y = oracle.all_reduce([x] * P, "f32", "sum")[0]
        np.testing.assert_array_equal(y, x * np.float32(P))
    else:
        y = oracle.all_reduce([h] * P, "bf16", "sum")[0]
        np.testing.assert_array_equal(y, si.to_bf16_bits(x * np.float32(P)))
        if P & (P - 1) == 0:
            np.testing.assert_array_equal(si.bf16_bits_to_f32(y), x * np.float32(P))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
def test_single_rank_is_identity(dtype):
    dist = "int20" if dtype == "i32" else "normal"
    x = si.rank_buffers(1, 777, dtype, dist)[0]
    for op in ("sum", "min", "max"):
        np.testing.assert_array_equal(oracle.all_reduce([x], dtype, op)[0], x)


@pytest.mark.parametrize("op", ["min", "max"])
def test_minmax_rank_permutation_invariant(op):
    xs = si.rank_buffers(5, 999, "f32", "uniform", seed=9)
    base = oracle.all_reduce(xs, "f32", op)[0]
    for perm in [(4, 3, 2, 1, 0), (2, 0, 4, 1, 3)]:
        np.testing.assert_array_equal(oracle.all_reduce([xs[i] for i in perm], "f32", op)[0], base)


# ---------------------------------------- reduce-scatter / all-gather / fold_at

@pytest.mark.parametrize("P", PS)
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "sum"), ("i32", "sum"),
                                      ("bf16", "max"), ("f32", "min")])
def test_reduce_scatter_then_all_gather_is_all_reduce(P, dtype, op):
    dist = "int20" if dtype == "i32" else "uniform"
    xs = si.rank_buffers(P, P * 513, dtype, dist, seed=P + 1)
    rs = oracle.reduce_scatter(xs, dtype, op)
    ag = oracle.all_gather(rs, dtype)
    ar = oracle.all_reduce(xs, dtype, op)
    for q in range(P):
        np.testing.assert_array_equal(ag[q], ar[q])
        np.testing.assert_array_equal(ar[q], ar[0])  # replicas identical


@pytest.mark.parametrize("P", PS)
def test_reduce_scatter_shard_s_is_slice_of_numpy_sum(P):
    xs = si.rank_buffers(P, P * 300, "f32", "uniform", seed=21)
    rs = oracle.reduce_scatter(xs, "f32", "sum")
    full = seq_sum_f32(xs)
    for s in range(P):
        np.testing.assert_array_equal(rs[s], np.split(full, P)[s])


@pytest.mark.parametrize("P", PS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
def test_all_gather_is_concatenation(P, dtype):
    dist = "int20" if dtype == "i32" else "normal"
    xs = si.rank_buffers(P, 301, dtype, dist, seed=4)
    ag = oracle.all_gather(xs, dtype)
    want = np.concatenate(xs)
    for y in ag:
        np.testing.assert_array_equal(y, want)


@pytest.mark.parametrize("dtype,op", [("bf16", "sum"), ("f32", "max"), ("i32", "sum")])
def test_fold_at_equals_full_allreduce(dtype, op):
    dist = "int20" if dtype == "i32" else "uniform"
    xs = si.rank_buffers(8, 10007, dtype, dist, seed=2)
    idx = si.sample_indices(10007, 500)
    np.testing.assert_array_equal(oracle.fold_at(xs, dtype, op, idx),
                                  oracle.all_reduce(xs, dtype, op)[0][idx.astype(np.int64)])


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.reduce_scatter(si.rank_buffers(3, 10, "f32", "uniform"), "f32", "sum")
    with pytest.raises(TypeError):
        oracle.all_reduce([np.zeros(4, np.float64)], "f32", "sum")


# ------------------------------------------------------------------ reshard

def global_iota(shape):
    return np.arange(int(np.prod(shape)), dtype=np.int32).reshape(shape)


@pytest.mark.parametrize("name", ["example_a.txt", "example_b.txt"])
def test_reshard_worked_examples(name):
    ex = load_example(name)
    shape = ex["shape"]
    G = global_iota(shape)
    src_dims, src_start, _ = ex["src"]
    dst_dims, dst_start, _ = ex["dst"]
    # the page's source holdings
    src_bufs = []
    for l in range(int(np.prod(src_dims))):
        (r0, r1), (c0, c1) = ex["hold"]["src"][src_start + l]
        src_bufs.append(np.ascontiguousarray(G[r0:r1, c0:c1]).ravel())
    dst = oracle.reshard(shape, ex["src"], ex["dst"], src_bufs, fill=-1)
    assert len(dst) == int(np.prod(dst_dims))
    for l, buf in enumerate(dst):
        (r0, r1), (c0, c1) = ex["hold"]["dst"][dst_start + l]
        np.testing.assert_array_equal(buf, G[r0:r1, c0:c1].ravel())


def test_example_a_source_holdings_follow_from_layout():
    ex = load_example("example_a.txt")
    G = global_iota(ex["shape"])
    blocks = local_blocks(G, ex["src"])
    for l, blk in enumerate(blocks):
        (r0, r1), (c0, c1) = ex["hold"]["src"][l]
        np.testing.assert_array_equal(blk, G[r0:r1, c0:c1].ravel())


def test_example_a_rejects_column_major_reading():
    """Numbering the destination mesh column-major would give ranks 4/5 rows
    [0:2]; the page says ranks 4/6, which is what the oracle produces."""
    ex = load_example("example_a.txt")
    G = global_iota(ex["shape"])
    src_bufs = local_blocks(G, ex["src"])
    dst = oracle.reshard(ex["shape"], ex["src"], ex["dst"], src_bufs)
    assert not np.array_equal(dst[1], G[0:2].ravel())  # rank 5 is not rows 0:2
    np.testing.assert_array_equal(dst[2], G[0:2].ravel())  # rank 6 is


def _tiny_layouts(ndim, shape):
    meshes = [[1], [2], [3], [4], [2, 2], [1, 3], [3, 1], [2, 3]]
    for dims in meshes:
        choices = [["R"] + [("S", d) for d in range(ndim)] for _ in dims]
        for pl in itertools.product(*choices):
            sharded = [p for p in pl if p != "R"]
            if len(sharded) > 1:
                continue
            yield dims, list(pl)


@pytest.mark.parametrize("shape", [(6,), (4, 6), (2, 3, 4), (5,), (7, 3), (3, 5, 2)])
def test_reshard_all_tiny_layouts_against_torch_chunk(shape):
    G = global_iota(shape)
    layouts = list(_tiny_layouts(len(shape), shape))
    # every ordered pair of layouts: meshes of 1-6 ranks, any placement with at
    # most one sharded axis
    for (sd, spl), (dd, dpl) in itertools.product(layouts, layouts):
        src = (sd, 0, spl)
        dst = (dd, int(np.prod(sd)) + 1, dpl)
        src_bufs = local_blocks(G, src)
        got = oracle.reshard(shape, src, dst, src_bufs, fill=-1)
        want = local_blocks(G, dst)
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)
        # point queries agree with the brute force
        for l, g in enumerate(got):
            idx = np.arange(g.size, dtype=np.uint64)
            np.testing.assert_array_equal(oracle.reshard_at(shape, src, dst, src_bufs, l, idx), g)


def test_reshard_shard_to_replicate_is_all_gather():
    P = 4
    xs = si.rank_buffers(P, 50, "bf16", "w002", seed=3)
    dst = oracle.reshard((P * 50,), ([P], 0, [("S", 0)]), ([3], P, ["R"]), xs)
    for y in dst:
        np.testing.assert_array_equal(y, np.concatenate(xs))


def test_reshard_replicate_to_shard_is_slicing():
    t = si.tensor((8, 5), "bf16", "w002", seed=8)
    dst = oracle.reshard((8, 5), ([2], 0, ["R"]), ([4], 2, [("S", 0)]), [t.ravel(), t.ravel()])
    for y, w in zip(dst, np.split(t, 4, axis=0)):
        np.testing.assert_array_equal(y, w.ravel())


def test_reshard_identical_layout_is_identity():
    xs = si.rank_buffers(4, 24, "f32", "normal", seed=6)
    dst = oracle.reshard((4, 24), ([4], 0, [("S", 0)]), ([4], 4, [("S", 0)]), xs)
    for y, x in zip(dst, xs):
        np.testing.assert_array_equal(y, x)


def test_reshard_detects_disagreeing_source_replicas():
    a = np.arange(8, dtype=np.int32)
    b = a.copy()
    b[3] += 1
    with pytest.raises(ValueError):
        oracle.reshard((8,), ([2], 0, ["R"]), ([1], 2, ["R"]), [a, b])


@pytest.mark.parametrize("bad", [
    dict(src=([2], 0, [("S", 0)]), dst=([2], 1, ["R"])),      # overlapping meshes
    dict(src=([2, 2], 0, [("S", 0), ("S", 0)]), dst=([1], 4, ["R"])),  # one dim sharded twice
    dict(src=([2], 0, [("S", 5)]), dst=([1], 2, ["R"])),      # no such tensor dim
])
def test_reshard_rejects_invalid_layouts(bad):
    bufs = [np.zeros(8, np.int32)] * 3
    with pytest.raises(ValueError):
        oracle.reshard((8,), bad["src"], bad["dst"], bufs)


def test_torch_available_for_library_checks():
    assert torch.tensor([1.0], dtype=torch.bfloat16).item() == 1.0


# ------------------------------------------------------------- fp16

@pytest.mark.parametrize(
    "f32_pattern, f16_pattern",
    [
        (0x3F800000, 0x3C00),  # 1.0
        (0x3F801000, 0x3C00),  # 1 + 2^-11: halfway, even below -> stays
        (0x3F803000, 0x3C02),  # 1 + 3*2^-11: halfway, odd below -> up to even
        (0x3F801001, 0x3C01),  # just above halfway -> up
        (0x477FE000, 0x7BFF),  # 65504, the largest half
        (0x477FEFFF, 0x7BFF),  # just below the overflow tie
        (0x477FF000, 0x7C00),  # 65520: tie between 65504 and 2^16 -> even -> inf
        (0x38800000, 0x0400),  # 2^-14, the smallest normal half
        (0x387FC000, 0x03FF),  # 1023 * 2^-24, the largest subnormal
        (0x33800000, 0x0001),  # 2^-24, the smallest subnormal
        (0x33000000, 0x0000),  # 2^-25: tie between 0 and 2^-24 -> 0
        (0x33000001, 0x0001),  # just above -> 2^-24
        (0x33C00000, 0x0002),  # 1.5 * 2^-24: tie between 1 and 2 -> 2
        (0xC0000000, 0xC000),  # -2
        (0x80000000, 0x8000),  # -0
        (0x7F800000, 0x7C00),  # +inf
        (0x7FC00001, 0x7E00),  # NaN -> canonical
    ],
)
def test_f16_rne_hand_worked(f32_pattern, f16_pattern):
    assert oracle.narrow_f16(bits_f32(f32_pattern)) == f16_pattern


def test_f16_narrow_and_widen_match_numpy():
    rng = np.random.default_rng(11)
    # values spread over the whole half range, subnormals and overflow included
    mags = np.exp2(rng.uniform(-27, 17, size=20000)).astype(np.float32)
    x = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    with np.errstate(over="ignore"):  # values past 65520 become inf on purpose
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.narrow_f16(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(got, want)
    h = np.arange(0, 2**16, 7, dtype=np.uint16)
    h = h[~np.isnan(h.view(np.float16))]
    wide = np.array([oracle.widen_f16(int(v)) for v in h], np.float32)
    np.testing.assert_array_equal(wide.view(np.uint32), h.view(np.float16).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("P", PS)
def test_allreduce_f16_sum_equals_fp32_fold_then_numpy_rne(P):
    xs = [x.astype(np.float16).view(np.uint16) for x in si.rank_buffers(P, 4000, "f32", "normal", seed=P)]
    ys = oracle.all_reduce(xs, "f16", "sum")
    want = seq_sum_f32([x.view(np.float16).astype(np.float32) for x in xs]).astype(np.float16)
    np.testing.assert_array_equal(ys[0], want.view(np.uint16))


# ------------------------------------------------------ reduce / broadcast

@pytest.mark.parametrize("P", PS)
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "max"), ("i32", "sum"), ("f16", "min")])
def test_reduce_is_the_fold_into_one_buffer(P, dtype, op):
    if dtype == "f16":
        xs = [x.astype(np.float16).view(np.uint16) for x in si.rank_buffers(P, 999, "f32", "uniform", seed=3)]
    else:
        xs = si.rank_buffers(P, 999, dtype, "int20" if dtype == "i32" else "uniform", seed=3)
    y = oracle.reduce(xs, dtype, op)
    if dtype == "f32" and op == "sum":
        np.testing.assert_array_equal(y, seq_sum_f32(xs))
    elif dtype == "i32":
        np.testing.assert_array_equal(y, np.sum(np.stack(xs).astype(np.int64), 0).astype(np.int32))
    elif dtype == "bf16":
        np.testing.assert_array_equal(y, si.to_bf16_bits(np.maximum.reduce([si.bf16_bits_to_f32(x) for x in xs])))
    else:
        np.testing.assert_array_equal(y, np.minimum.reduce([x.view(np.float16) for x in xs]).view(np.uint16))


@pytest.mark.parametrize("P", PS)
def test_broadcast_copies_the_root_buffer_everywhere(P):
    x = si.rank_buffers(1, 1001, "bf16", "normal", seed=P)[0]
    for y in oracle.broadcast(x, P, "bf16"):
        np.testing.assert_array_equal(y, x)


def test_uneven_shard_blocks_follow_torch_chunk():
    """9 rows over 4 ranks: pieces of ceil(9/4) = 3 rows, the last rank empty;
    10 over 4: 3, 3, 3, 1."""
    for D, want in [(9, [3, 3, 3, 0]), (10, [3, 3, 3, 1]), (3, [1, 1, 1, 0]), (1, [1, 0, 0, 0])]:
        sizes = [oracle.local_numel((D, 2), ([4], 0, [("S", 0)]), l) // 2 for l in range(4)]
        assert sizes == want
        assert sizes == [chunk_piece(np.zeros((D, 2)), 4, 0, c).shape[0] for c in range(4)]


def test_uneven_reshard_round_trip():
    t = si.tensor((11, 7), "f32", "normal", seed=12)
    a = ([3], 0, [("S", 0)])
    b = ([2, 2], 3, [("S", 1), "R"])
    c = ([1], 7, ["R"])
    mid = oracle.reshard((11, 7), a, b, local_blocks(t, a))
    back = oracle.reshard((11, 7), b, c, mid)
    np.testing.assert_array_equal(back[0], t.ravel())


# ------------------------------------------------- all-reduce + RMSNorm

@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_allreduce_rmsnorm_equals_torch_rms_norm_of_the_reduce(P, dtype):
    rows, hidden, eps = 6, 96, 1e-6
    xs = si.rank_buffers(P, rows * hidden, dtype, "normal", seed=P)
    gamma = si.rank_buffers(1, hidden, dtype, "uniform", seed=99)[0]
    ys = oracle.all_reduce_rmsnorm(xs, rows, hidden, gamma, eps, dtype)
    s = oracle.reduce(xs, dtype, "sum")  # the reduce-scatter's rounded values

    def widen(a):
        if dtype == "bf16":
            return si.bf16_bits_to_f32(a).astype(np.float64)
        if dtype == "f16":
            return a.view(np.float16).astype(np.float64)
        return a.astype(np.float64)

    S = torch.from_numpy(widen(s).reshape(rows, hidden))
    G = torch.from_numpy(widen(gamma))
    ref = torch.nn.functional.rms_norm(S, (hidden,), weight=G, eps=eps).numpy().astype(np.float32)
    if dtype == "bf16":
        want = si.to_bf16_bits(ref.ravel())
    elif dtype == "f16":
        want = ref.ravel().astype(np.float16).view(np.uint16)
    else:
        want = ref.ravel()
    for y in ys:
        np.testing.assert_array_equal(y, want)


def test_allreduce_rmsnorm_rows_are_unit_rms_with_unit_gamma():
    rows, hidden = 4, 512
    xs = si.rank_buffers(3, rows * hidden, "f32", "normal", seed=5)
    y = oracle.all_reduce_rmsnorm(xs, rows, hidden, np.ones(hidden, np.float32), 0.0, "f32")[0]
    rms = np.sqrt(np.mean(y.reshape(rows, hidden).astype(np.float64) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-6)


# ------------------------------------------------ fp8 staging quantization

def test_e4m3_code_values_match_torch_float8():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    np.testing.assert_array_equal(got, want)
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_rounding_matches_torch_in_range():
    rng = np.random.default_rng(3)
    y = (np.exp2(rng.uniform(-12, 8.8, 30000)) * rng.choice([-1, 1], 30000)).astype(np.float32)
    y = y[np.abs(y) <= 448]
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_nearest_sat(float(v)) for v in y], np.uint8)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("y, code", [
    (448.0, 0x7E), (449.0, 0x7E), (1e30, 0x7E), (-500.0, 0xFE),    # saturation
    (1.0625, 0x38), (1.1875, 0x3A),                                   # ties to even mantissa
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),                       # subnormal ties
    (-0.0, 0x80), (0.0, 0x00),
])
def test_e4m3_hand_worked(y, code):
    assert oracle.e4m3_nearest_sat(y) == code


def test_blockwise_quantization_round_trip_error_bound():
    x = si.rank_buffers(1, 128 * 40 + 17, "bf16", "w002", seed=8)[0]
    codes, scales = oracle.quantize_e4m3(x, "bf16")
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    deq = np.array([oracle.e4m3_value(int(c)) for c in codes]) * np.repeat(scales, 128)[: x.size]
    # each block's largest element maps to 448; E4M3 keeps 3 mantissa bits, so
    # a value within the normal range is off by at most 2^-4 of itself, and
    # anything in a block by at most half a subnormal step of that block
    for b in range(scales.size):
        sl = slice(128 * b, min(128 * (b + 1), x.size))
        amax = np.max(np.abs(xf[sl]))
        assert np.isclose(np.max(np.abs(deq[sl])), amax, rtol=2 ** -4)
        err = np.abs(deq[sl] - xf[sl])
        assert np.all(err <= np.maximum(np.abs(xf[sl]) * 2 ** -4, scales[b] * 2.0 ** -10) * 1.0001)


def test_quantization_scale_that_underflows_is_one():
    """A block whose amax / 448 rounds to zero in fp32 (amax = 2^-149, the
    smallest subnormal) is scaled like an all-zero block: scale 1, and every
    element, far below E4M3's smallest step, codes to a signed zero.  A block
    whose amax / 448 is a coarse subnormal keeps that scale, and its largest
    elements saturate at 448 instead of overflowing."""
    tiny = np.float32(2.0 ** -149)
    x = np.array([tiny, 0.0, -tiny, -0.0] * 32, np.float32)
    codes, scales = oracle.quantize_e4m3(x, "f32")
    assert scales.view(np.uint32)[0] == np.float32(1.0).view(np.uint32)
    assert list(codes[:4]) == [0x00, 0x00, 0x80, 0x80]
    amax = np.float32(3 * 2.0 ** -140)
    y = np.zeros(128, np.float32)
    y[0], y[1] = amax, -amax
    codes, scales = oracle.quantize_e4m3(y, "f32")
    s = scales[0]
    assert 0 < s < 2.0 ** -126 and s == np.float32(amax) / np.float32(448)
    assert amax / np.float64(s) > 448           # the quotient overshoots 448 ...
    assert codes[0] == 0x7E and codes[1] == 0xFE  # ... and saturates


def _e4m3_codes_from_quotients(q: np.ndarray) -> np.ndarray:
    """fp32 quotients -> E4M3 codes: saturate at +-448, then PyTorch's
    round-to-nearest-even conversion (which has no saturation of its own)."""
    t = torch.from_numpy(np.ascontiguousarray(q, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _blockwise_reference(xf: np.ndarray, block: int = 128):
    """The format written out with numpy and PyTorch only: per block an fp32
    amax, scale = amax / 448 in fp32 (1 when that is zero), code = E4M3 of the
    fp32 quotient x / scale."""
    nb = (xf.size + block - 1) // block
    scales = np.empty(nb, np.float32)
    q = np.empty(xf.size, np.float32)
    for b in range(nb):
        sl = slice(b * block, min((b + 1) * block, xf.size))
        amax = np.max(np.abs(xf[sl])).astype(np.float32)
        s = np.float32(amax / np.float32(448.0))
        s = np.float32(1.0) if s == 0 else s
        scales[b] = s
        q[sl] = xf[sl] / s
    return _e4m3_codes_from_quotients(q), scales


def _discriminating_blocks(rng, n_scales: int = 2000, keep: int = 64) -> np.ndarray:
    """128-element fp32 blocks, one per scale, each holding its amax and
    elements whose quotient x / scale lies within an fp32 ulp of a midpoint
    between two E4M3 values, kept only where the code of x / scale differs
    from the code of x * (1 / scale)."""
    amax = (rng.uniform(1, 2, n_scales) * np.exp2(rng.integers(-20, 20, n_scales))).astype(np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    vals = np.unique(vals[vals > 0])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = (mids[rng.integers(0, mids.size, n_scales)] * s).astype(np.float32)
    cands = [np.nextafter(x, np.float32(-np.inf), dtype=np.float32), x,
             np.nextafter(x, np.float32(np.inf), dtype=np.float32)]
    blocks = []
    for i in range(n_scales):
        good = [c[i] for c in cands
                if _e4m3_codes_from_quotients(np.array([c[i] / s[i]]))[0]
                != _e4m3_codes_from_quotients(np.array([c[i] * inv[i]]))[0]]
        if not good:
            continue
        y = (rng.uniform(-1, 1, 128) * amax[i]).astype(np.float32)
        y[0] = amax[i]
        for j, g in enumerate(good):
            y[1 + 2 * j], y[2 + 2 * j] = g, -g
        blocks.append(y)
        if len(blocks) == keep:
            break
    return np.concatenate(blocks)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_blockwise_quantization_equals_numpy_torch_chain(dtype):
    """orc_quantize_e4m3 bit for bit against the format rebuilt outside the
    oracle (numpy fp32 amax and division, PyTorch's E4M3 conversion), on
    ordinary blocks, an all-zero block, a block whose quotient underflows, a
    block with amax above 448 and a ragged last block."""
    rng = np.random.default_rng(41)
    n = 128 * 24 + 37
    if dtype == "f32":
        x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
        x[128:256] = 0.0
        x[256:384] = np.float32(2.0 ** -149) * rng.choice([-1, 0, 1], 128)
        x[384:512] = rng.uniform(-3000, 3000, 128).astype(np.float32)
        xs = x
    elif dtype == "bf16":
        x = si.rank_buffers(1, n, "bf16", "w002", seed=5)[0].copy()
        x[128:256] = 0
        big = si.to_bf16_bits(rng.uniform(-3000, 3000, 128).astype(np.float32))
        x[384:512] = big
        xs = x
    else:
        xf = (rng.standard_normal(n) * 10).astype(np.float16)
        xf[128:256] = 0
        xf[384:512] = rng.uniform(-60000, 60000, 128).astype(np.float16)
        xs = xf.view(np.uint16)
    codes, scales = oracle.quantize_e4m3(xs, dtype)
    if dtype == "f32":
        xf32 = xs
    elif dtype == "bf16":
        xf32 = si.bf16_bits_to_f32(xs)
    else:
        xf32 = xs.view(np.float16).astype(np.float32)
    want_codes, want_scales = _blockwise_reference(xf32)
    np.testing.assert_array_equal(scales.view(np.uint32), want_scales.view(np.uint32))
    np.testing.assert_array_equal(codes, want_codes)


def test_blockwise_quantization_chain_catches_reciprocal_and_early_clamp():
    """Blocks built on E4M3 rounding midpoints: the oracle matches the division
    x / scale there, while the two plausible slips -- multiplying by the fp32
    reciprocal, or clamping x (rather than the quotient) to +-448 -- give other
    codes on the same inputs, so the pin above would catch either."""
    rng = np.random.default_rng(43)
    x = _discriminating_blocks(rng)
    assert x.size == 64 * 128
    codes, scales = oracle.quantize_e4m3(x, "f32")
    want_codes, want_scales = _blockwise_reference(x)
    np.testing.assert_array_equal(scales.view(np.uint32), want_scales.view(np.uint32))
    np.testing.assert_array_equal(codes, want_codes)
    s = np.repeat(want_scales, 128)[: x.size]
    recip = _e4m3_codes_from_quotients(x * (np.float32(1.0) / s))
    assert np.count_nonzero(recip != codes) >= 64
    # clamping before the division: blocks whose amax exceeds 448
    big = (rng.uniform(-1, 1, 128 * 4) * 3000).astype(np.float32)
    codes_b, scales_b = oracle.quantize_e4m3(big, "f32")
    want_b, _ = _blockwise_reference(big)
    np.testing.assert_array_equal(codes_b, want_b)
    sb = np.repeat(scales_b, 128)
    early = _e4m3_codes_from_quotients(np.clip(big, -448.0, 448.0).astype(np.float32) / sb)
    assert np.count_nonzero(early != codes_b) >= 128
