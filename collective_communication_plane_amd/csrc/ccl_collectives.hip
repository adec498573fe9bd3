// Host side of the collectives: segments, alignment, launch shape, and the
// choice among the kernel families in ccl_coll_kernels.h.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ccl_coll_kernels.h"

namespace ccl {

namespace {

using DispatchFn = hipError_t (*)(const CollArgs &, const CollPath &, hipStream_t);

DispatchFn pick_dispatch(Kind kind, int dtype) {
  switch (kind) {
    case KIND_AR:
      return dtype == CCL_FLOAT32 ? dispatch_ar_f32
             : dtype == CCL_BFLOAT16 ? dispatch_ar_bf16
             : dtype == CCL_FLOAT16 ? dispatch_ar_f16
                                    : dispatch_ar_i32;
    case KIND_RS:
      return dtype == CCL_FLOAT32 ? dispatch_rs_f32
             : dtype == CCL_BFLOAT16 ? dispatch_rs_bf16
             : dtype == CCL_FLOAT16 ? dispatch_rs_f16
                                    : dispatch_rs_i32;
    default:
      return dtype_size(dtype) == 2 ? dispatch_ag_b16 : dispatch_ag_b32;
  }
}

}  // namespace

ccl_status_t launch_collective(const CollDesc &d, const Launch &l, hipStream_t stream) {
  CollArgs a{};
  const int esz = dtype_size(d.dtype);
  const int V = kVecBytes / esz;
  const uint64_t M = d.seg_elems;
  a.P = d.P;
  a.seg_elems = M;
  a.flags = (l.nt_load ? 1 : 0) | (l.nt_store ? 2 : 0);
  // Broadcast has one input, reduce one output; the other calls have P of each.
  const int n_in_ptrs = (d.kind == KIND_AG && d.single) ? 1 : d.P;
  const int n_out_ptrs = (d.kind == KIND_RS && d.single) ? 1 : d.P;
  for (int r = 0; r < n_in_ptrs; ++r) a.in[r] = (const char *)d.send[r];
  for (int r = 0; r < n_out_ptrs; ++r) a.out[r] = (char *)d.recv[r];
  const int nseg = (d.kind == KIND_AR || d.single) ? 1 : d.P;
  const int ni = d.kind == KIND_AG ? 1 : d.P;
  const int no = d.kind == KIND_RS ? 1 : d.P;

  // The outputs of a segment must share their address modulo 16; their
  // common misalignment becomes the scalar head, after which every output is
  // 16-byte aligned.  Inputs at another offset are realigned in registers.
  bool vec = true, realign = false;
  bool lines_aligned = true;  // every output's vector body starts on 256 bytes
  uint64_t max_nvec = 0;
  for (int s = 0; s < nseg && vec; ++s) {
    uintptr_t ob[CCL_MAX_RANKS];
    for (int q = 0; q < no; ++q) {
      const char *p = d.kind == KIND_AR ? a.out[q]
                      : d.kind == KIND_RS ? a.out[s]
                                          : a.out[q] + (uint64_t)s * M * esz;
      ob[q] = (uintptr_t)p;
    }
    const uintptr_t mis = ob[0] % kVecBytes;
    for (int q = 1; q < no; ++q)
      if (ob[q] % kVecBytes != mis) vec = false;
    uint64_t head = ((kVecBytes - mis) % kVecBytes) / esz;
    if (head > M) head = M;
    a.head[s] = (uint32_t)head;
    for (int q = 0; q < no; ++q)
      if ((ob[q] + head * esz) % 256) lines_aligned = false;
    a.nvec[s] = (M - head) / V;
    max_nvec = std::max<uint64_t>(max_nvec, a.nvec[s]);
    for (int r = 0; r < ni; ++r) {
      const char *p = d.kind == KIND_AR ? a.in[r]
                      : d.kind == KIND_RS ? a.in[r] + (uint64_t)s * M * esz
                                          : a.in[s];
      a.shift[s][r] = (uint8_t)(((uintptr_t)p + head * esz) % kVecBytes);
      if (a.shift[s][r]) realign = true;
    }
  }

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CCL_ERR_HIP;
  const int cus = device_cu_count(dev);
  if (cus <= 0) return CCL_ERR_HIP;

  const DispatchFn dispatch = pick_dispatch(d.kind, d.dtype);
  CollPath p{};
  p.op = d.op;
  p.stages = l.stages;
  p.occupancy = l.occupancy;
  p.nseg = nseg;
  hipError_t err;
  if (!vec) {
    const uint64_t total = (uint64_t)nseg * M;
    const uint64_t want = (total + kThreads - 1) / kThreads;
    p.path = PATH_SCALAR;
    p.grid = (unsigned)std::min<uint64_t>(std::max<uint64_t>(want, 1), (uint64_t)cus * 16);
    err = dispatch(a, p, stream);
    return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
  }

  uint64_t chunk_bytes = l.chunk_bytes;
  int occupancy = l.occupancy;
  int unroll = l.unroll;
  // All-reduce shapes by size and placement, from sweeps over P, per-rank
  // size and buffer layout (bf16; one torch tensor per rank and staggered
  // slabs, interleaved repeats):
  //  - 3 <= P <= 8 with 1-128 MiB per rank: 8 KiB chunks, unroll 2, <= 4 WGs
  //    per CU (+1.4-13.5 % at 32-128 MiB over the per-P shapes; past 128 MiB
  //    per rank the shape falls off, -7 to -16 % from 144-320 MiB by P);
  //  - P = 2 with 129-256 MiB per rank: unroll 1 (+11.5-17 % at 160-256 MiB;
  //    level at 128 MiB, -1 to -7 % from 288 MiB);
  //  - 6 <= P <= 16 from 512 MiB per rank, when every input starts at the same
  //    offset modulo 2 MiB (what separate framework allocations give): 16 KiB
  //    chunks, <= 3 WGs per CU (+1-19 %).  Inputs staggered against each
  //    other keep 4 KiB chunks, where 16 KiB ones lose 12-15 %.  At P = 5 the
  //    same inputs take 8 KiB chunks, <= 3 WGs per CU, the shape P = 3, 4
  //    write through with anyway: over two sets of nine random placements
  //    +4.3 and +4.7 % on average (+2 to +17 % at 512 MiB, within -3.1 to
  //    +7 % at 768 MiB-1 GiB), where 16 KiB chunks averaged -0.6 to -3.5 %;
  //    it loses 3-7 % at 384 MiB and 6 % on staggered inputs.
  const uint64_t per_rank = M * esz;
  bool congruent = true;  // every input at one offset modulo 2 MiB
  for (int r = 1; r < ni; ++r)
    congruent = congruent && ((uintptr_t)a.in[r] - (uintptr_t)a.in[0]) % (uint64_t(2) << 20) == 0;
  if (d.kind == KIND_AR && !realign && l.stages <= 1 && !l.chunk_set && !l.occupancy_set &&
      !l.unroll_set) {
    if (d.P >= 3 && d.P <= 8 && per_rank >= (uint64_t(1) << 20) &&
        per_rank <= (uint64_t(128) << 20)) {
      chunk_bytes = 8192;
      unroll = 2;
      occupancy = 4;
    } else if (d.P == 2 && per_rank > (uint64_t(128) << 20) && per_rank <= (uint64_t(256) << 20)) {
      unroll = 1;
    } else if (d.P >= 6 && per_rank >= (uint64_t(512) << 20) && congruent) {
      chunk_bytes = 16384;
      occupancy = 3;
    } else if (d.P == 5 && per_rank >= (uint64_t(512) << 20) && congruent) {
      chunk_bytes = 8192;
      occupancy = 3;
    }
  }
  // The realigning kernel reads two blocks per input vector and wants other
  // chunks and residency than the aligned kernels whose defaults it would
  // otherwise inherit (reduce-scatter at P = 3 and 12: 2800-3200 GB/s under
  // those, 4800-5800 with these).  Its loads stay cacheable: a lane's second
  // block is its neighbour's first, which a nontemporal load does not keep
  // for it (the ragged reduce-scatter ran 4-15 % slower with them).
  if (realign) {
    const bool many = d.kind == KIND_RS && d.P > 8;
    if (!l.chunk_set) chunk_bytes = many ? 8192 : 4096;
    if (!l.occupancy_set) occupancy = d.kind != KIND_AG ? (many ? 4 : 8) : d.P <= 6 ? 4 : 3;
    if (!l.nt_set && d.kind == KIND_RS) a.flags &= ~1;
  }
  // Write-through stores (register-direct kernel and LDS pipeline), by default where they
  // won in same-binary A/B runs on MI355X (bf16, separate kernel
  // instantiations): the reduce-scatter and reduce at P <= 8 (+3 % at P <= 4,
  // +1-8 % at P = 7, 8 from 64 to 512 MiB per rank; -0.4 to +0.8 % from
  // P = 9); the all-gather and broadcast at P = 2 (+7 %), at 7 <= P <= 16
  // with at most 256 MiB of input and at 4 <= P <= 6 with at most 64 MiB, with
  // >= 4 resident workgroups per CU from P = 9 on.  That rule follows
  // cold-MALL runs (three buffer sets used in turn): there write-through gains
  // 1-21 % at P = 2 and 7-12 and 1-5 % at P = 13-16, but at P = 4-6 with
  // 128-256 MiB of input nontemporal-only stores win by 2-10 %.  (Repeating
  // one call on the same buffers, the input stays in the MALL between calls
  // and write-through gains up to 30 % more; with 341-512 MiB of input it
  // loses 2-6 %, at P = 3 it loses, with 3 workgroups per CU up to 30 %.)  The
  // all-reduce, past the range of the 8 KiB / unroll-2 shape above: at P = 2
  // above 256 MiB per rank (+1-6 % at 384 MiB to 1 GiB), at P = 3 from
  // 256 MiB (P = 3-6 with 341-682 MiB per rank: +2-11 %, P = 3, 4 with 8 KiB
  // chunks and <= 3 workgroups per CU; P = 3 loses 3-6 % at 128-192 MiB), at
  // 4 <= P <= 8 above 128 MiB (P = 4-6 at 144-224 MiB: +1.6 to +2.8 % on
  // average over both layouts on two boxes, -1.3 to +12 % per cell, and at
  // 192 MiB +1-8 % in five runs of the defaults table; P = 7, 8: +2-11 % at
  // 136 MiB to 1 GiB, +3-4 % at the P = 8 x 256 MiB point), and at
  // 9 <= P <= 16 from 16 MiB (+0.5-8 % at 16-256 MiB and up to 1 GiB, one
  // cell at -0.1 %).  Only
  // where every chunk's stores
  // start on a 256-byte boundary: the all-gather at P = 8 with shards of
  // 2^24 + 8 elements ran 4086 GB/s with them against 5166 without, and every
  // shard size that is not a multiple of 256 bytes lost 10-43 %.  The stores
  // address a chunk through a buffer resource with 31-bit offsets.
  const uint64_t ag_in_bytes = (uint64_t)(d.single ? 1 : d.P) * M * esz;
  const uint64_t ar_wt_from = d.P == 2   ? (uint64_t(256) << 20) + 1
                              : d.P == 3  ? (uint64_t(256) << 20)
                              : d.P <= 8  ? (uint64_t(128) << 20) + 1
                                          : (uint64_t(16) << 20);
  bool wt = l.store_wt;
  if (!l.store_pol_set)
    wt = lines_aligned &&
         (d.kind == KIND_AG
              ? (d.P == 2 || (d.P >= 7 && ag_in_bytes <= (uint64_t(256) << 20)) ||
             (d.P >= 4 && d.P <= 6 && ag_in_bytes <= (uint64_t(64) << 20)))
          : d.kind == KIND_RS ? d.P <= 8
                              : d.P >= 2 && per_rank >= ar_wt_from);
  wt = wt && l.nt_store && !realign && chunk_bytes <= (uint64_t(1) << 30);
  if (wt) a.flags |= 4;
  if (wt && d.kind == KIND_AG && d.P >= 9 && !l.occupancy_set) occupancy = 4;
  // Write-through all-reduce shapes at few ranks (interleaved A/B, both
  // layouts): P = 2 above 256 MiB per rank with 4 KiB chunks, unroll 1 and
  // <= 6 WGs per CU, +0.1-9 % over 8 KiB / unroll 2 / <= 3 in all 18 cells at
  // 288 MiB-1 GiB (<= 4, 5, 7, 8 or uncapped trail <= 6); P = 3, 4 with 8 KiB
  // chunks and <= 3 WGs per CU (P = 4 at 256 MiB-1 GiB: the other shapes
  // tried within 1.2 % of it or behind, by up to 13 %), except at P = 4 from
  // 512 MiB per rank on inputs staggered against each other, where 4 KiB
  // chunks won all 12 cells of four stagger gaps at 512 MiB-1 GiB by 2.5-8.5 %
  // (at 384 MiB they lose 3-7 %; on congruent inputs 8 %; at P = 3 10 % on
  // both).  P = 1 has write-through only when asked for and keeps its own
  // shape (the <= 3 cap halves a copy's rate there).
  if (wt && d.kind == KIND_AR && d.P == 2) {
    if (!l.chunk_set) chunk_bytes = 4096;
    if (!l.unroll_set) unroll = 1;
    if (!l.occupancy_set) occupancy = 6;
  } else if (wt && d.kind == KIND_AR && d.P >= 3 && d.P <= 4) {
    const bool staggered_big = d.P == 4 && !congruent && per_rank >= (uint64_t(512) << 20);
    if (!l.chunk_set) chunk_bytes = staggered_big ? 4096 : 8192;
    if (!l.occupancy_set) occupancy = 3;
  }
  p.occupancy = occupancy;
  p.unroll = unroll;
  p.path = realign ? PATH_REALIGN : l.stages > 1 ? PATH_LDS : PATH_VEC;
  // The all-reduce kernel keeps slot 0's output stream cacheable (see the
  // kernel); the outputs are interchangeable, and the last one measured best
  // in that role (1-2 % over the first under the allocator's placement).
  if (d.kind == KIND_AR && d.P > 1) std::swap(a.out[0], a.out[d.P - 1]);
  a.chunk_vecs = chunk_bytes / kVecBytes;
  a.chunks_per_seg = std::max<uint64_t>(1, (max_nvec + a.chunk_vecs - 1) / a.chunk_vecs);
  a.total_chunks = a.chunks_per_seg * nseg;
  uint64_t grid = l.workgroups ? (uint64_t)l.workgroups : a.total_chunks;
  grid = std::min<uint64_t>(grid, a.total_chunks);
  grid = std::min<uint64_t>(grid, 1u << 30);
  p.grid = (unsigned)grid;
  p.lds = occupancy_lds(occupancy, 0);
  err = dispatch(a, p, stream);
  return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // namespace ccl
