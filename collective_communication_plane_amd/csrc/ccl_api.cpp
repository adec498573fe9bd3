// C ABI entry points of libccl: argument checks (fail-stop: nothing is
// enqueued unless every check passes), launch-config resolution, and dispatch
// to the kernels in ccl_collectives.hip / ccl_reshard.hip.
#include <cstdint>
#include <cstring>
#include <vector>

#include "ccl_internal.h"

namespace {

using ccl::dtype_size;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool mul_overflows(uint64_t a, uint64_t b) { return b != 0 && a > UINT64_MAX / b; }

ccl_status_t check_common(const void *const *send, void *const *recv, int nranks, int dtype) {
  if (nranks < 1 || nranks > CCL_MAX_RANKS) return CCL_ERR_INVALID_ARG;
  if (dtype_size(dtype) == 0) return CCL_ERR_INVALID_ARG;
  if (!send || !recv) return CCL_ERR_INVALID_ARG;
  const uintptr_t align = (uintptr_t)dtype_size(dtype);
  for (int r = 0; r < nranks; ++r) {
    if (!send[r] || !recv[r]) return CCL_ERR_INVALID_ARG;
    if (((uintptr_t)send[r] % align) || ((uintptr_t)recv[r] % align)) return CCL_ERR_INVALID_ARG;
  }
  return CCL_OK;
}

bool op_ok(int op) { return op == CCL_SUM || op == CCL_MIN || op == CCL_MAX; }

// Outputs must not overlap each other at all.
ccl_status_t check_outputs_disjoint(void *const *recv, int P, uint64_t bytes) {
  for (int a = 0; a < P; ++a)
    for (int b = a + 1; b < P; ++b) {
      Range ra{(uintptr_t)recv[a], (uintptr_t)recv[a] + bytes};
      Range rb{(uintptr_t)recv[b], (uintptr_t)recv[b] + bytes};
      if (overlap(ra, rb)) return CCL_ERR_ALIASING;
    }
  return CCL_OK;
}

}  // namespace

namespace ccl {

int device_cu_count(int dev) {
  static std::mutex mu;
  static int cached[64] = {0};
  if (dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -1;
    cached[dev] = n;
  }
  return cached[dev];
}

ccl_status_t resolve_launch(const ccl_launch_config_t *cfg, Op op, int P, Launch *out) {
  const OpDefaults d = default_launch(op, P);
  Launch l{d.chunk_bytes, 0, d.stages, d.unroll, true, true, d.occupancy};
  bool explicit_stages = false;
  if (cfg) {
    if (cfg->chunk_bytes) {
      if (cfg->chunk_bytes % kVecBytes || cfg->chunk_bytes < 1024 ||
          cfg->chunk_bytes > (uint64_t(1) << 32))
        return CCL_ERR_INVALID_ARG;
      l.chunk_bytes = cfg->chunk_bytes;
      l.chunk_set = true;
    }
    if (cfg->workgroups < 0 || cfg->workgroups > (1 << 24)) return CCL_ERR_INVALID_ARG;
    l.workgroups = cfg->workgroups;
    if (cfg->stages < 0 || cfg->stages > 4) return CCL_ERR_INVALID_ARG;
    if (cfg->stages) {
      l.stages = cfg->stages;
      explicit_stages = true;
      l.stages_set = true;
    }
    if (cfg->unroll < 0 || cfg->unroll > 4 || cfg->unroll == 3) return CCL_ERR_INVALID_ARG;
    if (cfg->unroll) {
      l.unroll = cfg->unroll;
      l.unroll_set = true;
    }
    if (cfg->nontemporal < 0 || cfg->nontemporal > 4) return CCL_ERR_INVALID_ARG;
    if (cfg->nontemporal == 4) {
      l.nt_load = l.nt_store = false;
      l.nt_set = true;
    } else if (cfg->nontemporal) {
      l.nt_load = cfg->nontemporal & 1;
      l.nt_store = (cfg->nontemporal >> 1) & 1;
      l.nt_set = true;
    }
    if (cfg->occupancy < 0 || cfg->occupancy > 32) return CCL_ERR_INVALID_ARG;
    if (cfg->store_policy < 0 || cfg->store_policy > 2) return CCL_ERR_INVALID_ARG;
    if (cfg->store_policy) {
      l.store_wt = cfg->store_policy == 1;
      l.store_pol_set = true;
    }
    if (cfg->occupancy) {
      l.occupancy = cfg->occupancy;
      l.occupancy_set = true;
    }
  }
  if ((op == OP_RESHARD || op == OP_RESHARD_FP8) && explicit_stages && l.stages != 1)
    return CCL_ERR_UNSUPPORTED;
  // the fused RMSNorm: 1 = one row at a time, 2 = two rows software-pipelined
  if (op == OP_RMSNORM) {
    if (l.stages > 2) return CCL_ERR_UNSUPPORTED;
    *out = l;
    return CCL_OK;
  }
  if (l.stages > 1 && l.chunk_bytes % kLdsTileBytes) return CCL_ERR_INVALID_ARG;
  *out = l;
  return CCL_OK;
}

}  // namespace ccl

extern "C" {

const char *ccl_get_error_string(ccl_status_t s) {
  switch (s) {
    case CCL_OK: return "success";
    case CCL_ERR_INVALID_ARG: return "invalid argument";
    case CCL_ERR_UNSUPPORTED: return "unsupported request";
    case CCL_ERR_ALIASING: return "illegal buffer overlap";
    case CCL_ERR_LAYOUT: return "invalid reshard layout";
    case CCL_ERR_HIP: return "HIP runtime error";
    case CCL_ERR_NOMEM: return "out of memory";
    case CCL_ERR_SCRATCH_LIMIT:
      return "request needs more scratch than the no-allocation entry point holds";
  }
  return "unknown status";
}

int ccl_version(void) { return 100; }

ccl_status_t ccl_all_reduce(const void *const *send, void *const *recv, int nranks, size_t count,
                            int dtype, int op, void *stream, const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_AR, nranks, &l);
  if (st) return st;
  if (nranks < 1 || nranks > CCL_MAX_RANKS || dtype_size(dtype) == 0 || !op_ok(op))
    return CCL_ERR_INVALID_ARG;
  if (count == 0) return CCL_OK;
  if ((st = check_common(send, recv, nranks, dtype))) return st;
  const uint64_t sz = dtype_size(dtype);
  if (mul_overflows(count, sz)) return CCL_ERR_INVALID_ARG;
  const uint64_t bytes = count * sz;
  if ((st = check_outputs_disjoint(recv, nranks, bytes))) return st;
  // An output may coincide exactly with an input: element i is read and then
  // written by the same lane.  Any other overlap would race.
  for (int q = 0; q < nranks; ++q)
    for (int r = 0; r < nranks; ++r) {
      Range y{(uintptr_t)recv[q], (uintptr_t)recv[q] + bytes};
      Range x{(uintptr_t)send[r], (uintptr_t)send[r] + bytes};
      if (overlap(x, y) && x.lo != y.lo) return CCL_ERR_ALIASING;
    }
  ccl::CollDesc d{ccl::KIND_AR, nranks, dtype, op, count, send, recv, false};
  return ccl::launch_collective(d, l, (hipStream_t)stream);
}

ccl_status_t ccl_reduce_scatter(const void *const *send, void *const *recv, int nranks,
                                size_t recvcount, int dtype, int op, void *stream,
                                const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_RS, nranks, &l);
  if (st) return st;
  if (nranks < 1 || nranks > CCL_MAX_RANKS || dtype_size(dtype) == 0 || !op_ok(op))
    return CCL_ERR_INVALID_ARG;
  if (recvcount == 0) return CCL_OK;
  if ((st = check_common(send, recv, nranks, dtype))) return st;
  const uint64_t sz = dtype_size(dtype);
  if (mul_overflows(recvcount, sz) || mul_overflows(recvcount * sz, (uint64_t)nranks))
    return CCL_ERR_INVALID_ARG;
  const uint64_t out_bytes = recvcount * sz, in_bytes = out_bytes * nranks;
  if ((st = check_outputs_disjoint(recv, nranks, out_bytes))) return st;
  // recv[s] may sit exactly on shard s of an input (the NCCL in-place form).
  for (int s = 0; s < nranks; ++s)
    for (int r = 0; r < nranks; ++r) {
      Range y{(uintptr_t)recv[s], (uintptr_t)recv[s] + out_bytes};
      Range x{(uintptr_t)send[r], (uintptr_t)send[r] + in_bytes};
      if (overlap(x, y) && y.lo != x.lo + (uint64_t)s * out_bytes) return CCL_ERR_ALIASING;
    }
  ccl::CollDesc d{ccl::KIND_RS, nranks, dtype, op, recvcount, send, recv, false};
  return ccl::launch_collective(d, l, (hipStream_t)stream);
}

ccl_status_t ccl_all_gather(const void *const *send, void *const *recv, int nranks,
                            size_t sendcount, int dtype, void *stream,
                            const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_AG, nranks, &l);
  if (st) return st;
  if (nranks < 1 || nranks > CCL_MAX_RANKS || dtype_size(dtype) == 0) return CCL_ERR_INVALID_ARG;
  if (sendcount == 0) return CCL_OK;
  if ((st = check_common(send, recv, nranks, dtype))) return st;
  const uint64_t sz = dtype_size(dtype);
  if (mul_overflows(sendcount, sz) || mul_overflows(sendcount * sz, (uint64_t)nranks))
    return CCL_ERR_INVALID_ARG;
  const uint64_t in_bytes = sendcount * sz, out_bytes = in_bytes * nranks;
  if ((st = check_outputs_disjoint(recv, nranks, out_bytes))) return st;
  // send[r] may sit exactly on slot r of an output (the NCCL in-place form).
  for (int q = 0; q < nranks; ++q)
    for (int r = 0; r < nranks; ++r) {
      Range y{(uintptr_t)recv[q], (uintptr_t)recv[q] + out_bytes};
      Range x{(uintptr_t)send[r], (uintptr_t)send[r] + in_bytes};
      if (overlap(x, y) && x.lo != y.lo + (uint64_t)r * in_bytes) return CCL_ERR_ALIASING;
    }
  ccl::CollDesc d{ccl::KIND_AG, nranks, dtype, CCL_SUM, sendcount, send, recv, false};
  return ccl::launch_collective(d, l, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Both RMSNorm entry points; noalloc: the split-row kernels' partial sums go
// to the fixed device array instead of the stream's library-allocated buffer.
ccl_status_t ar_rmsnorm(const void *const *send, void *const *recv, int nranks, size_t rows,
                        size_t hidden, const void *gamma, float eps, int dtype, void *stream,
                        const ccl_launch_config_t *cfg, bool noalloc) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_RMSNORM, nranks, &l);
  if (st) return st;
  if (nranks < 1 || nranks > CCL_MAX_RANKS) return CCL_ERR_INVALID_ARG;
  if (dtype != CCL_FLOAT32 && dtype != CCL_BFLOAT16 && dtype != CCL_FLOAT16)
    return CCL_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || eps > 1.f) return CCL_ERR_INVALID_ARG;  // also rejects NaN
  if (rows == 0) return CCL_OK;
  if (hidden == 0) return CCL_ERR_INVALID_ARG;
  const uint64_t sz = dtype_size(dtype);
  if (mul_overflows(hidden, sz) || mul_overflows(hidden * sz, rows)) return CCL_ERR_INVALID_ARG;
  if ((hidden * sz) % ccl::kVecBytes) return CCL_ERR_UNSUPPORTED;  // rows of whole vectors
  if (hidden * sz / ccl::kVecBytes > (uint64_t)ccl::kRmsMaxRowVecs) return CCL_ERR_UNSUPPORTED;
  if (!send || !recv || !gamma || (uintptr_t)gamma % ccl::kVecBytes) return CCL_ERR_INVALID_ARG;
  for (int r = 0; r < nranks; ++r) {
    if (!send[r] || !recv[r]) return CCL_ERR_INVALID_ARG;
    if ((uintptr_t)send[r] % ccl::kVecBytes || (uintptr_t)recv[r] % ccl::kVecBytes)
      return CCL_ERR_UNSUPPORTED;  // the fused kernel runs on 16-byte aligned rows only
  }
  const uint64_t bytes = rows * hidden * sz;
  if ((st = check_outputs_disjoint(recv, nranks, bytes))) return st;
  for (int q = 0; q < nranks; ++q) {
    Range y{(uintptr_t)recv[q], (uintptr_t)recv[q] + bytes};
    Range g{(uintptr_t)gamma, (uintptr_t)gamma + hidden * sz};
    if (overlap(y, g)) return CCL_ERR_ALIASING;
    for (int r = 0; r < nranks; ++r) {
      Range x{(uintptr_t)send[r], (uintptr_t)send[r] + bytes};
      if (overlap(x, y) && x.lo != y.lo) return CCL_ERR_ALIASING;
    }
  }
  // Defaults by row length.  Rows longer than 16 KiB per rank: the
  // row-pipelined kernel with one workgroup per CU (+2.5-4.6 % at 24-32 KiB);
  // up to 16 KiB: one workgroup per row, at most 3 per CU for rows of 4-8 KiB,
  // shorter and longer ones uncapped.
  const uint64_t row_bytes = hidden * sz;
  // chunk_bytes below the row length asks for the split-row kernels, whose
  // pieces are one vector per lane: 4 KiB per rank.  By default rows of at
  // least 8 KiB per rank take them at P >= 8 (bf16, 2 GiB of input: +1-9 %
  // on 8 KiB rows, +8-13 % on 16 KiB rows, +3-10 % on 24-32 KiB rows at
  // P = 8 and 12).  They move 1/P of the data twice more, which loses at
  // P <= 4 and sits within the run-to-run spread at P = 6 (-3 % to +4 %).
  const uint64_t max_pieces = uint64_t(1) << 31;
  bool split = false;
  if (l.chunk_set && l.chunk_bytes < row_bytes) {
    if (l.chunk_bytes != ccl::kSplitPieceBytes || (l.stages_set && l.stages != 1))
      return CCL_ERR_UNSUPPORTED;
    if (rows * ccl::rms_split_pieces(row_bytes) > max_pieces) return CCL_ERR_UNSUPPORTED;
    split = true;
  } else if (!l.chunk_set && !l.stages_set && nranks >= 8 && row_bytes >= 8192 &&
             rows * ccl::rms_split_pieces(row_bytes) <= max_pieces) {
    split = true;
  }
  // Their norm pass writes through past 256 MiB per rank, where every output
  // row starts on a 256-byte line (P = 8, 384 MiB per rank: +4-17 % over
  // nontemporal stores; at 256 MiB per rank the two are equal).
  if (split && !l.store_pol_set && rows * row_bytes > (uint64_t(256) << 20) &&
      row_bytes % 256 == 0) {
    bool lines = true;
    for (int q = 0; q < nranks; ++q) lines = lines && (uintptr_t)recv[q] % 256 == 0;
    l.store_wt = lines;
  } else if (split && !l.store_pol_set) {
    l.store_wt = false;
  }
  if (split) l.store_pol_set = true;
  // One-pass forms: rows longer than 16 KiB take the row-pipelined kernel at
  // P >= 6 (+1-5 % at 24-32 KiB); below P = 6 it loses up to 25 % to one
  // workgroup per row.
  if (!l.stages_set) l.stages = (row_bytes > 16384 && nranks >= 6) ? 2 : 1;
  if (!l.occupancy_set) {
    if (split) {
      l.occupancy = 4;   // fold pass
      l.occupancy2 = 2;  // norm pass
    } else if (l.stages == 2) {
      l.occupancy = 1;
    } else {
      l.occupancy = (row_bytes >= 4096 && row_bytes <= 8192) ? 3 : 0;
    }
  } else {
    l.occupancy2 = l.occupancy;
  }
  void *part = nullptr;
  if (split && noalloc) {
    if (ccl::rms_split_scratch_bytes(rows, row_bytes) > ccl::kNoAllocScratchBytes)
      return CCL_ERR_SCRATCH_LIMIT;
    if ((st = ccl::noalloc_scratch(&part))) return st;
  }
  ccl::RmsDesc d{nranks, dtype, rows, hidden, eps, send, recv, gamma};
  return ccl::launch_ar_rmsnorm(d, l, (hipStream_t)stream, split, part);
}

}  // namespace

extern "C" {

ccl_status_t ccl_all_reduce_rmsnorm(const void *const *send, void *const *recv, int nranks,
                                    size_t rows, size_t hidden, const void *gamma, float eps,
                                    int dtype, void *stream, const ccl_launch_config_t *cfg) {
  return ar_rmsnorm(send, recv, nranks, rows, hidden, gamma, eps, dtype, stream, cfg, false);
}

ccl_status_t ccl_all_reduce_rmsnorm_noalloc(const void *const *send, void *const *recv,
                                            int nranks, size_t rows, size_t hidden,
                                            const void *gamma, float eps, int dtype, void *stream,
                                            const ccl_launch_config_t *cfg) {
  return ar_rmsnorm(send, recv, nranks, rows, hidden, gamma, eps, dtype, stream, cfg, true);
}

ccl_status_t ccl_reduce(const void *const *send, void *recv, int nranks, size_t count, int dtype,
                        int op, int root, void *stream, const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_RS, nranks, &l);
  if (st) return st;
  if (nranks < 1 || nranks > CCL_MAX_RANKS || dtype_size(dtype) == 0 || !op_ok(op) || root < 0 ||
      root >= nranks)
    return CCL_ERR_INVALID_ARG;
  if (count == 0) return CCL_OK;
  void *const recv1[1] = {recv};
  if (!send || !recv || (uintptr_t)recv % (uintptr_t)dtype_size(dtype)) return CCL_ERR_INVALID_ARG;
  for (int r = 0; r < nranks; ++r)
    if (!send[r] || (uintptr_t)send[r] % (uintptr_t)dtype_size(dtype)) return CCL_ERR_INVALID_ARG;
  const uint64_t sz = dtype_size(dtype);
  if (mul_overflows(count, sz)) return CCL_ERR_INVALID_ARG;
  const uint64_t bytes = count * sz;
  for (int r = 0; r < nranks; ++r) {
    Range y{(uintptr_t)recv, (uintptr_t)recv + bytes};
    Range x{(uintptr_t)send[r], (uintptr_t)send[r] + bytes};
    if (overlap(x, y) && x.lo != y.lo) return CCL_ERR_ALIASING;
  }
  ccl::CollDesc d{ccl::KIND_RS, nranks, dtype, op, count, send, recv1, true};
  return ccl::launch_collective(d, l, (hipStream_t)stream);
}

ccl_status_t ccl_broadcast(const void *send, void *const *recv, int nranks, size_t count,
                           int dtype, int root, void *stream, const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_AG, nranks, &l);
  if (st) return st;
  if (nranks < 1 || nranks > CCL_MAX_RANKS || dtype_size(dtype) == 0 || root < 0 ||
      root >= nranks)
    return CCL_ERR_INVALID_ARG;
  if (count == 0) return CCL_OK;
  const void *const send1[1] = {send};
  if (!send || !recv || (uintptr_t)send % (uintptr_t)dtype_size(dtype)) return CCL_ERR_INVALID_ARG;
  for (int q = 0; q < nranks; ++q)
    if (!recv[q] || (uintptr_t)recv[q] % (uintptr_t)dtype_size(dtype)) return CCL_ERR_INVALID_ARG;
  const uint64_t sz = dtype_size(dtype);
  if (mul_overflows(count, sz)) return CCL_ERR_INVALID_ARG;
  const uint64_t bytes = count * sz;
  if ((st = check_outputs_disjoint(recv, nranks, bytes))) return st;
  for (int q = 0; q < nranks; ++q) {
    Range y{(uintptr_t)recv[q], (uintptr_t)recv[q] + bytes};
    Range x{(uintptr_t)send, (uintptr_t)send + bytes};
    if (overlap(x, y) && x.lo != y.lo) return CCL_ERR_ALIASING;
  }
  ccl::CollDesc d{ccl::KIND_AG, nranks, dtype, CCL_SUM, count, send1, recv, true};
  return ccl::launch_collective(d, l, (hipStream_t)stream);
}

ccl_status_t ccl_reshard_copy(const ccl_plan_t *plan, const void *const *src_bufs,
                              void *const *dst_bufs, void *stream,
                              const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_RESHARD, 0, &l);
  if (st) return st;
  if (!plan || !src_bufs || !dst_bufs) return CCL_ERR_INVALID_ARG;
  ccl_plan *p = const_cast<ccl_plan *>(plan);
  const uintptr_t align = (uintptr_t)p->elem_size;
  for (int i = 0; i < p->n_src; ++i)
    if (p->src_local_bytes[i] && (!src_bufs[i] || (uintptr_t)src_bufs[i] % align))
      return CCL_ERR_INVALID_ARG;
  for (int i = 0; i < p->n_dst; ++i)
    if (p->dst_local_bytes[i] && (!dst_bufs[i] || (uintptr_t)dst_bufs[i] % align))
      return CCL_ERR_INVALID_ARG;
  for (int a = 0; a < p->n_dst; ++a) {
    Range ra{(uintptr_t)dst_bufs[a], (uintptr_t)dst_bufs[a] + p->dst_local_bytes[a]};
    if (ra.lo == ra.hi) continue;
    for (int b = a + 1; b < p->n_dst; ++b) {
      Range rb{(uintptr_t)dst_bufs[b], (uintptr_t)dst_bufs[b] + p->dst_local_bytes[b]};
      if (rb.lo != rb.hi && overlap(ra, rb)) return CCL_ERR_ALIASING;
    }
    for (int s = 0; s < p->n_src; ++s) {
      Range rs{(uintptr_t)src_bufs[s], (uintptr_t)src_bufs[s] + p->src_local_bytes[s]};
      if (rs.lo != rs.hi && overlap(ra, rs)) return CCL_ERR_ALIASING;
    }
  }
  if (p->intervals.empty()) return CCL_OK;
  // Default shape by replica count (measured on MI355X over six layouts with
  // 4 to 32768 intervals): with one replica per destination shard, 16 KiB
  // chunks and at most 4 workgroups per CU (5-17 % over the general
  // default); with two or more, the source is loaded without the
  // nontemporal hint while the stores keep it (1-4 %).  With four or more
  // replicas the stores write through (+7.5-9.6 % at rho = 4 and +3.3-4.2 %
  // at rho = 8 on two tensors, level at rho <= 3), where every destination
  // chunk starts on a 256-byte line: partial lines written through cost more
  // than they save.
  const int rho = p->n_dst / p->n_dst_shards;
  if (rho == 1) {
    if (!l.chunk_set) l.chunk_bytes = 16384;
    if (!l.occupancy_set) l.occupancy = 4;
  } else if (!l.nt_set) {
    l.nt_load = false;
  }
  if (!l.store_pol_set) {
    bool lines = rho >= 4 && p->dst_offsets_aligned256 && l.chunk_bytes % 256 == 0;
    for (int i = 0; i < p->n_dst && lines; ++i) lines = (uintptr_t)dst_bufs[i] % 256 == 0;
    l.store_wt = lines;
    l.store_pol_set = true;
  }
  return ccl::reshard_launch(p, src_bufs, dst_bufs, l, (hipStream_t)stream);
}

ccl_status_t ccl_reshard_copy_fp8(const ccl_plan_t *plan, const void *const *src_bufs,
                                  void *const *dst_codes, float *const *dst_scales, void *stream,
                                  const ccl_launch_config_t *cfg) {
  ccl::Launch l;
  ccl_status_t st = ccl::resolve_launch(cfg, ccl::OP_RESHARD_FP8, 0, &l);
  if (st) return st;
  if (!plan || !src_bufs || !dst_codes || !dst_scales) return CCL_ERR_INVALID_ARG;
  ccl_plan *p = const_cast<ccl_plan *>(plan);
  if (p->dtype != CCL_FLOAT32 && p->dtype != CCL_BFLOAT16 && p->dtype != CCL_FLOAT16)
    return CCL_ERR_UNSUPPORTED;
  if (!p->fp8_blocks_ok || !p->offsets_aligned16) return CCL_ERR_UNSUPPORTED;
  const uint64_t esz = (uint64_t)p->elem_size;
  std::vector<Range> outs;
  for (int i = 0; i < p->n_src; ++i)
    if (p->src_local_bytes[i] && (!src_bufs[i] || (uintptr_t)src_bufs[i] % ccl::kVecBytes))
      return src_bufs[i] ? CCL_ERR_UNSUPPORTED : CCL_ERR_INVALID_ARG;
  for (int i = 0; i < p->n_dst; ++i) {
    const uint64_t n = p->dst_local_bytes[i] / esz;
    if (!n) continue;
    if (!dst_codes[i] || !dst_scales[i]) return CCL_ERR_INVALID_ARG;
    if ((uintptr_t)dst_codes[i] % ccl::kVecBytes) return CCL_ERR_UNSUPPORTED;
    if ((uintptr_t)dst_scales[i] % sizeof(float)) return CCL_ERR_INVALID_ARG;
    outs.push_back({(uintptr_t)dst_codes[i], (uintptr_t)dst_codes[i] + n});
    outs.push_back({(uintptr_t)dst_scales[i], (uintptr_t)dst_scales[i] + (n + 127) / 128 * 4});
  }
  for (size_t a = 0; a < outs.size(); ++a) {
    for (size_t b = a + 1; b < outs.size(); ++b)
      if (overlap(outs[a], outs[b])) return CCL_ERR_ALIASING;
    for (int s = 0; s < p->n_src; ++s) {
      Range rs{(uintptr_t)src_bufs[s], (uintptr_t)src_bufs[s] + p->src_local_bytes[s]};
      if (rs.lo != rs.hi && overlap(outs[a], rs)) return CCL_ERR_ALIASING;
    }
  }
  if (p->intervals.empty()) return CCL_OK;
  return ccl::reshard_fp8_launch(p, src_bufs, dst_codes, dst_scales, l, (hipStream_t)stream);
}

}  // extern "C"
