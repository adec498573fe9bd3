// Internal declarations shared by the libccl translation units.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#include "ccl.h"

namespace ccl {

constexpr int kVecBytes = 16;          // one dwordx4 per lane
constexpr int kThreads = 256;          // register-direct workgroup: 4 wave64s
constexpr int kLdsTileBytes = 4096;    // LDS pipeline: per-rank bytes per stage
// Launch defaults, from the launch sweep over chunk bytes, unroll, LDS stages
// and resident workgroups per CU on MI355X (2 GiB of input spread over P
// ranks, bf16).  The common thread: with 2P buffers streaming at once, capping
// residency keeps few DRAM pages open; with few buffers each workgroup has
// little in flight, so the cap is looser.
struct OpDefaults {
  uint64_t chunk_bytes;
  int stages;
  int unroll;
  int occupancy;
};

enum Op { OP_AR = 0, OP_RS = 1, OP_AG = 2, OP_RESHARD = 3, OP_RMSNORM = 4, OP_RESHARD_FP8 = 5 };

inline OpDefaults default_launch(Op op, int P) {
  switch (op) {
    case OP_AR:
      if (P == 1) return {8192, 1, 1, 8};
      if (P == 2) return {8192, 1, 2, 8};
      if (P <= 4) return {4096, 1, 1, 6};
      return {4096, 1, 1, 3};
    case OP_RS:
      if (P <= 2) return {8192, 1, 2, 4};
      if (P >= 9 && P <= 12) return {4096, 1, 1, 4};
      return {8192, 1, 2, 3};
    case OP_AG:
      if (P <= 2) return {8192, 1, 2, 4};
      if (P == 3) return {8192, 1, 2, 3};
      if (P <= 8) return {4096, 1, 1, 4};
      return {4096, 1, 1, 3};
    case OP_RMSNORM:
      return {16384, 1, 1, 0};
    case OP_RESHARD_FP8:
      return {32768, 1, 2, 0};
    default:
      return {32768, 1, 4, 2};
  }
}

inline int dtype_size(int dt) {
  switch (dt) {
    case CCL_FLOAT32: return 4;
    case CCL_BFLOAT16: return 2;
    case CCL_INT32: return 4;
    case CCL_FLOAT16: return 2;
    default: return 0;
  }
}

enum Kind { KIND_AR = 0, KIND_RS = 1, KIND_AG = 2 };

// A fully resolved launch configuration.
struct Launch {
  uint64_t chunk_bytes;
  int workgroups;  // 0 = derive from the chunk count
  int stages;      // 1 = register-direct, 2..4 = LDS pipeline
  int unroll;      // 1 or 2
  bool nt_load;
  bool nt_store;
  int occupancy;   // max resident workgroups per CU, 0 = no cap
  int occupancy2 = 0;  // the split-row RMSNorm's second (norm) pass
  bool chunk_set = false;      // chunk_bytes came from the caller
  bool unroll_set = false;     // unroll came from the caller
  bool stages_set = false;     // stages came from the caller
  bool occupancy_set = false;  // occupancy came from the caller
  bool nt_set = false;         // nontemporal hints came from the caller
  bool store_wt = true;        // nontemporal stores write through (st_wt)
  bool store_pol_set = false;  // store_wt came from the caller
};

// Dynamic LDS to request so that at most `occupancy` workgroups fit on a CU
// alongside `static_lds` bytes of their own; 0 when there is no cap.
inline size_t occupancy_lds(int occupancy, size_t static_lds) {
  constexpr size_t kLdsPerCu = 160 * 1024;
  if (occupancy <= 0) return 0;
  size_t per_wg = kLdsPerCu / (size_t)occupancy;
  per_wg &= ~size_t(511);
  return per_wg > static_lds ? per_wg - static_lds : 0;
}

// Collective launch description, all checks already passed.
struct CollDesc {
  Kind kind;
  int P;
  int dtype;
  int op;
  uint64_t seg_elems;  // AR: count, RS: recvcount, AG: sendcount
  const void *const *send;
  void *const *recv;
  bool single;         // one segment: reduce (KIND_RS) or broadcast (KIND_AG)
};

// Compute units of a device (cached after the first query); <= 0 on error.
int device_cu_count(int dev);

ccl_status_t resolve_launch(const ccl_launch_config_t *cfg, Op op, int P, Launch *out);

ccl_status_t launch_collective(const CollDesc &d, const Launch &l, hipStream_t stream);

// All-reduce with a row-wise RMSNorm between its halves, all checks passed.
struct RmsDesc {
  int P;
  int dtype;
  uint64_t rows;
  uint64_t hidden;
  float eps;
  const void *const *send;
  void *const *recv;
  const void *gamma;
};
constexpr int kRmsMaxRowVecs = 8 * kThreads;  // 16-byte vectors per row
// Split-row form: rows cut into pieces of one vector per lane (4 KiB per
// rank), a fold pass and a norm pass with one workgroup per piece each; the
// passes hand over one fp32 partial sum of squares per piece through device
// scratch.
constexpr uint64_t kSplitPieceBytes = (uint64_t)kThreads * kVecBytes;
inline uint64_t rms_split_pieces(uint64_t row_bytes) {
  return (row_bytes + kSplitPieceBytes - 1) / kSplitPieceBytes;
}
inline uint64_t rms_split_scratch_bytes(uint64_t rows, uint64_t row_bytes) {
  return rows * rms_split_pieces(row_bytes) * sizeof(float);
}
// split: run the split-row kernels.  Their partial sums go to part_buf when
// given (at least rms_split_scratch_bytes), else to the calling stream's own
// buffer, which the library allocates on first use and keeps.
ccl_status_t launch_ar_rmsnorm(const RmsDesc &d, const Launch &l, hipStream_t stream, bool split,
                               void *part_buf = nullptr);
// The no-allocation entry point's fixed scratch (CCL_NOALLOC_SCRATCH_BYTES)
// on the current device: its device address, looked up on first use.
constexpr size_t kNoAllocScratchBytes = CCL_NOALLOC_SCRATCH_BYTES;
ccl_status_t noalloc_scratch(void **out);

// ------------------------------------------------------------------ reshard

struct PlanInterval {
  int32_t src_local;   // index of the source rank inside the source mesh
  int32_t dst_shard;   // destination shard
  int32_t leader;      // global rank of the leading replica
  uint64_t src_off;    // bytes
  uint64_t dst_off;    // bytes
  uint64_t len;        // bytes
};

struct DevicePlanCache {
  int device = -1;
  void *table = nullptr;  // device copy of the interval, replica and chunk tables
  void *staging = nullptr;  // pinned host copy the upload reads (lives with the plan)
  hipEvent_t uploaded = nullptr;  // recorded on the uploading stream after the copy
  hipStream_t upload_stream = nullptr;
  bool upload_done = false;       // the event has been seen complete
  size_t rep_offset = 0;       // byte offset of the replica table
  size_t chunk_iv_offset = 0;  // byte offset of the chunk -> interval table (0: none)
  uint64_t chunk_bytes = 0;
  uint64_t total_chunks = 0;
};

}  // namespace ccl

struct ccl_plan {
  int32_t elem_size;
  int32_t dtype;
  int32_t src_start, dst_start;
  int32_t n_src, n_dst;                 // ranks in each mesh
  int32_t n_dst_shards;
  std::vector<uint64_t> src_local_bytes;  // per source-mesh rank
  std::vector<uint64_t> dst_local_bytes;  // per destination-mesh rank
  std::vector<std::vector<int32_t>> replicas;  // per dst shard: local dst indices, ascending
  std::vector<ccl::PlanInterval> intervals;
  bool offsets_aligned16 = true;         // every interval offset is a multiple of 16
  bool dst_offsets_aligned256 = true;    // every interval's destination offset is a multiple of 256
  bool fp8_blocks_ok = true;             // every 128-element destination block lies in one interval
  // Device-side state, created on first use.
  std::mutex mu;
  std::vector<ccl::DevicePlanCache> dev;
};

namespace ccl {
ccl_status_t reshard_launch(ccl_plan *plan, const void *const *src, void *const *dst,
                            const Launch &l, hipStream_t stream);
ccl_status_t reshard_fp8_launch(ccl_plan *plan, const void *const *src, void *const *codes,
                                float *const *scales, const Launch &l, hipStream_t stream);
void reshard_release(ccl_plan *plan);
}  // namespace ccl
