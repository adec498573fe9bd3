// Collective kernels for gfx950 (templates, included by ccl_coll_inst.hip): all-reduce, reduce-scatter (shard-in) and
// all-gather (shard-out) over P rank buffers resident in one GPU's HBM.
//
// Method (the "NCCL M2N vs T-CCL" digest, lqnn.cn news 207677):
//   s2.2  shard-in: the owner of a shard loads every rank's contribution and
//         reduces it locally -- no atomics, no reduction in memory.
//         shard-out: the owner loads its final shard once and stores that
//         copy to every destination.
//   s2.3  the logical tensor is cut into P shards, one per rank; each shard
//         is processed as a series of chunks.
//   s2.5  all-reduce = shard-in followed by shard-out.  On one GPU the two
//         fuse: the reduced value stays in VGPRs and is stored P times.
//
// Work decomposition.  A call is a list of "segments" (AR: one segment of
// `count` elements; RS: segment s = shard s; AG: segment s = rank s's shard).
// Each segment is cut into chunks of chunk_bytes per rank buffer; chunks are
// dealt to workgroups round-robin.  Inside a chunk every lane owns whole
// 16-byte vectors, so each output element has exactly one writer.  The
// register-direct kernel keeps `U` vectors per rank in flight per lane (P*U
// dwordx4 loads issued before the first fold) and folds in fp32 in rank
// order 0..P-1.  Segments whose buffers are not 16-byte aligned alike peel a
// scalar head and tail (< 8 elements each); buffers misaligned relative to
// each other use an element-wise kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "ccl_device.h"
#include "ccl_internal.h"

namespace ccl {

struct CollArgs {
  const char *in[CCL_MAX_RANKS];
  char *out[CCL_MAX_RANKS];
  uint64_t nvec[CCL_MAX_RANKS];   // 16-byte vectors in the body of segment s
  uint32_t head[CCL_MAX_RANKS];   // scalar elements before the body of segment s
  // shift[s][r]: byte offset, mod 16, of input r's element at the start of
  // segment s's vector body (the outputs are 16-byte aligned there).
  uint8_t shift[CCL_MAX_RANKS][CCL_MAX_RANKS];
  uint64_t seg_elems;             // M
  uint64_t chunk_vecs;
  uint64_t chunks_per_seg;
  uint64_t total_chunks;
  int P;
  // bit 0: nontemporal loads, bit 1: nontemporal stores, bit 2: those stores
  // write-through (register-direct kernel and LDS pipeline; the host sets it
  // only for chunks of at most 1 GiB)
  int flags;
};

// Which kernel family a launch uses, with its resolved launch shape.
enum CollPathKind { PATH_VEC = 0, PATH_LDS = 1, PATH_REALIGN = 2, PATH_SCALAR = 3 };

struct CollPath {
  int path;        // CollPathKind
  int op;          // ccl_op_t (ignored by copies)
  int unroll;      // register-direct vectors per lane per rank
  int stages;      // LDS ring depth
  int occupancy;   // resident workgroups per CU cap (0 = none)
  unsigned grid;
  size_t lds;      // dynamic LDS reserved to enforce the occupancy cap
  int nseg;        // segments (element-wise kernel only)
};

// One entry point per (kind, element type), each built in its own object.
hipError_t dispatch_ar_f32(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_ar_bf16(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_ar_f16(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_ar_i32(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_rs_f32(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_rs_bf16(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_rs_f16(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_rs_i32(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_ag_b16(const CollArgs &, const CollPath &, hipStream_t);
hipError_t dispatch_ag_b32(const CollArgs &, const CollPath &, hipStream_t);

namespace {

// Address of input r / output q of segment s, element e.
template <int KIND>
__device__ __forceinline__ const char *in_at(const CollArgs &a, int s, int r, uint64_t e,
                                             int esz) {
  if constexpr (KIND == KIND_AR) return a.in[r] + e * esz;
  else if constexpr (KIND == KIND_RS) return a.in[r] + ((uint64_t)s * a.seg_elems + e) * esz;
  else return a.in[s] + e * esz;
}

template <int KIND>
__device__ __forceinline__ char *out_at(const CollArgs &a, int s, int q, uint64_t e, int esz) {
  if constexpr (KIND == KIND_AR) return a.out[q] + e * esz;
  else if constexpr (KIND == KIND_RS) return a.out[s] + e * esz;
  else return a.out[q] + ((uint64_t)s * a.seg_elems + e) * esz;
}

// One element, any alignment: fold the inputs, store to every output.
template <int KIND, int DT, int OP>
__device__ __forceinline__ void scalar_element(const CollArgs &a, int s, uint64_t e) {
  constexpr int esz = (DT == CCL_BFLOAT16 || DT == CCL_FLOAT16) ? 2 : 4;
  const int ni = KIND == KIND_AG ? 1 : a.P;
  const int no = KIND == KIND_RS ? 1 : a.P;
  if constexpr (KIND == KIND_AG) {
    if constexpr (esz == 2) {
      const uint16_t v = *(const uint16_t *)in_at<KIND>(a, s, 0, e, esz);
      for (int q = 0; q < no; ++q) *(uint16_t *)out_at<KIND>(a, s, q, e, esz) = v;
    } else {
      const uint32_t v = *(const uint32_t *)in_at<KIND>(a, s, 0, e, esz);
      for (int q = 0; q < no; ++q) *(uint32_t *)out_at<KIND>(a, s, q, e, esz) = v;
    }
  } else if constexpr (DT == CCL_FLOAT16) {
    float acc = f16_lo(*(const uint16_t *)in_at<KIND>(a, s, 0, e, esz));
    for (int r = 1; r < ni; ++r)
      acc = fold_f32<OP>(acc, f16_lo(*(const uint16_t *)in_at<KIND>(a, s, r, e, esz)));
    const uint16_t y = (uint16_t)f16_rne(acc);
    for (int q = 0; q < no; ++q) *(uint16_t *)out_at<KIND>(a, s, q, e, esz) = y;
  } else if constexpr (DT == CCL_BFLOAT16) {
    float acc = bf16_lo(*(const uint16_t *)in_at<KIND>(a, s, 0, e, esz));
    for (int r = 1; r < ni; ++r)
      acc = fold_f32<OP>(acc, bf16_lo(*(const uint16_t *)in_at<KIND>(a, s, r, e, esz)));
    const uint16_t y = (uint16_t)bf16_rne(acc);
    for (int q = 0; q < no; ++q) *(uint16_t *)out_at<KIND>(a, s, q, e, esz) = y;
  } else if constexpr (DT == CCL_FLOAT32) {
    float acc = *(const float *)in_at<KIND>(a, s, 0, e, esz);
    for (int r = 1; r < ni; ++r) acc = fold_f32<OP>(acc, *(const float *)in_at<KIND>(a, s, r, e, esz));
    for (int q = 0; q < no; ++q) *(float *)out_at<KIND>(a, s, q, e, esz) = acc;
  } else {
    int32_t acc = *(const int32_t *)in_at<KIND>(a, s, 0, e, esz);
    for (int r = 1; r < ni; ++r)
      acc = fold_i32<OP>(acc, *(const int32_t *)in_at<KIND>(a, s, r, e, esz));
    for (int q = 0; q < no; ++q) *(int32_t *)out_at<KIND>(a, s, q, e, esz) = acc;
  }
}

// Waves per SIMD the register-direct kernel must leave room for, from the
// VGPRs its in-flight loads need (U x inputs x 4).  Without a target the
// register allocator sometimes takes nearly all 256 VGPRs for a small body
// (fp32 / fp16 / int32 all-reduce at P = 8, U = 1: 239 VGPRs plus 32 AGPRs of
// copies), which leaves one wave per SIMD and a third of the bandwidth.
template <int KIND, int PMAX, int U>
struct VecWaves {
  static constexpr int loads = U * (KIND == KIND_AG ? 1 : PMAX) * 4;
  static constexpr int value = loads <= 64 ? 4 : loads <= 160 ? 2 : 1;
};

// Register-direct kernel.  PMAX bounds P at compile time so every load of a
// lane's U x P vectors is issued before the first fold.
// WT: write-through stores (st_wt) as a compile-time choice, so that the
// nontemporal / plain kernel stays exactly what it is without them (a runtime
// branch among the three store paths slowed the nontemporal one).
//
// Cache hints.  With P nontemporal streams in flight, keeping exactly one of
// them on the default (cacheable) policy measured several percent faster
// than none and than two.  In the nontemporal paths below, slot 0 is that
// stream:
//  - reduce-scatter, reduce, all-gather and broadcast: input 0's loads;
//  - all-reduce: output 0's stores (the host puts the last output there);
//  - all-reduce with write-through stores: input 0's loads instead;
//  - all-reduce with two vectors per lane in flight (U = 2): input and output
//    (one cacheable stream ran 6 % slower than the two there).
// The nontemporal and the plain path of a group sit on the two sides of a
// branch on a run-time flag.  Left alone, the compiler treats a nontemporal
// access and a plain one to the same address there as one plain access, for
// whichever accesses it happens to merge.  An empty volatile asm statement
// (it emits nothing) at each end of a nontemporal group keeps them apart.
template <int KIND, int DT, int OP, int PMAX, int U, bool WT>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(VecWaves<KIND, PMAX, U>::value)))
    coll_vec_kernel(CollArgs a) {
  constexpr int esz = (DT == CCL_BFLOAT16 || DT == CCL_FLOAT16) ? 2 : 4;
  constexpr int V = kVecBytes / esz;  // elements per vector
  constexpr int NI = KIND == KIND_AG ? 1 : PMAX;
  constexpr int NO = KIND == KIND_RS ? 1 : PMAX;
  const int P = a.P;
  const int ni = KIND == KIND_AG ? 1 : P;
  const int no = KIND == KIND_RS ? 1 : P;
  const bool ntl = a.flags & 1, nts = a.flags & 2;
  // compile-time: which slot-0 stream stays cacheable (see above)
  constexpr bool pin0 = KIND != KIND_AR || WT || U > 1;
  constexpr bool pout0 = KIND == KIND_AR;
  // An all-reduce with U = 2 and nontemporal stores keeps the last rank's
  // input cacheable (it measured 1-3 % ahead of rank 0's): slot 0 loads rank
  // P - 1 and slot r rank r - 1, and the fold takes the slots in rank order.
  constexpr bool rot = KIND == KIND_AR && U > 1 && !WT;

  for (uint64_t c = blockIdx.x; c < a.total_chunks; c += gridDim.x) {
    const int s = (int)(c / a.chunks_per_seg);
    const uint64_t lc = c - (uint64_t)s * a.chunks_per_seg;
    const uint64_t nv = a.nvec[s];
    const uint64_t head = a.head[s];
    if (lc == 0) {
      // Scalar head and tail of the segment (fewer than V elements each).
      const uint64_t tail0 = head + nv * V;
      const uint64_t ntail = a.seg_elems - tail0;
      const uint64_t t = threadIdx.x;
      if (t < head) scalar_element<KIND, DT, OP>(a, s, t);
      else if (t - head < ntail) scalar_element<KIND, DT, OP>(a, s, tail0 + (t - head));
    }
    const uint64_t v0 = lc * a.chunk_vecs;
    const uint64_t v1 = min(v0 + a.chunk_vecs, nv);
    const char *ib[NI];
    char *ob[NO];
#pragma unroll
    for (int r = 0; r < NI; ++r)
      ib[r] = r >= ni ? nullptr
                      : in_at<KIND>(a, s, !rot ? r : r == 0 ? ni - 1 : r - 1, head, esz);
#pragma unroll
    for (int q = 0; q < NO; ++q) ob[q] = q < no ? out_at<KIND>(a, s, q, head, esz) : nullptr;

#pragma unroll 1  // U alone sets the vectors per rank a lane has in flight
    for (uint64_t v = v0 + threadIdx.x; v < v1; v += (uint64_t)kThreads * U) {
      // Every element of x is assigned on every path (zero where there is no
      // rank or no vector), so no value has to survive from the previous
      // iteration; otherwise the compiler carries all of them along and the
      // small fp32 / int32 bodies took ~240 VGPRs (one wave per SIMD).
      u32x4 x[U][NI];
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vv = v + (uint64_t)u * kThreads;
        const bool live = vv < v1;
        if (ntl) {
          // the cacheable slot-0 load goes last, after the hinted ones
          asm volatile("");
#pragma unroll
          for (int r = pin0 ? 1 : 0; r < NI; ++r)
            x[u][r] = (live && r < ni) ? ld_nt(ib[r] + vv * kVecBytes) : zero;
          asm volatile("");
          if constexpr (pin0) x[u][0] = live ? ld_plain(ib[0] + vv * kVecBytes) : zero;
        } else {
#pragma unroll
          for (int r = 0; r < NI; ++r)
            x[u][r] = (live && r < ni) ? ld_plain(ib[r] + vv * kVecBytes) : zero;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vv = v + (uint64_t)u * kThreads;
        if (vv < v1) {
          u32x4 y;
          if constexpr (KIND == KIND_AG) y = x[u][0];
          else if constexpr (!rot) y = fold_vec<DT, OP, NI>(x[u], ni);
          else {
            // back in rank order: slot r + 1 holds rank r, slot 0 rank ni - 1
            u32x4 xr[NI];
#pragma unroll
            for (int r = 0; r < NI; ++r) {
              const int next = r + 1 < NI ? r + 1 : 0;  // in bounds at compile time
              xr[r] = r + 1 < ni ? x[u][next] : x[u][0];
            }
            y = fold_vec<DT, OP, NI>(xr, ni);
          }
          if constexpr (WT) {
#pragma unroll
            for (int q = 0; q < NO; ++q)
              if (q < no) st_wt(ob[q] + v0 * kVecBytes, (vv - v0) * kVecBytes, y);
          } else if (nts) {
            // the cacheable slot-0 store goes last, after the hinted ones
            asm volatile("");
#pragma unroll
            for (int q = pout0 ? 1 : 0; q < NO; ++q)
              if (q < no) st_nt(ob[q] + vv * kVecBytes, y);
            asm volatile("");
            if constexpr (pout0) st_plain(ob[0] + vv * kVecBytes, y);
          } else {
#pragma unroll
            for (int q = 0; q < NO; ++q)
              if (q < no) st_plain(ob[q] + vv * kVecBytes, y);
          }
        }
      }
    }
  }
}

// Realigning kernel: the outputs of each segment are 16-byte aligned at the
// vector body, inputs may sit at any even byte offset from them.  An input at
// offset d is read as the two aligned 16-byte blocks that cover its 16 bytes
// and the wanted bytes are funnel-shifted out with v_alignbyte.  Both blocks
// contain at least one byte of the input range, so neither leaves the pages
// the input lives in.
__device__ __forceinline__ uint32_t pick4(int q, uint32_t w0, uint32_t w1, uint32_t w2,
                                          uint32_t w3) {
  return q == 0 ? w0 : q == 1 ? w1 : q == 2 ? w2 : w3;
}

__device__ __forceinline__ u32x4 realign16(u32x4 A, u32x4 B, int d) {
  const int q = d >> 2;
  const unsigned r = (unsigned)(d & 3);
  const uint32_t w[8] = {A[0], A[1], A[2], A[3], B[0], B[1], B[2], B[3]};
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = pick4(q, w[j], w[j + 1], w[j + 2], w[j + 3]);
    const uint32_t hi = pick4(q, w[j + 1], w[j + 2], w[j + 3], w[j + 4]);
    o[j] = __builtin_amdgcn_alignbyte(hi, lo, r);
  }
  return o;
}

template <int KIND, int DT, int OP, int PMAX>
__global__ void __launch_bounds__(kThreads) coll_realign_kernel(CollArgs a) {
  constexpr int esz = (DT == CCL_BFLOAT16 || DT == CCL_FLOAT16) ? 2 : 4;
  constexpr int V = kVecBytes / esz;
  constexpr int NI = KIND == KIND_AG ? 1 : PMAX;
  constexpr int NO = KIND == KIND_RS ? 1 : PMAX;
  const int P = a.P;
  const int ni = KIND == KIND_AG ? 1 : P;
  const int no = KIND == KIND_RS ? 1 : P;
  const bool ntl = a.flags & 1, nts = a.flags & 2;

  for (uint64_t c = blockIdx.x; c < a.total_chunks; c += gridDim.x) {
    const int s = (int)(c / a.chunks_per_seg);
    const uint64_t lc = c - (uint64_t)s * a.chunks_per_seg;
    const uint64_t nv = a.nvec[s];
    const uint64_t head = a.head[s];
    if (lc == 0) {
      const uint64_t tail0 = head + nv * V;
      const uint64_t ntail = a.seg_elems - tail0;
      const uint64_t t = threadIdx.x;
      if (t < head) scalar_element<KIND, DT, OP>(a, s, t);
      else if (t - head < ntail) scalar_element<KIND, DT, OP>(a, s, tail0 + (t - head));
    }
    const uint64_t v0 = lc * a.chunk_vecs;
    const uint64_t v1 = min(v0 + a.chunk_vecs, nv);
    const char *ib[NI];
    int sh[NI];
    char *ob[NO];
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      sh[r] = r < ni ? a.shift[s][r] : 0;
      ib[r] = r < ni ? in_at<KIND>(a, s, r, head, esz) - sh[r] : nullptr;  // aligned block
    }
#pragma unroll
    for (int q = 0; q < NO; ++q) ob[q] = q < no ? out_at<KIND>(a, s, q, head, esz) : nullptr;

    for (uint64_t v = v0 + threadIdx.x; v < v1; v += kThreads) {
      u32x4 x[NI];
      if constexpr (KIND == KIND_RS) {
        // Reduce-scatter (P inputs, one output): every rank's two blocks are
        // requested before the first one is realigned, so the P round trips
        // overlap.  Without a shift the second block repeats the first (the
        // block after it may lie outside the input).  The nontemporal choice
        // is made once around compile-time loads, since a load picked at run
        // time is merged into a plain one.
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 A[NI], B[NI];
        if (ntl) {
#pragma unroll
          for (int r = 0; r < NI; ++r) {
            A[r] = r < ni ? ld<true>(ib[r] + v * kVecBytes) : zero;
            B[r] = r < ni ? ld<true>(ib[r] + v * kVecBytes + (sh[r] ? kVecBytes : 0)) : zero;
          }
        } else {
#pragma unroll
          for (int r = 0; r < NI; ++r) {
            A[r] = r < ni ? ld<false>(ib[r] + v * kVecBytes) : zero;
            B[r] = r < ni ? ld<false>(ib[r] + v * kVecBytes + (sh[r] ? kVecBytes : 0)) : zero;
          }
        }
#pragma unroll
        for (int r = 0; r < NI; ++r) x[r] = r < ni ? realign16(A[r], B[r], sh[r]) : zero;
      } else {
        // All-reduce and all-gather: rank by rank, the second block only
        // where there is a shift, through cacheable loads.  With P outputs
        // as well, this measured faster than every load in flight at once,
        // and nontemporal loads gave no gain here.
#pragma unroll
        for (int r = 0; r < NI; ++r) {
          if (r < ni) {
            const char *p = ib[r] + v * kVecBytes;
            const u32x4 A = ld_plain(p);
            if (sh[r]) {
              const u32x4 B = ld_plain(p + kVecBytes);
              x[r] = realign16(A, B, sh[r]);
            } else {
              x[r] = A;
            }
          }
        }
      }
      u32x4 y;
      if constexpr (KIND == KIND_AG) y = x[0];
      else y = fold_vec<DT, OP, NI>(x, ni);
      // Every store nontemporal: the loads above already go through the
      // cache, and a cacheable output on top of them measured slower.  Fenced
      // as in coll_vec_kernel, without which the compiler merged one output's
      // store into the plain path's (all-gather 9-11 % slower, reduce-scatter
      // 4-5 %).
      if (nts) {
        asm volatile("");
#pragma unroll
        for (int q = 0; q < NO; ++q)
          if (q < no) st_nt(ob[q] + v * kVecBytes, y);
        asm volatile("");
      } else {
#pragma unroll
        for (int q = 0; q < NO; ++q)
          if (q < no) st_plain(ob[q] + v * kVecBytes, y);
      }
    }
  }
}

// Element-wise fallback for outputs that are not 16-byte aligned alike.
template <int KIND, int DT, int OP>
__global__ void __launch_bounds__(kThreads) coll_scalar_kernel(CollArgs a, int nseg) {
  const uint64_t total = (uint64_t)nseg * a.seg_elems;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * kThreads) {
    const int s = (int)(i / a.seg_elems);
    scalar_element<KIND, DT, OP>(a, s, i - (uint64_t)s * a.seg_elems);
  }
}

// ------------------------------------------------------------ LDS pipeline
//
// The staged form of the same fold ([digest] s2.3: each task becomes a series
// of windows fed through a multi-stage shared-memory pipeline, driven by
// asynchronous bulk loads with completion barriers).  On gfx950 the bulk load
// is global_load_lds_dwordx4, which moves 16 bytes per lane from HBM straight
// into LDS without touching VGPRs, and the completion barrier is the
// producer's s_waitcnt vmcnt followed by s_barrier.
//
// A workgroup is 4 consumer waves plus 4 producer waves.  The ring has S
// stages; a stage holds one 4 KiB tile of every input (the tile is 256
// vectors: one per consumer lane).  Producer wave p loads row p (64 vectors)
// of each input's tile; consumer wave w folds row w.  Per tile j:
//   producer: issue tile j+S-1 into the stage tile j-1 used, wait until tile
//             j has landed, barrier A_j, barrier B_j
//   consumer: barrier A_j, read stage j%S and fold, barrier B_j, store
// so up to S-1 tiles are in flight while a tile is folded and stored.  Every
// producer issues exactly one load per input per tile (lanes past the end of
// a chunk re-read its last vector, so the count of outstanding loads is exact
// and no load leaves the buffers).

constexpr int kLdsWaves = 4;                   // consumer waves = producer waves
constexpr int kLdsThreads = 2 * kLdsWaves * 64;
constexpr int kTileVecs = kLdsWaves * 64;      // vectors per input per tile

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void waitcnt_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int N = 0>
__device__ __forceinline__ void waitcnt_vm_le(int n) {
  if constexpr (N < 63) {
    if (n <= N) {
      waitcnt_vm<N>();
      return;
    }
    waitcnt_vm_le<N + 1>(n);
  } else {
    waitcnt_vm<63>();
  }
}

__device__ __forceinline__ void lgkm_wait_all() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
}

__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Walks a workgroup's chunks tile by tile (both roles walk the same sequence).
struct TileCursor {
  uint64_t c;       // current chunk
  uint64_t t;       // tile inside the chunk
  uint64_t v0, v1;  // vector range of the chunk
  int s;            // segment
  bool valid;
};

__device__ __forceinline__ void cursor_chunk(const CollArgs &a, TileCursor &k) {
  for (; k.c < a.total_chunks; k.c += gridDim.x) {
    k.s = (int)(k.c / a.chunks_per_seg);
    const uint64_t lc = k.c - (uint64_t)k.s * a.chunks_per_seg;
    k.v0 = lc * a.chunk_vecs;
    k.v1 = min(k.v0 + a.chunk_vecs, a.nvec[k.s]);
    k.t = 0;
    if (k.v1 > k.v0) {
      k.valid = true;
      return;
    }
  }
  k.valid = false;
}

__device__ __forceinline__ void cursor_begin(const CollArgs &a, TileCursor &k) {
  k.c = blockIdx.x;
  cursor_chunk(a, k);
}

__device__ __forceinline__ void cursor_next(const CollArgs &a, TileCursor &k) {
  ++k.t;
  if (k.v0 + k.t * kTileVecs >= k.v1) {
    k.c += gridDim.x;
    cursor_chunk(a, k);
  }
}

template <int KIND, int DT, int OP, int PMAX, int S>
__global__ void __launch_bounds__(kLdsThreads) coll_lds_kernel(CollArgs a) {
  constexpr int esz = (DT == CCL_BFLOAT16 || DT == CCL_FLOAT16) ? 2 : 4;
  constexpr int V = kVecBytes / esz;
  constexpr int NI = KIND == KIND_AG ? 1 : PMAX;
  constexpr int NO = KIND == KIND_RS ? 1 : PMAX;
  constexpr int kTileBytes = kTileVecs * kVecBytes;
  constexpr int kStageBytes = NI * kTileBytes;
  __shared__ __attribute__((aligned(16))) char lds[S * kStageBytes];

  const int P = a.P;
  const int ni = KIND == KIND_AG ? 1 : P;
  const int no = KIND == KIND_RS ? 1 : P;
  const bool ntl = a.flags & 1, nts = a.flags & 2, wts = a.flags & 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  if (wave >= kLdsWaves) {
    // ---------------------------------------------------------- producer
    const int p = wave - kLdsWaves;
    TileCursor issue;
    cursor_begin(a, issue);
    TileCursor need = issue;
    int inflight = 0;  // tiles issued and not yet waited for
    auto issue_tile = [&](const TileCursor &k, int stage) {
      const uint64_t head = a.head[k.s];
      uint64_t vv = k.v0 + k.t * kTileVecs + (uint64_t)p * 64 + lane;
      if (vv >= k.v1) vv = k.v1 - 1;
      char *dst = lds + stage * kStageBytes + p * 64 * kVecBytes;
      if (ntl && wts) {
        // with write-through stores input 0's loads stay cacheable, as in
        // coll_vec_kernel (the one cacheable stream of the call)
        __builtin_amdgcn_global_load_lds(
            (const void *)(in_at<KIND>(a, k.s, 0, head, esz) + vv * kVecBytes),
            (__attribute__((address_space(3))) void *)(dst), kVecBytes, 0, 0);
#pragma unroll
        for (int r = 1; r < NI; ++r)
          if (r < ni)
            __builtin_amdgcn_global_load_lds(
                (const void *)(in_at<KIND>(a, k.s, r, head, esz) + vv * kVecBytes),
                (__attribute__((address_space(3))) void *)(dst + r * kTileBytes), kVecBytes, 0, 2);
      } else if (ntl) {
#pragma unroll
        for (int r = 0; r < NI; ++r)
          if (r < ni)
            __builtin_amdgcn_global_load_lds(
                (const void *)(in_at<KIND>(a, k.s, r, head, esz) + vv * kVecBytes),
                (__attribute__((address_space(3))) void *)(dst + r * kTileBytes), kVecBytes, 0, 2);
      } else {
#pragma unroll
        for (int r = 0; r < NI; ++r)
          if (r < ni)
            __builtin_amdgcn_global_load_lds(
                (const void *)(in_at<KIND>(a, k.s, r, head, esz) + vv * kVecBytes),
                (__attribute__((address_space(3))) void *)(dst + r * kTileBytes), kVecBytes, 0, 0);
      }
    };
    int stage_issue = 0;
    for (int j = 0; j < S - 1 && issue.valid; ++j) {
      issue_tile(issue, stage_issue);
      stage_issue = stage_issue + 1 == S ? 0 : stage_issue + 1;
      ++inflight;
      cursor_next(a, issue);
    }
    while (need.valid) {
      if (issue.valid) {
        issue_tile(issue, stage_issue);
        stage_issue = stage_issue + 1 == S ? 0 : stage_issue + 1;
        ++inflight;
        cursor_next(a, issue);
      }
      // tile `need` is the oldest in flight: allow the younger ones to pend
      waitcnt_vm_le((inflight - 1) * ni);
      --inflight;
      wg_barrier();  // A: the tile has landed
      wg_barrier();  // B: consumers have read it
      cursor_next(a, need);
    }
  } else {
    // ---------------------------------------------------------- consumer
    const int w = wave;
    // Scalar head and tail of each segment, by the workgroup that owns the
    // segment's first chunk (also when the segment has no whole vector).
    for (uint64_t c = blockIdx.x; c < a.total_chunks; c += gridDim.x) {
      const int s = (int)(c / a.chunks_per_seg);
      if (c - (uint64_t)s * a.chunks_per_seg != 0) continue;
      const uint64_t head = a.head[s];
      const uint64_t tail0 = head + a.nvec[s] * V;
      const uint64_t ntail = a.seg_elems - tail0;
      const uint64_t t = threadIdx.x;
      if (t < head) scalar_element<KIND, DT, OP>(a, s, t);
      else if (t - head < ntail) scalar_element<KIND, DT, OP>(a, s, tail0 + (t - head));
    }
    TileCursor k;
    cursor_begin(a, k);
    int stage = 0;
    while (k.valid) {
      const int s = k.s;
      const uint64_t head = a.head[s];
      const uint64_t vv = k.v0 + k.t * kTileVecs + (uint64_t)w * 64 + lane;
      wg_barrier();  // A
      u32x4 x[NI];
      const char *src = lds + stage * kStageBytes + (w * 64 + lane) * kVecBytes;
#pragma unroll
      for (int r = 0; r < NI; ++r)
        if (r < ni) x[r] = *(const u32x4 *)(src + r * kTileBytes);
      lgkm_wait_all();
      wg_barrier();  // B
      stage = stage + 1 == S ? 0 : stage + 1;
      if (vv < k.v1) {
        u32x4 y;
        if constexpr (KIND == KIND_AG) y = x[0];
        else y = fold_vec<DT, OP, NI>(x, ni);
        // One cacheable stream per call, as in coll_vec_kernel.  Writing
        // through, that is input 0's loads (producer above) and every output
        // is written through.  Otherwise the inputs arrive through
        // nontemporal loads and output 0's stores stay cacheable (the host
        // puts the all-reduce's last output there); the reduce-scatter's
        // single output does not.  The nontemporal group is fenced as in
        // coll_vec_kernel: a per-store choice between the two hints was
        // merged by the compiler into plain stores to every output (10-15 %
        // slower for the all-reduce, 4-5 % for the all-gather).
        constexpr bool pout0 = KIND != KIND_RS;
        if (wts) {
          // from the wave's base in this tile, kept in scalar registers (see
          // st_wt)
          const uint64_t vbase = k.v0 + k.t * kTileVecs + (uint64_t)w * 64;
#pragma unroll
          for (int q = 0; q < NO; ++q)
            if (q < no)
              st_wt(wave_uniform(out_at<KIND>(a, s, q, head, esz) + vbase * kVecBytes),
                    (uint64_t)lane * kVecBytes, y);
        } else if (nts) {
          asm volatile("");
#pragma unroll
          for (int q = pout0 ? 1 : 0; q < NO; ++q)
            if (q < no) st_nt(out_at<KIND>(a, s, q, head, esz) + vv * kVecBytes, y);
          asm volatile("");
          if constexpr (pout0) st_plain(out_at<KIND>(a, s, 0, head, esz) + vv * kVecBytes, y);
        } else {
#pragma unroll
          for (int q = 0; q < NO; ++q)
            if (q < no) st_plain(out_at<KIND>(a, s, q, head, esz) + vv * kVecBytes, y);
        }
      }
      cursor_next(a, k);
    }
  }
}

// Largest stage count that keeps the ring within 128 KiB of LDS.
inline int lds_stages(int stages, int ni_max) {
  const int per_stage = ni_max * kTileVecs * kVecBytes;
  int s = stages;
  while (s > 2 && s * per_stage > 128 * 1024) --s;
  return s;
}

// ------------------------------------------------------------- dispatch

template <int KIND, int DT, int OP, int PMAX, bool WT>
void launch_vec_u(const CollArgs &a, int unroll, unsigned grid, size_t lds, hipStream_t st) {
  if (unroll == 1)
    hipLaunchKernelGGL((coll_vec_kernel<KIND, DT, OP, PMAX, 1, WT>), dim3(grid), dim3(kThreads), lds, st, a);
  else if (unroll == 2 || PMAX > 8)
    hipLaunchKernelGGL((coll_vec_kernel<KIND, DT, OP, PMAX, 2, WT>), dim3(grid), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((coll_vec_kernel<KIND, DT, OP, PMAX, 4, WT>), dim3(grid), dim3(kThreads), lds, st, a);
}

template <int KIND, int DT, int OP, int PMAX>
hipError_t launch_vec(const CollArgs &a, int unroll, unsigned grid, size_t lds, hipStream_t st) {
  if (a.flags & 4) launch_vec_u<KIND, DT, OP, PMAX, true>(a, unroll, grid, lds, st);
  else launch_vec_u<KIND, DT, OP, PMAX, false>(a, unroll, grid, lds, st);
  return hipGetLastError();
}

template <int KIND, int DT, int OP>
hipError_t launch_pmax(const CollArgs &a, int unroll, unsigned grid, size_t lds, hipStream_t st) {
  if (a.P <= 4) return launch_vec<KIND, DT, OP, 4>(a, unroll, grid, lds, st);
  if (a.P <= 8) return launch_vec<KIND, DT, OP, 8>(a, unroll, grid, lds, st);
  return launch_vec<KIND, DT, OP, 16>(a, unroll, grid, lds, st);
}

template <int KIND, int DT>
hipError_t launch_op(const CollArgs &a, int op, int unroll, unsigned grid, size_t lds,
                     hipStream_t st) {
  switch (op) {
    case CCL_SUM: return launch_pmax<KIND, DT, CCL_SUM>(a, unroll, grid, lds, st);
    case CCL_MIN: return launch_pmax<KIND, DT, CCL_MIN>(a, unroll, grid, lds, st);
    default: return launch_pmax<KIND, DT, CCL_MAX>(a, unroll, grid, lds, st);
  }
}

template <int KIND, int DT, int OP, int PMAX>
hipError_t launch_lds_s(const CollArgs &a, int stages, int occupancy, unsigned grid,
                        hipStream_t st) {
  constexpr int NI = KIND == KIND_AG ? 1 : PMAX;
  constexpr size_t kStage = (size_t)NI * kTileVecs * kVecBytes;
  const int s = lds_stages(stages, NI);
  if constexpr (kStage * 3 <= 128 * 1024) {
    if (s == 4 && kStage * 4 <= 128 * 1024)
      hipLaunchKernelGGL((coll_lds_kernel<KIND, DT, OP, PMAX, 4>), dim3(grid), dim3(kLdsThreads),
                         occupancy_lds(occupancy, 4 * kStage), st, a);
    else if (s >= 3)
      hipLaunchKernelGGL((coll_lds_kernel<KIND, DT, OP, PMAX, 3>), dim3(grid), dim3(kLdsThreads),
                         occupancy_lds(occupancy, 3 * kStage), st, a);
    else
      hipLaunchKernelGGL((coll_lds_kernel<KIND, DT, OP, PMAX, 2>), dim3(grid), dim3(kLdsThreads),
                         occupancy_lds(occupancy, 2 * kStage), st, a);
  } else {
    (void)s;
    hipLaunchKernelGGL((coll_lds_kernel<KIND, DT, OP, PMAX, 2>), dim3(grid), dim3(kLdsThreads),
                       occupancy_lds(occupancy, 2 * kStage), st, a);
  }
  return hipGetLastError();
}

template <int KIND, int DT, int OP>
hipError_t launch_lds_p(const CollArgs &a, int stages, int occ, unsigned grid, hipStream_t st) {
  if (a.P <= 4) return launch_lds_s<KIND, DT, OP, 4>(a, stages, occ, grid, st);
  if (a.P <= 8) return launch_lds_s<KIND, DT, OP, 8>(a, stages, occ, grid, st);
  return launch_lds_s<KIND, DT, OP, 16>(a, stages, occ, grid, st);
}

template <int KIND, int DT, int OP>
hipError_t launch_realign_p(const CollArgs &a, unsigned grid, size_t lds, hipStream_t st) {
  if (a.P <= 4)
    hipLaunchKernelGGL((coll_realign_kernel<KIND, DT, OP, 4>), dim3(grid), dim3(kThreads), lds, st, a);
  else if (a.P <= 8)
    hipLaunchKernelGGL((coll_realign_kernel<KIND, DT, OP, 8>), dim3(grid), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((coll_realign_kernel<KIND, DT, OP, 16>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int KIND, int DT, int OP>
hipError_t launch_scalar3(const CollArgs &a, int nseg, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((coll_scalar_kernel<KIND, DT, OP>), dim3(grid), dim3(kThreads), 0, st, a, nseg);
  return hipGetLastError();
}

template <int KIND, int DT, int OP>
hipError_t dispatch_path(const CollArgs &a, const CollPath &p, hipStream_t st) {
  switch (p.path) {
    case PATH_VEC: return launch_pmax<KIND, DT, OP>(a, p.unroll, p.grid, p.lds, st);
    case PATH_LDS: return launch_lds_p<KIND, DT, OP>(a, p.stages, p.occupancy, p.grid, st);
    case PATH_REALIGN: return launch_realign_p<KIND, DT, OP>(a, p.grid, p.lds, st);
    default: return launch_scalar3<KIND, DT, OP>(a, p.nseg, p.grid, st);
  }
}

}  // namespace

// The launches of one (kind, element type); copies ignore the op.
template <int KIND, int DT>
hipError_t dispatch_kind(const CollArgs &a, const CollPath &p, hipStream_t st) {
  if constexpr (KIND == KIND_AG) {
    return dispatch_path<KIND, DT, CCL_SUM>(a, p, st);
  } else {
    switch (p.op) {
      case CCL_SUM: return dispatch_path<KIND, DT, CCL_SUM>(a, p, st);
      case CCL_MIN: return dispatch_path<KIND, DT, CCL_MIN>(a, p, st);
      default: return dispatch_path<KIND, DT, CCL_MAX>(a, p, st);
    }
  }
}

}  // namespace ccl
