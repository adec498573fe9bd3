// Collective kernels for gfx950: all-reduce, reduce-scatter (shard-in) and
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
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ccl_internal.h"
#include "ccl_device.h"

namespace ccl {
namespace {

struct CollArgs {
  const char *in[CCL_MAX_RANKS];
  char *out[CCL_MAX_RANKS];
  uint64_t nvec[CCL_MAX_RANKS];   // 16-byte vectors in the body of segment s
  uint32_t head[CCL_MAX_RANKS];   // scalar elements before the body of segment s
  uint64_t seg_elems;             // M
  uint64_t chunk_vecs;
  uint64_t chunks_per_seg;
  uint64_t total_chunks;
  int P;
  int flags;                      // bit 0: nontemporal loads, bit 1: nontemporal stores
};

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
  constexpr int esz = DT == CCL_BFLOAT16 ? 2 : 4;
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

// Register-direct kernel.  PMAX bounds P at compile time so every load of a
// lane's U x P vectors is issued before the first fold.
template <int KIND, int DT, int OP, int PMAX, int U>
__global__ void __launch_bounds__(kThreads) coll_vec_kernel(CollArgs a) {
  constexpr int esz = DT == CCL_BFLOAT16 ? 2 : 4;
  constexpr int V = kVecBytes / esz;  // elements per vector
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
    for (int r = 0; r < NI; ++r) ib[r] = r < ni ? in_at<KIND>(a, s, r, head, esz) : nullptr;
#pragma unroll
    for (int q = 0; q < NO; ++q) ob[q] = q < no ? out_at<KIND>(a, s, q, head, esz) : nullptr;

    for (uint64_t v = v0 + threadIdx.x; v < v1; v += (uint64_t)kThreads * U) {
      u32x4 x[U][NI];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vv = v + (uint64_t)u * kThreads;
        if (vv < v1) {
          if (ntl) {
#pragma unroll
            for (int r = 0; r < NI; ++r)
              if (r < ni) x[u][r] = ld_nt(ib[r] + vv * kVecBytes);
          } else {
#pragma unroll
            for (int r = 0; r < NI; ++r)
              if (r < ni) x[u][r] = ld_plain(ib[r] + vv * kVecBytes);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vv = v + (uint64_t)u * kThreads;
        if (vv < v1) {
          u32x4 y;
          if constexpr (KIND == KIND_AG) y = x[u][0];
          else y = fold_vec<DT, OP, NI>(x[u], ni);
          if (nts) {
#pragma unroll
            for (int q = 0; q < NO; ++q)
              if (q < no) st_nt(ob[q] + vv * kVecBytes, y);
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

// Element-wise fallback for buffers that are not 16-byte aligned alike.
template <int KIND, int DT, int OP>
__global__ void __launch_bounds__(kThreads) coll_scalar_kernel(CollArgs a, int nseg) {
  const uint64_t total = (uint64_t)nseg * a.seg_elems;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * kThreads) {
    const int s = (int)(i / a.seg_elems);
    scalar_element<KIND, DT, OP>(a, s, i - (uint64_t)s * a.seg_elems);
  }
}

// ------------------------------------------------------------- dispatch

template <int KIND, int DT, int OP, int PMAX>
hipError_t launch_vec(const CollArgs &a, int unroll, unsigned grid, hipStream_t st) {
  if (unroll == 1)
    hipLaunchKernelGGL((coll_vec_kernel<KIND, DT, OP, PMAX, 1>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((coll_vec_kernel<KIND, DT, OP, PMAX, 2>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int KIND, int DT, int OP>
hipError_t launch_pmax(const CollArgs &a, int unroll, unsigned grid, hipStream_t st) {
  if (a.P <= 4) return launch_vec<KIND, DT, OP, 4>(a, unroll, grid, st);
  if (a.P <= 8) return launch_vec<KIND, DT, OP, 8>(a, unroll, grid, st);
  return launch_vec<KIND, DT, OP, 16>(a, unroll, grid, st);
}

template <int KIND, int DT>
hipError_t launch_op(const CollArgs &a, int op, int unroll, unsigned grid, hipStream_t st) {
  switch (op) {
    case CCL_SUM: return launch_pmax<KIND, DT, CCL_SUM>(a, unroll, grid, st);
    case CCL_MIN: return launch_pmax<KIND, DT, CCL_MIN>(a, unroll, grid, st);
    default: return launch_pmax<KIND, DT, CCL_MAX>(a, unroll, grid, st);
  }
}

template <int KIND>
hipError_t launch_dt(const CollArgs &a, int dt, int op, int unroll, unsigned grid, hipStream_t st) {
  if constexpr (KIND == KIND_AG) {
    // A copy: only the element size matters.
    if (dt == CCL_BFLOAT16) return launch_pmax<KIND, CCL_BFLOAT16, CCL_SUM>(a, unroll, grid, st);
    return launch_pmax<KIND, CCL_INT32, CCL_SUM>(a, unroll, grid, st);
  } else {
    switch (dt) {
      case CCL_FLOAT32: return launch_op<KIND, CCL_FLOAT32>(a, op, unroll, grid, st);
      case CCL_BFLOAT16: return launch_op<KIND, CCL_BFLOAT16>(a, op, unroll, grid, st);
      default: return launch_op<KIND, CCL_INT32>(a, op, unroll, grid, st);
    }
  }
}

template <int KIND, int DT, int OP>
hipError_t launch_scalar3(const CollArgs &a, int nseg, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((coll_scalar_kernel<KIND, DT, OP>), dim3(grid), dim3(kThreads), 0, st, a, nseg);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_scalar(const CollArgs &a, int nseg, int dt, int op, unsigned grid, hipStream_t st) {
  if constexpr (KIND == KIND_AG) {
    if (dt == CCL_BFLOAT16) return launch_scalar3<KIND, CCL_BFLOAT16, CCL_SUM>(a, nseg, grid, st);
    return launch_scalar3<KIND, CCL_INT32, CCL_SUM>(a, nseg, grid, st);
  } else {
#define CCL_SC(D)                                                               \
  switch (op) {                                                                 \
    case CCL_SUM: return launch_scalar3<KIND, D, CCL_SUM>(a, nseg, grid, st);   \
    case CCL_MIN: return launch_scalar3<KIND, D, CCL_MIN>(a, nseg, grid, st);   \
    default: return launch_scalar3<KIND, D, CCL_MAX>(a, nseg, grid, st);        \
  }
    switch (dt) {
      case CCL_FLOAT32: CCL_SC(CCL_FLOAT32)
      case CCL_BFLOAT16: CCL_SC(CCL_BFLOAT16)
      default: CCL_SC(CCL_INT32)
    }
#undef CCL_SC
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
  for (int r = 0; r < d.P; ++r) {
    a.in[r] = (const char *)d.send[r];
    a.out[r] = (char *)d.recv[r];
  }
  const int nseg = d.kind == KIND_AR ? 1 : d.P;
  const int ni = d.kind == KIND_AG ? 1 : d.P;
  const int no = d.kind == KIND_RS ? 1 : d.P;

  // Every buffer of a segment must share its address modulo 16 for the
  // vector path; the common misalignment becomes the scalar head.
  bool vec = true;
  uint64_t max_nvec = 0;
  for (int s = 0; s < nseg && vec; ++s) {
    uintptr_t base[2 * CCL_MAX_RANKS];
    int nb = 0;
    for (int r = 0; r < ni; ++r) {
      const char *p = d.kind == KIND_AR ? a.in[r]
                      : d.kind == KIND_RS ? a.in[r] + (uint64_t)s * M * esz
                                          : a.in[s];
      base[nb++] = (uintptr_t)p;
    }
    for (int q = 0; q < no; ++q) {
      const char *p = d.kind == KIND_AR ? a.out[q]
                      : d.kind == KIND_RS ? a.out[s]
                                          : a.out[q] + (uint64_t)s * M * esz;
      base[nb++] = (uintptr_t)p;
    }
    const uintptr_t mis = base[0] % kVecBytes;
    for (int i = 1; i < nb; ++i)
      if (base[i] % kVecBytes != mis) vec = false;
    uint64_t head = ((kVecBytes - mis) % kVecBytes) / esz;
    if (head > M) head = M;
    a.head[s] = (uint32_t)head;
    a.nvec[s] = (M - head) / V;
    max_nvec = std::max<uint64_t>(max_nvec, a.nvec[s]);
  }

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CCL_ERR_HIP;
  const int cus = device_cu_count(dev);
  if (cus <= 0) return CCL_ERR_HIP;

  hipError_t err;
  if (!vec) {
    const uint64_t total = (uint64_t)nseg * M;
    const uint64_t want = (total + kThreads - 1) / kThreads;
    const unsigned grid = (unsigned)std::min<uint64_t>(want, (uint64_t)cus * 16);
    switch (d.kind) {
      case KIND_AR: err = launch_scalar<KIND_AR>(a, nseg, d.dtype, d.op, grid, stream); break;
      case KIND_RS: err = launch_scalar<KIND_RS>(a, nseg, d.dtype, d.op, grid, stream); break;
      default: err = launch_scalar<KIND_AG>(a, nseg, d.dtype, d.op, grid, stream); break;
    }
    return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
  }

  if (l.stages > 1) return CCL_ERR_UNSUPPORTED;  // LDS pipeline: not built yet

  a.chunk_vecs = l.chunk_bytes / kVecBytes;
  a.chunks_per_seg = std::max<uint64_t>(1, (max_nvec + a.chunk_vecs - 1) / a.chunk_vecs);
  a.total_chunks = a.chunks_per_seg * nseg;
  uint64_t grid = l.workgroups ? (uint64_t)l.workgroups : a.total_chunks;
  grid = std::min<uint64_t>(grid, a.total_chunks);
  grid = std::min<uint64_t>(grid, 1u << 30);
  switch (d.kind) {
    case KIND_AR: err = launch_dt<KIND_AR>(a, d.dtype, d.op, l.unroll, (unsigned)grid, stream); break;
    case KIND_RS: err = launch_dt<KIND_RS>(a, d.dtype, d.op, l.unroll, (unsigned)grid, stream); break;
    default: err = launch_dt<KIND_AG>(a, d.dtype, d.op, l.unroll, (unsigned)grid, stream); break;
  }
  return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // namespace ccl
