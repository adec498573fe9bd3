// All-reduce with RMSNorm fused between its halves, for gfx950.
//
// The "nccl-extensions" roadmap page describes a Device API example that
// puts a Transformer RMSNorm between reduce-scatter and all-gather inside one
// kernel.  On one GPU the three steps fuse into a single pass over HBM: a
// workgroup owns whole rows (tokens); for each row it folds the P inputs in
// fp32 in rank order, rounds to the element type (the value a reduce-scatter
// would hand over), accumulates the row's sum of squares in fp32 (each lane
// over its elements, then a wave butterfly, then the four waves in order
// through LDS), scales by 1/sqrt(mean + eps) and gamma, and stores the result
// to all P outputs.  Every row is read completely before any of it is
// written, so the call may run in place.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ccl_device.h"
#include "ccl_internal.h"

namespace ccl {
namespace {

struct RmsArgs {
  const char *in[CCL_MAX_RANKS];
  char *out[CCL_MAX_RANKS];
  const char *gamma;
  uint64_t rows;
  uint32_t hidden;     // elements per row
  uint32_t row_vecs;   // 16-byte vectors per row
  float eps;
  int P;
};

// Up to 8 elements per 16-byte vector; fp32 uses the first 4.
template <int DT>
__device__ __forceinline__ void widen_vec(u32x4 v, float (&f)[8]) {
  if constexpr (DT == CCL_FLOAT32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]);
  } else if constexpr (DT == CCL_BFLOAT16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = bf16_lo(v[k]);
      f[2 * k + 1] = bf16_hi(v[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = f16_lo(v[k]);
      f[2 * k + 1] = f16_hi(v[k]);
    }
  }
}

template <int DT>
__device__ __forceinline__ u32x4 narrow_vec(const float (&f)[8]) {
  u32x4 v;
  if constexpr (DT == CCL_FLOAT32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __float_as_uint(f[k]);
  } else if constexpr (DT == CCL_BFLOAT16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = bf16_rne(f[2 * k]) | (bf16_rne(f[2 * k + 1]) << 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = f16_rne(f[2 * k]) | (f16_rne(f[2 * k + 1]) << 16);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// One workgroup per row (grid-strided).  The folded row is parked in dynamic
// LDS (row_vecs 16-byte vectors, in the element type, i.e. the value a
// reduce-scatter would hand over) between the two passes; each lane only
// reads back the vectors it wrote, so the block-wide barriers of the norm are
// the only synchronisation.  A lane keeps one vector per rank in flight:
// holding several (in registers) measured slower, since more concurrent
// streams only add DRAM page conflicts.
// NTL / NTS: nontemporal loads / stores (template arguments, see ld / st).
template <int DT, int PMAX, bool NTL, bool NTS>
__global__ void __launch_bounds__(kThreads) ar_rmsnorm_kernel(RmsArgs a) {
  constexpr int esz = DT == CCL_FLOAT32 ? 4 : 2;
  constexpr int V = kVecBytes / esz;
  extern __shared__ u32x4 row_buf[];
  __shared__ float wave_part[kThreads / 64];
  const int P = a.P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  for (uint64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint64_t base = row * (uint64_t)a.hidden * esz;
    float ss = 0.f;
#pragma unroll 1
    for (uint32_t v = threadIdx.x; v < a.row_vecs; v += kThreads) {
      u32x4 x[PMAX];
#pragma unroll
      for (int r = 0; r < PMAX; ++r)
        x[r] = r < P ? ld<NTL>(a.in[r] + base + (uint64_t)v * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 sv = fold_vec<DT, CCL_SUM, PMAX>(x, P);
      row_buf[v] = sv;
      float f[8];
      widen_vec<DT>(sv, f);
#pragma unroll
      for (int e = 0; e < V; ++e) ss += f[e] * f[e];
    }
    ss = wave_sum(ss);
    if (lane == 0) wave_part[wave] = ss;
    __syncthreads();
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) total += wave_part[w];
    __syncthreads();  // wave_part is reused by the next row
    const float inv = 1.0f / sqrtf(total / (float)a.hidden + a.eps);
#pragma unroll 2
    for (uint32_t v = threadIdx.x; v < a.row_vecs; v += kThreads) {
      float g[8], f[8], y[8];
      widen_vec<DT>(ld_plain(a.gamma + (uint64_t)v * kVecBytes), g);
      widen_vec<DT>(row_buf[v], f);
#pragma unroll
      for (int e = 0; e < V; ++e) y[e] = (f[e] * inv) * g[e];
      const u32x4 o = narrow_vec<DT>(y);
#pragma unroll
      for (int q = 0; q < PMAX; ++q)
        if (q < P) {
          char *d = a.out[q] + base + (uint64_t)v * kVecBytes;
          st<NTS>(d, o);
        }
    }
  }
}

template <int DT, bool NTL, bool NTS>
hipError_t launch_p(const RmsArgs &a, unsigned grid, size_t lds, hipStream_t st) {
  if (a.P <= 4) hipLaunchKernelGGL((ar_rmsnorm_kernel<DT, 4, NTL, NTS>), dim3(grid), dim3(kThreads), lds, st, a);
  else if (a.P <= 8) hipLaunchKernelGGL((ar_rmsnorm_kernel<DT, 8, NTL, NTS>), dim3(grid), dim3(kThreads), lds, st, a);
  else hipLaunchKernelGGL((ar_rmsnorm_kernel<DT, 16, NTL, NTS>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_nt(const RmsArgs &a, const Launch &l, unsigned grid, size_t lds, hipStream_t st) {
  if (l.nt_load && l.nt_store) return launch_p<DT, true, true>(a, grid, lds, st);
  if (l.nt_load) return launch_p<DT, true, false>(a, grid, lds, st);
  if (l.nt_store) return launch_p<DT, false, true>(a, grid, lds, st);
  return launch_p<DT, false, false>(a, grid, lds, st);
}

}  // namespace

ccl_status_t launch_ar_rmsnorm(const RmsDesc &d, const Launch &l, hipStream_t stream) {
  RmsArgs a{};
  const int esz = dtype_size(d.dtype);
  for (int r = 0; r < d.P; ++r) {
    a.in[r] = (const char *)d.send[r];
    a.out[r] = (char *)d.recv[r];
  }
  a.gamma = (const char *)d.gamma;
  a.rows = d.rows;
  a.hidden = (uint32_t)d.hidden;
  a.row_vecs = (uint32_t)(d.hidden * esz / kVecBytes);
  a.eps = d.eps;
  a.P = d.P;
  uint64_t grid = l.workgroups ? (uint64_t)l.workgroups : d.rows;
  grid = std::min<uint64_t>(std::min<uint64_t>(grid, d.rows), 1u << 30);
  // the row buffer, or more when the launch caps residency through LDS
  const size_t row_lds = (size_t)a.row_vecs * kVecBytes;
  const size_t lds = std::max(row_lds, occupancy_lds(l.occupancy, (kThreads / 64) * sizeof(float)));
  hipError_t err;
  switch (d.dtype) {
    case CCL_FLOAT32: err = launch_nt<CCL_FLOAT32>(a, l, (unsigned)grid, lds, stream); break;
    case CCL_BFLOAT16: err = launch_nt<CCL_BFLOAT16>(a, l, (unsigned)grid, lds, stream); break;
    default: err = launch_nt<CCL_FLOAT16>(a, l, (unsigned)grid, lds, stream); break;
  }
  return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // namespace ccl
