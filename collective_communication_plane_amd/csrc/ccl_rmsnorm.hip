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
// NTL: nontemporal loads (template argument, see ld); SP: store policy
// (StorePol: plain, nontemporal, or write-through from the row's base).
template <int DT, int PMAX, bool NTL, int SP>
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
        if (q < P) st_pol<SP>(a.out[q] + base, (uint64_t)v * kVecBytes, o);
    }
  }
}

// The row's inverse RMS from each lane's partial sum of squares: a wave
// butterfly, then the four waves in order through `part` (one slot per wave).
// One block-wide barrier; the caller alternates between two `part` arrays so
// that a wave cannot overwrite a slot another wave has yet to read.
__device__ __forceinline__ float row_inv_rms(float ss, float *part, uint32_t hidden, float eps) {
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) total += part[w];
  return 1.0f / sqrtf(total / (float)hidden + eps);
}

// The same computation as ar_rmsnorm_kernel, software-pipelined over a
// workgroup's rows so that reads and writes interleave.  The grid is
// persistent (workgroup w takes rows w, w + G, w + 2G, ...).  While the
// normalised row k is stored, 16-byte vector by 16-byte vector, the inputs of
// the workgroup's next row are loaded and folded into a second LDS row
// buffer: each lane keeps one vector per rank in flight for the next row and
// one per output for the current one, so HBM sees the all-reduce's mix of
// reads and writes instead of a whole row of reads followed by a whole row of
// writes.  Each lane only touches the row-buffer vectors it owns, so the one
// barrier per row (the norm's) is all the synchronisation there is; the sum
// of squares runs in the same order as ar_rmsnorm_kernel's, so both give
// identical bits.  Row k is read completely before any of it is stored, so
// the call may still run in place.
template <int DT, int PMAX, bool NTL, int SP>
__global__ void __launch_bounds__(kThreads) ar_rmsnorm_pipe_kernel(RmsArgs a) {
  constexpr int esz = DT == CCL_FLOAT32 ? 4 : 2;
  constexpr int V = kVecBytes / esz;
  extern __shared__ u32x4 row_bufs[];  // two rows of row_vecs vectors
  __shared__ float wave_part[2][kThreads / 64];
  const int P = a.P;
  const uint64_t row_bytes = (uint64_t)a.hidden * esz;
  uint64_t row = blockIdx.x;
  if (row >= a.rows) return;
  u32x4 *cur = row_bufs, *nxt = row_bufs + a.row_vecs;

  // prologue: fold the first row
  float ss = 0.f;
#pragma unroll 1
  for (uint32_t v = threadIdx.x; v < a.row_vecs; v += kThreads) {
    u32x4 x[PMAX];
#pragma unroll
    for (int r = 0; r < PMAX; ++r)
      x[r] = r < P ? ld<NTL>(a.in[r] + row * row_bytes + (uint64_t)v * kVecBytes)
                   : u32x4{0u, 0u, 0u, 0u};
    const u32x4 sv = fold_vec<DT, CCL_SUM, PMAX>(x, P);
    cur[v] = sv;
    float f[8];
    widen_vec<DT>(sv, f);
#pragma unroll
    for (int e = 0; e < V; ++e) ss += f[e] * f[e];
  }
  int par = 0;
  float inv = row_inv_rms(ss, wave_part[par], a.hidden, a.eps);

  for (;;) {
    const uint64_t next = row + gridDim.x;
    const bool more = next < a.rows;
    const uint64_t base = row * row_bytes, nbase = next * row_bytes;
    ss = 0.f;
#pragma unroll 1
    for (uint32_t v = threadIdx.x; v < a.row_vecs; v += kThreads) {
      const uint64_t off = (uint64_t)v * kVecBytes;
      // gamma first: vector loads complete in issue order, so the stores
      // below then wait only for gamma, not for the next row's inputs
      const u32x4 gv = ld_plain(a.gamma + off);
      u32x4 x[PMAX];
      if (more) {
#pragma unroll
        for (int r = 0; r < PMAX; ++r)
          x[r] = r < P ? ld<NTL>(a.in[r] + nbase + off) : u32x4{0u, 0u, 0u, 0u};
      }
      float g[8], f[8], y[8];
      widen_vec<DT>(gv, g);
      widen_vec<DT>(cur[v], f);
#pragma unroll
      for (int e = 0; e < V; ++e) y[e] = (f[e] * inv) * g[e];
      const u32x4 o = narrow_vec<DT>(y);
#pragma unroll
      for (int q = 0; q < PMAX; ++q)
        if (q < P) st_pol<SP>(a.out[q] + base, off, o);
      if (more) {
        const u32x4 sv = fold_vec<DT, CCL_SUM, PMAX>(x, P);
        nxt[v] = sv;
        float h[8];
        widen_vec<DT>(sv, h);
#pragma unroll
        for (int e = 0; e < V; ++e) ss += h[e] * h[e];
      }
    }
    if (!more) break;
    par ^= 1;
    inv = row_inv_rms(ss, wave_part[par], a.hidden, a.eps);
    u32x4 *t = cur;
    cur = nxt;
    nxt = t;
    row = next;
  }
}

template <int DT, bool NTL, int SP>
hipError_t launch_p(const RmsArgs &a, bool pipe, unsigned grid, size_t lds, hipStream_t st) {
  if (pipe) {
    if (a.P <= 4) hipLaunchKernelGGL((ar_rmsnorm_pipe_kernel<DT, 4, NTL, SP>), dim3(grid), dim3(kThreads), lds, st, a);
    else if (a.P <= 8) hipLaunchKernelGGL((ar_rmsnorm_pipe_kernel<DT, 8, NTL, SP>), dim3(grid), dim3(kThreads), lds, st, a);
    else hipLaunchKernelGGL((ar_rmsnorm_pipe_kernel<DT, 16, NTL, SP>), dim3(grid), dim3(kThreads), lds, st, a);
    return hipGetLastError();
  }
  if (a.P <= 4) hipLaunchKernelGGL((ar_rmsnorm_kernel<DT, 4, NTL, SP>), dim3(grid), dim3(kThreads), lds, st, a);
  else if (a.P <= 8) hipLaunchKernelGGL((ar_rmsnorm_kernel<DT, 8, NTL, SP>), dim3(grid), dim3(kThreads), lds, st, a);
  else hipLaunchKernelGGL((ar_rmsnorm_kernel<DT, 16, NTL, SP>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_nt(const RmsArgs &a, const Launch &l, bool pipe, unsigned grid, size_t lds,
                     hipStream_t st) {
  // Write-through stores only when the caller asks for them: against
  // nontemporal-only stores they measured -0.6 to -0.8 % on 16 KiB rows and
  // -0.4 to -0.7 % on 32 KiB rows (row-pipelined), in same-binary runs.
  const int sp = !l.nt_store ? ST_PLAIN : (l.store_pol_set && l.store_wt) ? ST_WT : ST_NT;
  if (l.nt_load) {
    if (sp == ST_WT) return launch_p<DT, true, ST_WT>(a, pipe, grid, lds, st);
    if (sp == ST_NT) return launch_p<DT, true, ST_NT>(a, pipe, grid, lds, st);
    return launch_p<DT, true, ST_PLAIN>(a, pipe, grid, lds, st);
  }
  if (sp == ST_WT) return launch_p<DT, false, ST_WT>(a, pipe, grid, lds, st);
  if (sp == ST_NT) return launch_p<DT, false, ST_NT>(a, pipe, grid, lds, st);
  return launch_p<DT, false, ST_PLAIN>(a, pipe, grid, lds, st);
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
  // stages = 2: the row-pipelined kernel on a persistent grid of (residency
  // cap, else 1) workgroups per CU; stages = 1: one workgroup per row.
  const bool pipe = l.stages == 2;
  uint64_t grid = d.rows;
  if (l.workgroups) {
    grid = (uint64_t)l.workgroups;
  } else if (pipe) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CCL_ERR_HIP;
    const int cus = device_cu_count(dev);
    if (cus <= 0) return CCL_ERR_HIP;
    grid = (uint64_t)cus * (uint64_t)(l.occupancy > 0 ? l.occupancy : 1);
  }
  grid = std::min<uint64_t>(std::min<uint64_t>(grid, d.rows), 1u << 30);
  // the row buffer(s), or more when the launch caps residency through LDS
  const size_t row_lds = (size_t)a.row_vecs * kVecBytes * (pipe ? 2 : 1);
  const size_t static_lds = (kThreads / 64) * sizeof(float) * (pipe ? 2 : 1);
  const size_t lds = std::max(row_lds, occupancy_lds(l.occupancy, static_lds));
  hipError_t err;
  switch (d.dtype) {
    case CCL_FLOAT32: err = launch_nt<CCL_FLOAT32>(a, l, pipe, (unsigned)grid, lds, stream); break;
    case CCL_BFLOAT16: err = launch_nt<CCL_BFLOAT16>(a, l, pipe, (unsigned)grid, lds, stream); break;
    default: err = launch_nt<CCL_FLOAT16>(a, l, pipe, (unsigned)grid, lds, stream); break;
  }
  return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // namespace ccl
