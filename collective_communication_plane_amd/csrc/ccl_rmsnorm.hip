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
#include <mutex>
#include <vector>

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

// ------------------------------------------------------------ split rows
//
// The same result from two kernels whose workgroups each own one piece of a
// row: 256 vectors, i.e. 4 KiB per rank, the plain all-reduce's unit, and a
// short-lived workgroup per piece.  A workgroup that owns a whole row walks
// 4 x 4 KiB per rank at P = 8 and runs ~15 % below the all-reduce; pieces
// of one row cannot wait for each other inside a kernel without giving most
// of that back (measured: pieces publishing partial sums to each other and
// polling ran at 4.5-4.9 TB/s against 5.8-6.3 for the same kernel without
// the wait), so the norm waits for a kernel boundary instead:
//   fold pass  folds the piece's P inputs in fp32 in rank order, rounds to
//              the element type (the reduce-scatter value s), parks s in
//              recv[0] at its own position, and writes the piece's sum of
//              squares (lanes, then a wave butterfly, then the four waves in
//              order) to part[row * K + piece];
//   norm pass  reads the row's K partial sums and adds them in piece order,
//              reads s back from recv[0] and gamma, and stores
//              s * inv * gamma to all P outputs, recv[0] included.
// Each position is read and then written by the same lane of the same piece
// in both passes, so the call may still run in place (recv[q] == send[r]).
// The cost over the one-pass kernels is one extra write and read of s
// (hidden * size bytes per row, 1/P of the input).
constexpr int kSplitPieceVecs = kThreads;  // one vector per lane

template <int DT, int PMAX, bool NTL>
__global__ void __launch_bounds__(kThreads) ar_rmsnorm_fold_kernel(RmsArgs a, float *part, int K) {
  constexpr int esz = DT == CCL_FLOAT32 ? 4 : 2;
  constexpr int V = kVecBytes / esz;
  __shared__ float wave_part[kThreads / 64];
  const int P = a.P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t row = blockIdx.x / (unsigned)K;
  const int piece = (int)(blockIdx.x - row * (unsigned)K);
  const uint32_t v = (uint32_t)piece * kSplitPieceVecs + threadIdx.x;
  const bool live = v < a.row_vecs;
  // lanes past the end of a short last piece re-read the row's last vector
  // (so every load is unconditional) and store nothing
  const uint32_t vc = live ? v : a.row_vecs - 1;
  const uint64_t row_base = row * (uint64_t)a.hidden * esz;

  // Every rank's load is issued before the first is used.  They go through
  // buffer resources over this row; ranks r >= P get an empty range, whose
  // loads return zero without touching memory, so no load sits behind a
  // per-rank branch (with branches the compiler copied one rank's result into
  // a register it had reserved and waited for the first loads there).  That
  // zero is turned into -0.0 by a uniform mask, and x + (-0.0) == x for every
  // x, -0.0 included, so folding all PMAX slots gives the P-rank fold bit for
  // bit without a per-rank branch in the fold either.
  constexpr uint32_t kNegZero = DT == CCL_FLOAT32 ? 0x80000000u : 0x80008000u;
  u32x4 x[PMAX];
#pragma unroll
  for (int r = 0; r < PMAX; ++r) {
    x[r] = ld_row<NTL>(a.in[r] + row_base, r < P ? a.row_vecs * kVecBytes : 0u,
                       (int)(vc * kVecBytes));
    x[r] ^= (r < P ? 0u : kNegZero);
  }
  const u32x4 sv = fold_vec<DT, CCL_SUM, PMAX>(x, PMAX);
  float f[8];
  widen_vec<DT>(sv, f);
  float ss = 0.f;
  if (live) {
#pragma unroll
    for (int e = 0; e < V; ++e) ss += f[e] * f[e];
    st_plain(a.out[0] + row_base + (uint64_t)v * kVecBytes, sv);
  }
  ss = wave_sum(ss);
  if (lane == 0) wave_part[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += wave_part[w];
    part[row * (unsigned)K + piece] = t;
  }
}

template <int DT, int PMAX, int SP>
__global__ void __launch_bounds__(kThreads) ar_rmsnorm_norm_kernel(RmsArgs a, const float *part,
                                                                    int K) {
  constexpr int esz = DT == CCL_FLOAT32 ? 4 : 2;
  constexpr int V = kVecBytes / esz;
  const int P = a.P;
  const uint64_t row = blockIdx.x / (unsigned)K;
  const int piece = (int)(blockIdx.x - row * (unsigned)K);
  const uint32_t v = (uint32_t)piece * kSplitPieceVecs + threadIdx.x;
  const bool live = v < a.row_vecs;
  const uint32_t vc = live ? v : a.row_vecs - 1;
  const uint64_t row_base = row * (uint64_t)a.hidden * esz;
  const u32x4 gv = ld_plain(a.gamma + (uint64_t)vc * kVecBytes);
  const u32x4 sv = ld_plain(a.out[0] + row_base + (uint64_t)vc * kVecBytes);
  float total = 0.f;
  for (int j = 0; j < K; ++j) total += part[row * (unsigned)K + j];
  const float inv = 1.0f / sqrtf(total / (float)a.hidden + a.eps);
  if (live) {
    float g[8], f[8], y[8];
    widen_vec<DT>(gv, g);
    widen_vec<DT>(sv, f);
#pragma unroll
    for (int e = 0; e < V; ++e) y[e] = (f[e] * inv) * g[e];
    const u32x4 o = narrow_vec<DT>(y);
    const uint64_t obase = row_base + (uint64_t)piece * kSplitPieceVecs * kVecBytes;
#pragma unroll
    for (int q = 0; q < PMAX; ++q)
      if (q < P) st_pol<SP>(a.out[q] + obase, (uint64_t)threadIdx.x * kVecBytes, o);
  }
}

template <int DT, int PMAX, bool NTL, int SP>
void launch_split_pm(const RmsArgs &a, float *part, int K, unsigned grid, size_t lds_fold,
                     size_t lds_norm, hipStream_t st) {
  hipLaunchKernelGGL((ar_rmsnorm_fold_kernel<DT, PMAX, NTL>), dim3(grid), dim3(kThreads), lds_fold,
                     st, a, part, K);
  hipLaunchKernelGGL((ar_rmsnorm_norm_kernel<DT, PMAX, SP>), dim3(grid), dim3(kThreads), lds_norm,
                     st, a, (const float *)part, K);
}

template <int DT, bool NTL, int SP>
hipError_t launch_split_p(const RmsArgs &a, float *part, int K, unsigned grid, size_t lds_fold,
                          size_t lds_norm, hipStream_t st) {
  if (a.P <= 4) launch_split_pm<DT, 4, NTL, SP>(a, part, K, grid, lds_fold, lds_norm, st);
  else if (a.P <= 8) launch_split_pm<DT, 8, NTL, SP>(a, part, K, grid, lds_fold, lds_norm, st);
  else launch_split_pm<DT, 16, NTL, SP>(a, part, K, grid, lds_fold, lds_norm, st);
  return hipGetLastError();
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

template <int DT>
hipError_t launch_split_nt(const RmsArgs &a, const Launch &l, float *part, int K, unsigned grid,
                           size_t lds_fold, size_t lds_norm, hipStream_t st) {
  const int sp = !l.nt_store ? ST_PLAIN : (l.store_pol_set && l.store_wt) ? ST_WT : ST_NT;
  if (l.nt_load) {
    if (sp == ST_WT) return launch_split_p<DT, true, ST_WT>(a, part, K, grid, lds_fold, lds_norm, st);
    if (sp == ST_NT) return launch_split_p<DT, true, ST_NT>(a, part, K, grid, lds_fold, lds_norm, st);
    return launch_split_p<DT, true, ST_PLAIN>(a, part, K, grid, lds_fold, lds_norm, st);
  }
  if (sp == ST_WT) return launch_split_p<DT, false, ST_WT>(a, part, K, grid, lds_fold, lds_norm, st);
  if (sp == ST_NT) return launch_split_p<DT, false, ST_NT>(a, part, K, grid, lds_fold, lds_norm, st);
  return launch_split_p<DT, false, ST_PLAIN>(a, part, K, grid, lds_fold, lds_norm, st);
}

// Partial sums of the split-row kernels, one buffer per (device, stream):
// calls on one stream are ordered, so they can share it; calls on different
// streams may overlap, so they must not.  Allocated on first use; a call
// that needs more allocates a larger buffer (at least twice the old one) and
// keeps the old one too, since queued kernels or a captured graph may still
// use it.  Every buffer lives until the process ends.  Every slot a call
// reads was written by the same call's fold pass, so nothing needs clearing.
// A stream in capture cannot allocate: *out is then null when the stream has
// no buffer large enough, and the caller runs a one-pass kernel instead.
struct StreamScratch {
  int device;
  hipStream_t stream;
  void *mem;
  size_t bytes;
};
std::mutex g_scratch_mu;
std::vector<StreamScratch> g_scratch;

ccl_status_t stream_scratch(int dev, hipStream_t st, size_t need, void **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  StreamScratch *e = nullptr;
  for (auto &x : g_scratch)
    if (x.device == dev && x.stream == st) e = &x;
  if (e && e->bytes >= need) {
    *out = e->mem;
    return CCL_OK;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) return CCL_ERR_HIP;
  if (cap != hipStreamCaptureStatusNone) {
    *out = nullptr;
    return CCL_OK;
  }
  const size_t bytes = std::max<size_t>({need, size_t(1) << 20, e ? 2 * e->bytes : 0});
  void *mem = nullptr;
  if (hipMalloc(&mem, bytes) != hipSuccess) return CCL_ERR_NOMEM;
  if (e) {
    e->mem = mem;  // the old buffer stays allocated (see above)
    e->bytes = bytes;
  } else {
    g_scratch.push_back(StreamScratch{dev, st, mem, bytes});
  }
  *out = mem;
  return CCL_OK;
}

}  // namespace

// The no-allocation entry point's partial sums: a fixed array in device
// memory, one copy per GPU the library runs on, held until the process ends.
// Its host-side name is not a device address; each device's address is looked
// up once (hipGetSymbolAddress with that device current) and kept.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void *g_noalloc_addr[kMaxDevices];
}  // namespace

ccl_status_t noalloc_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CCL_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CCL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_addr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CCL_ERR_HIP;
    g_noalloc_addr[dev] = ptr;
  }
  *out = g_noalloc_addr[dev];
  return CCL_OK;
}

ccl_status_t launch_ar_rmsnorm(const RmsDesc &d, const Launch &l_in, hipStream_t stream,
                               bool split, void *part_buf) {
  Launch l = l_in;
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
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CCL_ERR_HIP;
  const uint64_t row_bytes = (uint64_t)a.row_vecs * kVecBytes;
  void *part = part_buf;
  if (split && !part) {
    ccl_status_t st = stream_scratch(dev, stream, rms_split_scratch_bytes(d.rows, row_bytes), &part);
    if (st) return st;
    if (!part) {
      // in capture without scratch: the one-pass form this row length takes
      // by default (the same result within the documented bound, other bits);
      // the stages and residency cap the caller set still apply
      split = false;
      if (!l.stages_set) l.stages = (row_bytes > 16384 && d.P >= 6) ? 2 : 1;
      if (!l.occupancy_set)
        l.occupancy = l.stages == 2 ? 1 : (row_bytes >= 4096 && row_bytes <= 8192) ? 3 : 0;
      l.store_wt = false;
    }
  }
  if (split) {
    // one workgroup per piece in each pass; grid = rows x pieces (checked to
    // fit by the caller)
    const int K = (int)rms_split_pieces(row_bytes);
    const unsigned grid = (unsigned)(d.rows * (uint64_t)K);
    const size_t lds_fold = occupancy_lds(l.occupancy, 64);
    const size_t lds_norm = occupancy_lds(l.occupancy2, 0);
    float *pf = (float *)part;
    hipError_t err;
    switch (d.dtype) {
      case CCL_FLOAT32: err = launch_split_nt<CCL_FLOAT32>(a, l, pf, K, grid, lds_fold, lds_norm, stream); break;
      case CCL_BFLOAT16: err = launch_split_nt<CCL_BFLOAT16>(a, l, pf, K, grid, lds_fold, lds_norm, stream); break;
      default: err = launch_split_nt<CCL_FLOAT16>(a, l, pf, K, grid, lds_fold, lds_norm, stream); break;
    }
    return err == hipSuccess ? CCL_OK : CCL_ERR_HIP;
  }
  // stages = 2: the row-pipelined kernel on a persistent grid of (residency
  // cap, else 1) workgroups per CU; stages = 1: one workgroup per row.
  const bool pipe = l.stages == 2;
  uint64_t grid = d.rows;
  if (l.workgroups) {
    grid = (uint64_t)l.workgroups;
  } else if (pipe) {
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
