// Device helpers for the gfx950 kernels: 16-byte vector memory access with
// optional nontemporal hints, bf16 widening / round-to-nearest-even
// narrowing, and the element-wise fold in rank order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ccl.h"

namespace ccl {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_plain(const char *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ u32x4 ld_nt(const char *p) {
  return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ void st_plain(char *p, u32x4 v) { *(u32x4 *)p = v; }
__device__ __forceinline__ void st_nt(char *p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4 *)p); }

// The hint as a compile-time choice.  Selecting between ld_nt and ld_plain
// (or st_nt and st_plain) with a runtime flag is not enough: the compiler
// merges the two accesses into one and drops the nontemporal hint.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const char *p) {
  if constexpr (NT) return ld_nt(p);
  else return ld_plain(p);
}
template <bool NT>
__device__ __forceinline__ void st(char *p, u32x4 v) {
  if constexpr (NT) st_nt(p, v);
  else st_plain(p, v);
}

// Write-through streaming stores: buffer stores with the nontemporal and
// device-scope (sc1) cache-policy bits.  At device scope the L2 of the issuing
// XCD passes the line on to memory instead of holding it dirty.  Whether that
// is faster depends on the call (the launch code picks it per collective, P
// and size from measurements); it needs >= 4 resident workgroups per CU to
// cover its longer completion time, and whole 256-byte lines.  The buffer
// resource is built from `base`, which the callers keep uniform across the
// workgroup (a per-lane base would make the compiler loop over lanes): no
// stride, 2^31 - 1 bytes in range (the lane's byte offset from `base` is
// below 2^31), and the 32-bit data format that raw buffer accesses on
// gfx9-family parts take in the resource's last dword.
constexpr int kPolNtSc1 = 2 | 16;         // cache-policy bits: nt | sc1
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(char *base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, kRawBufferWord3);
}
__device__ __forceinline__ void st_wt(char *base, uint64_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, wt_rsrc(base), (int)off, 0, kPolNtSc1);
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_wt_b64(char *base, uint64_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, wt_rsrc(base), (int)off, 0, kPolNtSc1);
}
__device__ __forceinline__ void st_wt_b32(char *base, uint64_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, wt_rsrc(base), (int)off, 0, kPolNtSc1);
}

// A 16-byte load through a raw buffer resource over [base, base + bytes):
// `base` must be the same in every lane, `off` is the lane's byte offset.  A
// load outside the range (bytes = 0 makes every load so) returns zero and
// reads nothing.  NT: the nontemporal cache-policy bit.
template <bool NT>
__device__ __forceinline__ u32x4 ld_row(const char *base, uint32_t bytes, int off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kRawBufferWord3);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}

// A pointer the caller knows to be the same in every lane, moved to scalar
// registers so that a buffer resource can be built from it without a loop
// over lanes.
__device__ __forceinline__ char *wave_uniform(char *p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (char *)(((uint64_t)hi << 32) | lo);
}

// Store policy of the kernels that take it as a template argument.
enum StorePol { ST_PLAIN = 0, ST_NT = 1, ST_WT = 2 };
template <int POL>
__device__ __forceinline__ void st_pol(char *base, uint64_t off, u32x4 v) {
  if constexpr (POL == ST_WT) st_wt(base, off, v);
  else if constexpr (POL == ST_NT) st_nt(base + off, v);
  else st_plain(base + off, v);
}

// bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32 one.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits (in the low 16 bits), round to nearest, ties to even;
// NaN becomes the canonical quiet NaN 0x7fc0.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? 0x7fc0u : r;
}

// fp16 <-> fp32: widening is exact; narrowing rounds to nearest even (the
// default rounding mode), fp16 denormals kept.
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t f16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// One fold step.  min/max are compare-and-select so a tie (including +0 vs
// -0) keeps the accumulated (earlier-rank) value.
template <int OP>
__device__ __forceinline__ float fold_f32(float acc, float v) {
  if constexpr (OP == CCL_SUM) return acc + v;
  else if constexpr (OP == CCL_MIN) return (v < acc) ? v : acc;
  else return (v > acc) ? v : acc;
}

template <int OP>
__device__ __forceinline__ int32_t fold_i32(int32_t acc, int32_t v) {
  if constexpr (OP == CCL_SUM) return (int32_t)((uint32_t)acc + (uint32_t)v);
  else if constexpr (OP == CCL_MIN) return (v < acc) ? v : acc;
  else return (v > acc) ? v : acc;
}

// Fold the first n (runtime, <= NI) vectors of x element-wise in rank order.
template <int DT, int OP, int NI>
__device__ __forceinline__ u32x4 fold_vec(const u32x4 (&x)[NI], int n) {
  u32x4 y;
  if constexpr (DT == CCL_FLOAT16) {
    float a[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[2 * k] = f16_lo(x[0][k]);
      a[2 * k + 1] = f16_hi(x[0][k]);
    }
#pragma unroll
    for (int r = 1; r < NI; ++r) {
      if (r < n) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a[2 * k] = fold_f32<OP>(a[2 * k], f16_lo(x[r][k]));
          a[2 * k + 1] = fold_f32<OP>(a[2 * k + 1], f16_hi(x[r][k]));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = f16_rne(a[2 * k]) | (f16_rne(a[2 * k + 1]) << 16);
  } else if constexpr (DT == CCL_BFLOAT16) {
    float a[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[2 * k] = bf16_lo(x[0][k]);
      a[2 * k + 1] = bf16_hi(x[0][k]);
    }
#pragma unroll
    for (int r = 1; r < NI; ++r) {
      if (r < n) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a[2 * k] = fold_f32<OP>(a[2 * k], bf16_lo(x[r][k]));
          a[2 * k + 1] = fold_f32<OP>(a[2 * k + 1], bf16_hi(x[r][k]));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = bf16_rne(a[2 * k]) | (bf16_rne(a[2 * k + 1]) << 16);
  } else if constexpr (DT == CCL_FLOAT32) {
    float a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = __uint_as_float(x[0][k]);
#pragma unroll
    for (int r = 1; r < NI; ++r)
      if (r < n) {
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = fold_f32<OP>(a[k], __uint_as_float(x[r][k]));
      }
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = __float_as_uint(a[k]);
  } else {
    int32_t a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = (int32_t)x[0][k];
#pragma unroll
    for (int r = 1; r < NI; ++r)
      if (r < n) {
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = fold_i32<OP>(a[k], (int32_t)x[r][k]);
      }
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = (uint32_t)a[k];
  }
  return y;
}

}  // namespace ccl
