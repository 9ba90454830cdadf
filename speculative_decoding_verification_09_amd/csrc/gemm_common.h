// Pieces shared by the scoring-GEMM kernels (gfx950, bf16 MFMA).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l
// holds A[row l%16][k 8*(l/16) .. +7], B[k 8*(l/16) .. +7][col l%16], and
// receives D[rows 4*(l/16) .. +3][col l%16].
#pragma once

#include <atomic>

#include "internal.h"

namespace specdec {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPad = 8;  // bf16 padding per LDS row: 16 bytes, spreads rows over banks

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7f800000u) == 0x7f800000u) return (b >> 16) | ((b & 0x7fffffu) ? 0x40u : 0u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// W is read exactly once per call, so its loads are marked nontemporal: the
// memory system then streams it without keeping it in the caches (a plain
// streaming read measured 6.9 TB/s this way against 6.4 TB/s without).
template <bool NTL>
__device__ __forceinline__ u32x4 load_w16(const uint16_t* p) {
  return NTL ? __builtin_nontemporal_load((const u32x4*)p) : *(const u32x4*)p;
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Stores one lane's 4 consecutive outputs Y[n][v0 .. v0+3] (v0 < V).
template <bool OUT_BF16>
__device__ __forceinline__ void store4(void* Y, size_t base, int64_t v0, int64_t V, const f32x4& a) {
  const bool vec = (V & 3) == 0;
  if (OUT_BF16) {
    uint16_t* y = (uint16_t*)Y + base;
    if (vec) {
      *(u32x2*)y = u32x2{bf16_rne(a[0]) | (bf16_rne(a[1]) << 16), bf16_rne(a[2]) | (bf16_rne(a[3]) << 16)};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v0 + j < V) y[j] = (uint16_t)bf16_rne(a[j]);
    }
  } else {
    float* y = (float*)Y + base;
    if (vec) {
      *(f32x4*)y = a;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v0 + j < V) y[j] = a[j];
    }
  }
}

template <class K>
inline hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Compute units of the current device, cached per device.  Host threads may
// call this at once: each slot is an atomic, and two threads that both miss
// store the same value.
inline int device_cus() {
  static std::atomic<int> cached[64];  // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace gemm
}  // namespace specdec
