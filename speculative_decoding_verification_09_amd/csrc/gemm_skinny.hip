// Skinny-N bf16 scoring GEMM for gfx950: Y[n, v] = sum_k X[n, k] * W[v, k].
//
// The verification pass scores N = B*(gamma+1) positions with one read of the
// output-layer weights ("LLM Inference & Speculative Decoding", section 0: a
// linear layer over N << d tokens moves ~2*d_in*d_out bytes for 2*N*d_in*d_out
// flops, so its intensity is about N flop/byte; "Speculative Decoding:
// Mathematical Foundations ...", "Prefill vs. Verification Arithmetic
// Intensity").  For N up to a few hundred the work is bound by streaming W
// from HBM, so the kernel is built around reading every W byte exactly once:
//
//   * W rows go on the M side of v_mfma_f32_16x16x32_bf16.  Each lane loads 16
//     bytes (8 bf16 along k) of one W row straight from global memory into the
//     A-operand registers: no LDS round trip, no conversion, no VALU FMAs.
//     A wave owns 16*R consecutive vocabulary rows for the whole k range and
//     prefetches the next k-chunk of W while the matrix cores work on the
//     current one.
//   * X (tiny: N x d) is staged in LDS in k-chunks, double buffered, shared by
//     the waves of a workgroup; lanes read their B-operand fragments from it.
//     Token columns beyond N are zero rows in LDS.  All N columns are handled
//     in one workgroup (NT column tiles of 16), so W is never re-read for
//     N <= 512.
//   * Accumulation is fp32 in the MFMA accumulators; results are written as
//     fp32 (or bf16, round to nearest even) with 16-byte (8-byte) stores.
//
// MFMA operand layout of 16x16x32 bf16 (checked on the device): lane l holds
// A[row l%16][k 8*(l/16) .. +7], B[k 8*(l/16) .. +7][col l%16], and receives
// D[rows 4*(l/16) .. +3][col l%16].
#include "internal.h"

namespace specdec {
namespace {

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

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// NT: 16-wide token tiles per workgroup; R: 16-row vocabulary tiles per wave;
// KC: k elements per chunk; NW: waves per workgroup.
template <int NT, int R, int KC, int NW, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void skinny_gemm_kernel(const uint16_t* __restrict__ X,
                                                              const uint16_t* __restrict__ W, void* __restrict__ Y,
                                                              int N, int d, int V, int n_base) {
  constexpr int kThreads = NW * 64;
  constexpr int kSteps = KC / 32;          // MFMA k-steps per chunk
  constexpr int kRow = KC + kPad;          // LDS row pitch (bf16)
  constexpr int kBuf = NT * 16 * kRow;     // one LDS buffer (bf16)
  constexpr int kUnits = KC / 8;           // 16-byte units per X row per chunk
  constexpr int kXPT = (NT * 16 * kUnits + kThreads - 1) / kThreads;
  extern __shared__ __align__(16) uint16_t xs[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int m = lane & 15;
  const int g = lane >> 4;
  const int ncols = min(N - n_base, NT * 16);
  const uint16_t* Xb = X + (size_t)n_base * d;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // Token rows beyond N stay zero in both buffers.
  {
    const int pad_units = (NT * 16 - ncols) * (kRow / 8);
    for (int i = tid; i < 2 * pad_units; i += kThreads) {
      const int buf = i / pad_units, rem = i - buf * pad_units;
      const int r = ncols + rem / (kRow / 8), u = rem % (kRow / 8);
      *(u32x4*)(xs + buf * kBuf + r * kRow + u * 8) = zero;
    }
  }

  // This lane's W rows (clamped into range; rows >= V are computed but never stored).
  const int64_t vwave = (int64_t)blockIdx.x * (NW * 16 * R) + wv * 16 * R;
  const uint16_t* wp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t v = vwave + 16 * r + m;
    v = v < V ? v : (int64_t)V - 1;
    wp[r] = W + (size_t)v * d + 8 * g;
  }

  u32x4 xr[kXPT];
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int i = tid + j * kThreads;
      const int n = i / kUnits, u = i - n * kUnits;
      const int k = c * KC + u * 8;
      xr[j] = (n < ncols && k < d) ? *(const u32x4*)(Xb + (size_t)n * d + k) : zero;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int i = tid + j * kThreads;
      const int n = i / kUnits, u = i - n * kUnits;
      if (n < ncols) *(u32x4*)(xs + buf * kBuf + n * kRow + u * 8) = xr[j];
    }
  };
  auto load_w = [&](u32x4(&dst)[kSteps][R], int c) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int k = c * KC + 32 * s + 8 * g;
#pragma unroll
      for (int r = 0; r < R; ++r) dst[s][r] = k < d ? *(const u32x4*)(wp[r] + c * KC + 32 * s) : zero;
    }
  };

  f32x4 acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4(&wa)[kSteps][R], int buf) {
    const uint16_t* xb = xs + buf * kBuf;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 bf[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) bf[t] = *(const u32x4*)(xb + (t * 16 + m) * kRow + 32 * s + 8 * g);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[r][t] = mfma(wa[s][r], bf[t], acc[r][t]);
    }
  };

  const int nch = (d + KC - 1) / KC;
  u32x4 wa[kSteps][R], wb[kSteps][R];
  load_x(0);
  load_w(wa, 0);
  store_x(0);
  __syncthreads();
  // Two chunks per trip so the prefetch registers swap roles without copies.
  // X for the next chunk is loaded before W so that waiting for it does not
  // also wait for the W prefetch (loads complete in issue order).
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) {
      load_x(c + 1);
      load_w(wb, c + 1);
    }
    compute(wa, 0);
    if (c + 1 < nch) store_x(1);
    __syncthreads();
    if (c + 1 >= nch) break;
    if (c + 2 < nch) {
      load_x(c + 2);
      load_w(wa, c + 2);
    }
    compute(wb, 1);
    if (c + 2 < nch) store_x(0);
    __syncthreads();
  }

  // Epilogue: lane holds tokens n = 16t + m, vocabulary rows v0 .. v0+3.
  const bool vec = (V & 3) == 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t v0 = vwave + 16 * r + 4 * g;
    if (v0 >= V) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = t * 16 + m;
      if (n >= ncols) continue;
      const size_t base = (size_t)(n_base + n) * V + v0;
      const f32x4 a = acc[r][t];
      if (OUT_BF16) {
        uint16_t* y = (uint16_t*)Y + base;
        if (vec) {
          u32x2 pk = {bf16_rne(a[0]) | (bf16_rne(a[1]) << 16), bf16_rne(a[2]) | (bf16_rne(a[3]) << 16)};
          *(u32x2*)y = pk;
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
  }
}

template <int NT, int R, int KC, int NW>
hipError_t launch_shape(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V, bool out_bf16,
                        hipStream_t stream) {
  constexpr int kRowsPerBlock = NW * 16 * R;
  constexpr size_t kLds = 2ull * NT * 16 * (KC + kPad) * sizeof(uint16_t);
  const dim3 grid((unsigned)((V + kRowsPerBlock - 1) / kRowsPerBlock));
  for (int64_t n0 = 0; n0 < N; n0 += NT * 16) {
    if (out_bf16) {
      auto k = skinny_gemm_kernel<NT, R, KC, NW, true>;
      if (kLds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(k, grid, dim3(NW * 64), kLds, stream, X, W, Y, (int)N, (int)d, (int)V, (int)n0);
    } else {
      auto k = skinny_gemm_kernel<NT, R, KC, NW, false>;
      if (kLds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(k, grid, dim3(NW * 64), kLds, stream, X, W, Y, (int)N, (int)d, (int)V, (int)n0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_skinny_gemm(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V,
                              bool out_bf16, hipStream_t stream) {
  if (N <= 16) return launch_shape<1, 2, 256, 4>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 32) return launch_shape<2, 2, 256, 4>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 64) return launch_shape<4, 2, 256, 4>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 128) return launch_shape<8, 2, 128, 4>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 256) return launch_shape<16, 1, 64, 4>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 384) return launch_shape<24, 1, 64, 4>(X, W, Y, N, d, V, out_bf16, stream);
  return launch_shape<32, 1, 32, 4>(X, W, Y, N, d, V, out_bf16, stream);
}

}  // namespace specdec
