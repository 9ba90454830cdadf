// Skinny-N bf16 scoring GEMM for gfx950: Y[n, v] = sum_k X[n, k] * W[v, k].
//
// The verification pass scores N = B*(gamma+1) positions with one read of the
// output-layer weights ("LLM Inference & Speculative Decoding", section 0: a
// linear layer over N << d tokens moves ~2*d_in*d_out bytes for 2*N*d_in*d_out
// flops, so its intensity is about N flop/byte; "Speculative Decoding:
// Mathematical Foundations ...", "Prefill vs. Verification Arithmetic
// Intensity").  For N up to a few hundred the work is bound by streaming W
// from HBM, so every kernel here reads each W byte exactly once.
//
// W rows go on the M side of v_mfma_f32_16x16x32_bf16 and are loaded from
// global memory straight into A-operand registers (no LDS round trip, no
// conversion, no VALU FMAs).  X is tiny and sits in LDS.  Operand layout of
// 16x16x32 bf16 (checked on the device): lane l holds A[row l%16][k
// 8*(l/16) .. +7], B[k 8*(l/16) .. +7][col l%16], and receives D[rows
// 4*(l/16) .. +3][col l%16].
//
// Weight layouts.
//   row-major: W[V][d] as given.
//   packed:    16-row tiles; inside tile t, k-step s (32 k values) is one
//              contiguous 1 KB block in which lane l = 16*g + m finds its 16
//              bytes W[16t + m][32s + 8g .. +7].  A wave's A-operand load is
//              then one fully contiguous 1 KB read, and a tile is read front to
//              back.  Rows past V are zero.  specdec_pack_weights builds it once.
//
// Kernels.
//   sweep  (packed, N <= 8, X fits in LDS): persistent, one workgroup per CU.
//          A workgroup takes one 16-row tile at a time; its 8 waves split the
//          tile's k range and each streams a contiguous slice, the next work
//          unit prefetched into a second register buffer; partial sums meet in
//          LDS in a fixed order.  At any moment the whole GPU reads within a
//          window of about (#CUs x tile size), which keeps HBM streaming close
//          to a plain sequential read.
//   tiled  (any layout, any N): each wave owns 16*R vocabulary rows for the
//          whole k range; X is staged through LDS in k-chunks, double
//          buffered; NT 16-wide token tiles cover up to 16*NT tokens without
//          re-reading W.
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

// ---------------------------------------------------------------------------
// Packing: Wp[((t * nsteps + s) * 64 + l) * 8 + e] = W[16t + l%16][32s + 8(l/16) + e].
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wp,
                                                   int64_t V, int64_t d) {
  const int64_t nsteps = d / 32;
  const int64_t total = ((V + 15) / 16) * nsteps * 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t l = i & 63, ts = i >> 6, s = ts % nsteps, t = ts / nsteps;
    const int64_t v = t * 16 + (l & 15), k = s * 32 + 8 * (l >> 4);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (v < V) val = *(const u32x4*)(W + v * d + k);
    *(u32x4*)(Wp + i * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Sweep kernel (packed W, small N).  Work unit u = (tile, k-group): tile
// t = blockIdx.x + (u / ngroups) * gridDim.x, group u % ngroups.  Wave w owns
// k-steps [w*spw, (w+1)*spw) of every tile, taken SPW at a time.
template <int NW, int SPW, bool NTL, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void sweep_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
                                                        void* __restrict__ Y, int N, int d, int V) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, m = lane & 15, g = lane >> 4;
  const int pitch = d + kPad;
  const int nsteps = d >> 5;
  const int ntiles = (V + 15) >> 4;
  const int spw = (nsteps + NW - 1) / NW;        // k-steps per wave and tile
  const int ngroups = (spw + SPW - 1) / SPW;     // register groups per wave and tile
  uint16_t* xs = lds;
  f32x4* red = (f32x4*)(lds + (((size_t)N * pitch + 7) & ~(size_t)7));
  for (int i = tid; i < N * (d >> 3); i += NW * 64) {
    const int n = i / (d >> 3), u = i - n * (d >> 3);
    *(u32x4*)(xs + n * pitch + u * 8) = *(const u32x4*)(X + (size_t)n * d + u * 8);
  }
  __syncthreads();
  const bool live = m < N;
  const int my0 = wv * spw;                       // first k-step of this wave
  const int my1 = min(my0 + spw, nsteps);         // one past the last
  const int64_t units = (int64_t)((ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x) * ngroups;

  auto load = [&](u32x4(&dst)[SPW], int64_t u) {
    const int t = (int)blockIdx.x + (int)(u / ngroups) * (int)gridDim.x;
    const int s0 = my0 + (int)(u % ngroups) * SPW;
    const uint16_t* p = Wp + ((size_t)t * nsteps + s0) * 512 + lane * 8;
#pragma unroll
    for (int s = 0; s < SPW; ++s) dst[s] = (s0 + s < my1) ? load_w16<NTL>(p + (size_t)s * 512) : u32x4{0u, 0u, 0u, 0u};
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const u32x4(&a)[SPW], int64_t u) {
    const int grp = (int)(u % ngroups);
    const int s0 = my0 + grp * SPW;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (s0 + s < my1) {
        const u32x4 bf = live ? *(const u32x4*)(xs + m * pitch + (s0 + s) * 32 + 8 * g) : u32x4{0u, 0u, 0u, 0u};
        acc = mfma(a[s], bf, acc);
      }
    }
    if (grp != ngroups - 1) return;
    // Last group of the tile: sum the waves' partials in a fixed order.
    red[wv * 64 + lane] = acc;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (wv == 0) {
      f32x4 sum = red[lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const f32x4 o = red[w * 64 + lane];
        sum[0] += o[0];
        sum[1] += o[1];
        sum[2] += o[2];
        sum[3] += o[3];
      }
      const int t = (int)blockIdx.x + (int)(u / ngroups) * (int)gridDim.x;
      const int64_t v0 = (int64_t)t * 16 + 4 * g;
      if (live && v0 < V) store4<OUT_BF16>(Y, (size_t)m * V + v0, v0, V, sum);
    }
    __syncthreads();
  };
  u32x4 a0[SPW], a1[SPW];
  if (units > 0) load(a0, 0);
  for (int64_t u = 0; u < units; u += 2) {
    if (u + 1 < units) load(a1, u + 1);
    consume(a0, u);
    if (u + 1 >= units) break;
    if (u + 2 < units) load(a0, u + 2);
    consume(a1, u + 1);
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel.  NT: 16-wide token tiles per workgroup; R: 16-row vocabulary
// tiles per wave; KC: k per chunk; NW: waves per workgroup.
template <int NT, int R, int KC, int NW, bool PACKED, bool NTL, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void tiled_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                        void* __restrict__ Y, int N, int d, int V, int n_base) {
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
  const int nsteps = d >> 5;

  // Token rows beyond N stay zero in both buffers.
  {
    const int pad_units = (NT * 16 - ncols) * (kRow / 8);
    for (int i = tid; i < 2 * pad_units; i += kThreads) {
      const int buf = i / pad_units, rem = i - buf * pad_units;
      const int r = ncols + rem / (kRow / 8), u = rem % (kRow / 8);
      *(u32x4*)(xs + buf * kBuf + r * kRow + u * 8) = zero;
    }
  }

  // This lane's W rows (row-major: clamped into range; rows >= V are never stored).
  const int64_t vwave = (int64_t)blockIdx.x * (NW * 16 * R) + wv * 16 * R;
  const uint16_t* wp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (PACKED) {
      wp[r] = W + ((size_t)((vwave >> 4) + r) * nsteps) * 512 + lane * 8;
    } else {
      int64_t v = vwave + 16 * r + m;
      v = v < V ? v : (int64_t)V - 1;
      wp[r] = W + (size_t)v * d + 8 * g;
    }
  }
  const int64_t ntiles = ((int64_t)V + 15) >> 4;

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
      for (int r = 0; r < R; ++r) {
        if (PACKED) {
          const bool ok = (c * KC + 32 * s) < d && (vwave >> 4) + r < ntiles;
          dst[s][r] = ok ? load_w16<NTL>(wp[r] + (size_t)(c * kSteps + s) * 512) : zero;
        } else {
          dst[s][r] = k < d ? load_w16<NTL>(wp[r] + c * KC + 32 * s) : zero;
        }
      }
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
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 bf = *(const u32x4*)(xb + (t * 16 + m) * kRow + 32 * s + 8 * g);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = mfma(wa[s][r], bf, acc[r][t]);
      }
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
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t v0 = vwave + 16 * r + 4 * g;
    if (v0 >= V) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = t * 16 + m;
      if (n >= ncols) continue;
      store4<OUT_BF16>(Y, (size_t)(n_base + n) * V + v0, v0, V, acc[r][t]);
    }
  }
}

template <class K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int NT, int R, int KC, int NW, bool PACKED, bool NTL>
hipError_t launch_tiled(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V, bool out_bf16,
                        hipStream_t stream) {
  constexpr int kRowsPerBlock = NW * 16 * R;
  constexpr size_t kLds = 2ull * NT * 16 * (KC + kPad) * sizeof(uint16_t);
  const dim3 grid((unsigned)((V + kRowsPerBlock - 1) / kRowsPerBlock));
  auto k = out_bf16 ? tiled_kernel<NT, R, KC, NW, PACKED, NTL, true> : tiled_kernel<NT, R, KC, NW, PACKED, NTL, false>;
  hipError_t e = allow_lds(k, kLds);
  if (e != hipSuccess) return e;
  for (int64_t n0 = 0; n0 < N; n0 += NT * 16) {
    hipLaunchKernelGGL(k, grid, dim3(NW * 64), kLds, stream, X, W, Y, (int)N, (int)d, (int)V, (int)n0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

constexpr int kSweepWaves = 8;
constexpr int kSweepGroup = 16;

size_t sweep_lds_bytes(int64_t N, int64_t d) {
  return (((size_t)N * (size_t)(d + kPad) + 7) & ~(size_t)7) * sizeof(uint16_t) + (size_t)kSweepWaves * 64 * 16;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

int64_t packed_weight_elems(int64_t V, int64_t d) { return ((V + 15) / 16) * 16 * d; }

hipError_t launch_pack_weights(const uint16_t* W, uint16_t* Wp, int64_t V, int64_t d, hipStream_t stream) {
  const int64_t total = ((V + 15) / 16) * (d / 32) * 64;
  const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, Wp, V, d);
  return hipGetLastError();
}

hipError_t launch_skinny_gemm(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V,
                              bool out_bf16, bool packed, hipStream_t stream) {
  // Shapes chosen by measurement on MI355X (streaming rate of W per N range).
  if (packed) {
    const size_t lds = sweep_lds_bytes(N, d);
    if (N <= 8 && lds <= 150 * 1024) {
      auto k = out_bf16 ? sweep_kernel<kSweepWaves, kSweepGroup, true, true>
                        : sweep_kernel<kSweepWaves, kSweepGroup, true, false>;
      hipError_t e = allow_lds(k, lds);
      if (e != hipSuccess) return e;
      const int64_t ntiles = (V + 15) / 16;
      const int64_t grid = ntiles < device_cus() ? ntiles : device_cus();
      hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kSweepWaves * 64), lds, stream, X, W, Y, (int)N, (int)d, (int)V);
      return hipGetLastError();
    }
    if (N <= 32) return launch_tiled<4, 2, 64, 4, true, true>(X, W, Y, N, d, V, out_bf16, stream);
    return launch_tiled<4, 1, 128, 8, true, true>(X, W, Y, N, d, V, out_bf16, stream);
  }
  if (N <= 16) return launch_tiled<1, 1, 256, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 32) return launch_tiled<2, 2, 128, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
  return launch_tiled<4, 2, 128, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
}

}  // namespace specdec
