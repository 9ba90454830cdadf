// Scoring GEMM Y[n, v] = sum_k X[n, k] * W[v, k] for more positions than the
// sweep kernel takes, and for row-major weights; plus the dispatcher.
//
// Tiled kernel (any layout, any N): each wave owns 16*R vocabulary rows for
// the whole k range, loading them straight into MFMA A-operand registers; X
// is staged through LDS in k-chunks, double buffered; NT 16-wide token tiles
// cover up to 16*NT tokens without re-reading W.
//
// Panel kernel (packed W, N in the tens to hundreds): the same register-direct
// W stream, with X staged in LDS in the MFMA's own lane order (one contiguous
// 1 KB block per 16 tokens x 32 k, so staging writes and operand reads are
// both conflict-free), all token tiles of a pass kept in accumulators, and
// several token passes over the same W rows placed on one XCD back to back so
// that only the first reads them from HBM.  A 16-row W block fetched into
// registers feeds NT MFMAs, and an X block read from LDS feeds R of them.
#include "gemm_common.h"

namespace specdec {
namespace gemm {
namespace {

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
// ---------------------------------------------------------------------------
// Panel kernel.  Grid: vocabulary blocks of NW*R 16-row tiles x token passes
// of NT*16 tokens, launched in an order where block id i runs on XCD i % 8 and
// the passes of one vocabulary block take consecutive slots of one XCD.
// KS: MFMA k-steps (32 k each) per LDS chunk.
template <int NT, int R, int NW, int KS, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void panel_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
                                                        void* __restrict__ Y, int N, int d, int V, int npass) {
  constexpr int kThreads = NW * 64;
  constexpr int kBlocks = NT * KS;                   // 1 KB X blocks per chunk
  constexpr int kXPT = (kBlocks * 64 + kThreads - 1) / kThreads;
  constexpr int kBufElems = kBlocks * 512;           // bf16 per LDS buffer
  extern __shared__ __align__(16) uint16_t xs[];

  const int nsteps = d >> 5;
  const int ntiles = (V + 15) >> 4;
  const int nvb = (ntiles + NW * R - 1) / (NW * R);
  const int id = (int)blockIdx.x;
  const int slot = id >> 3;
  const int vb = (id & 7) + 8 * (slot / npass);
  if (vb >= nvb) return;
  const int n0 = (slot % npass) * NT * 16;
  const int ncols = min(N - n0, NT * 16);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, m = lane & 15, g = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int vt0 = vb * NW * R + wv * R;              // this wave's first 16-row tile
  const uint16_t* wbase = Wp + (size_t)vt0 * nsteps * 512 + lane * 8;

  // X staging: unit u (16 bytes) = block b = u / 64 (token tile b / KS, k-step
  // b % KS of the chunk), lane position l = u % 64.  Rows past N read row N-1:
  // they only feed output columns that are never stored.
  u32x4 xr[kXPT];
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int u = tid + j * kThreads;
      if (kXPT * kThreads == kBlocks * 64 || u < kBlocks * 64) {
        const int b = u >> 6, l = u & 63;
        const int t = b / KS, s = c * KS + b % KS;
        const int n = min(n0 + t * 16 + (l & 15), N - 1);
        xr[j] = s < nsteps ? *(const u32x4*)(X + (size_t)n * d + s * 32 + 8 * (l >> 4)) : zero;
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int u = tid + j * kThreads;
      if (kXPT * kThreads == kBlocks * 64 || u < kBlocks * 64) *(u32x4*)(xs + buf * kBufElems + u * 8) = xr[j];
    }
  };
  auto load_w = [&](u32x4(&dst)[KS][R], int c) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int ks = c * KS + s;
#pragma unroll
      for (int r = 0; r < R; ++r)
        dst[s][r] = (ks < nsteps && vt0 + r < ntiles) ? load_w16<true>(wbase + ((size_t)r * nsteps + ks) * 512) : zero;
    }
  };

  f32x4 acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4(&wa)[KS][R], int buf, int c) {
    const uint16_t* xb = xs + buf * kBufElems + lane * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (c * KS + s >= nsteps) break;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 bf = *(const u32x4*)(xb + (t * KS + s) * 512);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = mfma(wa[s][r], bf, acc[r][t]);
      }
    }
  };

  const int nch = (nsteps + KS - 1) / KS;
  u32x4 wa[KS][R], wb[KS][R];
  load_x(0);
  load_w(wa, 0);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) {
      load_x(c + 1);
      load_w(wb, c + 1);
    }
    compute(wa, 0, c);
    if (c + 1 < nch) store_x(1);
    __syncthreads();
    if (c + 1 >= nch) break;
    if (c + 2 < nch) {
      load_x(c + 2);
      load_w(wa, c + 2);
    }
    compute(wb, 1, c + 1);
    if (c + 2 < nch) store_x(0);
    __syncthreads();
  }

  // Lane holds tokens n0 + 16t + m, vocabulary rows 16*(vt0 + r) + 4g .. +3.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t v0 = (int64_t)(vt0 + r) * 16 + 4 * g;
    if (v0 >= V) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = t * 16 + m;
      if (n >= ncols) continue;
      store4<OUT_BF16>(Y, (size_t)(n0 + n) * V + v0, v0, V, acc[r][t]);
    }
  }
}

template <int NT, int R, int NW, int KS>
constexpr size_t panel_lds_bytes() {
  return 2ull * NT * KS * 1024;
}

template <int NT, int R, int NW, int KS>
hipError_t launch_panel(const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d, int64_t V, bool out_bf16,
                        hipStream_t stream) {
  constexpr size_t kLds = panel_lds_bytes<NT, R, NW, KS>();
  static_assert(kLds <= 160 * 1024, "panel LDS");
  auto k = out_bf16 ? panel_kernel<NT, R, NW, KS, true> : panel_kernel<NT, R, NW, KS, false>;
  hipError_t e = allow_lds(k, kLds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (V + 15) / 16;
  const int64_t nvb = (ntiles + NW * R - 1) / (NW * R);
  const int64_t npass = (N + NT * 16 - 1) / (NT * 16);
  const int64_t grid = 8 * ((nvb + 7) / 8) * npass;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(NW * 64), kLds, stream, X, Wp, Y, (int)N, (int)d, (int)V,
                     (int)npass);
  return hipGetLastError();
}

}  // namespace
}  // namespace gemm

hipError_t launch_skinny_gemm(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V,
                              bool out_bf16, bool packed, hipStream_t stream) {
  using namespace gemm;
  // Shapes chosen by measurement on MI355X (streaming rate of W per N range).
  if (packed) {
    if (sweep_applies(N, d)) return launch_sweep(X, W, Y, N, d, V, out_bf16, stream);
    if (N <= 32) return launch_tiled<4, 2, 64, 4, true, true>(X, W, Y, N, d, V, out_bf16, stream);
    return launch_tiled<4, 1, 128, 8, true, true>(X, W, Y, N, d, V, out_bf16, stream);
  }
  if (N <= 16) return launch_tiled<1, 1, 256, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 32) return launch_tiled<2, 2, 128, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
  return launch_tiled<4, 2, 128, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
}

}  // namespace specdec
