// Packed weight layout and the sweep kernel: the scoring GEMM
// Y[n, v] = sum_k X[n, k] * W[v, k] for few positions (N <= 8).
//
// The verification pass scores N = B*(gamma+1) positions with one read of the
// output-layer weights ("LLM Inference & Speculative Decoding", section 0: a
// linear layer over N << d tokens moves ~2*d_in*d_out bytes for 2*N*d_in*d_out
// flops, so its intensity is about N flop/byte; "Speculative Decoding:
// Mathematical Foundations ...", "Prefill vs. Verification Arithmetic
// Intensity").  At these N the work is bound by streaming W from HBM, so the
// kernel reads each W byte exactly once.
//
// W rows go on the M side of the MFMA and are loaded from global memory
// straight into A-operand registers (no LDS round trip, no conversion, no VALU
// FMAs).  X is tiny and sits in LDS.
//
// Packed layout: 16-row tiles; inside tile t, k-step s (32 k values) is one
// contiguous 1 KB block in which lane l = 16*g + m finds its 16 bytes
// W[16t + m][32s + 8g .. +7].  A wave's A-operand load is then one fully
// contiguous 1 KB read, and a tile is read front to back.  Rows past V are
// zero.  specdec_pack_weights builds it once.
//
// Sweep kernel: persistent, one workgroup per CU.  A workgroup takes one
// 16-row tile at a time; its 8 waves split the tile's k range and each streams
// a contiguous slice, the next work unit prefetched into a second register
// buffer; partial sums meet in LDS in a fixed order.  At any moment the whole
// GPU reads within a window of about (#CUs x tile size), which keeps HBM
// streaming close to a plain sequential read.
#include "gemm_common.h"

namespace specdec {
namespace gemm {
namespace {

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

constexpr int kSweepWaves = 8;
constexpr int kSweepGroup = 16;

size_t sweep_lds_bytes(int64_t N, int64_t d) {
  return (((size_t)N * (size_t)(d + kPad) + 7) & ~(size_t)7) * sizeof(uint16_t) + (size_t)kSweepWaves * 64 * 16;
}

}  // namespace

bool sweep_applies(int64_t N, int64_t d) { return N <= 8 && sweep_lds_bytes(N, d) <= 150 * 1024; }

hipError_t launch_sweep(const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d, int64_t V, bool out_bf16,
                        hipStream_t stream) {
  const size_t lds = sweep_lds_bytes(N, d);
  auto k = out_bf16 ? sweep_kernel<kSweepWaves, kSweepGroup, true, true>
                    : sweep_kernel<kSweepWaves, kSweepGroup, true, false>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (V + 15) / 16;
  const int64_t grid = ntiles < device_cus() ? ntiles : device_cus();
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kSweepWaves * 64), lds, stream, X, Wp, Y, (int)N, (int)d, (int)V);
  return hipGetLastError();
}

}  // namespace gemm

int64_t packed_weight_elems(int64_t V, int64_t d) { return ((V + 15) / 16) * 16 * d; }

hipError_t launch_pack_weights(const uint16_t* W, uint16_t* Wp, int64_t V, int64_t d, hipStream_t stream) {
  const int64_t total = ((V + 15) / 16) * (d / 32) * 64;
  const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
  hipLaunchKernelGGL(gemm::pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, Wp, V, d);
  return hipGetLastError();
}

}  // namespace specdec
