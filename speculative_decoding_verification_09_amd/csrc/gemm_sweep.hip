// Packed weight layout and the sweep kernel: the scoring GEMM
// Y[n, v] = sum_k X[n, k] * W[v, k] for few positions (N <= 16: one MFMA column tile).
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
// Sweep kernel (packed W, small N).  The kernel can split the k range into
// groups of spk k-steps (KG = ceil(nsteps / spk) groups): block b takes group
// b % KG of the tiles t = b / KG + j * (gridDim.x / KG), holds only that slice
// of X in LDS, and writes its partial sums to slice b % KG of Y (fp32
// [KG][N][V]).  The planner runs it with one group (spk = nsteps), where Y is
// the output.
// Inside a block, wave w owns k-steps [w*spw, (w+1)*spw) of the group, taken
// SPW at a time; a work unit u is (tile u / ngroups, register group
// u % ngroups).
//
// Inside the main loop every global load is issued unconditionally, with its
// address clamped into the wave's k range where a register group runs past it
// (those values are never used): the compiler can then count outstanding loads
// exactly and keeps the next unit's loads in flight while the current unit
// computes, instead of draining all of them at each branch join.
//
// Statistics epilogue (EPI 1: softmax at temperature T, EPI 2: argmax), used
// by the whole verification step with one k-group: wave 0 folds every tile's
// finished logits into a running per-lane state (max of a = z * fl32(1/T) and
// an fp64 sum of fp32 exp(a - max), rescaled when the max grows; or the
// largest z with its lowest index), records the logit of each row's drafted
// token from the tile that holds it, and at the end leaves one partial per
// (row, workgroup).  With draft logits, the workgroups that have one tile
// fewer (they finish first) also summarise a slice of every draft row, one
// wave per row (few rows here: B*(gamma+1) <= 16).
template <int NW, int SPW, bool NTL, bool OUT_BF16, int EPI>
__global__ __launch_bounds__(NW * 64) void sweep_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
                                                        void* __restrict__ Y, int N, int d, int V, int spk,
                                                        FusedStats fs) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
  if (EPI == 1 && fs.done != nullptr) {  // the draw kernel's counters, for the step that follows
    const int64_t gid = (int64_t)blockIdx.x * (NW * 64) + tid;
    if (gid < fs.B) fs.done[gid] = 0u;
  }
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int nsteps = d >> 5;
  const int ntiles = (V + 15) >> 4;
  const int kgs = (nsteps + spk - 1) / spk;
  const int kg = (int)blockIdx.x % kgs;
  const int stream = (int)blockIdx.x / kgs, nstream = (int)gridDim.x / kgs;
  const int ks0 = kg * spk;                       // first k-step of the group
  const int kw = min(spk, nsteps - ks0);          // k-steps in the group (>= 1)
  const int pitch = spk * 32 + kPad;
  const int spw = (kw + NW - 1) / NW;             // k-steps per wave and tile
  const int ngroups = (spw + SPW - 1) / SPW;      // register groups per wave and tile
  uint16_t* xs = lds;
  f32x4* red = (f32x4*)(lds + (((size_t)N * pitch + 7) & ~(size_t)7));
  const int units_per_row = kw * 4;               // 16-byte units of one X row slice
  for (int i = tid; i < N * units_per_row; i += NW * 64) {
    const int n = i / units_per_row, u = i - n * units_per_row;
    *(u32x4*)(xs + n * pitch + u * 8) = *(const u32x4*)(X + (size_t)n * d + (size_t)ks0 * 32 + u * 8);
  }
  __syncthreads();
  const bool live = m < N;
  const int mx = live ? m : N - 1;                // lanes past N read a valid row; their column is not stored
  const int my0 = wv * spw;                       // first k-step of this wave, relative to ks0
  const int my1 = min(my0 + spw, kw);             // one past the last
  const int last = max(0, min(my1, kw) - 1);      // a k-step of the group this wave may address
  const int64_t units = stream < ntiles ? (int64_t)((ntiles - stream + nstream - 1) / nstream) * ngroups : 0;
  float* part = (float*)Y + (size_t)kg * N * V;   // this group's slice when the k range is split

  // Statistics state of lane (token m, rows 4g .. 4g+3 of each tile).
  float st_m = -INFINITY;
  double st_s = 0.0;
  int st_i = 0x7fffffff;
  int st_x = -1;  // drafted token of this lane's row, if any
  if (EPI == 1 && live) {
    const int g1 = (int)fs.gamma + 1;
    const int bq = m / g1, iq = m - bq * g1;
    if (iq < fs.gamma) {
      const int32_t x = fs.tokens[bq * fs.gamma + iq];
      st_x = x < 0 ? 0 : (x >= V ? V - 1 : x);
    }
  }

  auto load = [&](u32x4(&dst)[SPW], int64_t u) {
    const int t = stream + (int)(u / ngroups) * nstream;
    const int s0 = my0 + (int)(u % ngroups) * SPW;
    const uint16_t* p = Wp + ((size_t)t * nsteps + ks0) * 512 + lane * 8;
#pragma unroll
    for (int s = 0; s < SPW; ++s) dst[s] = load_w16<NTL>(p + (size_t)min(s0 + s, last) * 512);
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const u32x4(&a)[SPW], int64_t u) {
    const int grp = (int)(u % ngroups);
    const int s0 = my0 + grp * SPW;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (s0 + s < my1) {
        const u32x4 bf = *(const u32x4*)(xs + mx * pitch + (s0 + s) * 32 + 8 * g);
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
      const int t = stream + (int)(u / ngroups) * nstream;
      const int64_t v0 = (int64_t)t * 16 + 4 * g;
      if (live && v0 < V) {
        if (kgs == 1)
          store4<OUT_BF16>(Y, (size_t)m * V + v0, v0, V, sum);
        else
          store4<false>(part, (size_t)m * V + v0, v0, V, sum);
        if (EPI == 1) {  // terms 2^(z * c1 - max * log2(e)), c1 = fl32(1/T) * log2(e)
          constexpr float kLog2e = 1.4426950408889634f;
          float zt = -INFINITY;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v0 + j < V) zt = fmaxf(zt, sum[j]);
          const float mt = zt * fs.inv_t;  // = max of fl32(z * fl32(1/T)) over the four
          if (mt > st_m) {
            if (st_s > 0.0) st_s *= (double)__builtin_amdgcn_exp2f((st_m - mt) * kLog2e);
            st_m = mt;
          }
          const float c1 = fs.inv_t * kLog2e, c2 = st_m * kLog2e;
          float s4 = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v0 + j < V) s4 += __builtin_amdgcn_exp2f(fmaf(sum[j], c1, -c2));
          st_s += (double)s4;
        } else if (EPI == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v0 + j < V && (sum[j] > st_m || (sum[j] == st_m && (int)v0 + j < st_i))) {
              st_m = sum[j];
              st_i = (int)v0 + j;
            }
        }
        if (EPI == 1 && st_x >= v0 && st_x < v0 + 4) fs.zx[m] = sum[st_x - (int)v0];
      }
    }
    __syncthreads();
  };
  if (units <= 0) return;
  // Two units per trip so the prefetch registers swap roles without copies;
  // the loop body loads only units that exist, and the last one or two units
  // are peeled off so that no load is issued past the end.
  u32x4 a0[SPW], a1[SPW];
  load(a0, 0);
  int64_t u = 0;
  for (; u + 2 < units; u += 2) {
    load(a1, u + 1);
    consume(a0, u);
    load(a0, u + 2);
    consume(a1, u + 1);
  }
  if (u + 1 < units) {
    load(a1, u + 1);
    consume(a0, u);
    consume(a1, u + 1);
  } else {
    consume(a0, u);
  }
  if (EPI == 0) return;

  // Partials of the target rows: combine the four lanes of each token.
  if (wv == 0) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float om = __shfl_xor(st_m, o);
      if (EPI == 1) {
        const double os = __shfl_xor(st_s, o);
        const float M = fmaxf(st_m, om);
        st_s = (st_s > 0.0 ? st_s * exp((double)st_m - (double)M) : 0.0) +
               (os > 0.0 ? os * exp((double)om - (double)M) : 0.0);
        st_m = M;
      } else {
        const int oi = __shfl_xor(st_i, o);
        if (om > st_m || (om == st_m && oi < st_i)) {
          st_m = om;
          st_i = oi;
        }
      }
    }
    if (g == 0 && live) {
      const size_t slot = (size_t)m * fs.pstride + blockIdx.x;
      fs.cmax[slot] = st_m;
      if (EPI == 1)
        fs.csum[slot] = st_s;
      else
        fs.cidx[slot] = st_i;
    }
  }
  if (EPI != 1 || fs.draft == nullptr) return;

  // Draft rows: workgroups with the smaller tile count take consecutive
  // vocabulary slices (a multiple of 4 entries each); the others leave empty
  // partials.  Wave w takes draft rows w, w + NW, ...  A lane loads sixteen
  // entries at a time, all before any use; the fp64 sum is rescaled when the
  // running maximum grows (only for slices past 1024 entries).
  const int G = (int)gridDim.x;
  const int rem = ntiles % G;
  const int ndraft = rem == 0 ? G : G - rem;
  const int rank = rem == 0 ? (int)blockIdx.x : (int)blockIdx.x - rem;
  const int L = (((V + ndraft - 1) / ndraft) + 3) & ~3;
  const int s0 = rank >= 0 ? min(rank * L, V) : V, s1 = rank >= 0 ? min(s0 + L, V) : V;
  const int nd = (int)(fs.B * fs.gamma);
  for (int j = wv; j < nd; j += NW) {
    const float* row = fs.draft + (size_t)j * V;
    constexpr int kPer = 16;
    float mx = -INFINITY;
    double sm = 0.0;
    for (int c0 = s0; c0 < s1; c0 += 64 * kPer) {
      float a[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int v = c0 + 64 * e + lane;
        a[e] = v < s1 ? row[v] * fs.inv_t : -INFINITY;
      }
      float bm = a[0];
#pragma unroll
      for (int e = 1; e < kPer; ++e) bm = fmaxf(bm, a[e]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
      const float mn = fmaxf(mx, bm);  // wave-uniform
      if (mn == -INFINITY) continue;
      if (sm > 0.0) sm *= exp((double)mx - (double)mn);
      mx = mn;
#pragma unroll
      for (int e = 0; e < kPer; ++e) sm += (double)expf(a[e] - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
    if (lane == 0) {
      const size_t slot = (size_t)(N + j) * fs.pstride + blockIdx.x;
      fs.cmax[slot] = mx;
      fs.csum[slot] = sm;
      const int32_t x = fs.tokens[j];
      const int xc = x < 0 ? 0 : (x >= V ? V - 1 : x);
      if (xc >= s0 && xc < s1) fs.zx[N + j] = row[xc];
    }
  }
}

constexpr int kSweepWaves = 8;
constexpr int kSweepGroup = 16;
constexpr size_t kSweepLdsLimit = 150 * 1024;

size_t sweep_lds_bytes(int64_t N, int64_t spk) {
  return (((size_t)N * (size_t)(spk * 32 + kPad) + 7) & ~(size_t)7) * sizeof(uint16_t) +
         (size_t)kSweepWaves * 64 * 16;
}

}  // namespace

SweepPlan plan_sweep(int64_t N, int64_t d, int64_t V, int cus) {
  SweepPlan p{};
  const int64_t nsteps = d / 32, ntiles = (V + 15) / 16;
  // One k-group: X whole in LDS (the dispatcher takes the panel kernel otherwise).
  if (N > 16 || nsteps < 1 || sweep_lds_bytes(N, nsteps) > kSweepLdsLimit) return p;
  p.ok = true;
  p.spk = nsteps;
  p.kgroups = 1;
  p.grid = ntiles < cus ? ntiles : cus;
  return p;
}

hipError_t launch_sweep(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d,
                        int64_t V, bool out_bf16, hipStream_t stream) {
  const size_t lds = sweep_lds_bytes(N, p.spk);
  auto k = out_bf16 ? sweep_kernel<kSweepWaves, kSweepGroup, true, true, 0>
                    : sweep_kernel<kSweepWaves, kSweepGroup, true, false, 0>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  const FusedStats none{};
  hipLaunchKernelGGL(k, dim3((unsigned)p.grid), dim3(kSweepWaves * 64), lds, stream, X, Wp, Y, (int)N, (int)d, (int)V,
                     (int)p.spk, none);
  return hipGetLastError();
}

}  // namespace gemm

namespace gemm {

hipError_t launch_sweep_with_stats(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, float* Y, int64_t N,
                                   int64_t d, int64_t V, const FusedStats& fs, int64_t* nparts, hipStream_t stream) {
  const size_t lds = sweep_lds_bytes(N, p.spk);
  auto k = fs.greedy ? sweep_kernel<kSweepWaves, kSweepGroup, true, false, 2>
                     : sweep_kernel<kSweepWaves, kSweepGroup, true, false, 1>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)p.grid), dim3(kSweepWaves * 64), lds, stream, X, Wp, (void*)Y, (int)N, (int)d,
                     (int)V, (int)p.spk, fs);
  e = hipGetLastError();
  if (e == hipSuccess) *nparts = p.grid;
  return e;
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
