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
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
      wp[r] = W;
    } else {
      int64_t v = vwave + 16 * r + m;
      v = v < V ? v : (int64_t)V - 1;
      wp[r] = W + (size_t)v * d;
    }
  }
  const int64_t ntiles = ((int64_t)V + 15) >> 4;

  // Global loads are issued unconditionally from clamped addresses and the
  // values past the edges replaced by zeros with a select, so the compiler
  // can count outstanding loads and keep the prefetch in flight.
  u32x4 xr[kXPT];
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int i = tid + j * kThreads;
      const int n = i / kUnits, u = i - n * kUnits;
      const int k = c * KC + u * 8;
      const u32x4 v = *(const u32x4*)(Xb + (size_t)min(n, ncols - 1) * d + min(k, d - 8));
      xr[j] = (n < ncols && k < d) ? v : zero;
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
          const int64_t tile = min((vwave >> 4) + r, ntiles - 1);
          const int step = min(c * kSteps + s, nsteps - 1);
          const u32x4 v = load_w16<NTL>(W + ((size_t)tile * nsteps + step) * 512 + lane * 8);
          dst[s][r] = ok ? v : zero;
        } else {
          const u32x4 v = load_w16<NTL>(wp[r] + min(k, d - 8));
          dst[s][r] = k < d ? v : zero;
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
  // The last one or two chunks are peeled off so that the loop body loads
  // without conditions and no load is issued past the end.
  int c = 0;
  for (; c + 2 < nch; c += 2) {
    load_x(c + 1);
    load_w(wb, c + 1);
    compute(wa, 0);
    store_x(1);
    __syncthreads();
    load_x(c + 2);
    load_w(wa, c + 2);
    compute(wb, 1);
    store_x(0);
    __syncthreads();
  }
  if (c + 1 < nch) {
    load_x(c + 1);
    load_w(wb, c + 1);
    compute(wa, 0);
    store_x(1);
    __syncthreads();
    compute(wb, 1);
  } else {
    compute(wa, 0);
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
// Statistics epilogue of the panel kernel (see below).  xs: the kernel's LDS,
// free once the main loop has ended.
// The drafted token of each of a lane's NT tokens (n0 + 16t + lane % 16),
// clamped into [0, V), or -1 for a token without one: loaded before the main
// loop (EPI 1 only), so that no global load round trip waits at its end.
template <int NT, int EPI>
__device__ __forceinline__ void drafted_tokens(const FusedStats& fs, int V, int n0, int ncols, int lane,
                                               int (&xd)[NT]) {
  const int m = lane & 15;
  const int g1 = (int)fs.gamma + 1;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    xd[t] = -1;
    if (EPI == 1 && t * 16 + m < ncols) {
      const int n = n0 + t * 16 + m;
      const int bq = n / g1, iq = n - bq * g1;
      if (iq < fs.gamma) {
        const int32_t x = fs.tokens[bq * fs.gamma + iq];
        xd[t] = x < 0 ? 0 : (x >= V ? V - 1 : x);
      }
    }
  }
}

template <int NT, int R, int NW, int EPI>
__device__ __forceinline__ void panel_stats(const f32x4 (&acc)[R][NT], uint16_t* xs, const FusedStats& fs, int V,
                                            int n0, int ncols, int vt0, int vb, int wv, int lane,
                                            const int (&xd)[NT]) {
  constexpr int kTok = NT * 16;
  const int m = lane & 15, g = lane >> 4;
  float* lm = (float*)xs;                                     // [NW][kTok] wave maxima
  double* ls = (double*)((char*)xs + 4 * NW * kTok);          // [NW][kTok] wave sums (8-byte aligned)
  int* li = (int*)((char*)xs + 12 * NW * kTok);               // [NW][kTok] argmax indices
  __syncthreads();  // every wave is done with the X buffers
  // Pass 1: per-token maxima (with the lowest index at T == 0) over the wave's
  // rows; at T > 0 the max of a = z * fl32(1/T) is fl32(max z * fl32(1/T)).
  // Bitwise tests and selects throughout, and each shuffle round issued for
  // all NT tokens before any of them is merged: with short-circuit tests every
  // element and every merge became a branch, and each token's two shuffles
  // waited in turn, which at one wave per SIMD cost microseconds here.
  float pm[NT];
  int pi[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    pm[t] = -INFINITY;
    pi[t] = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = (vt0 + r) * 16 + 4 * g + j;
        const float a = acc[r][t][j];
        bool take = a > pm[t];
        if (EPI == 2) take = take | ((a == pm[t]) & (v < pi[t]));
        take = take & (v < V);
        pm[t] = take ? a : pm[t];
        pi[t] = take ? v : pi[t];
      }
  }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    float om[NT];
    int oi[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      om[t] = __shfl_xor(pm[t], o);
      if (EPI == 2) oi[t] = __shfl_xor(pi[t], o);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (EPI == 2) {
        const bool take = (om[t] > pm[t]) | ((om[t] == pm[t]) & (oi[t] < pi[t]));
        pm[t] = take ? om[t] : pm[t];
        pi[t] = take ? oi[t] : pi[t];
      } else {
        pm[t] = om[t] > pm[t] ? om[t] : pm[t];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (g == 0) {
      lm[wv * kTok + t * 16 + m] = EPI == 1 ? pm[t] * fs.inv_t : pm[t];
      if (EPI == 2) li[wv * kTok + t * 16 + m] = pi[t];
    }
    if (EPI == 1 && xd[t] >= 0) {  // the drafted token's logit, from the lane that holds it
      const int rel = xd[t] - vt0 * 16 - 4 * g;  // = 16r + j when this lane holds it
      bool hit = false;
      float zv = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (rel == 16 * r + j) {  // static indices only: acc stays in registers
            hit = true;
            zv = acc[r][t][j];
          }
      if (hit) fs.zx[n0 + t * 16 + m] = zv;
    }
  }
  __syncthreads();
  if (EPI == 2) {
    for (int tk = wv * 64 + lane; tk < kTok; tk += NW * 64) {
      if (tk >= ncols) continue;
      float M = -INFINITY;
      int I = 0x7fffffff;
      for (int w = 0; w < NW; ++w) {  // fixed order
        const float om = lm[w * kTok + tk];
        const int oi = li[w * kTok + tk];
        if (om > M || (om == M && oi < I)) {
          M = om;
          I = oi;
        }
      }
      const size_t slot = (size_t)(n0 + tk) * fs.pstride + vb;
      fs.cmax[slot] = M;
      fs.cidx[slot] = I;
    }
    return;
  }
  // Pass 2: exp(a - M) against the workgroup maximum M of each token, each term
  // 2^(z * c1 - c2) with c1 = fl32(1/T) * log2(e), c2 = M * log2(e) (one FMA
  // into the hardware base-2 exponential); the four terms of a vocabulary tile
  // are added in fp32, the tiles in fp64.
  const float c1 = fs.inv_t * 1.4426950408889634f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float M = lm[t * 16 + m];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, lm[w * kTok + t * 16 + m]);
    double ps = 0.0;
    if (M > -INFINITY) {
      const float c2 = M * 1.4426950408889634f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int v = (vt0 + r) * 16 + 4 * g;
        float s4 = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (v + j < V) s4 += __builtin_amdgcn_exp2f(fmaf(acc[r][t][j], c1, -c2));
        ps += (double)s4;
      }
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    if (g == 0) ls[wv * kTok + t * 16 + m] = ps;
    pm[t] = M;
  }
  __syncthreads();
  for (int tk = wv * 64 + lane; tk < kTok; tk += NW * 64) {
    if (tk >= ncols) continue;
    float M = lm[tk];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, lm[w * kTok + tk]);
    double S = 0.0;
    for (int w = 0; w < NW; ++w) S += ls[w * kTok + tk];  // fixed order
    const size_t slot = (size_t)(n0 + tk) * fs.pstride + vb;
    fs.cmax[slot] = M;
    fs.csum[slot] = S;
  }
}

// ---------------------------------------------------------------------------
// Draft-row statistics on the workgroups of a panel grid that have no work
// item (the grid is a multiple of 8).  Idle workgroup e of E takes
// vocabulary slice e of every draft row (a multiple of 4 entries); wave w takes
// the rows w, w + NW, ...  One pass per row: each lane keeps the running max
// of its z and its sum of exp(a - fl32(max z * fl32(1/T))), the terms formed as
// in the statistics epilogue and the sum rescaled when the max grows, with
// four 16-byte loads in flight; the lanes then meet in the same (max a, sum)
// form.  Writes slot e of each draft row, and the drafted token's logit from
// the slice that holds it.
template <int NW>
__device__ void idle_draft_stats(const FusedStats& fs, int N, int V, int e, int E, int wv, int lane) {
  constexpr float kL2e = 1.4426950408889634f;
  const int L = (((V + E - 1) / E) + 3) & ~3;
  const int s0 = min(e * L, V), s1 = min(s0 + L, V);
  const int nd = (int)(fs.B * fs.gamma);
  const float c1 = fs.inv_t * kL2e;
  const bool vec = (V & 3) == 0;
  for (int j = wv; j < nd; j += NW) {
    const float* row = fs.draft + (size_t)j * V;
    float zm = -INFINITY;
    double s = 0.0;
    for (int v0 = s0 + 4 * lane; v0 < s1; v0 += 1024) {
      float z[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = v0 + 256 * u;
        if (vec && v + 3 < s1) {
          const f32x4 t = *(const f32x4*)(row + v);
          z[4 * u + 0] = t[0];
          z[4 * u + 1] = t[1];
          z[4 * u + 2] = t[2];
          z[4 * u + 3] = t[3];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) z[4 * u + q] = v + q < s1 ? row[v + q] : -INFINITY;
        }
      }
      float bm = z[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) bm = fmaxf(bm, z[i]);
      if (bm > zm) {
        if (s > 0.0) s *= (double)__builtin_amdgcn_exp2f((zm * fs.inv_t - bm * fs.inv_t) * kL2e);
        zm = bm;
      }
      if (zm > -INFINITY) {
        const float c2 = zm * fs.inv_t * kL2e;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) s4[i >> 2] += __builtin_amdgcn_exp2f(fmaf(z[i], c1, -c2));
        s += (double)s4[0] + (double)s4[1] + (double)s4[2] + (double)s4[3];
      }
    }
    float M = zm;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (M > -INFINITY && s > 0.0) s *= (double)__builtin_amdgcn_exp2f((zm * fs.inv_t - M * fs.inv_t) * kL2e);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) {
      const size_t slot = (size_t)(N + j) * fs.pstride + e;
      fs.cmax[slot] = M * fs.inv_t;
      fs.csum[slot] = M > -INFINITY ? s : 0.0;
      const int32_t x = fs.tokens[j];
      const int xc = x < 0 ? 0 : (x >= V ? V - 1 : x);
      if (xc >= s0 && xc < s1) fs.zx[N + j] = row[xc];
    }
  }
}

// Index e and count E of the idle workgroups of a grid laid out as the panel
// kernel's (8 * ceil(items / 8) slots per token pass, items = vocabulary
// blocks x k-groups); -1 for a workgroup with a work item.
__device__ __forceinline__ int idle_index(int id, int items, int npass, int& E) {
  const int rem = items & 7;
  E = rem ? (8 - rem) * npass : 0;
  const int slot = id >> 3;
  const int gi = (id & 7) + 8 * (slot / npass);
  return gi >= items ? (slot % npass) * (8 - rem) + ((id & 7) - rem) : -1;
}

// Writes a block's outputs Y[n0 + n][vb*NW*R*16 + v] (lane: tokens n0 + 16t +
// lane % 16, rows 16*(vb*NW*R + wv*R + r) + 4*(lane / 16) .. +3) through LDS,
// one token tile at a time, so that consecutive lanes write consecutive 16
// bytes of one row of Y (a token's rows of the block are contiguous) instead
// of 64-byte pieces of 16 rows.  The token rows in LDS are padded by 16 bytes,
// which spreads a wave's writes over the banks.  st: 16 * (NW*R*16 + 4) floats
// of LDS whose previous users are done at the first barrier.
template <int NT, int R, int NW, bool OUT_BF16>
__device__ __forceinline__ void store_block(const f32x4 (&acc)[R][NT], float* st, void* Y, int V, int n0, int ncols,
                                            int vb, int wv, int lane) {
  constexpr int kThreads = NW * 64;
  constexpr int kRows = NW * R * 16;  // vocabulary rows of the block
  constexpr int kPitch = kRows + 4;   // floats per token row in LDS
  const int m = lane & 15, g = lane >> 4, tid = wv * 64 + lane;
  const int64_t vbase = (int64_t)vb * kRows;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    __syncthreads();  // the previous users of the LDS are done
#pragma unroll
    for (int r = 0; r < R; ++r) *(f32x4*)(st + m * kPitch + (wv * R + r) * 16 + 4 * g) = acc[r][t];
    __syncthreads();
    for (int i = tid; i < 16 * (kRows / 4); i += kThreads) {
      const int tok = i / (kRows / 4), q = i - tok * (kRows / 4);
      const int n = t * 16 + tok;
      const int64_t v0 = vbase + 4 * q;
      if (n < ncols && v0 < V)
        store4<OUT_BF16>(Y, (size_t)(n0 + n) * V + v0, v0, V, *(const f32x4*)(st + tok * kPitch + 4 * q));
    }
  }
}

// ---------------------------------------------------------------------------
// Panel kernel.  Work items are (vocabulary block, k-group, token pass): a
// vocabulary block is NW*R 16-row tiles, a token pass NT*16 tokens, and a
// k-group cpk chunks of KS MFMA k-steps (32 k each).  Block id i runs on XCD
// i % 8; the token passes of one (vocabulary block, k-group) take consecutive
// slots of one XCD, so the W rows they share are read from HBM once.  With one
// k-group the block writes Y; otherwise it writes fp32 partials to slice
// `group` of Y ([groups][N][V]), which are then summed in group order.
//
// Statistics epilogue (EPI 1: softmax at temperature T, EPI 2: argmax; one
// k-group only), for the whole verification step: every wave reduces its
// 16*R vocabulary rows per token, the NW wave partials meet in LDS, and the
// workgroup leaves one partial per (row, vocabulary block), plus the logit of
// each drafted token from the lane that holds it.  With the argmax, Y may be
// null: the scores are then not stored.
template <int NT, int R, int NW, int KS, bool OUT_BF16, int EPI>
__global__ __launch_bounds__(NW * 64) void panel_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
                                                        void* __restrict__ Y, int N, int d, int V, int npass, int cpk,
                                                        FusedStats fs) {
  constexpr int kThreads = NW * 64;
  constexpr int kBlocks = NT * KS;                   // 1 KB X blocks per chunk
  constexpr int kXPT = (kBlocks * 64 + kThreads - 1) / kThreads;
  constexpr int kBufElems = kBlocks * 512;           // bf16 per LDS buffer
  extern __shared__ __align__(16) uint16_t xs[];

  const int nsteps = d >> 5;
  const int ntiles = (V + 15) >> 4;
  const int nvb = (ntiles + NW * R - 1) / (NW * R);
  const int nch_all = (nsteps + KS - 1) / KS;
  const int ngroups = (nch_all + cpk - 1) / cpk;
  const int id = (int)blockIdx.x;
  if (EPI == 1 && fs.done != nullptr) {  // the draw kernel's counters, for the step that follows
    const int64_t gid = (int64_t)id * kThreads + threadIdx.x;
    if (gid < fs.B) fs.done[gid] = 0u;
  }
  const int slot = id >> 3;
  const int gi = (id & 7) + 8 * (slot / npass);
  if (gi >= nvb * ngroups) {
    if (EPI == 1 && fs.draft != nullptr) {  // the launcher hands the draft rows to the idle workgroups
      int E;
      const int e = idle_index(id, nvb * ngroups, npass, E);
      idle_draft_stats<NW>(fs, N, V, e, E, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63);
    }
    return;
  }
  const int vb = gi % nvb, group = gi / nvb;
  const int c0 = group * cpk, c1 = min(c0 + cpk, nch_all);
  // Chunk c of the loop reads chunk pc(c): with one k-group, the k range
  // rotated by a per-block offset, so that the blocks streaming at the same
  // moment read different offsets within their W rows rather than all the
  // same one (measured at N = 64, d = 8192, V = 128256: 313.0 -> 310.4 us).
  // It also sets the order in which the block's k-steps are summed.  With
  // several k-groups the blocks of a group keep reading the same X chunk at
  // the same time, which the XCD's L2 then serves once (rotated there, the
  // scattered X reads missed in L2: 86.9 against 79.7 us at N = 64 on
  // 28672 -> 8192, 108.8 against 98.2 us at N = 128).
  const int krot = c1 > c0 && ngroups == 1 ? (vb * 37) % (c1 - c0) : 0;
  auto pc = [&](int c) {
    const int q = c - c0 + krot;
    return c0 + (q >= c1 - c0 ? q - (c1 - c0) : q);
  };
  const int n0 = (slot % npass) * NT * 16;
  const int ncols = min(N - n0, NT * 16);

  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
  int xd[NT];
  drafted_tokens<NT, EPI>(fs, V, n0, ncols, lane, xd);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int vt0 = vb * NW * R + wv * R;              // this wave's first 16-row tile

  // Global loads are issued without conditions, their addresses clamped into
  // the buffer where a row, tile or k-step lies past the end (such values are
  // never used), so that the compiler counts outstanding loads exactly and
  // keeps the prefetch in flight across the computation.
  //
  // X staging: unit u (16 bytes) = block b = u / 64 (token tile b / KS, k-step
  // b % KS of the chunk), lane position l = u % 64.  Rows past N read row N-1:
  // they only feed output columns that are never stored.
  u32x4 xr[kXPT];
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int u = (tid + j * kThreads) % (kBlocks * 64);
      const int b = u >> 6, l = u & 63;
      const int t = b / KS, s = min(pc(c) * KS + b % KS, nsteps - 1);
      const int n = min(n0 + t * 16 + (l & 15), N - 1);
      xr[j] = *(const u32x4*)(X + (size_t)n * d + s * 32 + 8 * (l >> 4));
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int u = tid + j * kThreads;
      if (kXPT * kThreads == kBlocks * 64 || u < kBlocks * 64) *(u32x4*)(xs + buf * kBufElems + u * 8) = xr[j];
    }
  };
  // One wave-uniform row base per vocabulary tile (clamped into the buffer)
  // and one lane offset: the loads take a scalar base and a 32-bit offset.
  const uint16_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wrow[r] = Wp + (size_t)min(vt0 + r, ntiles - 1) * nsteps * 512;
  auto load_w = [&](u32x4(&dst)[KS][R], int c) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = min(pc(c) * KS + s, nsteps - 1) * 512 + lane * 8;
#pragma unroll
      for (int r = 0; r < R; ++r) dst[s][r] = load_w16<true>(wrow[r] + off);
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
      if (pc(c) * KS + s >= nsteps) break;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 bf = *(const u32x4*)(xb + (t * KS + s) * 512);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = mfma(wa[s][r], bf, acc[r][t]);
      }
    }
  };

  // Chunk c + 1 is fetched while chunk c computes.  The loop body only loads
  // chunks that exist; the last one or two chunks are peeled off so that no
  // load is issued past the end.
  u32x4 wa[KS][R], wb[KS][R];
  load_x(c0);
  load_w(wa, c0);
  store_x(0);
  __syncthreads();
  int c = c0;
  for (; c + 2 < c1; c += 2) {
    load_x(c + 1);
    load_w(wb, c + 1);
    compute(wa, 0, c);
    store_x(1);
    __syncthreads();
    load_x(c + 2);
    load_w(wa, c + 2);
    compute(wb, 1, c + 1);
    store_x(0);
    __syncthreads();
  }
  if (c + 1 < c1) {
    load_x(c + 1);
    load_w(wb, c + 1);
    compute(wa, 0, c);
    store_x(1);
    __syncthreads();
    compute(wb, 1, c + 1);
  } else {
    compute(wa, 0, c);
  }

  if (EPI != 0) panel_stats<NT, R, NW, EPI>(acc, xs, fs, V, n0, ncols, vt0, vb, wv, lane, xd);

  // Lane holds tokens n0 + 16t + m, vocabulary rows 16*(vt0 + r) + 4g .. +3.
  if (ngroups > 1) {  // fp32 partials of this k-group
    float* part = (float*)Y + (size_t)group * N * V;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t v0 = (int64_t)(vt0 + r) * 16 + 4 * g;
      if (v0 >= V) continue;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + m;
        if (n < ncols) store4<false>(part, (size_t)(n0 + n) * V + v0, v0, V, acc[r][t]);
      }
    }
    return;
  }
  if (EPI == 2 && Y == nullptr) return;  // a greedy step that keeps no logits
  store_block<NT, R, NW, OUT_BF16>(acc, (float*)xs, Y, V, n0, ncols, vb, wv, lane);
}

// Deep panel kernel, for many positions, where the work is bound by the matrix
// cores rather than by HBM.  One wave per SIMD: the four waves of a block share
// a token pass of NT*16 positions staged through LDS, each wave owns R
// vocabulary tiles, and its R x NT accumulator tiles live in the matrix-core
// registers.  Each step is one MFMA k-step (32 k) and one barrier; the W
// fragments of the next D-1 steps and the X rows of the next F steps are in
// flight in registers meanwhile, so that a load has D-1 (W) or F (X) steps of
// matrix work to arrive in.  Work items and their order on the XCDs are those
// of the panel kernel, with k-groups of cpk steps; W loads are nontemporal
// only when a single token pass reads W (NTL), since with several passes the
// passes of one vocabulary block share W through the XCD's L2.
//
// The token passes of a vocabulary block split N evenly (ptok positions each, a
// multiple of 16, at most NT*16), so that they take equally long: the passes
// that read the same W rows then stay level with each other, and the later
// ones find those rows in the XCD's L2 instead of fetching them from HBM again
// (measured at N = 320: passes of 192 and 128 positions fetched 1.59x the
// bytes of W from HBM).  FULL: every pass holds NT whole tiles of positions,
// so the matrix steps run without a per-tile test.
//
// Measured at N = 320, d = 5120, V = 152064 (two passes of 160): about 530 us
// per launch, against about 420 us with the W loads left out and 470 us with
// every W load an L2 hit.  The X ring bounds the W prefetch: the wait for the
// X rows stored at a step (loaded F steps before) is a count of outstanding
// loads, which also waits for every W load issued before them, so a W ring
// deeper than F bought nothing (D = 8 ran 2-3% slower, its registers spilling
// into copies) and F is held to 4 by the register file.
template <int NT, int R, int D, int F, bool NTL, bool OUT_BF16, int EPI, bool PX = false, bool FULL = false>
__global__ __launch_bounds__(256) void deep_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
                                                   void* __restrict__ Y, int N, int d, int V, int npass, int cpk,
                                                   int ptok, FusedStats fs) {
  constexpr int NW = 4, kThreads = NW * 64;
  constexpr int kXU = NT * 64;                            // 16-byte X units per step
  constexpr int kXPT = (kXU + kThreads - 1) / kThreads;  // per thread
  static_assert(NT % 2 == 0 && D == 4 && F == D, "deep kernel ring shapes");
  constexpr int kBufElems = NT * 512;  // bf16 per LDS buffer: NT fragments of 16 x 32
  extern __shared__ __align__(16) uint16_t xs[];

  const int nsteps = d >> 5;
  const int ntiles = (V + 15) >> 4;
  const int nvb = (ntiles + NW * R - 1) / (NW * R);
  const int ngroups = (nsteps + cpk - 1) / cpk;
  const int id = (int)blockIdx.x;
  if (EPI == 1 && fs.done != nullptr) {  // the draw kernel's counters, for the step that follows
    const int64_t gid = (int64_t)id * kThreads + threadIdx.x;
    if (gid < fs.B) fs.done[gid] = 0u;
  }
  const int slot = id >> 3;
  const int gi = (id & 7) + 8 * (slot / npass);
  if (gi >= nvb * ngroups) return;
  const int vb = gi % nvb, group = gi / nvb;
  const int s0 = group * cpk, s1 = min(s0 + cpk, nsteps);
  const int n0 = (slot % npass) * ptok;
  const int ncols = min(N - n0, ptok);

  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
  int xd[NT];
  drafted_tokens<NT, EPI>(fs, V, n0, ncols, lane, xd);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int vt0 = vb * NW * R + wv * R;

  // Loads are issued without conditions, steps past the group's end clamped
  // to its last step (such values are never used), so that the compiler
  // counts outstanding loads exactly.  X unit u = tid + 256 j: token tile
  // u / 64, lane position u % 64; rows past N read row N-1.
  const uint16_t* xrow[kXPT];
#pragma unroll
  for (int j = 0; j < kXPT; ++j) {
    const int u = tid + j * kThreads, l = u & 63;
    if (PX) {
      const int tile = min((n0 >> 4) + (u >> 6), ((N + 15) >> 4) - 1);
      xrow[j] = X + (size_t)tile * nsteps * 512 + l * 8;
    } else {
      const int n = min(n0 + (u >> 6) * 16 + (l & 15), N - 1);
      xrow[j] = X + (size_t)n * d + 8 * (l >> 4);
    }
  }
  // Unit j of a thread exists when tid + 256 j < kXU, that is (kXU being a
  // multiple of 64) when 64 wv + 256 j < kXU: a test on the wave index, which
  // compiles to a scalar branch.
  auto has_unit = [&](int j) { return kXU % kThreads == 0 || wv * 64 + j * kThreads < kXU; };
  auto load_x = [&](u32x4(&dst)[kXPT], int s) {
    const int sc = min(s, s1 - 1) * (PX ? 512 : 32);
#pragma unroll
    for (int j = 0; j < kXPT; ++j)
      if (has_unit(j)) dst[j] = *(const u32x4*)(xrow[j] + sc);
  };
  auto store_x = [&](const u32x4(&src)[kXPT], int buf) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j)
      if (has_unit(j)) *(u32x4*)(xs + buf * kBufElems + (tid + j * kThreads) * 8) = src[j];
  };
  const uint16_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wrow[r] = Wp + (size_t)min(vt0 + r, ntiles - 1) * nsteps * 512;
  auto load_w = [&](u32x4(&dst)[R], int s) {
    const int off = min(s, s1 - 1) * 512 + lane * 8;
#pragma unroll
    for (int r = 0; r < R; ++r) dst[r] = load_w16<NTL>(wrow[r] + off);
  };

  f32x4 acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Step i (from s0) uses W ring slot i % D; X of step j is staged in
  // register slot j % F.
  u32x4 wr[D][R], xr[F][kXPT], bf[2][NT];
  auto read_b = [&](u32x4(&dst)[NT], int buf) {
    const uint16_t* xb = xs + buf * kBufElems + lane * 8;
#pragma unroll
    for (int t = 0; t < NT; ++t) dst[t] = *(const u32x4*)(xb + t * 512);
  };
  // Token tiles past N (in the last token pass) skip their MFMAs; the test is
  // uniform over the workgroup.
  const int ntv = min(NT, (ncols + 15) >> 4);
  auto mfmas = [&](const u32x4(&wa)[R], const u32x4(&b)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (FULL || t < ntv) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = mfma(wa[r], b[t], acc[r][t]);
      }
  };
  // X of step j goes to LDS buffer j % 4 three steps ahead (at step j - 3) and
  // its B fragments are read into registers one step ahead (at step j - 1);
  // the workgroup meets at a barrier after every odd step only, which is
  // enough: a store and its reads are always separated by one, and so are the
  // reads of a buffer and its next store, four steps on.
  //
  // Prologue: X of steps 0 to 2 into LDS, then the loads in flight at the top
  // of every trip, in the order the trips issue them (W of step j, then X of
  // step j + 3), so that the compiler's wait counts at the loop head are those
  // of the steady state.
#pragma unroll
  for (int j = 0; j < 3; ++j) load_x(xr[j], s0 + j);
#pragma unroll
  for (int j = 0; j < 3; ++j) store_x(xr[j], j);
  __syncthreads();
  read_b(bf[0], 0);
  __syncthreads();  // buffer 0 is stored again at step 1
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_w(wr[j], s0 + j);
    __builtin_amdgcn_sched_barrier(0);
    load_x(xr[(j + 3) % F], s0 + j + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  // One step; I = i % D is a compile-time index.  Steps past the group's end
  // (in its last trip) skip their MFMAs only.
  auto step = [&](auto I_, int s) {
    constexpr int I = decltype(I_)::value;
    read_b(bf[(I + 1) & 1], (I + 1) & 3);  // X of step s + 1
    __builtin_amdgcn_sched_barrier(0);     // issue those reads before the MFMAs
    if (s < s1) mfmas(wr[I], bf[I & 1]);
    load_w(wr[I], s + D);
    store_x(xr[(I + 3) % F], (I + 3) & 3);  // X of step s + 3
    load_x(xr[(I + 3) % F], s + 3 + F);
    if (I & 1) __syncthreads();
  };
  for (int s = s0; s < s1; s += D) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    step(std::integral_constant<int, 2>{}, s + 2);
    step(std::integral_constant<int, 3>{}, s + 3);
  }

  if (EPI != 0) panel_stats<NT, R, NW, EPI>(acc, xs, fs, V, n0, ncols, vt0, vb, wv, lane, xd);

  // Stored straight from the accumulators (staging them through LDS as the
  // panel kernel does measured slower here: this kernel is bound by the
  // matrix cores, and the staging adds two barriers per token tile).  A
  // greedy step that keeps no logits passes a null Y.
  if (EPI == 2 && Y == nullptr) return;
  const bool split = ngroups > 1;
  float* part = (float*)Y + (size_t)group * N * V;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t v0 = (int64_t)(vt0 + r) * 16 + 4 * g;
    if (v0 >= V) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = t * 16 + m;
      if (n >= ncols) continue;
      if (split)
        store4<false>(part, (size_t)(n0 + n) * V + v0, v0, V, acc[r][t]);
      else
        store4<OUT_BF16>(Y, (size_t)(n0 + n) * V + v0, v0, V, acc[r][t]);
    }
  }
}

// Sums the k-group partials P [groups][N][V] in group order into Y.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, void* __restrict__ Y,
                                                            int64_t N, int64_t V, int groups) {
  const int64_t NV = N * V;
  if ((V & 3) == 0) {
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < NV; i += (int64_t)gridDim.x * 1024) {
      f32x4 s = *(const f32x4*)(P + i);
      for (int gq = 1; gq < groups; ++gq) {
        const f32x4 o = *(const f32x4*)(P + (size_t)gq * NV + i);
        s[0] += o[0];
        s[1] += o[1];
        s[2] += o[2];
        s[3] += o[3];
      }
      const int64_t v0 = i % V;
      store4<OUT_BF16>(Y, (size_t)i, v0, V, s);
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < NV; i += (int64_t)gridDim.x * 256) {
      float s = P[i];
      for (int gq = 1; gq < groups; ++gq) s += P[(size_t)gq * NV + i];
      if (OUT_BF16)
        ((uint16_t*)Y)[i] = (uint16_t)bf16_rne(s);
      else
        ((float*)Y)[i] = s;
    }
  }
}

hipError_t launch_reduce(const float* P, void* Y, int64_t N, int64_t V, int64_t groups, bool out_bf16,
                         hipStream_t stream) {
  const int64_t work = (V & 3) == 0 ? (N * V) / 4 : N * V;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  auto k = out_bf16 ? splitk_reduce_kernel<true> : splitk_reduce_kernel<false>;
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, stream, P, Y, N, V, (int)groups);
  return hipGetLastError();
}

// Launch geometry of one panel configuration for a shape (ptok: positions
// per token pass of the deep kernel).
struct PanelPlan {
  int64_t npass, cpk, groups, grid, ptok;
};

// Splits the k range into groups only when the (vocabulary block, token pass)
// work items would leave more than 15% of the CUs idle: then into as many
// groups (each at least 4 chunks) as fill the CUs in one round.  A streaming
// CU reads about 27 GB/s, so an idle CU is bandwidth lost (28672 -> 8192 at
// N = 64: 7 groups on 224 CUs took 81.3 us, 8 groups on 256 took 79.8 us),
// while a second round of items, or every extra group's fp32 partials N x V
// written and read back, costs more than it gains.
PanelPlan plan_panel(int64_t N, int64_t d, int64_t V, int NT, int R, int NW, int KS, int cus) {
  PanelPlan p{};
  const int64_t ntiles = (V + 15) / 16, nvb = (ntiles + NW * R - 1) / (NW * R);
  const int64_t nch = (d / 32 + KS - 1) / KS;
  p.npass = (N + NT * 16 - 1) / (NT * 16);
  const int64_t items = nvb * p.npass, want = (cus * 85 + 99) / 100;
  int64_t gq = items >= want ? 1 : (cus / items > 1 ? cus / items : 1);
  const int64_t gmax = nch / 4 > 1 ? nch / 4 : 1;
  if (gq > gmax) gq = gmax;
  p.cpk = (nch + gq - 1) / gq;
  p.groups = (nch + p.cpk - 1) / p.cpk;
  p.grid = 8 * ((nvb * p.groups + 7) / 8) * p.npass;
  return p;
}

// Two X buffers for the main loop; the output staging afterwards takes one
// token tile of the block (16 padded rows of NW*R*16 floats).
template <int NT, int R, int NW, int KS>
constexpr size_t panel_lds_bytes() {
  constexpr size_t x = 2ull * NT * KS * 1024, y = 16ull * (NW * R * 16 + 4) * sizeof(float);
  return x > y ? x : y;
}

template <int NT, int R, int NW, int KS>
hipError_t launch_panel(const PanelPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d,
                        int64_t V, bool out_bf16, hipStream_t stream, const FusedStats* fs = nullptr) {
  constexpr size_t kLds = panel_lds_bytes<NT, R, NW, KS>();
  static_assert(kLds <= 160 * 1024, "panel LDS");
  // The statistics epilogue reuses the X buffers: NW*NT*16 entries of 4 + 8 + 4 bytes.
  static_assert((size_t)NW * NT * 16 * 16 <= kLds, "panel statistics LDS");
  auto k = out_bf16 ? panel_kernel<NT, R, NW, KS, true, 0> : panel_kernel<NT, R, NW, KS, false, 0>;
  if (fs) k = fs->greedy ? panel_kernel<NT, R, NW, KS, false, 2> : panel_kernel<NT, R, NW, KS, false, 1>;
  hipError_t e = allow_lds(k, kLds);
  if (e != hipSuccess) return e;
  const FusedStats none{};
  hipLaunchKernelGGL(k, dim3((unsigned)p.grid), dim3(NW * 64), kLds, stream, X, Wp, Y, (int)N, (int)d, (int)V,
                     (int)p.npass, (int)p.cpk, fs ? *fs : none);
  return hipGetLastError();
}

// The deep kernel takes a plan from plan_panel with NW = 4 and KS = 1 (its
// chunks are single k-steps).
template <int NT, int R, int D, bool PX = false>
hipError_t launch_deep(const PanelPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d,
                       int64_t V, bool out_bf16, hipStream_t stream, const FusedStats* fs = nullptr) {
  constexpr size_t kLds = 4ull * NT * 1024;
  static_assert((size_t)4 * NT * 16 * 16 <= kLds, "deep statistics LDS");
  auto pick = [&](auto ntl, auto full) {
    constexpr bool L = decltype(ntl)::value, FU = decltype(full)::value;
    auto k = out_bf16 ? deep_kernel<NT, R, D, D, L, true, 0, PX, FU> : deep_kernel<NT, R, D, D, L, false, 0, PX, FU>;
    if (fs) k = fs->greedy ? deep_kernel<NT, R, D, D, L, false, 2, PX, FU> : deep_kernel<NT, R, D, D, L, false, 1, PX, FU>;
    return k;
  };
  // Every token pass full (NT tiles of live positions): no per-tile test.
  const bool full = p.ptok == NT * 16 && N % p.ptok == 0;
  auto k = p.npass == 1 ? (full ? pick(std::true_type{}, std::true_type{}) : pick(std::true_type{}, std::false_type{}))
                        : (full ? pick(std::false_type{}, std::true_type{}) : pick(std::false_type{}, std::false_type{}));
  hipError_t e = allow_lds(k, kLds);
  if (e != hipSuccess) return e;
  const FusedStats none{};
  hipLaunchKernelGGL(k, dim3((unsigned)p.grid), dim3(256), kLds, stream, X, Wp, Y, (int)N, (int)d, (int)V,
                     (int)p.npass, (int)p.cpk, (int)p.ptok, fs ? *fs : none);
  return hipGetLastError();
}

// The panel configurations the dispatcher uses, by N (chosen by measurement).
struct PanelShape {
  int NT, R, NW, KS;
  bool deep = false;  // deep kernel (NW = 4, KS = 1) over packed X
};
// Shapes (token tiles x vocabulary tiles per wave, waves, k-steps per chunk)
// chosen from timings of every candidate on the LM heads (V = 128256 and
// 152064, d = 4096 to 8192) and the decoder projections (8192 <-> 28672):
// short vocabularies take narrow vocabulary blocks so that one round of
// blocks covers the CUs without splitting k; long ones take 64 rows per wave.
// Past 64 positions the work turns MFMA-bound and more token tiles per wave
// win.  The 8x4 shape does not fit its registers without spilling (it is
// still the fastest there), so the statistics epilogue never uses it.
PanelShape panel_shape(int64_t N, int64_t d, int64_t V, bool with_stats) {
  const bool big_v = V >= 65536;
  // With d a multiple of 128 (whole trips of four k-steps), the deep kernel
  // (128 x 64 tiles per wave, one wave per SIMD) past 128 positions, and past
  // 64 with the statistics epilogue; at 65 to 128 positions without it the
  // 8x4 and 8x2 panels measured as fast or faster.
  // Its token pass is 128 positions, or on long vocabularies 192 where that
  // takes fewer passes (N = 129-192, 257-384, ...): each pass streams all of
  // W from L2 into the CUs, the kernel's limit, so at N = 320, V = 152064
  // two passes of 192 ran the step ~22 us (3.5%) faster than passes of 128,
  // 128 and 64.  Where passes of 160 are as few, the kernel takes ten token
  // tiles instead of twelve: at N = 320 both passes then fill every tile and
  // skip the per-tile tests (the launch 1.4% faster).  On the 28672-row projection at N = 512 three passes of 192
  // took 329 us against 257 us for four of 128: with 112 vocabulary blocks
  // the work items fill the CUs in fewer, more uneven rounds.
  if (d % 128 == 0 && (N > 128 || (N > 64 && with_stats))) {
    if (!(big_v && (N + 191) / 192 < (N + 127) / 128)) return PanelShape{8, 4, 4, 1, true};
    return PanelShape{(N + 159) / 160 == (N + 191) / 192 ? 10 : 12, 4, 4, 1, true};
  }
  if (N <= 64) {
    if (!big_v) return N <= 32 ? PanelShape{4, 1, 8, 4} : PanelShape{4, 2, 8, 2};
    return d <= 4096 ? PanelShape{4, 2, 8, 2} : PanelShape{4, 4, 8, 2};
  }
  if (N <= 128) return big_v && !with_stats ? PanelShape{8, 4, 8, 2} : PanelShape{8, 2, 8, 2};
  return big_v || with_stats ? PanelShape{4, 4, 8, 2} : PanelShape{8, 4, 8, 2};
}

hipError_t launch_panel_shape(const PanelShape& s, const PanelPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y,
                              int64_t N, int64_t d, int64_t V, bool out_bf16, hipStream_t stream,
                              const FusedStats* fs = nullptr) {
  if (s.deep && s.NT == 12) return launch_deep<12, 4, 4, true>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (s.deep && s.NT == 10) return launch_deep<10, 4, 4, true>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (s.deep) return launch_deep<8, 4, 4, true>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (s.NT == 4 && s.R == 1) return launch_panel<4, 1, 8, 4>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (s.NT == 4 && s.R == 2) return launch_panel<4, 2, 8, 2>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (s.NT == 4) return launch_panel<4, 4, 8, 2>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (s.R == 2) return launch_panel<8, 2, 8, 2>(p, X, Wp, Y, N, d, V, out_bf16, stream, fs);
  if (fs) return hipErrorNotSupported;
  return launch_panel<8, 4, 8, 2>(p, X, Wp, Y, N, d, V, out_bf16, stream, nullptr);
}

// The deep kernel's copy of X: ceil(N / 16) 16-row tiles in the packed
// weight layout (one 1 KB block per tile and k-step), so that its X loads are
// whole 1 KB blocks like its W loads.
size_t xpack_bytes(int64_t N, int64_t d) {
  return ((size_t)((N + 15) / 16) * 16 * d * sizeof(uint16_t) + 255) & ~(size_t)255;
}

// What the dispatcher will run for a shape, and the workspace it needs: the
// sweep kernel's tile queue; or the packed X (deep kernel), then the k-group
// partials.
struct GemmPlan {
  enum Kind { kSweep, kPanel, kTiled } kind;
  SweepPlan sweep;
  PanelShape shape;
  PanelPlan panel;
  size_t xpack;  // bytes of packed X at the start of the workspace
  size_t workspace;
};

GemmPlan plan_gemm(int64_t N, int64_t d, int64_t V, bool packed, bool with_stats = false) {
  GemmPlan g{};
  const int cus = device_cus();
  g.kind = GemmPlan::kTiled;
  if (!packed) return g;
  // The sweep kernel wins on long vocabularies with X whole in LDS (d up to
  // 4096 at 16 positions); elsewhere the panel kernel streams W faster.
  g.sweep = plan_sweep(N, d, V, cus);
  if (g.sweep.ok && V >= 65536 && d <= 4096) {
    g.kind = GemmPlan::kSweep;
    g.workspace = kSweepTicketBytes;
    return g;
  }
  g.kind = GemmPlan::kPanel;
  g.shape = panel_shape(N, d, V, with_stats);
  g.panel = plan_panel(N, d, V, g.shape.NT, g.shape.R, g.shape.NW, g.shape.KS, cus);
  if (g.shape.deep) {
    // k-groups of whole trips of four k-steps.
    const int64_t nsteps = d / 32, ntiles = (V + 15) / 16, nvb = (ntiles + 15) / 16;
    g.panel.cpk = (g.panel.cpk + 3) / 4 * 4;
    g.panel.groups = (nsteps + g.panel.cpk - 1) / g.panel.cpk;
    // Equal token passes: the 16-row token tiles spread evenly over the passes.
    const int64_t ntok_tiles = (N + 15) / 16;
    g.panel.ptok = 16 * ((ntok_tiles + g.panel.npass - 1) / g.panel.npass);
    g.panel.grid = 8 * ((nvb * g.panel.groups + 7) / 8) * g.panel.npass;
    g.xpack = xpack_bytes(N, d);
  }
  g.workspace = g.xpack;
  if (g.panel.groups > 1) g.workspace += (size_t)g.panel.groups * N * V * sizeof(float);
  return g;
}

// Workgroups of a panel grid without a work item: the items
// (vocabulary blocks x k-groups) are rounded up to a multiple of 8 per token
// pass.
int64_t idle_workgroups(const GemmPlan& g, int64_t V) {
  const int64_t ntiles = (V + 15) / 16, rows = (int64_t)g.shape.NW * g.shape.R;
  const int64_t items = (ntiles + rows - 1) / rows * g.panel.groups, rem = items % 8;
  return rem ? (8 - rem) * g.panel.npass : 0;
}

// Whether `idle` workgroups can summarise nd draft rows well within the GEMM:
// each reads its share at about 5 GB/s per wave (measured on the 8-wave
// panel), against W streamed at about 6.5 TB/s; the share must take at most
// 60% of the GEMM's time.
bool idle_drafts_fit(const GemmPlan& g, int64_t nd, int64_t d, int64_t V, int64_t idle) {
  const double share = 4.0 * (double)nd * (double)V / (double)idle;
  const double t_idle = share / (5e9 * g.shape.NW), t_gemm = 2.0 * (double)V * (double)d / 6.5e12;
  return t_idle <= 0.6 * t_gemm;
}

}  // namespace
}  // namespace gemm

int64_t gemm_stats_parts(int64_t N, int64_t d, int64_t V, int64_t pstride, bool required) {
  using namespace gemm;
  if (N > kFusedStatsMaxRows) return 0;
  const GemmPlan g = plan_gemm(N, d, V, true, true);
  // At 65-128 positions with d <= 4096 the deep kernel with an epilogue is
  // slower than the plain 8x4 panel followed by the statistics kernel
  // (measured, V = 128256, d = 4096: 8 trees of 16 nodes 248.6 us against
  // 235-241 us for the tree step; a softmax step at N = 128, 264-268 us
  // against 240-253 us).  With d = 8192 the epilogue pays for itself
  // (N = 96: 402-403 us fused against 416-419 us).  A step without logits
  // takes the epilogue all the same.
  if (!required && g.kind == GemmPlan::kPanel && g.shape.deep && N <= 128 && d <= 4096) return 0;
  int64_t parts = 0;
  if (g.kind == GemmPlan::kSweep) {
    parts = g.sweep.grid;
  } else if (g.kind == GemmPlan::kPanel && g.panel.groups == 1) {
    const int64_t ntiles = (V + 15) / 16, rows = (int64_t)g.shape.NW * g.shape.R;
    parts = (ntiles + rows - 1) / rows;
  }
  return parts > 0 && parts <= kFusedStatsMaxParts && parts <= pstride ? parts : 0;
}

size_t gemm_stats_scratch_bytes(int64_t N, int64_t d, int64_t V) {
  const gemm::GemmPlan g = gemm::plan_gemm(N, d, V, true, true);
  return g.kind == gemm::GemmPlan::kSweep ? g.workspace : g.xpack;
}

hipError_t launch_gemm_with_stats(const uint16_t* X, const uint16_t* Wp, float* Y, int64_t N, int64_t d, int64_t V,
                                  const FusedStats& fs, int64_t* nparts, int64_t* nparts_draft, void* scratch,
                                  hipStream_t stream, bool required) {
  using namespace gemm;
  if (Y == nullptr && !fs.greedy) return hipErrorInvalidValue;
  const int64_t parts = gemm_stats_parts(N, d, V, fs.pstride, required);
  if (parts == 0) return hipErrorNotSupported;
  const GemmPlan g = plan_gemm(N, d, V, true, true);
  if (g.xpack > 0) {
    if (scratch == nullptr) return hipErrorInvalidValue;
    const hipError_t e = launch_pack_weights(X, (uint16_t*)scratch, N, d, stream);
    if (e != hipSuccess) return e;
    X = (const uint16_t*)scratch;
  }
  if (g.kind == GemmPlan::kSweep) {
    // The sweep kernel also summarises the (at most 15) draft rows itself, in
    // the same slots as the target rows.
    const hipError_t e = launch_sweep_with_stats(g.sweep, X, Wp, Y, N, d, V, fs, scratch, nparts, stream);
    if (e == hipSuccess) *nparts = *nparts_draft = parts;
    return e;
  }
  // Many draft rows: the workgroups of the grid that have no vocabulary block
  // summarise them during the GEMM when they can finish well within it;
  // otherwise the statistics kernel does first, one partial per 2048-entry
  // chunk.  Either way the panel (or deep) kernel forms the target rows'.
  int64_t dparts = parts;
  FusedStats run = fs;
  if (fs.draft != nullptr) {
    const int64_t idle = g.shape.deep ? 0 : idle_workgroups(g, V);  // the deep kernel's grid is busy for longer
    if (idle > 0 && idle_drafts_fit(g, fs.B * fs.gamma, d, V, idle)) {
      dparts = idle;
    } else {
      const hipError_t e = launch_draft_stats(fs, N, V, &dparts, stream);
      if (e != hipSuccess) return e;
      run.draft = nullptr;
    }
  }
  const hipError_t e = launch_panel_shape(g.shape, g.panel, X, Wp, Y, N, d, V, false, stream, &run);
  if (e == hipSuccess) {
    *nparts = parts;
    *nparts_draft = dparts;
  }
  return e;
}

size_t gemm_workspace_bytes(int64_t N, int64_t d, int64_t V, bool packed) {
  return gemm::plan_gemm(N, d, V, packed).workspace;
}

const char* scoring_kernel_name(int64_t N, int64_t d, int64_t V, bool packed) {
  const gemm::GemmPlan g = gemm::plan_gemm(N, d, V, packed);
  switch (g.kind) {
    case gemm::GemmPlan::kSweep: return "sweep_kernel";
    case gemm::GemmPlan::kPanel: return g.shape.deep ? "deep_kernel" : "panel_kernel";
    default: return "tiled_kernel";
  }
}

hipError_t launch_skinny_gemm(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V,
                              bool out_bf16, bool packed, void* workspace, hipStream_t stream) {
  using namespace gemm;
  const GemmPlan g = plan_gemm(N, d, V, packed);
  if (g.workspace > 0 && !workspace) return hipErrorInvalidValue;
  switch (g.kind) {
    case GemmPlan::kSweep: {
      return launch_sweep(g.sweep, X, W, Y, N, d, V, out_bf16, workspace, stream);
    }
    case GemmPlan::kPanel: {
      if (g.xpack > 0) {
        const hipError_t e = launch_pack_weights(X, (uint16_t*)workspace, N, d, stream);
        if (e != hipSuccess) return e;
        X = (const uint16_t*)workspace;
      }
      float* part = (float*)((char*)workspace + g.xpack);
      if (g.panel.groups == 1) return launch_panel_shape(g.shape, g.panel, X, W, Y, N, d, V, out_bf16, stream);
      hipError_t e = launch_panel_shape(g.shape, g.panel, X, W, part, N, d, V, false, stream);
      return e != hipSuccess ? e : launch_reduce(part, Y, N, V, g.panel.groups, out_bf16, stream);
    }
    default:
      break;
  }
  // Row-major weights.
  if (N <= 16) return launch_tiled<1, 1, 256, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
  if (N <= 32) return launch_tiled<2, 2, 128, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
  return launch_tiled<4, 2, 128, 4, false, false>(X, W, Y, N, d, V, out_bf16, stream);
}

}  // namespace specdec
