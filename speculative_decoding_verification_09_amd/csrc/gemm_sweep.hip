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
// a contiguous slice, the next tile prefetched into a second register buffer;
// partial sums meet in LDS in a fixed order.  At any moment the whole GPU
// reads within a window of about (#CUs x tile size), which keeps HBM
// streaming close to a plain sequential read; the last tiles come from a
// queue, so that every workgroup finishes at about the same time.
#include <chrono>

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
// Sweep kernel (packed W, small N).  Persistent, one workgroup per CU.  A
// workgroup takes one 16-row tile at a time; its 8 waves split the tile's k
// range (wave w owns k-steps [w*spw, (w+1)*spw), spw <= SPW: d up to
// NW*SPW*32), each loading its slice straight into A-operand registers, and
// the partial sums meet in LDS in a fixed order.
//
// Tiles come in two phases.  First a fixed share: workgroup b takes tiles b,
// b + G, ..., b + (S-1)*G (G = grid size, S*G about 85% of the tiles), the
// next tile's loads in flight while the current one computes.  Then a queue:
// a ticket counter hands out the remaining tiles in the order asked for.  HBM does not serve every
// CU equally fast (measured on the LM-head sweep: with fixed shares only, the
// workgroups on four of the eight XCDs finished 11-15% later than those on
// the other four, whatever tiles they were given), so fixed shares alone
// leave half the chip idle at the end; with the queue every workgroup
// finishes within about one tile of the others.  The queue is kept to the
// last 15% because each ticket is a device-scope atomic on one address, and
// handing out every tile that way measurably slowed the whole stream.
// In the queue phase thread 0 asks for the next ticket right after the
// current tile's loads go out, and reads the answer once they have been
// used.
//
// The counter lives in the caller's workspace, which holds anything on entry.
// Workgroup 0 zeroes it as its first act and then publishes a tag unique to
// this launch (from the host, 64 bits) next to it, with release order; every
// workgroup reads that word one tile before its first ticket and asks only
// once it holds this launch's tag.  A launch thus never needs a separate
// reset (measured: a one-thread reset kernel before the sweep cost 1.5 us of
// the 166 us one-sequence step).  Waiting for the tag ends: workgroup 0 runs
// its first instructions without waiting on anything, and the grid (at most
// one workgroup per CU) is resident as a whole.  The wait is bounded all the
// same; past the bound a workgroup takes no queue tile (the bound, about a
// second, is never reached while the grid is resident).
//
// Every global load is issued unconditionally, with its address clamped into
// the wave's k range (those values are never used): the compiler can then
// count outstanding loads exactly and keeps the next tile's loads in flight
// while the current tile computes, instead of draining all of them at each
// branch join.
//
// Statistics epilogue (EPI 1: softmax at temperature T, EPI 2: argmax; with
// the argmax, Y may be null and the scores are then not stored), used by the
// verification step: wave 0 folds every tile's finished logits into a
// running per-lane state (max of a = z * fl32(1/T) and an fp64 sum of fp32
// exp(a - max), rescaled when the max grows; or the largest z with its lowest
// index), records the logit of each row's drafted token from the tile that
// holds it, and at the end leaves one partial per (row, workgroup).  With
// draft logits, workgroup b first summarises the 2048-entry slices b, b + G,
// ... of every draft row (few rows here: B*gamma <= 15), before its first
// tile; the queue evens out the difference.
constexpr int kDraftSlice = 2048;

constexpr int kTagSpinLimit = 1 << 22;  // polls of the launch tag, each after a short sleep

template <int NW, int SPW, bool NTL, bool OUT_BF16, int EPI>
__global__ __launch_bounds__(NW * 64) void sweep_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
                                                        void* __restrict__ Y, int N, int d, int V, int S,
                                                        unsigned* __restrict__ tickets, uint64_t tag, FusedStats fs) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int sh_tile;  // the next queue tile, passed from thread 0 to the workgroup
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
  uint64_t* const ready = (uint64_t*)(tickets + 2);  // the launch tag, 8 bytes after the counter
  if (blockIdx.x == 0 && tid == 0) {
    __hip_atomic_store(tickets, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ready, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (EPI == 1 && fs.done != nullptr) {  // the draw kernel's counters, for the step that follows
    const int64_t gid = (int64_t)blockIdx.x * (NW * 64) + tid;
    if (gid < fs.B) fs.done[gid] = 0u;
  }
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int nsteps = d >> 5;
  const int ntiles = (V + 15) >> 4;
  const int G = (int)gridDim.x;
  const int qbase = S * G;  // the first tile of the queue (S * G <= ntiles)
  // Ticket k names tile qbase + k; past the last tile, ntiles (no tile).
  auto tile_of = [&](unsigned k) { return k < (unsigned)(ntiles - qbase) ? qbase + (int)k : ntiles; };
  auto ask = [&]() { return __hip_atomic_fetch_add(tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  // Thread 0: the tag word as last read (read early, one tile ahead of the
  // first ticket), and the first ticket once it shows this launch's tag.
  uint64_t seen = 0;
  auto read_tag = [&]() { seen = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto first_ask = [&]() {
    for (int i = 0; seen != tag && i < kTagSpinLimit; ++i) {
      __builtin_amdgcn_s_sleep(2);
      read_tag();
    }
    return seen == tag ? ask() : 0xffffffffu;  // past the bound: no queue tile
  };
  if (S == 0 && tid == 0) {  // no fixed share: the first tile comes from the queue
    read_tag();
    sh_tile = tile_of(first_ask());
  }
  const int pitch = nsteps * 32 + kPad;
  const int spw = (nsteps + NW - 1) / NW;         // k-steps per wave and tile (<= SPW)
  uint16_t* xs = lds;
  f32x4* red = (f32x4*)(lds + (((size_t)N * pitch + 7) & ~(size_t)7));
  const int units_per_row = nsteps * 4;           // 16-byte units of one X row
  for (int i = tid; i < N * units_per_row; i += NW * 64) {
    const int n = i / units_per_row, u = i - n * units_per_row;
    *(u32x4*)(xs + n * pitch + u * 8) = *(const u32x4*)(X + (size_t)n * d + u * 8);
  }

  if (EPI == 1 && fs.draft != nullptr) {
    // Draft rows: wave w takes rows w and w + NW; a lane loads its 32 entries
    // of a slice before any use, and the fp64 sum is rescaled when the running
    // maximum grows.  Workgroups without a slice leave empty partials.
    const int nd = (int)(fs.B * fs.gamma);
    const int nsl = (V + kDraftSlice - 1) / kDraftSlice;
    for (int j = wv; j < nd; j += NW) {
      const float* row = fs.draft + (size_t)j * V;
      constexpr int kPer = kDraftSlice / 64;
      float mx = -INFINITY;
      double sm = 0.0;
      for (int c = (int)blockIdx.x; c < nsl; c += G) {
        // Loads from clamped indices first, all in flight together (guarded
        // loads compiled to one round trip per entry), then the mask.
        float a[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) a[e] = row[min(c * kDraftSlice + 64 * e + lane, V - 1)];
#pragma unroll
        for (int e = 0; e < kPer; ++e) a[e] = c * kDraftSlice + 64 * e + lane < V ? a[e] * fs.inv_t : -INFINITY;
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
        if ((xc / kDraftSlice) % G == (int)blockIdx.x) fs.zx[N + j] = row[xc];
      }
    }
  }
  __syncthreads();

  const bool live = m < N;
  const int mx = live ? m : N - 1;                // lanes past N read a valid row; their column is not stored
  const int my0 = wv * spw;                       // first k-step of this wave
  const int my1 = min(my0 + spw, nsteps);         // one past the last
  const int last = max(0, my1 - 1);               // a k-step this wave may address

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

  auto load = [&](u32x4(&dst)[SPW], int t) {
    const uint16_t* p = Wp + (size_t)t * nsteps * 512 + lane * 8;
#pragma unroll
    for (int s = 0; s < SPW; ++s) dst[s] = load_w16<NTL>(p + (size_t)min(my0 + s, last) * 512);
  };
  unsigned ticket = 0u;  // thread 0: the ticket asked for during the current tile
  // Tile t from registers a.  With pass_on, thread 0 turns its ticket into
  // the next queue tile for the workgroup, between the two barriers.
  auto consume = [&](const u32x4(&a)[SPW], int t, bool pass_on) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (my0 + s < my1) {
        const u32x4 bf = *(const u32x4*)(xs + mx * pitch + (my0 + s) * 32 + 8 * g);
        acc = mfma(a[s], bf, acc);
      }
    }
    // Sum the waves' partials in a fixed order.
    red[wv * 64 + lane] = acc;
    __syncthreads();
    if (wv == 0) {
      if (pass_on && lane == 0) sh_tile = tile_of(ticket);
      f32x4 sum = red[lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const f32x4 o = red[w * 64 + lane];
        sum[0] += o[0];
        sum[1] += o[1];
        sum[2] += o[2];
        sum[3] += o[3];
      }
      const int64_t v0 = (int64_t)t * 16 + 4 * g;
      if (live && v0 < V) {
        if (EPI != 2 || Y != nullptr) store4<OUT_BF16>(Y, (size_t)m * V + v0, v0, V, sum);
        if (EPI == 1) {  // terms 2^(z * c1 - max * log2(e)), c1 = fl32(1/T) * log2(e)
          constexpr float kLog2e = 1.4426950408889634f;
          float zt = -INFINITY;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (v0 + q < V) zt = fmaxf(zt, sum[q]);
          const float mt = zt * fs.inv_t;  // = max of fl32(z * fl32(1/T)) over the four
          if (mt > st_m) {
            if (st_s > 0.0) st_s *= (double)__builtin_amdgcn_exp2f((st_m - mt) * kLog2e);
            st_m = mt;
          }
          const float c1 = fs.inv_t * kLog2e, c2 = st_m * kLog2e;
          float s4 = 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (v0 + q < V) s4 += __builtin_amdgcn_exp2f(fmaf(sum[q], c1, -c2));
          st_s += (double)s4;
        } else if (EPI == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (v0 + q < V && (sum[q] > st_m || (sum[q] == st_m && (int)v0 + q < st_i))) {
              st_m = sum[q];
              st_i = (int)v0 + q;
            }
        }
        if (EPI == 1 && st_x >= v0 && st_x < v0 + 4) fs.zx[m] = sum[st_x - (int)v0];
      }
    }
    __syncthreads();
  };

  // Fixed share: two tiles per trip so the prefetch registers swap roles
  // without copies; the last one or two tiles are peeled off so that no load
  // is issued past the share, and the last one also passes on the first
  // queue tile.
  if (S > 0) {
    const int b = (int)blockIdx.x;
    u32x4 a0[SPW], a1[SPW];
    if (S == 1 && tid == 0) read_tag();
    load(a0, b);
    int j = 0;
    for (; j + 2 < S; j += 2) {
      if (j + 4 >= S && tid == 0) read_tag();  // the last trip: a tile or two ahead of the first ticket
      load(a1, b + (j + 1) * G);
      consume(a0, b + j * G, false);
      load(a0, b + (j + 2) * G);
      consume(a1, b + (j + 1) * G, false);
    }
    if (j + 1 < S) {
      if (j == 0 && tid == 0) read_tag();
      load(a1, b + (j + 1) * G);
      consume(a0, b + j * G, false);
      if (tid == 0) ticket = first_ask();
      consume(a1, b + (j + 1) * G, true);
    } else {
      if (tid == 0) ticket = first_ask();
      consume(a0, b + j * G, true);
    }
  }
  // Queue: one tile at a time (a second register set for prefetching
  // measured no faster here).  Thread 0 asks for the next ticket right after
  // the tile's loads go out and passes it on while the tile is reduced.
  // Every wave reads the tile index after the barrier that follows its
  // publication, so all waves take the same tiles and meet at the same
  // barriers.
  for (;;) {
    const int t = __builtin_amdgcn_readfirstlane(sh_tile);
    if (t >= ntiles) break;
    u32x4 a[SPW];
    load(a, t);
    if (tid == 0) ticket = ask();
    consume(a, t, true);
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
}

// A tag unique to each launch in this process (a bijective mix of a counter
// that starts at a value drawn from the clock and an address), never 0.
uint64_t next_launch_tag() {
  static std::atomic<uint64_t> counter{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                                       ((uint64_t)(uintptr_t)&counter << 17)};
  uint64_t z = counter.fetch_add(0x9e3779b97f4a7c15ull, std::memory_order_relaxed) + 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return z ? z : 1;
}

constexpr int kSweepWaves = 8;
constexpr int kSweepGroup = 16;
constexpr size_t kSweepLdsLimit = 150 * 1024;

size_t sweep_lds_bytes(int64_t N, int64_t d) {
  return (((size_t)N * (size_t)(d + kPad) + 7) & ~(size_t)7) * sizeof(uint16_t) + (size_t)kSweepWaves * 64 * 16;
}

template <bool OUT_BF16, int EPI>
hipError_t launch_sweep_kernel(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N,
                               int64_t d, int64_t V, void* tickets, const FusedStats& fs, hipStream_t stream) {
  if (tickets == nullptr) return hipErrorInvalidValue;
  const size_t lds = sweep_lds_bytes(N, d);
  auto k = sweep_kernel<kSweepWaves, kSweepGroup, true, OUT_BF16, EPI>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  // The fixed share: about 85% of the tiles (measured on the LM-head sweep:
  // 80-90% equally fast, 70% and 95% slower).
  const int64_t ntiles = (V + 15) / 16;
  const int S = (int)(ntiles * 17 / (20 * p.grid));
  hipLaunchKernelGGL(k, dim3((unsigned)p.grid), dim3(kSweepWaves * 64), lds, stream, X, Wp, Y, (int)N, (int)d, (int)V, S,
                     (unsigned*)tickets, next_launch_tag(), fs);
  return hipGetLastError();
}

}  // namespace

SweepPlan plan_sweep(int64_t N, int64_t d, int64_t V, int cus) {
  SweepPlan p{};
  const int64_t nsteps = d / 32, ntiles = (V + 15) / 16;
  // X whole in LDS and one register group per wave and tile (the dispatcher
  // takes the panel kernel otherwise).
  if (N > 16 || nsteps < 1 || nsteps > kSweepWaves * kSweepGroup || sweep_lds_bytes(N, d) > kSweepLdsLimit) return p;
  p.ok = true;
  p.grid = ntiles < cus ? ntiles : cus;
  return p;
}

hipError_t launch_sweep(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d,
                        int64_t V, bool out_bf16, void* tickets, hipStream_t stream) {
  const FusedStats none{};
  return out_bf16 ? launch_sweep_kernel<true, 0>(p, X, Wp, Y, N, d, V, tickets, none, stream)
                  : launch_sweep_kernel<false, 0>(p, X, Wp, Y, N, d, V, tickets, none, stream);
}

hipError_t launch_sweep_with_stats(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, float* Y, int64_t N,
                                   int64_t d, int64_t V, const FusedStats& fs, void* tickets, int64_t* nparts,
                                   hipStream_t stream) {
  const hipError_t e = fs.greedy ? launch_sweep_kernel<false, 2>(p, X, Wp, Y, N, d, V, tickets, fs, stream)
                                 : launch_sweep_kernel<false, 1>(p, X, Wp, Y, N, d, V, tickets, fs, stream);
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
