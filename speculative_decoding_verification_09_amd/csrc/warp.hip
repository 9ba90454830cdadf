// Top-k / top-p warping of a row before the rule ("Speculative decoding."
// lesson, "Why the output is exactly p": the sampling settings reshape p before
// the rule and q before drafting; "Speculative Decoding: Draft, Verify,
// Accept", "Correctness": the rule then reproduces that reshaped p).  The
// reading taken: temperature, then top-k, then top-p; entries ranked by logit
// (larger first), ties by index (lower first); top-k keeps the first k; top-p
// keeps the shortest prefix of the top-k survivors whose probability reaches
// top_p (at least one entry); the sampling kernels renormalise what is kept.
//
// Every kept set is a prefix of that ranking, so a row's warping is one cut
// (cut_key, cut_idx) in the order of order_key and index.  One workgroup per
// row finds it:
//   top-k: a radix select over the 32-bit keys, 8 bits a level, each level a
//     histogram of the digit under the prefix found so far (LDS integer
//     atomics into 16 padded copies, lane l using copy l % 16, so lanes of one
//     wave that hit the same digit mostly hit different addresses), then the
//     tie at the cut resolved in index order with a workgroup prefix sum;
//   top-p: the same select weighted by the masses of the top-k survivors.  The
//     mass of v is fp32 exp((z_v - max z) * fl32(1/T)) (the difference first,
//     so the error stays near (1 + |z_v - max z| / T) * 2^-23 relative however
//     large the logits are) held as an integer with 40 fraction bits, so every
//     sum is exact and independent of the order of the atomics; the cut is the
//     first entry at which the running mass reaches ceil(top_p * total), at
//     least one entry.
// Totals stay below 2^64 for V <= 2^23.  The row is read from L2 after the
// first pass (a 128K-entry row is 512 KB).
#include "internal.h"

namespace specdec {
namespace {

constexpr int kWarpThreads = 1024;
constexpr int kWaves = kWarpThreads / 64;
constexpr int kCopies = 16;
constexpr int kBinPitch = 257;  // padded so copies start on different banks
constexpr double kFix = 1099511627776.0;  // 2^40

typedef unsigned long long u64;

__device__ __forceinline__ u64 mass_fixed(float z, float inv_t, float zmax) {
  const float e = expf((z - zmax) * inv_t);
  return e > 0.0f ? (u64)((double)e * kFix) : 0ull;  // 0 for -inf logits and NaN
}

__device__ __forceinline__ float block_max(float v, float* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if (lane == 0) lds[wv] = v;
  __syncthreads();
  float r = lds[0];
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, lds[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ u64 block_sum(u64 v, u64* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) lds[wv] = v;
  __syncthreads();
  u64 r = 0;
  for (int w = 0; w < kWaves; ++w) r += lds[w];
  __syncthreads();
  return r;
}

// Exclusive prefix sum over the workgroup in thread order.
__device__ __forceinline__ u64 block_exclusive(u64 v, u64* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  u64 x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wv] = x;
  __syncthreads();
  u64 before = 0;
  for (int w = 0; w < wv; ++w) before += lds[w];
  __syncthreads();
  return before + x - v;
}

struct Shared {
  u64 hist[kCopies * kBinPitch];
  u64 tot[256];
  u64 red[kWaves];
  float redf[kWaves];
  u64 above;
  uint32_t digit;
  int idx;
};

// One radix level: among entries whose key matches `prefix` under `mask` and
// that the cut (lk, li) keeps, weigh the digit at `shift` (count, or mass when
// MASS); scanning digits from 255 down, take the one where the running weight
// first reaches `need`, and lower `need` by the weight of the digits above it.
template <bool MASS>
__device__ void radix_level(const float* __restrict__ row, int V, uint32_t& prefix, uint32_t& mask, int shift,
                            u64& need, uint32_t lk, int li, float inv_t, float zmax, Shared& sh) {
  for (int b = threadIdx.x; b < kCopies * kBinPitch; b += kWarpThreads) sh.hist[b] = 0;
  __syncthreads();
  u64* mine = sh.hist + (threadIdx.x & (kCopies - 1)) * kBinPitch;
  for (int v = threadIdx.x; v < V; v += kWarpThreads) {
    const float z = row[v];
    const uint32_t k = order_key(z);
    if ((k & mask) == prefix && warp_kept(k, v, lk, li))
      atomicAdd(mine + ((k >> shift) & 0xffu), MASS ? mass_fixed(z, inv_t, zmax) : 1ull);
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    u64 t = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) t += sh.hist[c * kBinPitch + threadIdx.x];
    sh.tot[threadIdx.x] = t;
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // wave 0: lane l holds digits 255-4l down to 252-4l
    const int lane = threadIdx.x;
    u64 h[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = sh.tot[255 - 4 * lane - j];
      local += h[j];
    }
    u64 incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u64 y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const u64 before = incl - local;
    const u64 hit = __ballot(before < need && incl >= need);
    const int l = hit ? __builtin_ctzll(hit) : 63;  // none: only if need exceeds the total
    if (lane == l) {
      u64 run = before;
      int j = 0;
      while (j < 3 && run + h[j] < need) run += h[j++];
      sh.digit = (uint32_t)(255 - 4 * lane - j);
      sh.above = run;
    }
  }
  __syncthreads();
  prefix |= sh.digit << shift;
  mask |= 0xffu << shift;
  need = need > sh.above ? need - sh.above : 0;
  __syncthreads();
}

// Among entries with key == ck that the cut (lk, li) keeps, in index order,
// the index at which the running weight first reaches `need` (thread t takes a
// contiguous slice, so thread order is index order).
template <bool MASS>
__device__ int tie_index(const float* __restrict__ row, int V, uint32_t ck, u64 need, uint32_t lk, int li,
                         float inv_t, float zmax, Shared& sh) {
  const int chunk = (V + kWarpThreads - 1) / kWarpThreads;
  const int v0 = min((int)threadIdx.x * chunk, V), v1 = min(v0 + chunk, V);
  u64 w = 0;
  for (int v = v0; v < v1; ++v) {
    const float z = row[v];
    const uint32_t k = order_key(z);
    if (k == ck && warp_kept(k, v, lk, li)) w += MASS ? mass_fixed(z, inv_t, zmax) : 1ull;
  }
  const u64 before = block_exclusive(w, sh.red);
  if (threadIdx.x == 0) sh.idx = -1;
  __syncthreads();
  if (before < need && before + w >= need) {  // exactly one thread, unless need exceeds the total
    u64 run = before;
    for (int v = v0; v < v1; ++v) {
      const float z = row[v];
      const uint32_t k = order_key(z);
      if (k == ck && warp_kept(k, v, lk, li)) {
        run += MASS ? mass_fixed(z, inv_t, zmax) : 1ull;
        if (run >= need) {
          sh.idx = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  const int r = sh.idx;
  __syncthreads();
  return r < 0 ? V - 1 : r;
}

__global__ __launch_bounds__(kWarpThreads) void warp_cut_kernel(const float* __restrict__ target,
                                                                const float* __restrict__ draft, int64_t n_target,
                                                                int64_t V64, float inv_t, int64_t top_k, float top_p,
                                                                uint32_t* __restrict__ cut_key,
                                                                int32_t* __restrict__ cut_idx) {
  __shared__ Shared sh;
  const int V = (int)V64;
  const int64_t r = blockIdx.x;
  const float* row = r < n_target ? target + (size_t)r * V : draft + (size_t)(r - n_target) * V;
  uint32_t ck = 0u;  // (0, INT_MAX) keeps every entry
  int ci = 0x7fffffff;
  float zm = -INFINITY;
  for (int v = threadIdx.x; v < V; v += kWarpThreads) zm = fmaxf(zm, row[v]);
  const float zmax = block_max(zm, sh.redf);  // the top entry's mass is 1, every other <= 1
  if (top_k > 0 && top_k < V) {
    uint32_t prefix = 0, mask = 0;
    u64 need = (u64)top_k;
    for (int shift = 24; shift >= 0; shift -= 8)
      radix_level<false>(row, V, prefix, mask, shift, need, ck, ci, inv_t, zmax, sh);
    ci = tie_index<false>(row, V, prefix, need, ck, ci, inv_t, zmax, sh);
    ck = prefix;
  }
  if (top_p < 1.0f) {
    u64 total = 0;
    for (int v = threadIdx.x; v < V; v += kWarpThreads) {
      const float z = row[v];
      if (warp_kept(order_key(z), v, ck, ci)) total += mass_fixed(z, inv_t, zmax);
    }
    total = block_sum(total, sh.red);
    const double t = ceil((double)top_p * (double)total);
    u64 need = t < 1.0 ? 1ull : (u64)t;
    if (need > total) need = total;
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8)
      radix_level<true>(row, V, prefix, mask, shift, need, ck, ci, inv_t, zmax, sh);
    ci = tie_index<true>(row, V, prefix, need, ck, ci, inv_t, zmax, sh);
    ck = prefix;
  }
  if (threadIdx.x == 0) {
    cut_key[r] = ck;
    cut_idx[r] = ci;
  }
}

}  // namespace

hipError_t launch_warp_cuts(const float* target, const float* draft, int64_t n_target, int64_t n_rows, int64_t V,
                            float inv_t, int64_t top_k, float top_p, uint32_t* cut_key, int32_t* cut_idx,
                            hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(warp_cut_kernel, dim3((unsigned)n_rows), dim3(kWarpThreads), 0, stream, target, draft, n_target,
                     V, inv_t, top_k, top_p, cut_key, cut_idx);
  return hipGetLastError();
}

}  // namespace specdec
