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
// (cut_key, cut_idx).  Ranking entries by the 55-bit composite
// (order_key(z) << 23) | (2^23 - 1 - index), larger first, is exactly that
// order, and the cut is the entry at which the running weight (1 per entry
// for top-k; for top-p the mass) first reaches a target.  One workgroup per
// row finds it:
//   * the 12 high bits of the key (sign, exponent, 3 mantissa bits) split the
//     row into 4096 buckets: one coalesced pass histograms them in LDS (with
//     the row maximum), and a workgroup scan from the top bucket finds the
//     bucket of the cut;
//   * a second pass copies the candidates into LDS: for top-k every entry at
//     or above that bucket when they are at most kCap (top-p then runs on the
//     same candidates, with no further pass), else that bucket alone;
//   * in LDS the candidates of the top-k case are sorted by composite (a
//     bitonic network), so the top-k cut is the k-th of them and the top-p cut
//     the first rank where the prefix mass reaches the target; elsewhere the
//     cut is the crossing of the running weight in composite order, found by
//     a single wave ranking up to 64 candidates directly, or by radix levels
//     of 12 bits over the composite;
//   * a bucket with more than kCap entries is split by a second global level
//     on the next 12 key bits, and one still too full (runs of equal logits)
//     by the last 8 bits; equal keys are then cut in index order by an
//     ordered scan over wave-contiguous ranges.
// For a small top-k of a long row a sampled threshold replaces the histogram:
// one pass collects every entry above it together with the row maximum, and
// the histogram passes run only when that catch is too small or too large.
// The threshold comes from small histograms of the sample's top buckets, and
// the pass compares values (the largest of each four first), forming keys
// only for the entries it collects.
// The kernel also leaves the warped row's statistics for the draw (the max
// and sum of exponentials over the kept entries, the drafted token's logit),
// so a warped step needs no separate statistics pass.
// The mass of v is fp32 exp((z_v - max z) * fl32(1/T)) (the difference first,
// so its error stays near (1 + |z_v - max z| / T) * 2^-23 relative however
// large the logits are) as an integer with 40 fraction bits: every sum is
// exact and independent of the order of the atomics.  The top-p target is
// ceil(top_p * total), at least 1.  Totals stay below 2^64 and indices fit
// the composite for V <= 2^23.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;  // 12-bit digits
constexpr int kCap = 2048;   // candidates held in LDS
constexpr int kIdxBits = 23;
constexpr uint32_t kIdxMask = (1u << kIdxBits) - 1;

typedef unsigned long long u64;

struct Cut {
  uint32_t key;
  int32_t idx;
};

struct Shared {
  u64 mass[kBins];      // per-bin masses (top-p)
  uint32_t cnt[kBins];  // per-bin counts
  u64 comp[kCap];       // candidates: composite
  u64 cw[kCap];         // candidates: mass (top-p)
  u64 red[kWaves];
  float redf[kWaves];
  u64 above;
  uint32_t ncand;
  uint32_t bin;
  int found;
};

// floor(e * 2^40) for e = 2^((z - zmax) * (fl32(1/T) * log2(e))) in [0, 1]
// (the difference first, then one rounding more than z/T - max/T itself, then
// the hardware base-2 exponential): 256 e is exact in fp32, its integer part
// h counts units of 2^32, and its fraction 256 e - h times 2^32, exact too,
// truncates to the rest.  0 for -inf logits and wherever e underflows.
__device__ __forceinline__ u64 mass_fixed(float z, float inv_t, float zmax) {
  const float s = __builtin_amdgcn_exp2f((z - zmax) * (inv_t * 1.4426950408889634f)) * 256.0f;
  return ((u64)(uint32_t)s << 32) | (u64)(uint32_t)(__builtin_amdgcn_fractf(s) * 4294967296.0f);
}
__device__ __forceinline__ u64 composite(uint32_t key, int v) {
  return ((u64)key << kIdxBits) | (u64)(kIdxMask - (uint32_t)v);
}
__device__ __forceinline__ float key_value(uint32_t key) {  // inverse of order_key
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Loads from the row through global-memory instructions.  The row is always
// device memory; in the functions kept out of line its pointer arrives
// without that knowledge, and generic loads would share their wait counter
// with the LDS operations of the same loop.
__device__ __forceinline__ float4 load_row4(const float* p) {
  typedef float v4 __attribute__((ext_vector_type(4)));
  const v4 t = *(const __attribute__((address_space(1))) v4*)p;
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float load_row1(const float* p) {
  return *(const __attribute__((address_space(1))) float*)p;
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

// Bins nb-1 down to 0 (thread t holds nb-1-4t .. nb-4-4t): the bin where the
// running weight first reaches `need`, and the weight of the bins above it.
template <bool MASS>
__device__ void scan_bins(int nb, u64 need, Shared& sh, uint32_t& bin, u64& above) {
  u64 h[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = nb - 1 - 4 * (int)threadIdx.x - j;
    h[j] = d >= 0 ? (MASS ? sh.mass[d] : (u64)sh.cnt[d]) : 0ull;
    local += h[j];
  }
  if (threadIdx.x == 0) {  // kept if no bin crosses (need above the total)
    sh.bin = 0;
    sh.above = 0;
  }
  const u64 before = block_exclusive(local, sh.red);
  if (before < need && before + local >= need) {
    u64 run = before;
    int sel = 3;
#pragma unroll
    for (int j = 0; j < 3; ++j) {  // static indices: h stays in registers
      if (sel == 3 && run + h[j] >= need) sel = j;
      if (sel == 3) run += h[j];
    }
    sh.bin = (uint32_t)(nb - 1 - 4 * (int)threadIdx.x - sel);
    sh.above = run;
  }
  __syncthreads();
  bin = sh.bin;
  above = sh.above;
  __syncthreads();
}

__device__ __forceinline__ void clear_bins(Shared& sh, bool mass) {
  for (int b = threadIdx.x; b < kBins; b += kThreads) {
    sh.cnt[b] = 0;
    if (mass) sh.mass[b] = 0;
  }
  __syncthreads();
}

// Calls f(v, z) for every entry of the row; wave w takes the contiguous range
// [w*R, (w+1)*R) (R a multiple of 256) in steps of 256 entries, lane l the 4
// entries at 4l, four steps' loads issued together.
template <bool VEC, class F, int U = 4>
__device__ __forceinline__ void for_row(const float* __restrict__ row, int V, int R, F&& f) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b0 = w * R, b1 = min(b0 + R, V);
  for (int base = b0; base < b1; base += U * 256) {
    float z[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = base + 256 * u + 4 * lane;
      if (VEC && v + 3 < b1) {
        const float4 t = load_row4(row + v);
        z[u][0] = t.x;
        z[u][1] = t.y;
        z[u][2] = t.z;
        z[u][3] = t.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[u][e] = v + e < b1 ? load_row1(row + v + e) : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = base + 256 * u + 4 * lane + e;
        if (v < b1) f(v, z[u][e]);
      }
  }
}

// The collecting pass: the running max zm of the row's entries, and A(z, v)
// for every entry with z >= zt, over the same ranges as for_row with eight
// 16-byte loads in flight per lane.  Steps that lie wholly inside the wave's
// range load without tests.
template <bool VEC, class A>
__device__ __forceinline__ void collect_row(const float* __restrict__ row, int V, int R, float zt, float& zm, A&& append) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b0 = w * R, b1 = min(b0 + R, V);
  for (int base = b0; base < b1; base += U * 256) {
    float z[U][4];
    const bool whole = VEC && base + U * 256 <= b1;  // wave-uniform
    if (whole) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float4 t = load_row4(row + base + 256 * u + 4 * lane);
        z[u][0] = t.x;
        z[u][1] = t.y;
        z[u][2] = t.z;
        z[u][3] = t.w;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float g = fmaxf(fmaxf(z[u][0], z[u][1]), fmaxf(z[u][2], z[u][3]));
        zm = fmaxf(zm, g);
        if (g >= zt) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (z[u][e] >= zt) append(z[u][e], base + 256 * u + 4 * lane + e);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = base + 256 * u + 4 * lane + e;
          z[u][e] = v < b1 ? load_row1(row + v) : -INFINITY;
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = base + 256 * u + 4 * lane + e;
          if (v < b1) {
            zm = fmaxf(zm, z[u][e]);
            if (z[u][e] >= zt) append(z[u][e], v);
          }
        }
    }
  }
}

// The cut among the n candidates in LDS: the candidate (those with composite >=
// floor only) at which the running weight in composite order first reaches
// need.  Returns its composite, or 0 if the weights never reach need.
template <bool MASS>
__device__ u64 lds_select(int n, u64 need, u64 floor, Shared& sh) {
  if (n <= 64) {  // one wave ranks every candidate directly
    if (threadIdx.x == 0) sh.found = -1;
    __syncthreads();
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      const u64 ci = i < n ? sh.comp[i] : 0ull;
      const u64 wi = (i < n && ci >= floor) ? (MASS ? sh.cw[i] : 1ull) : 0ull;
      u64 before = 0;
      for (int j = 0; j < n; ++j) {
        const u64 cj = sh.comp[j];
        if (cj > ci && cj >= floor) before += MASS ? sh.cw[j] : 1ull;
      }
      if (wi > 0 && before < need && before + wi >= need) sh.found = i;
    }
    __syncthreads();
    const int f = sh.found;
    const u64 r = f >= 0 ? sh.comp[f] : 0ull;
    __syncthreads();
    return r;
  }
  u64 prefix = 0;
  int hi = 32 + kIdxBits;  // composite bits [0, hi) still open
  while (hi > 0) {
    const int width = hi < 12 ? hi : 12, lo = hi - width;
    clear_bins(sh, MASS);
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const u64 c = sh.comp[i];
      if (c >= floor && (c >> hi) == (prefix >> hi)) {
        const uint32_t d = (uint32_t)((c >> lo) & ((1ull << width) - 1));
        atomicAdd(&sh.cnt[d], 1u);
        if (MASS) atomicAdd(&sh.mass[d], sh.cw[i]);
      }
    }
    __syncthreads();
    uint32_t d;
    u64 above;
    scan_bins<MASS>(1 << width, need, sh, d, above);
    need = need > above ? need - above : 0;
    prefix |= (u64)d << lo;
    hi = lo;
  }
  return prefix;
}

// Calls f(v, z) for every entry of the row over the same ranges as for_row,
// U 16-byte loads in flight per lane; steps that lie wholly inside the wave's
// range load and call without per-entry tests.
template <bool VEC, int U = 8, class F>
__device__ __forceinline__ void for_row_lean(const float* __restrict__ row, int V, int R, F&& f) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b0 = w * R, b1 = min(b0 + R, V);
  for (int base = b0; base < b1; base += U * 256) {
    float z[U][4];
    if (VEC && base + U * 256 <= b1) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float4 t = load_row4(row + base + 256 * u + 4 * lane);
        z[u][0] = t.x;
        z[u][1] = t.y;
        z[u][2] = t.z;
        z[u][3] = t.w;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) f(base + 256 * u + 4 * lane + e, z[u][e]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = base + 256 * u + 4 * lane + e;
          z[u][e] = v < b1 ? load_row1(row + v) : 0.0f;
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = base + 256 * u + 4 * lane + e;
          if (v < b1) f(v, z[u][e]);
        }
    }
  }
}

// The value zt with order_key(z) >= t exactly for the non-NaN z >= zt (the
// keys below that of -inf, and those above that of +inf, are no float's; a
// NaN zt compares false).
__device__ __forceinline__ float key_floor_value(uint32_t t) {
  return t <= 0x007fffffu ? -INFINITY : (t > 0xff800000u ? __uint_as_float(0x7fc00000u) : key_value(t));
}

// Top-p alone over a long row, from a window of keys around the cut.  The
// sample of the collecting path (16 entries per thread), weighed by its
// masses, puts the cut in a 12-bit key bucket bc.  One pass over the row then
// takes every entry's mass (the row's total), the masses above the window of
// buckets bc - 4 .. bc + 3 (per thread, no atomics), and the window's
// histogram of masses at 11-bit resolution (4096 bins of 2^11 keys).  The
// bin where the running mass from the top reaches the target is compacted
// into LDS and the cut found among its entries, as select_cut's last step
// does.  That compacting pass also sums the warped statistics' terms of the
// entries above the bin (all of them kept), and those of the kept candidates
// are added after the cut: zpart is this thread's share of Z (the terms as the
// statistics pass forms them, in another order).  Returns false (LDS changed,
// nothing else) when the cut lies outside the window or its bin holds more
// than kCap entries; the full passes then run.
template <bool VEC>
__device__ __noinline__ bool top_p_window(const float* __restrict__ row, int V, int R, float top_p, float inv_t, float zmax,
                             Shared& sh, Cut& cut, double& zpart) {
  const int q = V / (16 * kThreads);
  u64 stot = 0;
  clear_bins(sh, true);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int v0 = 16 * q * (int)threadIdx.x + 4 * u;  // v0 + 3 < 16 q kThreads <= V
    float z[4];
    if (VEC) {
      const float4 t = load_row4(row + v0);
      z[0] = t.x;
      z[1] = t.y;
      z[2] = t.z;
      z[3] = t.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = load_row1(row + v0 + e);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u64 m = mass_fixed(z[e], inv_t, zmax);
      if (m > 0) atomicAdd(&sh.mass[order_key(z[e]) >> 20], m);
      stot += m;
    }
  }
  const u64 S = block_sum(stot, sh.red);  // its barriers also order the atomics before the scan
  if (S == 0) return false;
  const double ts = ceil((double)top_p * (double)S);
  const u64 sneed = ts < 1.0 ? 1ull : (ts > (double)S ? S : (u64)ts);
  uint32_t bc;
  u64 sabove;
  scan_bins<true>(kBins, sneed, sh, bc, sabove);
  const uint32_t blo = bc >= 4 ? bc - 4 : 0u;
  const u64 whi = (u64)min(bc + 4u, (uint32_t)kBins) << 20;  // window: keys [blo << 20, whi)
  const uint32_t wlo = blo << 20;
  const float zwlo = key_floor_value(wlo);
  const float zwhi = whi > 0xffffffffull ? __uint_as_float(0x7fc00000u) : key_floor_value((uint32_t)whi);

  clear_bins(sh, true);
  u64 tot = 0, hi = 0;
  for_row_lean<VEC, 4>(row, V, R, [&](int v, float z) {
    const u64 m = mass_fixed(z, inv_t, zmax);
    tot += m;
    if (z >= zwhi) {
      hi += m;
    } else if (z >= zwlo && m > 0) {
      atomicAdd(&sh.mass[(order_key(z) - wlo) >> 11], m);
    }
  });
  tot = block_sum(tot, sh.red);
  hi = block_sum(hi, sh.red);  // also orders the atomics before the scan
  const double t = ceil((double)top_p * (double)tot);
  u64 need = t < 1.0 ? 1ull : (t > (double)tot ? tot : (u64)t);
  if (tot == 0 || hi >= need) return false;
  need -= hi;
  uint32_t f;
  u64 above;
  scan_bins<true>(kBins, need, sh, f, above);
  const bool found = above + sh.mass[f] >= need;  // else the window holds less than need
  __syncthreads();
  if (!found) return false;
  need -= above;
  const uint32_t flo = wlo + (f << 11);
  const u64 fhi = (u64)flo + 2048;
  const float zflo = key_floor_value(flo);
  const float zfhi = fhi > 0xffffffffull ? __uint_as_float(0x7fc00000u) : key_floor_value((uint32_t)fhi);
  // The statistics' terms 2^(z * c1 - c2), as the statistics pass forms them.
  const float c1 = inv_t * 1.4426950408889634f, c2 = (zmax * inv_t) * 1.4426950408889634f;
  if (threadIdx.x == 0) sh.ncand = 0;
  __syncthreads();
  double zs = 0.0;
  for_row_lean<VEC, 4>(row, V, R, [&](int v, float z) {
    if (z >= zfhi) {  // above the cut's bin: kept
      zs += (double)__builtin_amdgcn_exp2f(fmaf(z, c1, -c2));
    } else if (z >= zflo) {
      // In the bin.  Only entries of positive mass can be kept: the cut's own
      // mass is positive, and masses do not decrease with z.
      const u64 m = mass_fixed(z, inv_t, zmax);
      if (m > 0) {
        const uint32_t sl = atomicAdd(&sh.ncand, 1u);
        if (sl < (uint32_t)kCap) {
          sh.comp[sl] = composite(order_key(z), v);
          sh.cw[sl] = m;
        }
      }
    }
  });
  __syncthreads();
  const uint32_t napp = sh.ncand;
  __syncthreads();
  if (napp > (uint32_t)kCap) return false;
  const int n = (int)napp;
  const u64 c = lds_select<true>(n, need, 0ull, sh);
  cut = Cut{(uint32_t)(c >> kIdxBits), (int32_t)(kIdxMask - (uint32_t)(c & kIdxMask))};
  for (int i = threadIdx.x; i < n; i += kThreads) {  // the kept candidates: composites at or above the cut's
    const u64 ci = sh.comp[i];
    if (ci >= c) zs += (double)__builtin_amdgcn_exp2f(fmaf(key_value((uint32_t)(ci >> kIdxBits)), c1, -c2));
  }
  zpart = zs;
  return true;
}

// Copies into LDS the entries kept by `lim` (positive mass when MASS) whose
// key has `prefix` in the bits under `mask`.  Returns how many there are.
template <bool MASS, bool VEC>
__device__ int compact(const float* __restrict__ row, int V, int R, uint32_t mask, uint32_t prefix, bool at_or_above,
                       Cut lim, float inv_t, float zmax, Shared& sh) {
  if (threadIdx.x == 0) sh.ncand = 0;
  __syncthreads();
  for_row<VEC>(row, V, R, [&](int v, float z) {
    const uint32_t k = order_key(z);
    const bool in = at_or_above ? (k & mask) >= prefix : (k & mask) == prefix;
    if (in && warp_kept(k, v, lim.key, lim.idx)) {
      const u64 m = MASS ? mass_fixed(z, inv_t, zmax) : 1ull;
      if (m > 0) {
        const uint32_t s = atomicAdd(&sh.ncand, 1u);
        if (s < (uint32_t)kCap) {
          sh.comp[s] = composite(k, v);
          if (MASS) sh.cw[s] = m;
        }
      }
    }
  });
  __syncthreads();
  const int n = (int)min(sh.ncand, (uint32_t)kCap);
  __syncthreads();
  return n;
}

// The r-th (1-based) entry in index order among those with key == ck kept by
// lim: each wave counts its contiguous range, the waves' counts are scanned,
// and the wave holding the crossing walks its range in order with ballots.
template <bool VEC>
__device__ int ordered_tie(const float* __restrict__ row, int V, int R, uint32_t ck, u64 r, Cut lim, Shared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u64 c = 0;
  for_row<VEC>(row, V, R, [&](int v, float z) {
    const uint32_t k = order_key(z);
    if (k == ck && warp_kept(k, v, lim.key, lim.idx)) ++c;
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  const u64 before = block_exclusive(lane == 0 ? c : 0ull, sh.red);  // lane 0 of each wave carries its count
  const u64 wb = __shfl(before, 0);
  if (threadIdx.x == 0) sh.found = V - 1;
  __syncthreads();
  if (wb < r && wb + c >= r) {  // wave-uniform
    const int b0 = w * R, b1 = min(b0 + R, V);
    u64 run = wb;
    for (int base = b0; base < b1; base += 256) {
      const int v = base + 4 * lane;
      int cnt = 0;
      bool hit[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hit[e] = false;
        if (v + e < b1) {
          const uint32_t k = order_key(load_row1(row + v + e));
          hit[e] = k == ck && warp_kept(k, v + e, lim.key, lim.idx);
        }
        cnt += hit[e];
      }
      u64 incl = (u64)cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u64 y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const u64 total = __shfl(incl, 63);
      if (run + total >= r) {
        const u64 lb = run + incl - (u64)cnt;  // matches before this lane's four
        if (lb < r && lb + (u64)cnt >= r) {
          u64 q = lb;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (hit[e] && ++q == r) sh.found = v + e;
        }
        break;
      }
      run += total;
    }
  }
  __syncthreads();
  const int f = sh.found;
  __syncthreads();
  return f;
}

// The cut at which the running weight over the entries kept by lim (in rank
// order) first reaches need, given the 12-bit level-1 histograms in sh of
// those entries (counts, and masses when MASS).
template <bool MASS, bool VEC>
__device__ Cut select_cut(const float* __restrict__ row, int V, int R, u64 need, Cut lim, float inv_t, float zmax,
                          Shared& sh) {
  uint32_t b;
  u64 above;
  scan_bins<MASS>(kBins, need, sh, b, above);
  need -= above;
  uint32_t prefix = b << 20, mask = 0xfff00000u;
  int n = (int)sh.cnt[b];
  __syncthreads();
  if (n > kCap) {  // level 2: key bits 19..8 of the bucket's entries
    clear_bins(sh, MASS);
    for_row<VEC>(row, V, R, [&](int v, float z) {
      const uint32_t k = order_key(z);
      if ((k & mask) == prefix && warp_kept(k, v, lim.key, lim.idx)) {
        const u64 m = MASS ? mass_fixed(z, inv_t, zmax) : 1ull;
        if (m > 0) {
          atomicAdd(&sh.cnt[(k >> 8) & 0xfffu], 1u);
          if (MASS) atomicAdd(&sh.mass[(k >> 8) & 0xfffu], m);
        }
      }
    });
    __syncthreads();
    scan_bins<MASS>(kBins, need, sh, b, above);
    need -= above;
    prefix |= b << 8;
    mask = 0xffffff00u;
    n = (int)sh.cnt[b];
    __syncthreads();
    if (n > kCap) {  // level 3: the last 8 bits, then equal keys in index order
      clear_bins(sh, MASS);
      for_row<VEC>(row, V, R, [&](int v, float z) {
        const uint32_t k = order_key(z);
        if ((k & mask) == prefix && warp_kept(k, v, lim.key, lim.idx)) {
          const u64 m = MASS ? mass_fixed(z, inv_t, zmax) : 1ull;
          if (m > 0) {
            atomicAdd(&sh.cnt[k & 0xffu], 1u);
            if (MASS) atomicAdd(&sh.mass[k & 0xffu], m);
          }
        }
      });
      __syncthreads();
      scan_bins<MASS>(256, need, sh, b, above);
      need -= above;
      const uint32_t ck = prefix | b;
      u64 r = need;
      if (MASS) {  // every entry with this key weighs the same
        const u64 m = mass_fixed(key_value(ck), inv_t, zmax);
        r = m > 0 ? (need + m - 1) / m : 1;
      }
      return Cut{ck, ordered_tie<VEC>(row, V, R, ck, r, lim, sh)};
    }
  }
  n = compact<MASS, VEC>(row, V, R, mask, prefix, false, lim, inv_t, zmax, sh);
  const u64 c = lds_select<MASS>(n, need, 0ull, sh);
  return Cut{(uint32_t)(c >> kIdxBits), (int32_t)(kIdxMask - (uint32_t)(c & kIdxMask))};
}

// Sorts sh.comp[0, n) into descending order by rank (n <= 2 * kThreads): the
// rank of a candidate is the number of candidates above it (composites are
// distinct), counted by each thread for its two over the whole list (reads
// that every lane of a wave makes at once), then each is written to its rank.
// No stage or barrier per step of a network; waves past n skip the count.
__device__ void sort_desc_rank(int n, Shared& sh) {
  const int t = threadIdx.x;
  const u64 a = t < n ? sh.comp[t] : 0ull;
  const u64 b = t + kThreads < n ? sh.comp[t + kThreads] : 0ull;
  int ra = 0, rb = 0;
  if (__builtin_amdgcn_readfirstlane(t >> 6) * 64 < n) {  // the wave holds a candidate
    for (int j = 0; j < n; ++j) {
      const u64 c = sh.comp[j];
      ra += c > a;
      rb += c > b;
    }
  }
  __syncthreads();  // every count is done before the list is overwritten
  if (t < n) sh.comp[ra] = a;
  if (t + kThreads < n) sh.comp[rb] = b;
  __syncthreads();
}

// Sorts sh.comp[0, n) into descending order (n <= kCap): by rank up to 512
// candidates (measured: the b8 warped step 3 us faster than a one-wave
// bitonic network, whose stages wait on shuffles in turn), else a bitonic
// network over the next power of two, the padding zeros (below every
// composite of a real entry but a possible 0, which then sorts among them)
// last.
__device__ void sort_desc(int n, Shared& sh) {
  if (n <= 512) {
    sort_desc_rank(n, sh);
    return;
  }
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = n + threadIdx.x; i < P; i += kThreads) sh.comp[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (P >> 1); t += kThreads) {
        const int i = 2 * stride * (t / stride) + (t % stride), j = i + stride;
        const bool desc = (i & size) == 0;  // the final merge (size == P) is descending
        const u64 a = sh.comp[i], b = sh.comp[j];
        if ((a < b) == desc) {
          sh.comp[i] = b;
          sh.comp[j] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Both cuts from n candidates in LDS that include every entry of the row's
// top k (top_k <= n): sorted, the top-k cut is the top_k-th; top-p then runs
// over those top_k entries in rank order (masses exact in fixed point).
// Returns how many entries the cut keeps: ranks [0, that) of sh.comp.
__device__ int cuts_from_candidates(int n, int64_t top_k, bool tp, float top_p, float inv_t, float zmax, Shared& sh,
                                    Cut& cut) {
  sort_desc(n, sh);
  const int kk = (int)top_k;  // top_k < V <= 2^23 and top_k <= n <= kCap
  const u64 ck = sh.comp[kk - 1];
  cut = Cut{(uint32_t)(ck >> kIdxBits), (int32_t)(kIdxMask - (uint32_t)(ck & kIdxMask))};
  if (!tp) return kk;
  if (kk <= 128) {  // one wave, no workgroup scans: lane l holds ranks 2l and 2l + 1
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      u64 m[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * lane + e;
        m[e] = i < kk ? mass_fixed(key_value((uint32_t)(sh.comp[i] >> kIdxBits)), inv_t, zmax) : 0ull;
      }
      u64 incl = m[0] + m[1];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u64 y = (u64)__shfl_up((long long)incl, o);
        if (lane >= o) incl += y;
      }
      const u64 total = (u64)__shfl((long long)incl, 63);
      const double t = ceil((double)top_p * (double)total);
      u64 need = t < 1.0 ? 1ull : (u64)t;
      if (need > total) need = total;
      int f = -1;
      if (need > 0) {
        u64 run = incl - (m[0] + m[1]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if (m[e] > 0 && run < need && run + m[e] >= need) f = 2 * lane + e;
          run += m[e];
        }
      }
      const uint64_t hit = __ballot(f >= 0);
      const int fw = hit ? __shfl(f, __builtin_ctzll(hit)) : -1;
      if (lane == 0) sh.found = fw;
    }
    __syncthreads();
    const int f = sh.found;
    if (f >= 0) {
      const u64 cp = sh.comp[f];
      cut = Cut{(uint32_t)(cp >> kIdxBits), (int32_t)(kIdxMask - (uint32_t)(cp & kIdxMask))};
    }
    __syncthreads();
    return f >= 0 ? f + 1 : kk;
  }
  // Thread t holds ranks 2t and 2t + 1.
  u64 m[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = 2 * (int)threadIdx.x + e;
    m[e] = i < kk ? mass_fixed(key_value((uint32_t)(sh.comp[i] >> kIdxBits)), inv_t, zmax) : 0ull;
  }
  const u64 before = block_exclusive(m[0] + m[1], sh.red);
  const u64 total = block_sum(m[0] + m[1], sh.red);
  const double t = ceil((double)top_p * (double)total);
  u64 need = t < 1.0 ? 1ull : (u64)t;
  if (need > total) need = total;
  if (threadIdx.x == 0) sh.found = -1;
  __syncthreads();
  if (need > 0) {
    u64 run = before;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * (int)threadIdx.x + e;
      if (m[e] > 0 && run < need && run + m[e] >= need) sh.found = i;
      run += m[e];
    }
  }
  __syncthreads();
  const int f = sh.found;
  if (f >= 0) {
    const u64 cp = sh.comp[f];
    cut = Cut{(uint32_t)(cp >> kIdxBits), (int32_t)(kIdxMask - (uint32_t)(cp & kIdxMask))};
  }
  __syncthreads();
  return f >= 0 ? f + 1 : kk;
}

__device__ __forceinline__ double block_sum_f64(double v, u64* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) lds[wv] = __double_as_longlong(v);
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < kWaves; ++w) r += __longlong_as_double(lds[w]);  // fixed order
  __syncthreads();
  return r;
}

// A key t0 with at least `need` of the sample's keys at or above it, close
// above the need-th largest, from two small histograms near the top of the
// sample: counts of the 16 12-bit buckets at and below the bucket of the
// largest key (LDS atomics only from the few samples that fall there), then of
// the 256 next-8-bit sub-buckets of the bucket where the count from the top
// reaches `need`; each is scanned by one wave.  Returns 0 (no threshold) when
// those 16 buckets hold fewer than `need` samples.  Uses sh.cnt[0, 272).
__device__ uint32_t sample_threshold_near_top(const uint32_t (&ks)[16], uint32_t need, Shared& sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t km = ks[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) km = max(km, ks[e]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) km = max(km, (uint32_t)__shfl_xor((int)km, o));
  if (threadIdx.x < 16 + 256) sh.cnt[threadIdx.x] = 0u;
  if (lane == 0) sh.redf[wv] = __uint_as_float(km);
  __syncthreads();
  uint32_t kmax = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) kmax = max(kmax, __float_as_uint(sh.redf[w]));
  const uint32_t kb = kmax >> 20;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t d = kb - (ks[e] >> 20);  // bucket distance below the top one
    if (d < 16u) atomicAdd(&sh.cnt[d], 1u);
  }
  __syncthreads();
  if (wv == 0) {  // buckets kb, kb - 1, ... in lanes 0..15: where the count from the top reaches need
    const uint32_t c = lane < 16 ? sh.cnt[lane] : 0u;
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
      if (lane >= o) incl += y;
    }
    const uint64_t hit = __ballot(lane < 16 && incl >= need);
    if (lane == 0) sh.bin = hit ? kb - (uint32_t)__builtin_ctzll(hit) : 0xffffffffu;
    const int l = hit ? __builtin_ctzll(hit) : 0;
    const uint32_t above = (uint32_t)__shfl((int)(incl - c), l);
    if (lane == 0) sh.above = above;
  }
  __syncthreads();
  const uint32_t b = sh.bin;
  const uint32_t need2 = need - (uint32_t)sh.above;
  if (b == 0xffffffffu) {
    __syncthreads();  // every thread has read sh.bin before it is written again
    return 0u;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if ((ks[e] >> 20) == b) atomicAdd(&sh.cnt[16 + ((ks[e] >> 12) & 0xffu)], 1u);
  __syncthreads();
  if (wv == 0) {  // sub-buckets 255 .. 0, four per lane from the top
    uint32_t h[4], local = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = sh.cnt[16 + 255 - 4 * lane - j];
      local += h[j];
    }
    uint32_t incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
      if (lane >= o) incl += y;
    }
    const uint64_t hit = __ballot(incl >= need2);  // the total of bucket b is at least need2
    const int l = hit ? __builtin_ctzll(hit) : 63;
    if (lane == l) {
      uint32_t run = incl - local;
      int sel = 3;
#pragma unroll
      for (int j = 0; j < 3; ++j) {  // static indices: h stays in registers
        if (sel == 3 && run + h[j] >= need2) sel = j;
        if (sel == 3) run += h[j];
      }
      sh.bin = (b << 20) | ((uint32_t)(255 - 4 * lane - sel) << 12);
    }
  }
  __syncthreads();
  const uint32_t t0 = sh.bin;
  __syncthreads();
  return t0 == 0u ? 1u : t0;  // 0 is kept for "no threshold"; key 0 is no float's
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void warp_cut_kernel(const float* __restrict__ target,
                                                            const float* __restrict__ draft, int64_t n_target,
                                                            int64_t V64, float inv_t, int64_t top_k, float top_p,
                                                            uint32_t* __restrict__ cut_key,
                                                            int32_t* __restrict__ cut_idx, WarpStats so) {
  __shared__ Shared sh;
  const int V = (int)V64;
  const int64_t r = blockIdx.x;
  const float* row = r < n_target ? target + (size_t)r * V : draft + (size_t)(r - n_target) * V;
  const int R = ((V + kWaves * 256 - 1) / (kWaves * 256)) * 256;
  const bool tk = top_k > 0 && top_k < V, tp = top_p < 1.0f;
  // Thread 0: the row's drafted token and its logit, loaded now for the end.
  int xt = -1;
  float zx = 0.0f;
  if (threadIdx.x == 0) {
    const int64_t g1 = so.gamma + 1;
    const bool is_target = r < n_target;
    const int64_t b = is_target ? r / g1 : (r - n_target) / (so.gamma > 0 ? so.gamma : 1);  // draft rows: gamma > 0
    const int64_t i = is_target ? r - b * g1 : (r - n_target) - b * so.gamma;
    if (i < so.gamma) {
      const int32_t x = so.tokens[b * so.gamma + i];
      xt = x < 0 ? 0 : (x >= V ? V - 1 : x);
      zx = row[xt];
    }
  }
  Cut cut{0u, 0x7fffffff};  // keeps every entry
  bool done_p = false;
  int nk = -1;  // when the kept entries are ranks [0, nk) of the sorted candidates in LDS
  bool have_zpart = false;  // the top-p window's share of the warped Z
  double zpart = 0.0;
  float zmax;
  // A small top-k of a long row, in one pass: a sample of 16 entries per
  // thread spread over the row, histogrammed by key (12 bits, then the next 12 within the
  // bucket), gives a threshold t0 at the sample entry whose count from the top
  // stands for about 3*top_k row entries; the pass then takes the row maximum and
  // collects every entry at or above t0 into LDS.  At least top_k of them,
  // none lost to overflow: they hold the whole top k (the k-th largest key is
  // at or above t0), and both cuts come from them.  Otherwise the passes
  // below run as if nothing had been collected.  (Histogramming every entry
  // of the row by bucket serialised on the LDS atomics of the crowded
  // buckets: the one-pass path measured much faster.)
  const bool collect = tk && top_k <= kCap / 4 && V >= 16 * kThreads;
  if (collect) {
    // Sample entries 16*q*t + 4u + e of thread t (u, e < 4; q >= 1): 16384 in
    // all, sixteen consecutive ones (one 64-byte line) at each of 1024 evenly
    // spaced places, so the sample touches a quarter of the lines that
    // sixteen scattered entries per thread would.
    const int q = V / (16 * kThreads);
    uint32_t ks[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v0 = 16 * q * (int)threadIdx.x + 4 * u;  // v0 + 3 < 16 q kThreads <= V
      if (VEC) {
        const float4 t = load_row4(row + v0);
        ks[4 * u + 0] = order_key(t.x);
        ks[4 * u + 1] = order_key(t.y);
        ks[4 * u + 2] = order_key(t.z);
        ks[4 * u + 3] = order_key(t.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ks[4 * u + e] = order_key(load_row1(row + v0 + e));
      }
    }
    // The s0-th largest sample stands for about 3*top_k row entries (mean);
    // fewer than top_k row entries at or above it would need s0 of the row's
    // top top_k - 1 in the sample, far out in the tail.
    const u64 s0 = (u64)((3 * top_k * 16 * kThreads + V - 1) / V);  // >= 1
    uint32_t t0 = sample_threshold_near_top(ks, (uint32_t)s0, sh);
    if (t0 == 0u) {  // the top 16 buckets hold fewer than s0 samples: full 12-bit histograms
      clear_bins(sh, false);
#pragma unroll
      for (int e = 0; e < 16; ++e) atomicAdd(&sh.cnt[ks[e] >> 20], 1u);
      __syncthreads();
      uint32_t b0, b1;
      u64 above0, above1;
      scan_bins<false>(kBins, s0, sh, b0, above0);
      // ... refined by the sample's next 12 key bits within that bucket
      clear_bins(sh, false);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((ks[e] >> 20) == b0) atomicAdd(&sh.cnt[(ks[e] >> 8) & 0xfffu], 1u);
      __syncthreads();
      scan_bins<false>(kBins, s0 - above0, sh, b1, above1);
      t0 = (b0 << 20) | (b1 << 8);
    }
    if (threadIdx.x == 0) sh.ncand = 0;
    __syncthreads();
    // order_key(z) >= t0 holds exactly for the non-NaN z >= zt (the keys
    // below that of -inf, and those above that of +inf, are no float's), so
    // the pass tests values: per four entries their largest against zt, and
    // the four one by one only when it passes (for about 3*top_k of the row's
    // entries), which keeps the pass at a few vector instructions per entry.
    const float zt = t0 <= 0x007fffffu ? -INFINITY : (t0 > 0xff800000u ? __uint_as_float(0x7fc00000u) : key_value(t0));
    float zm = -INFINITY;
    auto append = [&](float z, int v) {
      const uint32_t s = atomicAdd(&sh.ncand, 1u);
      if (s < (uint32_t)kCap) sh.comp[s] = composite(order_key(z), v);
    };
    collect_row<VEC>(row, V, R, zt, zm, append);  // eight 16-byte loads in flight per lane
    zmax = block_max(zm, sh.redf);  // its barriers order the appends
    const uint32_t napp = sh.ncand;
    __syncthreads();
    if (napp >= (uint32_t)top_k && napp <= (uint32_t)kCap) {
      nk = cuts_from_candidates((int)napp, top_k, tp, top_p, inv_t, zmax, sh, cut);
      done_p = tp;
    } else {  // the level-1 histogram in a pass of its own
      clear_bins(sh, false);
      for_row<VEC>(row, V, R, [&](int, float z) { atomicAdd(&sh.cnt[order_key(z) >> 20], 1u); });
      __syncthreads();
    }
  } else {
    // Pass 1: the row maximum, and the top-k level-1 histogram.
    if (tk) clear_bins(sh, false);
    float zm = -INFINITY;
    for_row<VEC>(row, V, R, [&](int /*v*/, float z) {
      zm = fmaxf(zm, z);
      if (tk) atomicAdd(&sh.cnt[order_key(z) >> 20], 1u);
    });
    zmax = block_max(zm, sh.redf);
    // Top-p alone over a long row: from a window around the cut when it holds it.
    if (!tk && tp && V >= 16 * kThreads && top_p_window<VEC>(row, V, R, top_p, inv_t, zmax, sh, cut, zpart)) {
      done_p = true;
      have_zpart = true;
    }
  }
  if (tk && nk < 0) {
    uint32_t b;
    u64 above;
    scan_bins<false>(kBins, (u64)top_k, sh, b, above);
    const u64 held = above + sh.cnt[b];
    __syncthreads();
    if (held <= (u64)kCap) {
      // Every entry at or above the cut's bucket fits in LDS: both cuts from there.
      const int n = compact<false, VEC>(row, V, R, 0xfff00000u, b << 20, true, cut, inv_t, zmax, sh);
      nk = cuts_from_candidates(n, top_k, tp, top_p, inv_t, zmax, sh, cut);
      done_p = tp;
    } else {
      cut = select_cut<false, VEC>(row, V, R, (u64)top_k, cut, inv_t, zmax, sh);
    }
  }
  if (tp && !done_p) {
    nk = -1;
    clear_bins(sh, true);
    u64 part = 0;
    for_row<VEC>(row, V, R, [&](int v, float z) {
      const uint32_t k = order_key(z);
      if (warp_kept(k, v, cut.key, cut.idx)) {
        const u64 m = mass_fixed(z, inv_t, zmax);
        if (m > 0) {
          atomicAdd(&sh.cnt[k >> 20], 1u);
          atomicAdd(&sh.mass[k >> 20], m);
          part += m;
        }
      }
    });
    const u64 total = block_sum(part, sh.red);  // its barriers also order the atomics before the scan
    const double t = ceil((double)top_p * (double)total);
    u64 need = t < 1.0 ? 1ull : (u64)t;
    if (need > total) need = total;
    if (need > 0) cut = select_cut<true, VEC>(row, V, R, need, cut, inv_t, zmax, sh);
  }
  if (threadIdx.x == 0) {
    cut_key[r] = cut.key;
    cut_idx[r] = cut.idx;
  }
  // The warped row's statistics, as the statistics pass would leave them (one
  // partial in slot 0, the row's other slots empty): the max of a = z *
  // fl32(1/T) over the kept entries (the row maximum: the first entry in rank
  // order is always kept) and Z = sum over them of exp(a - max), each term
  // 2^(z * c1 - c2) with c1 = fl32(1/T) * log2(e), c2 = max * log2(e), fp32
  // terms summed in fp64; and the drafted token's logit (-inf when the cut
  // drops it).  The kept entries are the candidates' ranks [0, nk) when the
  // cut came from them; the top-p window has summed them itself; otherwise
  // one more pass over the row.
  const float mx = zmax * inv_t;
  double zsum = 0.0;
  if (mx > -INFINITY) {
    const float c1 = inv_t * 1.4426950408889634f, c2 = mx * 1.4426950408889634f;
    if (have_zpart) {
      zsum = zpart;
    } else if (nk >= 0) {
      for (int i = threadIdx.x; i < nk; i += kThreads)
        zsum += (double)__builtin_amdgcn_exp2f(fmaf(key_value((uint32_t)(sh.comp[i] >> kIdxBits)), c1, -c2));
    } else {
      const ValueCut vc = value_cut(cut.key, cut.idx);
      for_row_lean<VEC, 4>(row, V, R, [&](int v, float z) {
        if (value_kept(z, v, vc.z, vc.idx)) zsum += (double)__builtin_amdgcn_exp2f(fmaf(z, c1, -c2));
      });
    }
  }
  zsum = block_sum_f64(zsum, sh.red);
  const size_t base = (size_t)r * so.pstride;
  for (int c = threadIdx.x; c < so.nch; c += kThreads) {
    so.cmax[base + c] = c == 0 ? mx : -INFINITY;
    so.csum[base + c] = c == 0 ? zsum : 0.0;
  }
  if (threadIdx.x == 0 && xt >= 0) so.zx[r] = warp_kept(order_key(zx), xt, cut.key, cut.idx) ? zx : -INFINITY;
  if (r == 0)
    for (int64_t t = threadIdx.x; t < so.B; t += kThreads) so.done[t] = 0u;
}

}  // namespace

hipError_t launch_warp_cuts(const float* target, const float* draft, int64_t n_target, int64_t n_rows, int64_t V,
                            float inv_t, int64_t top_k, float top_p, uint32_t* cut_key, int32_t* cut_idx,
                            const WarpStats& so, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if ((V & 3) == 0)
    hipLaunchKernelGGL(warp_cut_kernel<true>, dim3((unsigned)n_rows), dim3(kThreads), 0, stream, target, draft,
                       n_target, V, inv_t, top_k, top_p, cut_key, cut_idx, so);
  else
    hipLaunchKernelGGL(warp_cut_kernel<false>, dim3((unsigned)n_rows), dim3(kThreads), 0, stream, target, draft,
                       n_target, V, inv_t, top_k, top_p, cut_key, cut_idx, so);
  return hipGetLastError();
}

}  // namespace specdec
