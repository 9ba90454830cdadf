// Paged KV cache with speculative rollback, on the device ("LLM Inference &
// Speculative Decoding", section 1: paged block allocation, block tables and
// instant rollback of rejected speculative tokens; "Speculative decoding."
// lesson, "The KV cache has to forget").
//
// State (caller-owned device memory):
//   pools   [num_blocks][heads][block_size][head_dim] keys and values
//   tables  [R][max_blocks] physical block of each logical block
//   lens    [R] tokens held by each request; request r uses ceil(lens/bs)
//           logical blocks, token t at block t / bs, offset t % bs
//   stack   [num_blocks] free blocks, top[0] of them; the top is stack[top-1]
// A batch is served in request order, as one request at a time would be:
// allocation takes blocks from the top of the stack, and rollback pushes a
// request's trailing blocks back, its last logical block first.  The
// bookkeeping runs in one workgroup with exclusive prefix sums over the
// requests (so the result never depends on scheduling); copies of keys and
// values run over the whole grid in 16-byte units.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kBookThreads = 1024;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t nblocks(int64_t len, int64_t bs) { return (len + bs - 1) / bs; }

// Exclusive prefix sum over the workgroup (kBookThreads threads, 16 waves);
// returns the exclusive value for this thread and the workgroup total.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* lds, int64_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wv] = x;
  __syncthreads();
  int64_t before = 0;
  total = 0;
  for (int w = 0; w < kBookThreads / 64; ++w) {
    if (w < wv) before += lds[w];
    total += lds[w];
  }
  __syncthreads();  // lds reusable
  return before + x - v;
}

__global__ __launch_bounds__(256) void kv_init_kernel(int32_t* __restrict__ stack, int32_t* __restrict__ top,
                                                      int32_t* __restrict__ lens, int64_t R, int64_t num_blocks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < num_blocks) stack[i] = (int32_t)(num_blocks - 1 - i);
  if (i < R) lens[i] = 0;
  if (i == 0) top[0] = (int32_t)num_blocks;
}

// Allocation for n_new tokens per request: all or nothing.  status: 0, 1 (the
// free blocks do not cover the batch), 2 (a request would need more than
// max_blocks).  old_lens receives each request's length before the append.
__global__ __launch_bounds__(kBookThreads) void kv_alloc_kernel(int32_t* __restrict__ tables, int32_t* __restrict__ lens,
                                                                int32_t* __restrict__ stack, int32_t* __restrict__ top,
                                                                int64_t R, int64_t n_new, int64_t bs, int64_t max_blocks,
                                                                int32_t* __restrict__ old_lens,
                                                                int32_t* __restrict__ status) {
  __shared__ int64_t lds[kBookThreads / 64];
  const int tid = threadIdx.x;
  // Pass 1: blocks needed in all, and whether some table is too short.
  int64_t need = 0, bad = 0;
  for (int64_t r = tid; r < R; r += kBookThreads) {
    const int64_t nb_new = nblocks(lens[r] + n_new, bs);
    bad |= nb_new > max_blocks;
    need += nb_new - nblocks(lens[r], bs);
  }
  int64_t tot_need, tot_bad;
  block_exclusive_scan(need, lds, tot_need);
  block_exclusive_scan(bad, lds, tot_bad);
  const int64_t avail = top[0];
  const int32_t st = tot_bad ? 2 : (tot_need > avail ? 1 : 0);
  if (st != 0) {
    if (tid == 0) status[0] = st;
    return;  // uniform: nothing changes
  }
  // Pass 2: hand out blocks in request order.
  int64_t carry = 0;
  for (int64_t r0 = 0; r0 < R; r0 += kBookThreads) {
    const int64_t r = r0 + tid;
    int64_t len = 0, nb_old = 0, nr = 0;
    if (r < R) {
      len = lens[r];
      nb_old = nblocks(len, bs);
      nr = nblocks(len + n_new, bs) - nb_old;
    }
    int64_t chunk_total;
    const int64_t before = carry + block_exclusive_scan(nr, lds, chunk_total);
    if (r < R) {
      for (int64_t j = 0; j < nr; ++j) tables[r * max_blocks + nb_old + j] = stack[avail - 1 - (before + j)];
      old_lens[r] = (int32_t)len;
      lens[r] = (int32_t)(len + n_new);
    }
    carry += chunk_total;
  }
  if (tid == 0) {
    top[0] = (int32_t)(avail - carry);
    status[0] = 0;
  }
}

// Copies the new keys and values ([R][heads][n_new][head_dim]) into their
// blocks, one 16-byte unit per thread; nothing if the allocation failed.
__global__ __launch_bounds__(256) void kv_scatter_kernel(uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool,
                                                         const int32_t* __restrict__ tables,
                                                         const int32_t* __restrict__ old_lens,
                                                         const uint8_t* __restrict__ knew,
                                                         const uint8_t* __restrict__ vnew, int64_t R, int64_t n_new,
                                                         int64_t heads, int64_t bs, int64_t row_units,
                                                         int64_t max_blocks, int64_t num_blocks,
                                                         const int32_t* __restrict__ status) {
  if (status[0] != 0) return;
  const int64_t total = R * heads * n_new * row_units;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t u = idx % row_units, rest = idx / row_units;
    const int64_t i = rest % n_new, rh = rest / n_new, h = rh % heads, r = rh / heads;
    const int64_t pos = old_lens[r] + i;
    const int64_t phys = tables[r * max_blocks + pos / bs];
    if (phys < 0 || phys >= num_blocks) continue;  // a table the caller left inconsistent: never write outside the pool
    const int64_t dst = ((phys * heads + h) * bs + pos % bs) * row_units + u;
    ((u32x4*)kpool)[dst] = ((const u32x4*)knew)[idx];
    ((u32x4*)vpool)[dst] = ((const u32x4*)vnew)[idx];
  }
}

// Rollback: request r keeps keep_lens[r] tokens (or, after a verification
// step of gamma drafts that fed gamma+1 positions, lens[r] - (gamma+1) +
// num_emitted[r]: the text grew by num_emitted tokens and the last one is not
// yet in the cache).  Trailing blocks go back to the stack, last logical block
// first, requests in order.  A request asked to grow (or shrink below 0) is
// left as it is and status becomes 3.
__global__ __launch_bounds__(kBookThreads) void kv_rollback_kernel(const int32_t* __restrict__ tables,
                                                                   int32_t* __restrict__ lens,
                                                                   int32_t* __restrict__ stack,
                                                                   int32_t* __restrict__ top,
                                                                   const int32_t* __restrict__ keep_lens,
                                                                   const int32_t* __restrict__ num_emitted,
                                                                   int64_t gamma, int64_t R, int64_t bs,
                                                                   int64_t max_blocks, int64_t num_blocks,
                                                                   int32_t* __restrict__ status) {
  __shared__ int64_t lds[kBookThreads / 64];
  const int tid = threadIdx.x;
  const int64_t base = top[0];
  int64_t carry = 0, bad = 0;
  for (int64_t r0 = 0; r0 < R; r0 += kBookThreads) {
    const int64_t r = r0 + tid;
    int64_t len = 0, keep = 0, freed = 0;
    bool ok = false;
    if (r < R) {
      len = lens[r];
      keep = keep_lens ? (int64_t)keep_lens[r] : len - (gamma + 1) + (int64_t)num_emitted[r];
      ok = keep >= 0 && keep <= len;
      bad |= !ok;
      if (ok) freed = nblocks(len, bs) - nblocks(keep, bs);
    }
    int64_t chunk_total;
    const int64_t before = carry + block_exclusive_scan(freed, lds, chunk_total);
    if (r < R && ok) {
      const int64_t have = nblocks(len, bs);
      for (int64_t j = 0; j < freed; ++j) {
        const int64_t slot = base + before + j, logical = have - 1 - j;
        if (slot < num_blocks && logical < max_blocks) stack[slot] = tables[r * max_blocks + logical];
      }
      lens[r] = (int32_t)keep;
    }
    carry += chunk_total;
  }
  int64_t tot_bad;
  block_exclusive_scan(bad, lds, tot_bad);
  if (tid == 0) {
    top[0] = (int32_t)(base + carry < num_blocks ? base + carry : num_blocks);
    status[0] = tot_bad ? 3 : 0;
  }
}

// Contiguous keys and values: out[r][h][t][:] for t < min(lens[r], max_len).
// Grid y runs over (request, head) pairs, grid x over the 16-byte units of
// one pair's max_len rows, so a unit's token and offset come from 32-bit
// arithmetic (shifts when the row and block sizes are powers of two); each
// thread moves two units of K and two of V per trip, with streaming
// (nontemporal) loads and stores: the copy is touched once.
__global__ __launch_bounds__(256) void kv_gather_kernel(const uint8_t* __restrict__ kpool,
                                                        const uint8_t* __restrict__ vpool,
                                                        const int32_t* __restrict__ tables,
                                                        const int32_t* __restrict__ lens, int64_t R, int64_t heads,
                                                        int64_t bs, int64_t row_units, int64_t max_blocks,
                                                        int64_t num_blocks, int64_t max_len, int ru_shift, int bs_shift,
                                                        uint8_t* __restrict__ kout, uint8_t* __restrict__ vout) {
  const int ru = (int)row_units, bsi = (int)bs;
  const int per = (int)(max_len * row_units);  // units of one (request, head) pair
  const int stride = (int)gridDim.x * 256;
  for (int64_t rh = blockIdx.y; rh < R * heads; rh += gridDim.y) {
    const int64_t r = rh / heads, h = rh - r * heads;
    const int len = (int)min((int64_t)lens[r], max_len);
    const int32_t* tab = tables + r * max_blocks;
    const int64_t out0 = rh * (int64_t)per;
    auto src_of = [&](int i, int64_t& src) {  // false where the unit is not written
      const int t = ru_shift >= 0 ? i >> ru_shift : i / ru;
      const int u = i - t * ru;
      if (t >= len) return false;
      const int lb = bs_shift >= 0 ? t >> bs_shift : t / bsi;
      if (lb >= max_blocks) return false;
      const int64_t phys = tab[lb];
      if (phys < 0 || phys >= num_blocks) return false;
      src = ((phys * heads + h) * bs + (t - lb * bsi)) * row_units + u;
      return true;
    };
    for (int i = blockIdx.x * 256 + threadIdx.x; i < per; i += 2 * stride) {
      const int i2 = i + stride;
      int64_t s0 = 0, s1 = 0;
      const bool w0 = src_of(i, s0);
      const bool w1 = i2 < per && src_of(i2, s1);
      u32x4 k0, v0, k1, v1;
      if (w0) {
        k0 = __builtin_nontemporal_load((const u32x4*)kpool + s0);
        v0 = __builtin_nontemporal_load((const u32x4*)vpool + s0);
      }
      if (w1) {
        k1 = __builtin_nontemporal_load((const u32x4*)kpool + s1);
        v1 = __builtin_nontemporal_load((const u32x4*)vpool + s1);
      }
      if (w0) {
        __builtin_nontemporal_store(k0, (u32x4*)kout + out0 + i);
        __builtin_nontemporal_store(v0, (u32x4*)vout + out0 + i);
      }
      if (w1) {
        __builtin_nontemporal_store(k1, (u32x4*)kout + out0 + i2);
        __builtin_nontemporal_store(v1, (u32x4*)vout + out0 + i2);
      }
    }
  }
}

inline unsigned grid_for(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

hipError_t launch_kv_init(int32_t* stack, int32_t* top, int32_t* lens, int64_t R, int64_t num_blocks,
                          hipStream_t stream) {
  hipLaunchKernelGGL(kv_init_kernel, dim3(grid_for(R > num_blocks ? R : num_blocks)), dim3(256), 0, stream, stack, top,
                     lens, R, num_blocks);
  return hipGetLastError();
}

hipError_t launch_kv_append(const KvArgs& a, const void* knew, const void* vnew, int64_t n_new, int32_t* old_lens,
                            hipStream_t stream) {
  hipLaunchKernelGGL(kv_alloc_kernel, dim3(1), dim3(kBookThreads), 0, stream, a.tables, a.lens, a.stack, a.top, a.R,
                     n_new, a.block_size, a.max_blocks, old_lens, a.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = a.heads * a.head_dim * a.elem / 16;
  hipLaunchKernelGGL(kv_scatter_kernel, dim3(grid_for(a.R * n_new * units)), dim3(256), 0, stream, (uint8_t*)a.kpool,
                     (uint8_t*)a.vpool, a.tables, old_lens, (const uint8_t*)knew, (const uint8_t*)vnew, a.R, n_new,
                     a.heads, a.block_size, a.head_dim * a.elem / 16, a.max_blocks, a.num_blocks, a.status);
  return hipGetLastError();
}

hipError_t launch_kv_rollback(const KvArgs& a, const int32_t* keep_lens, const int32_t* num_emitted, int64_t gamma,
                              hipStream_t stream) {
  hipLaunchKernelGGL(kv_rollback_kernel, dim3(1), dim3(kBookThreads), 0, stream, a.tables, a.lens, a.stack, a.top,
                     keep_lens, num_emitted, gamma, a.R, a.block_size, a.max_blocks, a.num_blocks, a.status);
  return hipGetLastError();
}

hipError_t launch_kv_gather(const KvArgs& a, int64_t max_len, void* kout, void* vout, hipStream_t stream) {
  const int64_t units = a.head_dim * a.elem / 16;
  // One pair's units are indexed in 32 bits.
  if (max_len * units > INT32_MAX / 2) return hipErrorInvalidValue;
  auto log2_or_neg = [](int64_t x) { return x > 0 && (x & (x - 1)) == 0 ? __builtin_ctzll((uint64_t)x) : -1; };
  const int64_t pairs = a.R * a.heads, per = max_len * units;
  const int64_t gx = (per + 511) / 512;  // two units per thread
  const dim3 grid((unsigned)(gx < 1 ? 1 : (gx > 4096 ? 4096 : gx)), (unsigned)(pairs < 65535 ? pairs : 65535));
  hipLaunchKernelGGL(kv_gather_kernel, grid, dim3(256), 0, stream, (const uint8_t*)a.kpool, (const uint8_t*)a.vpool,
                     a.tables, a.lens, a.R, a.heads, a.block_size, units, a.max_blocks, a.num_blocks, max_len,
                     log2_or_neg(units), log2_or_neg(a.block_size), (uint8_t*)kout, (uint8_t*)vout);
  return hipGetLastError();
}

}  // namespace specdec
