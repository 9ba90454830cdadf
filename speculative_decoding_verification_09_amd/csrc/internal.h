// Internal interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specdec {

// Y[n, v] = sum_k X[n, k] W[v, k]; X [N, d] bf16; W [V, d] bf16 row-major or
// in the packed tile layout; Y fp32 or bf16.
// The workspace must hold gemm_workspace_bytes(N, d, V, packed) bytes (may be
// null when that is 0).
hipError_t launch_skinny_gemm(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V,
                              bool out_bf16, bool packed, void* workspace, hipStream_t stream);

namespace gemm {
// The sweep kernel (packed W, at most 16 positions, X whole in LDS; ok is
// false when X does not fit).  tickets: 16 bytes of device memory for its tile
// queue (a counter and a launch tag), initialised by the launch itself.
struct SweepPlan {
  bool ok;
  int64_t grid;
};
constexpr size_t kSweepTicketBytes = 256;
SweepPlan plan_sweep(int64_t N, int64_t d, int64_t V, int cus);
hipError_t launch_sweep(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d,
                        int64_t V, bool out_bf16, void* tickets, hipStream_t stream);
}  // namespace gemm
struct FusedStats;
namespace gemm {
// The sweep kernel with the statistics epilogue (fp32 logits).
hipError_t launch_sweep_with_stats(const SweepPlan& p, const uint16_t* X, const uint16_t* Wp, float* Y, int64_t N,
                                   int64_t d, int64_t V, const FusedStats& fs, void* tickets, int64_t* nparts,
                                   hipStream_t stream);
}  // namespace gemm

// Bytes of device workspace the scoring GEMM needs for this shape (0: none).
size_t gemm_workspace_bytes(int64_t N, int64_t d, int64_t V, bool packed);

// Packed tile layout of W [V, d] (d % 32 == 0): ceil(V/16)*16*d elements.
int64_t packed_weight_elems(int64_t V, int64_t d);
hipError_t launch_pack_weights(const uint16_t* W, uint16_t* Wp, int64_t V, int64_t d, hipStream_t stream);

struct RejectArgs {
  const float* target;     // [B, gamma+1, V]
  const float* draft;      // [B, gamma, V] logits or probabilities
  int draft_kind;          // 0 logits, 1 probabilities
  const int32_t* tokens;   // [B, gamma]
  float temperature;       // 0: greedy
  const float* uniforms;   // [B, gamma+1, 2]
  int64_t B, gamma, V;
  int32_t* out_tokens;     // [B, gamma+1]
  int32_t* out_num;        // [B]
  float* out_probs;        // [B, gamma, 2] or null
  void* workspace;
  size_t workspace_bytes;
  int64_t top_k = 0;       // keep the top_k largest logits of a row; <= 0 or >= V: no top-k
  float top_p = 1.0f;      // then the shortest prefix with mass >= top_p; >= 1: no top-p
};

// True when the step warps its rows (T > 0 with an active top-k or top-p).
inline bool warp_active(const RejectArgs& a) {
  return a.temperature > 0.0f && ((a.top_k > 0 && a.top_k < a.V) || a.top_p < 1.0f);
}

size_t reject_workspace_bytes(int64_t B, int64_t gamma, int64_t V);
// Statistics pass over a.target (and draft logits), then the draw or the
// greedy rule; with warping, the per-row cuts are found first.
hipError_t launch_reject_sample(const RejectArgs& a, hipStream_t stream);

// e^x for x <= 0 (the weights of the draw, the masses of the top-p cut). x
// log2(e) is carried as its rounded product h plus a correction l (that
// product's rounding error and the tail of log2(e)), and 2^(h + l) =
// 2^h (1 + l ln 2) up to a relative 2^-34, as |l| < 2^-16 for |x| <= 128. The
// hardware base-2 exponential gives 2^h. x is clamped at -128, where e^x lies
// below the smallest subnormal, so a -inf logit weighs exactly 0.
__device__ __forceinline__ float exp_nonpos(float x) {
  constexpr float kLog2eHi = 1.4426950408889634f;
  constexpr float kLog2eLo = 1.925963e-08f;  // log2(e) minus its float value
  constexpr float kLn2 = 0.6931472f;
  x = fmaxf(x, -128.0f);
  const float h = x * kLog2eHi;
  const float l = fmaf(x, kLog2eLo, fmaf(x, kLog2eHi, -h));
  const float e = __builtin_amdgcn_exp2f(h);
  return fmaf(e, l * kLn2, e);
}

// Order-preserving integer image of an fp32 logit (larger value, larger key;
// -0 and +0 map to one key).  A warped row keeps entry v iff
// key(z_v) > cut_key, or key(z_v) == cut_key and v <= cut_idx: the entries
// ranked by logit, ties by lower index, cut after one of them.
__device__ __forceinline__ uint32_t order_key(float z) {
  uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ bool warp_kept(uint32_t key, int64_t v, uint32_t cut_key, int32_t cut_idx) {
  return key > cut_key || (key == cut_key && v <= (int64_t)cut_idx);
}
// A warp cut (key ck, index ci: entry v with key k kept iff k > ck, or k == ck
// and v <= ci) as a test on values: a non-NaN z is kept iff z > cz, or
// z == cz and v <= the returned index.  Keys order values (-0 and +0 share
// one key and compare equal), so at the key of a float this is the key test;
// keys below that of -inf keep every entry, keys above that of +inf none (a
// NaN cz compares false), and the one key no float has (that -0 would have
// without sharing) keeps exactly the z >= -0.
struct ValueCut {
  float z;
  int32_t idx;
};
__device__ __forceinline__ ValueCut value_cut(uint32_t ck, int32_t ci) {
  if (ck < 0x007fffffu) return {-INFINITY, 0x7fffffff};
  if (ck > 0xff800000u) return {__uint_as_float(0x7fc00000u), -1};
  if (ck == 0x7fffffffu) return {__uint_as_float(0x80000001u), -1};
  return {__uint_as_float((ck & 0x80000000u) ? (ck & 0x7fffffffu) : ~ck), ci};
}
__device__ __forceinline__ bool value_kept(float z, int64_t v, float cz, int32_t ci) {
  return z > cz || (z == cz && v <= (int64_t)ci);
}

// Where the warp cut kernel leaves each warped row's statistics, in the
// layout of the statistics pass: per row, pstride slots of (max of z/T, sum of
// exp(z/T - max)), of which nch are read; the drafted token's logit; and the
// draw kernel's per-sequence counters, zeroed.
struct WarpStats {
  float* cmax;
  double* csum;
  float* zx;
  int64_t pstride, nch;
  const int32_t* tokens;  // [B, gamma]
  int64_t gamma, B;
  uint32_t* done;         // [B]
};
// One workgroup per row: rows [0, n_target) of target, then rows of draft.
// Writes each row's cut and its statistics after warping.
hipError_t launch_warp_cuts(const float* target, const float* draft, int64_t n_target, int64_t n_rows, int64_t V,
                            float inv_t, int64_t top_k, float top_p, uint32_t* cut_key, int32_t* cut_idx,
                            const WarpStats& so, hipStream_t stream);

// Softmax (or argmax) statistics formed by the scoring kernel itself, as an
// epilogue: for every row, one partial per workgroup of that kernel, in the
// reject workspace's partial slots.  Target rows are [0, B*(gamma+1)), draft
// rows B*(gamma+1) + b*gamma + i.
constexpr int64_t kFusedStatsMaxParts = 1024;  // workgroups (partials per row)
constexpr int64_t kFusedStatsMaxRows = 512;   // B*(gamma+1)
struct FusedStats {
  float* cmax;            // [row][pstride]: max of z/T (greedy: max of z)
  double* csum;           // [row][pstride]: sum of exp(z/T - max)
  int32_t* cidx;          // [row][pstride]: lowest index of the max (greedy)
  float* zx;              // [row]: logit of the drafted token
  int64_t pstride;
  const float* draft;     // draft logits [B, gamma, V] to summarise, or null
  const int32_t* tokens;  // [B, gamma]
  int64_t B, gamma;
  float inv_t;            // fl32(1/T); 1 when greedy
  bool greedy;
  uint32_t* done;         // [B]: the draw kernel's per-sequence counters, zeroed by the softmax epilogue (or null)
};
// Points fs at the workspace of a; false when the shape cannot take fused statistics.
bool reject_fused_stats(const RejectArgs& a, FusedStats* fs);
// The stages after the statistics, reading nparts partials per target row and
// nparts_draft per draft row.
hipError_t launch_reject_after_fused(const RejectArgs& a, int64_t nparts, int64_t nparts_draft, hipStream_t stream);
// The draft rows' partials in the fused slot layout, one per 2048-entry chunk
// (their count in *nparts); independent of the scoring kernel.
hipError_t launch_draft_stats(const FusedStats& fs, int64_t n_target, int64_t V, int64_t* nparts, hipStream_t stream);
// Partials per row that launch_gemm_with_stats will produce for this shape
// (0: the shape does not take the statistics epilogue, or, unless required,
// is faster without it).  required: the caller keeps no logits, so the
// epilogue is taken wherever the kernels can form it.
int64_t gemm_stats_parts(int64_t N, int64_t d, int64_t V, int64_t pstride, bool required = false);
// Slots per row of the reject workspace's partials, when its shape can take
// partials from the scoring kernel (B*(gamma+1) rows within the limit); 0
// otherwise.
int64_t reject_fusable_stride(int64_t B, int64_t gamma, int64_t V);
// Device scratch that launch_gemm_with_stats needs for this shape (the packed
// copy of X of the deep kernel, the sweep kernel's tile queue; 0 for the
// panel kernel), 256-byte multiple.
size_t gemm_stats_scratch_bytes(int64_t N, int64_t d, int64_t V);
// The scoring GEMM with the statistics epilogue (packed W, sweep, panel or
// deep kernel without k-groups, at most kFusedStatsMaxParts partials per row);
// the same launch summarises the draft rows.  scratch: at least
// gemm_stats_scratch_bytes, disjoint from the statistics arrays.  Y may be
// null with the argmax epilogue (fs.greedy): the logits are then not stored.
// Returns the partial counts of target and draft rows, or
// hipErrorNotSupported, launching nothing, for shapes it does not take.
hipError_t launch_gemm_with_stats(const uint16_t* X, const uint16_t* Wp, float* Y, int64_t N, int64_t d, int64_t V,
                                  const FusedStats& fs, int64_t* nparts, int64_t* nparts_draft, void* scratch,
                                  hipStream_t stream, bool required = false);
// Name of the kernel that computes the scores of this shape (the one that
// dominates a step's time).
const char* scoring_kernel_name(int64_t N, int64_t d, int64_t V, bool packed);

// Tree verification (greedy), M <= 64 nodes per tree.
struct TreeArgs {
  const float* logits;       // [B, M, V]
  const int32_t* parents;    // [B, M]
  const int32_t* node_tokens;  // [B, M]
  int64_t B, M, V;
  int32_t* out_tokens;       // [B, M]
  int32_t* out_num;          // [B]
  int32_t* out_nodes;        // [B, M]
  void* workspace;
};
size_t tree_workspace_bytes(int64_t B, int64_t M, int64_t V);
hipError_t launch_tree_mask(const int32_t* parents, int64_t B, int64_t M, uint64_t* out_mask, int32_t* out_depth,
                            float* out_additive, hipStream_t stream);
// Points fs at the tree workspace for the scoring kernel's argmax epilogue; false if the shape cannot take it.
bool tree_fused_stats(const TreeArgs& t, FusedStats* fs);
// The greedy tree rule; nparts > 0: argmax partials already in the workspace
// (from the scoring kernel), else a statistics pass over t.logits first.
hipError_t launch_tree_greedy(const TreeArgs& t, int64_t nparts, hipStream_t stream);

// Paged KV cache (see paged_kv.hip).
struct KvArgs {
  void* kpool;           // [num_blocks][heads][block_size][head_dim] elements of elem bytes
  void* vpool;
  int32_t* tables;       // [R][max_blocks]
  int32_t* lens;         // [R]
  int32_t* stack;        // [num_blocks] free blocks
  int32_t* top;          // [1] number of free blocks
  int32_t* status;       // [1]
  int64_t R, num_blocks, heads, block_size, head_dim, elem, max_blocks;
};
hipError_t launch_kv_init(int32_t* stack, int32_t* top, int32_t* lens, int64_t R, int64_t num_blocks,
                          hipStream_t stream);
// old_lens: [R] int32 scratch (the lengths before the append).
hipError_t launch_kv_append(const KvArgs& a, const void* knew, const void* vnew, int64_t n_new, int32_t* old_lens,
                            hipStream_t stream);
hipError_t launch_kv_rollback(const KvArgs& a, const int32_t* keep_lens, const int32_t* num_emitted, int64_t gamma,
                              hipStream_t stream);
hipError_t launch_kv_gather(const KvArgs& a, int64_t max_len, void* kout, void* vout, hipStream_t stream);

}  // namespace specdec
