// Rejection-sampling verification kernels for gfx950.
//
// The rule ("LLM Inference & Speculative Decoding", section 2, acceptance
// rule, residual distribution and bonus token; "Speculative Decoding:
// Mathematical Foundations ...", "The Modified Rejection Sampling Algorithm"
// and "Greedy Decoding Equivalence"; "Speculative decoding." lesson, "Draft,
// then verify" and "The acceptance rule"):
//   row i keeps the drafted x_i iff u_i < min(1, p_i(x_i) / max(q_i(x_i), 1e-12));
//   the step emits x_0 .. x_{k-1} for the first rejected row k and then one
//   token drawn from (p_k - q_k)+ (p_k itself if that has no mass), or, when
//   all gamma are kept, one token drawn from the bonus row p_gamma.
//   Draws are inverse CDF in vocabulary order: the smallest v with
//   u * S < C_v, C the running sum of the (unnormalised) weights, S their total.
//   At T == 0 the rule is greedy: keep x_i iff it is the row's argmax (lowest
//   index on ties); emit the argmax at the first mismatch or as the bonus.
//
// Launches on the caller's stream; kernel boundaries order every step (no
// inter-wave signalling inside a launch, no host synchronisation):
//   1. stats: one wave per (row, 2048-entry vocabulary chunk) of every target
//      row and, for draft logits at T > 0, every draft row.  T > 0: chunk max
//      m_c of a = z * (1/T) and s_c = sum exp(a - m_c) (fp32 terms summed in
//      fp64); the wave whose chunk holds the row's drafted token also records
//      that logit.  T == 0: chunk max value and its lowest index.
//   2. draw sums (T > 0): workgroups of 16 waves over consecutive 1024-entry
//      chunks of one sequence.  The waves first merge the sequence's rows in
//      parallel into LDS (M = max m_c, Z = sum s_c exp(m_c - M) in fp64, and
//      p_i(x_i) or q_i(x_i) of the drafted token, fp64 rounded once to fp32);
//      then lane i takes row i, every accept test is taken at once and the
//      first rejection k found with a ballot, and each wave sums its chunk of
//      the weights of row k: r_v = max(0, p_v - q_v) and p_v (fp32 values,
//      fp64 sums).  The chunk-0 wave writes the kept prefix, the count, the
//      probabilities and a per-sequence draw descriptor.
//   3. select (T > 0): one wave per sequence finds the chunk holding u * S with
//      an fp64 prefix sum over the chunk totals, rescans that chunk with an
//      fp64 running sum in vocabulary order and writes the token.
//   2'. greedy decide (T == 0): one wave per sequence merges the argmax
//      partials of its rows (lane i <-> row i) and applies the greedy rule.
// p, q, (p - q)+ and p/q are fp32 values, as the first source asks for T > 0
// (section 4, failure mode 1); normalisers and running sums are fp64.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kStatChunk = 2048;   // vocabulary entries per statistics work item (one wave)
constexpr int kDrawChunk = 1024;   // vocabulary entries per draw work item (one wave)
constexpr int kGreedyWaves = 8;    // waves of the greedy rule's workgroup (one per sequence)
constexpr int kWavesPerBlock = 4;
constexpr float kQFloor = 1e-12f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kMaxFusedParts = kFusedStatsMaxParts;
constexpr int64_t kMaxFusedRows = kFusedStatsMaxRows;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int64_t stat_chunks(int64_t V) { return (V + kStatChunk - 1) / kStatChunk; }
__host__ __device__ inline int64_t draw_chunks(int64_t V) { return (V + kDrawChunk - 1) / kDrawChunk; }
__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Where the step of one sequence ends and how to weigh that row.
struct DrawDesc {
  int32_t k;       // row index (gamma for the bonus row)
  float mp, ip;    // target row: max of a and 1/Z
  float mq, iq;    // draft row (draft logits only)
  float u;         // the uniform that drives the draw
  int32_t xk;      // drafted token of row k (one-hot drafts), -1 on the bonus row
  float pz, qz;    // warp cuts of the target and draft rows k as values (see value_cut)
  int32_t pi, qi;
  float pad;
};

// Workspace layout, every array 16-byte aligned.  Each row has pstride slots
// for softmax partials: one per statistics chunk, or, when the scoring kernel
// forms them itself (at most kMaxFusedParts workgroups, B*(gamma+1) <= kMaxFusedRows), one
// per workgroup of that kernel.
struct Layout {
  size_t off_cmax, off_csum, off_cidx;      // per (row, partial slot)
  size_t off_zx;                            // per row
  size_t off_desc;                          // per sequence
  size_t off_sres, off_sp;                  // per (sequence, draw chunk)
  size_t off_wkey, off_widx;                // per row: warp cut
  size_t off_done;                          // per sequence: draw workgroups finished
  int64_t pstride;
  size_t total;
};

__host__ __device__ inline int64_t partial_stride(int64_t B, int64_t gamma, int64_t V) {
  const int64_t sc = stat_chunks(V);
  const bool fusable = B * (gamma + 1) <= kMaxFusedRows;
  return fusable && sc < kMaxFusedParts ? kMaxFusedParts : sc;
}

__host__ __device__ inline Layout make_layout(int64_t B, int64_t gamma, int64_t V) {
  Layout L;
  const size_t rows = (size_t)(B * (2 * gamma + 1));
  L.pstride = partial_stride(B, gamma, V);
  const size_t rc = rows * (size_t)L.pstride;
  const size_t ndc = (size_t)(B * draw_chunks(V));
  size_t o = 0;
  L.off_cmax = o; o = align16(o + rc * sizeof(float));
  L.off_csum = o; o = align16(o + rc * sizeof(double));
  L.off_cidx = o; o = align16(o + rc * sizeof(int32_t));
  L.off_zx = o;   o = align16(o + rows * sizeof(float));
  L.off_desc = o; o = align16(o + (size_t)B * sizeof(DrawDesc));
  L.off_sres = o; o = align16(o + ndc * sizeof(double));
  L.off_sp = o;   o = align16(o + ndc * sizeof(double));
  L.off_wkey = o; o = align16(o + rows * sizeof(uint32_t));
  L.off_widx = o; o = align16(o + rows * sizeof(int32_t));
  L.off_done = o; o = align16(o + (size_t)B * sizeof(uint32_t));
  L.total = o;
  return L;
}

struct Ws {
  float* cmax;     // per (row, slot): max of a = z / T (greedy: max of z)
  double* csum;    // per (row, slot): sum exp(a - slot max)
  int32_t* cidx;   // per (row, slot): lowest index of the max (greedy)
  float* zx;       // per drafted row: logit of the drafted token
  DrawDesc* desc;  // per sequence
  double* sres;    // per (sequence, draw chunk): sum of the residual weights
  double* sp;      // per (sequence, draw chunk): sum of p
  uint32_t* wkey;  // per row: warp cut key (read only by the warped kernels)
  int32_t* widx;   // per row: warp cut index
  uint32_t* done;  // per sequence: draw workgroups finished (zeroed by the statistics pass)
  int64_t pstride; // slots per row
  int64_t nparts;  // slots in use per target row
  int64_t nparts_d;  // slots in use per draft row
};

inline Ws bind(void* base, const Layout& L, int64_t nparts, int64_t nparts_d = -1) {
  char* b = (char*)base;
  return Ws{(float*)(b + L.off_cmax), (double*)(b + L.off_csum), (int32_t*)(b + L.off_cidx), (float*)(b + L.off_zx),
            (DrawDesc*)(b + L.off_desc), (double*)(b + L.off_sres), (double*)(b + L.off_sp),
            (uint32_t*)(b + L.off_wkey), (int32_t*)(b + L.off_widx), (uint32_t*)(b + L.off_done), L.pstride,
            nparts, nparts_d < 0 ? nparts : nparts_d};
}

// ---------------------------------------------------------------------------
// Wave-wide helpers (64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ void wave_argmax(float& val, int& idx) {  // larger wins, ties to the lower index
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(val, o);
    const int oi = __shfl_xor(idx, o);
    if (ov > val || (ov == val && oi < idx)) {
      val = ov;
      idx = oi;
    }
  }
}
__device__ __forceinline__ double wave_inclusive_scan(double x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int clamp_token(int32_t t, int64_t V) { return t < 0 ? 0 : (t >= V ? (int)(V - 1) : t); }

// ---------------------------------------------------------------------------
// 1. Chunk statistics.  Target rows are [0, B*(gamma+1)) (row b*(gamma+1) + i),
//    draft rows [B*(gamma+1), B*(2*gamma+1)) (row B*(gamma+1) + b*gamma + i).
//    Lane l of a wave takes the 32 entries 256*j + 4*l + e (j < 8, e < 4) of
//    its 2048-entry chunk (1 KB per load instruction).  Rows [row0, n_rows)
//    are summarised.  The first n_done threads also zero the draw kernel's
//    per-sequence counters.  (Warped rows are summarised by the warp cut
//    kernel itself.)
template <bool VEC, bool GREEDY>
__global__ __launch_bounds__(kWavesPerBlock * 64) void stats_kernel(const float* __restrict__ target,
                                                                     const float* __restrict__ draft,
                                                                     const int32_t* __restrict__ tokens,
                                                                     int64_t n_target_rows, int64_t row0,
                                                                     int64_t n_rows, int64_t gamma, int64_t V,
                                                                     float inv_t, Ws ws, int64_t n_done) {
  constexpr int PL = kStatChunk / 64;
  const int lane = threadIdx.x & 63;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < n_done) ws.done[gid] = 0u;
  const int64_t nch = stat_chunks(V);
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= (n_rows - row0) * nch) return;
  const int64_t r = row0 + item / nch, c = item - (r - row0) * nch;
  const bool is_target = r < n_target_rows;
  const float* row = is_target ? target + (size_t)r * V : draft + (size_t)(r - n_target_rows) * V;
  const int64_t c0 = c * kStatChunk;
  float x[PL];
#pragma unroll
  for (int j = 0; j < PL / 4; ++j) {
    const int64_t v = c0 + 256 * j + 4 * lane;
    if (VEC && v + 3 < V) {
      const f32x4 t = __builtin_nontemporal_load((const f32x4*)(row + v));
      x[4 * j + 0] = t[0];
      x[4 * j + 1] = t[1];
      x[4 * j + 2] = t[2];
      x[4 * j + 3] = t[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = (v + e < V) ? row[v + e] : -INFINITY;
    }
  }
  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < PL; ++e) {
      const int64_t idx = c0 + 256 * (e >> 2) + 4 * lane + (e & 3);
      if (idx < V && (x[e] > bv || (x[e] == bv && (int)idx < bi))) {
        bv = x[e];
        bi = (int)idx;
      }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
      ws.cmax[r * ws.pstride + c] = bv;
      ws.cidx[r * ws.pstride + c] = bi;
    }
    return;
  }
  // The drafted token of this row, if it falls in this chunk.
  const int64_t g1 = gamma + 1;
  const int64_t b = is_target ? r / g1 : (r - n_target_rows) / gamma;
  const int64_t i = is_target ? r - b * g1 : (r - n_target_rows) - b * gamma;
  if (i < gamma && lane == 0) {
    const int xt = clamp_token(tokens[b * gamma + i], V);
    if (xt >= c0 && xt < c0 + kStatChunk) {
      ws.zx[r] = row[xt];
    }
  }
  // The chunk max of a = z * fl32(1/T) is fl32(max z * fl32(1/T)) (the product
  // is monotonic in z).  Each term exp(a - max) is formed as 2^(z * c1 - c2)
  // with c1 = fl32(1/T) * log2(e), c2 = max * log2(e): one FMA into the
  // hardware base-2 exponential, its argument rounded about as much as
  // fl32(z / T) - max is.  Four fp32 terms are added before each fp64 add.
  float zm = -INFINITY;
#pragma unroll
  for (int e = 0; e < PL; ++e) zm = fmaxf(zm, x[e]);
  const float mx = wave_max(zm) * inv_t;
  double sum = 0.0;
  if (mx > -INFINITY) {
    const float c1 = inv_t * kLog2e, c2 = mx * kLog2e;
#pragma unroll
    for (int e = 0; e < PL; e += 4) {
      const float s4 = (__builtin_amdgcn_exp2f(fmaf(x[e], c1, -c2)) + __builtin_amdgcn_exp2f(fmaf(x[e + 1], c1, -c2))) +
                       (__builtin_amdgcn_exp2f(fmaf(x[e + 2], c1, -c2)) + __builtin_amdgcn_exp2f(fmaf(x[e + 3], c1, -c2)));
      sum += (double)s4;
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) {
    ws.cmax[r * ws.pstride + c] = mx;
    ws.csum[r * ws.pstride + c] = sum;
  }
}

// Merges the partials of row r with one wave: M = max m_c, Z = sum s_c
// exp(m_c - M) (fp64 sum; each rescale factor is the hardware base-2
// exponential of fp32 (m_c - M) * log2(e), relative error about 1e-7 where a
// partial carries weight), and the probability of the drafted token
// exp(a_x - M)/Z (fp64, rounded once to fp32; 0 for rows without a drafted
// token).  Partials are read 256 at a time, all loads of a batch issued before
// any reduction.
__device__ __forceinline__ void merge_row(const Ws& ws, int64_t r, bool drafted, int64_t nch, float inv_t, int lane,
                                          double& M_out, double& Z_out, float& px_out) {
  constexpr int kPer = 4;  // partials per lane and batch
  const size_t base = (size_t)r * ws.pstride;
  const float zx = drafted ? ws.zx[r] : 0.0f;  // loaded with the partials
  float M = -INFINITY;
  double z = 0.0;
  for (int64_t c0 = 0; c0 < nch; c0 += 64 * kPer) {
    float cm[kPer];
    double cs[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t c = c0 + 64 * j + lane;
      cm[j] = c < nch ? ws.cmax[base + c] : -INFINITY;
      cs[j] = c < nch ? ws.csum[base + c] : 0.0;
    }
    float bm = cm[0];
#pragma unroll
    for (int j = 1; j < kPer; ++j) bm = fmaxf(bm, cm[j]);
    bm = wave_max(bm);
    const float Mn = fmaxf(M, bm);
    if (z > 0.0) z *= exp((double)M - (double)Mn);  // wave-uniform: every lane holds the same M
    M = Mn;
    double zb = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (cs[j] > 0.0) zb += cs[j] * (double)__builtin_amdgcn_exp2f((cm[j] - M) * kLog2e);
    z += wave_sum(zb);
  }
  M_out = (double)M;
  Z_out = z;
  px_out = drafted ? (float)(exp((double)(zx * inv_t) - (double)M) / z) : 0.0f;
}

// Weights of the draw at entry v: p_v and r_v = max(0, p_v - q_v), fp32.
// q is read (draft logits or probabilities), or, for a one-hot draft, 1 at the
// drafted token and 0 elsewhere.
struct DrawRow {
  const float* zp;  // target logits of the row
  const float* zq;  // draft logits or probabilities of the row (null on the bonus row and for one-hot drafts)
  float mp, ip, mq, iq, inv_t;
  int kind;         // draft kind: 0 logits, 1 probabilities, 2 one-hot
  bool has_q;       // the step ends on a drafted row (a residual), not on the bonus row
  int xk;           // the drafted token of that row (one-hot drafts)
  float pz, qz;     // warp cuts of the two rows as values (WARP only), see value_cut
  int32_t pi, qi;
};

// WARP: p_v (and q_v of draft logits) is 0 where the row's warp cut drops v.
template <bool WARP>
__device__ __forceinline__ void weights(const DrawRow& R, int64_t v, float zp, float zq, float& p, float& r) {
  p = exp_nonpos(zp * R.inv_t - R.mp) * R.ip;
  if (WARP && !value_kept(zp, v, R.pz, R.pi)) p = 0.0f;
  if (R.has_q) {
    float q = R.kind == 2 ? (v == R.xk ? 1.0f : 0.0f) : (R.kind == 1 ? zq : exp_nonpos(zq * R.inv_t - R.mq) * R.iq);
    if (WARP && R.kind == 0 && !value_kept(zq, v, R.qz, R.qi)) q = 0.0f;
    const float dlt = p - q;
    r = dlt > 0.0f ? dlt : 0.0f;
  } else {
    r = p;
  }
}

template <bool WARP>
__device__ __forceinline__ DrawRow make_row(const float* __restrict__ target, const float* __restrict__ draft,
                                            int draft_kind, int64_t B, int64_t b, int64_t gamma, int64_t V,
                                            const DrawDesc& D, float inv_t, const Ws& ws) {
  DrawRow R;
  R.zp = target + (size_t)(b * (gamma + 1) + D.k) * V;
  R.has_q = D.k < gamma;
  R.zq = R.has_q && draft_kind != 2 ? draft + (size_t)(b * gamma + D.k) * V : nullptr;
  R.mp = D.mp;
  R.ip = D.ip;
  R.mq = D.mq;
  R.iq = D.iq;
  R.inv_t = inv_t;
  R.kind = draft_kind;
  R.xk = D.xk;
  R.pz = WARP ? D.pz : -INFINITY;
  R.pi = WARP ? D.pi : 0x7fffffff;
  R.qz = WARP ? D.qz : -INFINITY;
  R.qi = WARP ? D.qi : 0x7fffffff;
  return R;
}

// Loads lane's 16 entries of a 1024-entry chunk, coalesced (entry 4j + e at
// chunk offset 256j + 4*lane + e).  Entries past V read as fill.
template <bool VEC>
__device__ __forceinline__ void load_chunk16(const float* __restrict__ row, int64_t V, int64_t c0, int lane, float fill,
                                             float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t v = c0 + 256 * j + 4 * lane;
    if (VEC && v + 3 < V) {
      const f32x4 t = *(const f32x4*)(row + v);
      x[4 * j + 0] = t[0];
      x[4 * j + 1] = t[1];
      x[4 * j + 2] = t[2];
      x[4 * j + 3] = t[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = (v + e < V) ? row[v + e] : fill;
    }
  }
}

// 3. Select (T > 0), by one wave of the last draw workgroup of sequence b to
//    finish: the residual's weights, or p when the residual has no mass or the
//    step ends on the bonus row.
template <bool VEC, bool WARP>
__device__ void select_seq(const float* __restrict__ target, const float* __restrict__ draft, int draft_kind,
                           int64_t B, int64_t b, int64_t gamma, int64_t V, float inv_t,
                           int32_t* __restrict__ out_tokens, const Ws& ws, const DrawDesc& D, int lane) {
  const int64_t ndc = draw_chunks(V);
  const int64_t g1 = gamma + 1;
  // The first 64*K chunk totals of both weights (all of them up to V = 262144)
  // in one round of loads, kept in registers for the search below.
  constexpr int K = 4;
  const double* pr = ws.sres + b * ndc;
  const double* pp = ws.sp + b * ndc;
  double cr[K], cp[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t c = 64 * k + lane;
    cr[k] = c < ndc ? pr[c] : 0.0;
    cp[k] = c < ndc ? pp[c] : 0.0;
  }
  const DrawRow R = make_row<WARP>(target, draft, draft_kind, B, b, gamma, V, D, inv_t, ws);
  double lr = 0.0, lp = 0.0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    lr += cr[k];
    lp += cp[k];
  }
  for (int64_t j0 = 64 * K; j0 < ndc; j0 += 64) {  // longer vocabularies
    lr += j0 + lane < ndc ? pr[j0 + lane] : 0.0;
    lp += j0 + lane < ndc ? pp[j0 + lane] : 0.0;
  }
  double tot = R.has_q ? wave_sum(lr) : 0.0;
  const bool use_p = !(tot > 0.0);
  if (use_p) tot = wave_sum(lp);
  const double* part = use_p ? pp : pr;
  const double t = (double)D.u * tot;
  // First chunk whose running total passes t (or, if rounding leaves none,
  // the last chunk with mass), 64 chunks at a time in vocabulary order.
  int64_t cs = -1, clast = 0;
  double before = 0.0, run = 0.0;
  for (int64_t j0 = 0; j0 < ndc && cs < 0; j0 += 64) {
    double pj = 0.0;
    if (j0 < 64 * K) {  // from registers, by static indices only
      const int k = (int)(j0 >> 6);
#pragma unroll
      for (int q = 0; q < K; ++q)
        if (q == k) pj = use_p ? cp[q] : cr[q];
    } else {
      pj = j0 + lane < ndc ? part[j0 + lane] : 0.0;
    }
    const double incl = run + wave_inclusive_scan(pj, lane);
    const uint64_t hit = ballot(j0 + lane < ndc && t < incl);
    const uint64_t pos = ballot(j0 + lane < ndc && pj > 0.0);
    if (pos) clast = j0 + 63 - __builtin_clzll(pos);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      cs = j0 + l;
      before = __shfl(incl - pj, l);
    }
    run = __shfl(incl, 63);
  }
  if (cs < 0) {
    cs = clast;
    before = run - part[clast];
  }
  // Rescan: lane l takes the 16 consecutive entries starting at cs*1024 + 16*l.
  const int64_t s0 = cs * kDrawChunk + 16 * (int64_t)lane;
  float w[16];
  double lsum = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t v = s0 + 4 * j;
    float ap[4], aq[4];
    if (VEC && v + 3 < V) {
      const f32x4 a = *(const f32x4*)(R.zp + v);
      ap[0] = a[0]; ap[1] = a[1]; ap[2] = a[2]; ap[3] = a[3];
      if (R.zq) {
        const f32x4 bq = *(const f32x4*)(R.zq + v);
        aq[0] = bq[0]; aq[1] = bq[1]; aq[2] = bq[2]; aq[3] = bq[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ap[e] = v + e < V ? R.zp[v + e] : -INFINITY;
        if (R.zq) aq[e] = v + e < V ? R.zq[v + e] : (R.kind == 1 ? 0.0f : -INFINITY);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float p, r;
      weights<WARP>(R, v + e, ap[e], R.zq ? aq[e] : 0.0f, p, r);
      w[4 * j + e] = use_p ? p : r;
      lsum += (double)w[4 * j + e];
    }
  }
  const double incl = wave_inclusive_scan(lsum, lane);
  double C = before + (incl - lsum);
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    C += (double)w[e];
    if (w[e] > 0.0f) {
      lastpos = (int)(s0 + e);
      if (hit < 0 && t < C) hit = (int)(s0 + e);
    }
  }
  const uint64_t hits = ballot(hit >= 0);
  lastpos = wave_max_i(lastpos);
  int tok = hits ? __shfl(hit, __builtin_ctzll(hits)) : lastpos;
  if (tok < 0 || tok >= V) tok = 0;  // no positive weight anywhere (non-finite inputs)
  if (lane == 0) out_tokens[b * g1 + D.k] = tok;
}

// 2. Draw sums (T > 0).  A workgroup of WB waves takes WB consecutive chunks of
//    one sequence.  Its waves first merge the sequence's rows in parallel (one
//    row per wave at a time) into LDS; after one barrier every wave reads the
//    statistics of all rows from LDS, lane i <-> row i.  Each workgroup then
//    counts itself done on the sequence's counter (a device-scope atomic with
//    release order, so its chunk totals are visible first); the last of them
//    acquires and runs the select (3) with one wave.  No workgroup waits for
//    another.
constexpr int kMaxRows = 2 * 63 + 1;
template <int WB, bool VEC, bool WARP>
__global__ __launch_bounds__(WB * 64) void draw_sum_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int draft_kind,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int64_t B, int64_t gamma, int64_t V,
    float inv_t, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num, float* __restrict__ out_probs,
    Ws ws) {
  __shared__ double sh_m[kMaxRows], sh_z[kMaxRows];
  __shared__ float sh_px[kMaxRows];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t ndc = draw_chunks(V);
  const int64_t gps = (ndc + WB - 1) / WB;  // workgroups per sequence
  const int64_t b = blockIdx.x / gps;
  const int64_t c = (blockIdx.x - b * gps) * WB + wv;
  const int64_t g1 = gamma + 1;
  const bool q_probs = draft_kind == 1;
  const bool q_onehot = draft_kind == 2;
  const int64_t nch = ws.nparts;
  // Per-row inputs that do not depend on the statistics, loaded first (lane i <-> row i).
  const bool has_row = lane < g1;
  const bool drafted = lane < gamma;
  const float u_acc = drafted ? uniforms[(b * g1 + lane) * 2 + 0] : 0.0f;
  const float u_smp = has_row ? uniforms[(b * g1 + lane) * 2 + 1] : 0.0f;
  const int xi = drafted ? clamp_token(tokens[b * gamma + lane], V) : 0;
  const float q_given = drafted && q_probs ? draft[(size_t)(b * gamma + lane) * V + xi] : (q_onehot ? 1.0f : 0.0f);
  // The warp cuts of the rows (lane i <-> target row i and draft row i), loaded now so that no load waits once
  // the row where the step ends is known.
  uint32_t ck_t = 0u, ck_d = 0u;
  int32_t ci_t = 0x7fffffff, ci_d = 0x7fffffff;
  if (WARP && has_row) {
    ck_t = ws.wkey[b * g1 + lane];
    ci_t = ws.widx[b * g1 + lane];
  }
  if (WARP && drafted && draft_kind == 0) {
    ck_d = ws.wkey[B * g1 + b * gamma + lane];
    ci_d = ws.widx[B * g1 + b * gamma + lane];
  }
  // Rows of the sequence: j < g1 target row j, then draft row j - g1 (draft logits).
  const int nrows = (int)(draft_kind != 0 ? g1 : g1 + gamma);
  for (int j = wv; j < nrows; j += WB) {
    const int64_t r = j < g1 ? b * g1 + j : B * g1 + b * gamma + (j - g1);
    const bool row_drafted = j < g1 ? j < gamma : true;
    double M, Z;
    float px;
    merge_row(ws, r, row_drafted, j < g1 ? nch : ws.nparts_d, inv_t, lane, M, Z, px);
    if (lane == 0) {
      sh_m[j] = M;
      sh_z[j] = Z;
      sh_px[j] = px;
    }
  }
  __syncthreads();
  const bool active = c < ndc;  // waves past the last chunk only take part in the barriers
  const int64_t item = b * ndc + c;
  const double rmt = has_row ? sh_m[lane] : 0.0, rzt = has_row ? sh_z[lane] : 1.0;
  const float p_x = drafted ? sh_px[lane] : 0.0f;
  const bool ql = drafted && draft_kind == 0;
  const double rmq = ql ? sh_m[g1 + lane] : 0.0, rzq = ql ? sh_z[g1 + lane] : 1.0;
  const float q_x = ql ? sh_px[g1 + lane] : q_given;

  bool reject = false;
  if (drafted) {
    const float ratio = p_x / (q_x > kQFloor ? q_x : kQFloor);
    const float thr = ratio < 1.0f ? ratio : 1.0f;
    reject = !(u_acc < thr);
  }
  const uint64_t rej = ballot(reject);
  const int k = rej ? (int)__builtin_ctzll(rej) : (int)gamma;
  DrawDesc D;
  D.k = k;
  D.mp = (float)__shfl(rmt, k);
  D.ip = (float)(1.0 / __shfl(rzt, k));
  const int kq = k < gamma ? k : 0;
  D.mq = (float)__shfl(rmq, kq);
  D.iq = (float)(1.0 / __shfl(rzq, kq));
  D.u = __shfl(u_smp, k);
  D.xk = k < gamma ? __shfl(xi, k) : -1;
  D.pz = D.qz = -INFINITY;
  D.pi = D.qi = 0x7fffffff;
  if (WARP) {
    const ValueCut cp = value_cut((uint32_t)__shfl((int)ck_t, k), __shfl(ci_t, k));
    D.pz = cp.z;
    D.pi = cp.idx;
    if (k < gamma && draft_kind == 0) {
      const ValueCut cq = value_cut((uint32_t)__shfl((int)ck_d, k), __shfl(ci_d, k));
      D.qz = cq.z;
      D.qi = cq.idx;
    }
  }
  D.pad = 0.0f;

  if (c == 0) {
    if (has_row && lane != k) out_tokens[b * g1 + lane] = lane < k ? xi : -1;
    if (drafted && out_probs) {
      out_probs[(b * gamma + lane) * 2 + 0] = p_x;
      out_probs[(b * gamma + lane) * 2 + 1] = q_x;
    }
    if (lane == 0) {
      out_num[b] = k + 1;
      ws.desc[b] = D;
    }
  }
  const DrawRow R = make_row<WARP>(target, draft, draft_kind, B, b, gamma, V, D, inv_t, ws);
  if (active) {
    const int64_t c0 = c * kDrawChunk;
    float zp[16], zq[16];
    load_chunk16<VEC>(R.zp, V, c0, lane, -INFINITY, zp);
    if (R.zq) load_chunk16<VEC>(R.zq, V, c0, lane, q_probs ? 0.0f : -INFINITY, zq);
    double sr = 0.0, sp = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float p, r;
      weights<WARP>(R, c0 + 256 * (e >> 2) + 4 * lane + (e & 3), zp[e], R.zq ? zq[e] : 0.0f, p, r);
      sr += (double)r;
      sp += (double)p;
    }
    sr = wave_sum(sr);
    sp = wave_sum(sp);
    if (lane == 0) {
      ws.sres[item] = sr;
      ws.sp[item] = sp;
    }
  }
  __shared__ int sh_last;
  __syncthreads();  // every wave's chunk totals are written
  if (threadIdx.x == 0)  // counted with release order: the totals are visible before the count
    sh_last = __hip_atomic_fetch_add(&ws.done[b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(gps - 1);
  __syncthreads();
  if (sh_last && wv == 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other workgroups' totals
    select_seq<VEC, WARP>(target, draft, draft_kind, B, b, gamma, V, inv_t, out_tokens, ws, D, lane);
  }
}

// 2''. Small vocabularies (V <= kSmallV, T > 0, no warping): the whole rule
//     for one sequence in one wave, for batches of many short rows (such as
//     many trials over a few tokens), where a workgroup per sequence and
//     per-chunk partials in the workspace would leave the GPU mostly idle.
//     The arithmetic is that of kernels 1-3 with one statistics chunk and one
//     draw chunk per row, so both paths give the same bits: lane l holds
//     entries 4l .. 4l+3 of a row (row max and sum of the four fp32 terms, as
//     in the statistics kernel; weights and their totals, as in the draw
//     kernel), and the final rescan takes 16 consecutive entries per lane, as
//     in the select.  Rows are loaded four at a time.
constexpr int kSmallV = 256;
template <bool VEC>
__device__ __forceinline__ void load4(const float* __restrict__ row, int64_t V, int lane, float fill, float (&x)[4]) {
  const int64_t v = 4 * (int64_t)lane;
  if (VEC && v + 3 < V) {
    const f32x4 t = *(const f32x4*)(row + v);
    x[0] = t[0];
    x[1] = t[1];
    x[2] = t[2];
    x[3] = t[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v + e < V ? row[v + e] : fill;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kWavesPerBlock * 64) void small_rule_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int draft_kind,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int64_t B, int64_t gamma, int64_t V,
    float inv_t, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num, float* __restrict__ out_probs) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (b >= B) return;  // whole waves; no barriers below
  const int64_t g1 = gamma + 1;
  const bool q_logits = draft_kind == 0;
  const bool has_row = lane < g1, drafted = lane < gamma;
  const float u_acc = drafted ? uniforms[(b * g1 + lane) * 2 + 0] : 0.0f;
  const float u_smp = has_row ? uniforms[(b * g1 + lane) * 2 + 1] : 0.0f;
  const int xi = drafted ? clamp_token(tokens[b * gamma + lane], V) : 0;
  const float q_given = drafted && draft_kind == 1 ? draft[(size_t)(b * gamma + lane) * V + xi]
                                                  : (draft_kind == 2 ? 1.0f : 0.0f);
  // Row j < g1: target row j; g1 <= j < g1 + gamma: draft row j - g1 (draft logits).  Lane i keeps the
  // statistics of target row i (and draft row i): the max of a, Z and the drafted token's probability.
  const int nrows = (int)(q_logits ? g1 + gamma : g1);
  float mt = 0.0f, mq = 0.0f, px = 0.0f, qx = q_given;
  double zt = 1.0, zq = 1.0;
  const float c1 = inv_t * kLog2e;
  for (int j0 = 0; j0 < nrows; j0 += 4) {
    float x[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // rows past the last read the last one again (never used)
      const int j = min(j0 + q, nrows - 1);
      const float* row = j < g1 ? target + (size_t)(b * g1 + j) * V : draft + (size_t)(b * gamma + (j - g1)) * V;
      load4<VEC>(row, V, lane, -INFINITY, x[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q;
      if (j >= nrows) break;
      const int i = j < g1 ? j : j - (int)g1;  // position of the row
      const float mx = wave_max(fmaxf(fmaxf(x[q][0], x[q][1]), fmaxf(x[q][2], x[q][3]))) * inv_t;
      double s = 0.0;
      if (mx > -INFINITY) {
        const float c2 = mx * kLog2e;
        const float s4 = (__builtin_amdgcn_exp2f(fmaf(x[q][0], c1, -c2)) + __builtin_amdgcn_exp2f(fmaf(x[q][1], c1, -c2))) +
                         (__builtin_amdgcn_exp2f(fmaf(x[q][2], c1, -c2)) + __builtin_amdgcn_exp2f(fmaf(x[q][3], c1, -c2)));
        s = (double)s4;
      }
      const double Z = wave_sum(s);
      // The drafted token's logit, from the lane that holds it.
      const int xr = i < gamma ? __shfl(xi, i) : 0;
      float zx = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) zx = (xr & 3) == e ? x[q][e] : zx;
      zx = __shfl(zx, xr >> 2);
      const float pr = i < gamma ? (float)(exp((double)(zx * inv_t) - (double)mx) / Z) : 0.0f;
      if (lane == i) {
        if (j < g1) {
          mt = mx;
          zt = Z;
          px = pr;
        } else {
          mq = mx;
          zq = Z;
          qx = pr;
        }
      }
    }
  }
  bool reject = false;
  if (drafted) {
    const float ratio = px / (qx > kQFloor ? qx : kQFloor);
    const float thr = ratio < 1.0f ? ratio : 1.0f;
    reject = !(u_acc < thr);
  }
  const uint64_t rej = ballot(reject);
  const int k = rej ? (int)__builtin_ctzll(rej) : (int)gamma;
  if (has_row && lane != k) out_tokens[b * g1 + lane] = lane < k ? xi : -1;
  if (drafted && out_probs) {
    out_probs[(b * gamma + lane) * 2 + 0] = px;
    out_probs[(b * gamma + lane) * 2 + 1] = qx;
  }
  if (lane == 0) out_num[b] = k + 1;
  // The draw at row k, with the draw kernel's weights.
  DrawDesc D;
  D.k = k;
  D.mp = __shfl(mt, k);
  D.ip = (float)(1.0 / __shfl(zt, k));
  const int kq = k < gamma ? k : 0;
  D.mq = __shfl(mq, kq);
  D.iq = (float)(1.0 / __shfl(zq, kq));
  D.u = __shfl(u_smp, k);
  D.xk = k < gamma ? __shfl(xi, k) : -1;
  D.pz = D.qz = -INFINITY;
  D.pi = D.qi = 0x7fffffff;
  D.pad = 0.0f;
  DrawRow R;
  R.zp = target + (size_t)(b * g1 + k) * V;
  R.has_q = k < gamma;
  R.zq = R.has_q && draft_kind != 2 ? draft + (size_t)(b * gamma + k) * V : nullptr;
  R.mp = D.mp;
  R.ip = D.ip;
  R.mq = D.mq;
  R.iq = D.iq;
  R.inv_t = inv_t;
  R.kind = draft_kind;
  R.xk = D.xk;
  R.pz = R.qz = -INFINITY;
  R.pi = R.qi = 0x7fffffff;
  float zp4[4], zq4[4];
  load4<VEC>(R.zp, V, lane, -INFINITY, zp4);
  if (R.zq) load4<VEC>(R.zq, V, lane, draft_kind == 1 ? 0.0f : -INFINITY, zq4);
  double sr = 0.0, sp = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float p, r;
    weights<false>(R, 4 * lane + e, zp4[e], R.zq ? zq4[e] : 0.0f, p, r);
    sr += (double)r;
    sp += (double)p;
  }
  double tot = R.has_q ? wave_sum(sr) : 0.0;
  const bool use_p = !(tot > 0.0);
  if (use_p) tot = wave_sum(sp);
  const double t = (double)D.u * tot;
  // Rescan: lane l takes the 16 consecutive entries starting at 16l (one chunk, nothing before it).
  const int64_t s0 = 16 * (int64_t)lane;
  float w[16];
  double lsum = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t v = s0 + 4 * j;
    float ap[4], aq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ap[e] = v + e < V ? R.zp[v + e] : -INFINITY;
      if (R.zq) aq[e] = v + e < V ? R.zq[v + e] : (R.kind == 1 ? 0.0f : -INFINITY);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float p, r;
      weights<false>(R, v + e, ap[e], R.zq ? aq[e] : 0.0f, p, r);
      w[4 * j + e] = use_p ? p : r;
      lsum += (double)w[4 * j + e];
    }
  }
  const double incl = wave_inclusive_scan(lsum, lane);
  double C = incl - lsum;
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    C += (double)w[e];
    if (w[e] > 0.0f) {
      lastpos = (int)(s0 + e);
      if (hit < 0 && t < C) hit = (int)(s0 + e);
    }
  }
  const uint64_t hits = ballot(hit >= 0);
  lastpos = wave_max_i(lastpos);
  int tok = hits ? __shfl(hit, __builtin_ctzll(hits)) : lastpos;
  if (tok < 0 || tok >= V) tok = 0;  // no positive weight anywhere (non-finite inputs)
  if (lane == 0) out_tokens[b * g1 + k] = tok;
}

// 2'. Greedy decide (T == 0): one workgroup per sequence.  Wave w merges the
//     chunk partials of rows w, w + kGreedyWaves, ... (each lane issuing four
//     loads at a time), leaving row i's argmax in LDS; wave 0 then compares
//     the drafted tokens with them, lane i <-> row i.
__global__ __launch_bounds__(kGreedyWaves * 64) void greedy_kernel(const int32_t* __restrict__ tokens, int64_t gamma,
                                                                    int64_t V,
                                                                    int32_t* __restrict__ out_tokens,
                                                                    int32_t* __restrict__ out_num, Ws ws) {
  __shared__ int sh_best[64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t b = blockIdx.x;
  const int64_t g1 = gamma + 1;
  const int64_t nch = ws.nparts;
  for (int64_t r = w; r < g1; r += kGreedyWaves) {
    const size_t base = (size_t)(b * g1 + r) * ws.pstride;
    float cv = -INFINITY;
    int ci = 0x7fffffff;
    for (int64_t c0 = 0; c0 < nch; c0 += 4 * 64) {
      float v[4];
      int ix[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        v[u] = -INFINITY;
        ix[u] = 0x7fffffff;
        if (c < nch) {
          v[u] = ws.cmax[base + c];
          ix[u] = ws.cidx[base + c];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v[u] > cv || (v[u] == cv && ix[u] < ci)) {
          cv = v[u];
          ci = ix[u];
        }
    }
    wave_argmax(cv, ci);
    if (lane == 0) sh_best[r] = (ci >= 0 && ci < V) ? ci : 0;  // all-NaN row: any in-range id
  }
  __syncthreads();
  if (w != 0) return;
  const bool drafted = lane < gamma;
  const int xi = drafted ? clamp_token(tokens[b * gamma + lane], V) : 0;
  const int mine = lane < g1 ? sh_best[lane] : 0;
  const uint64_t miss = ballot(drafted && xi != mine);
  const int k = miss ? (int)__builtin_ctzll(miss) : (int)gamma;
  const int gk = __shfl(mine, k);
  if (lane < g1) out_tokens[b * g1 + lane] = lane < k ? xi : (lane == k ? gk : -1);  // gamma + 1 <= 64 lanes
  if (lane == 0) out_num[b] = k + 1;
}

// ---------------------------------------------------------------------------
// Tree verification ([LLMI] section 3, tree attention mask and depth offsets;
// [MATH] "SpecInfer and Tree-Based Verification").  One wave per tree of
// M <= 64 nodes, lane i <-> node i.  parents[0] is ignored (node 0 is the
// root); a node whose parent is not in [0, i) is detached: its own only
// ancestor, depth 0, never accepted.

// Parent of lane i's node if its link is well formed, else -1.
__device__ __forceinline__ int tree_link(const int32_t* __restrict__ parents, int64_t base, int i, int M) {
  if (i >= M || i == 0) return -1;
  const int p = parents[base + i];
  return (p >= 0 && p < i) ? p : -1;
}

// Ancestor-or-self bit mask and depth of lane i's node: every lane climbs one
// link per round, reading its current node's parent from the lane that holds
// it (M rounds bound every path).
__device__ __forceinline__ void tree_walk(int par, int i, int M, uint64_t& bits, int& depth) {
  bits = 0;
  depth = 0;
  int cur = i < M ? i : -1;
  for (int step = 0; step < M; ++step) {
    const int pc = __shfl(par, cur < 0 ? 0 : cur);
    if (cur >= 0) {
      bits |= (uint64_t)1 << cur;
      if (pc >= 0) ++depth;
      cur = pc;
    }
  }
}

__global__ __launch_bounds__(kWavesPerBlock * 64) void tree_mask_kernel(const int32_t* __restrict__ parents, int64_t B,
                                                                         int M, uint64_t* __restrict__ out_mask,
                                                                         int32_t* __restrict__ out_depth,
                                                                         float* __restrict__ out_additive) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (b >= B) return;
  const int64_t base = b * M;
  const int par = tree_link(parents, base, lane, M);
  uint64_t bits;
  int depth;
  tree_walk(par, lane, M, bits, depth);
  if (lane >= M) return;
  out_mask[base + lane] = bits;
  out_depth[base + lane] = depth;
  if (out_additive) {
    float* row = out_additive + (size_t)(base + lane) * M;
    for (int j = 0; j < M; ++j) row[j] = ((bits >> j) & 1) ? 0.0f : -INFINITY;
  }
}

// Greedy tree rule on the argmax partials of the B*M rows (row b*M + i scores
// the position after node i).  Node i >= 1 is accepted iff its parent is and
// its token is the parent row's argmax (lowest index on ties); the deepest
// accepted node a (lowest index among equals) ends the kept path.  Its
// ancestors, in index order, are the path from the root.  One workgroup per
// tree: its waves merge the rows' partials in parallel (row i by wave i % 16,
// four partials per lane in flight), then wave 0 applies the rule.
constexpr int kTreeWaves = 16;
__global__ __launch_bounds__(kTreeWaves * 64) void tree_greedy_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ node_tokens, int M, int64_t V,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num, int32_t* __restrict__ out_nodes, Ws ws) {
  __shared__ int sh_best[64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t b = blockIdx.x;
  const int64_t base = b * M;
  const int64_t nch = ws.nparts;
  for (int i = wv; i < M; i += kTreeWaves) {
    const size_t rb = (size_t)(base + i) * ws.pstride;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int64_t c0 = 0; c0 < nch; c0 += 4 * 64) {
      float v[4];
      int ix[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // clamped addresses: the four loads go out together
        const int64_t c = c0 + 64 * j + lane;
        const int64_t cc = c < nch ? c : nch - 1;
        v[j] = ws.cmax[rb + cc];
        ix[j] = ws.cidx[rb + cc];
        if (c >= nch) {
          v[j] = -INFINITY;
          ix[j] = 0x7fffffff;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v[j] > bv || (v[j] == bv && ix[j] < bi)) {
          bv = v[j];
          bi = ix[j];
        }
    }
    wave_argmax(bv, bi);
    if (lane == 0) sh_best[i] = (bi >= 0 && bi < V) ? bi : 0;  // all-NaN row: any in-range id
  }
  __syncthreads();
  if (wv != 0) return;  // no barrier below
  const int par = tree_link(parents, base, lane, M);
  const int tok = lane < M ? node_tokens[base + lane] : -1;
  const int best = lane < M ? sh_best[lane] : 0;
  uint64_t bits;
  int depth;
  tree_walk(par, lane, M, bits, depth);
  // Acceptance, one level per round (parents come before children).
  bool acc = lane == 0;
  for (int step = 0; step < M; ++step) {
    const bool pacc = __shfl(acc ? 1 : 0, par < 0 ? 0 : par) != 0;
    const int pbest = __shfl(best, par < 0 ? 0 : par);
    if (lane > 0 && lane < M) acc = par >= 0 && pacc && tok == pbest;
  }
  // Deepest accepted node, lowest index among equals.
  const int key = acc && lane < M ? depth * 64 + (63 - lane) : -1;
  const int kmax = wave_max_i(key);
  const int a = 63 - (kmax & 63);
  const uint64_t path = __shfl((unsigned long long)bits, a);
  const int n = __shfl(depth, a) + 1;
  const int a_best = __shfl(best, a);
  if (lane < M) {
    if ((path >> lane) & 1) {
      const int rank = __builtin_popcountll(path & (((uint64_t)1 << lane) - 1));
      out_nodes[base + rank] = lane;
      if (rank > 0) out_tokens[base + rank - 1] = tok;
    }
    if (lane >= n) {
      out_nodes[base + lane] = -1;
      out_tokens[base + lane] = -1;
    }
    if (lane == 0) {
      out_tokens[base + n - 1] = a_best;
      out_num[b] = n;
    }
  }
}

inline unsigned blocks_for(int64_t items, int per) { return (unsigned)((items + per - 1) / per); }

}  // namespace

size_t reject_workspace_bytes(int64_t B, int64_t gamma, int64_t V) { return make_layout(B, gamma, V).total; }

int64_t reject_fusable_stride(int64_t B, int64_t gamma, int64_t V) {
  const Layout L = make_layout(B, gamma, V);
  return B * (gamma + 1) > kMaxFusedRows || L.pstride < kMaxFusedParts ? 0 : L.pstride;
}

bool reject_fused_stats(const RejectArgs& a, FusedStats* fs) {
  const Layout L = make_layout(a.B, a.gamma, a.V);
  if (a.B * (a.gamma + 1) > kMaxFusedRows || L.pstride < kMaxFusedParts || warp_active(a)) return false;
  const Ws ws = bind(a.workspace, L, 0);
  const bool greedy = a.temperature == 0.0f;
  fs->cmax = ws.cmax;
  fs->csum = ws.csum;
  fs->cidx = ws.cidx;
  fs->zx = ws.zx;
  fs->pstride = L.pstride;
  fs->draft = (!greedy && a.draft_kind == 0 && a.gamma > 0) ? a.draft : nullptr;
  fs->done = greedy ? nullptr : ws.done;
  fs->tokens = a.tokens;
  fs->B = a.B;
  fs->gamma = a.gamma;
  fs->inv_t = greedy ? 1.0f : (float)(1.0 / (double)a.temperature);
  fs->greedy = greedy;
  return true;
}

namespace {

// The stages after the statistics: the draw (T > 0) or the greedy rule.
hipError_t launch_decide(const RejectArgs& a, const Ws& ws, hipStream_t stream) {
  const bool greedy = a.temperature == 0.0f;
  const bool vec = (a.V & 3) == 0;
  const float inv_t = greedy ? 1.0f : (float)(1.0 / (double)a.temperature);
  if (greedy) {
    hipLaunchKernelGGL(greedy_kernel, dim3((unsigned)a.B), dim3(kGreedyWaves * 64), 0, stream, a.tokens, a.gamma,
                       a.V, a.out_tokens, a.out_num, ws);
    return hipGetLastError();
  }
  const int64_t ndc = draw_chunks(a.V);
  const bool warp = warp_active(a);
#define SPECDEC_DRAW(WB, V4, WP)                                                                                    \
  hipLaunchKernelGGL((draw_sum_kernel<WB, V4, WP>), dim3((unsigned)(a.B * ((ndc + WB - 1) / WB))), dim3(WB * 64), 0, \
                     stream, a.target, a.draft, a.draft_kind, a.tokens, a.uniforms, a.B, a.gamma, a.V, inv_t,          \
                     a.out_tokens, a.out_num, a.out_probs, ws)
  if (warp) {
    if (ndc >= 16) {
      if (vec) SPECDEC_DRAW(16, true, true); else SPECDEC_DRAW(16, false, true);
    } else {
      if (vec) SPECDEC_DRAW(4, true, true); else SPECDEC_DRAW(4, false, true);
    }
  } else if (ndc >= 16) {
    if (vec) SPECDEC_DRAW(16, true, false); else SPECDEC_DRAW(16, false, false);
  } else {
    if (vec) SPECDEC_DRAW(4, true, false); else SPECDEC_DRAW(4, false, false);
  }
#undef SPECDEC_DRAW
  return hipGetLastError();
}

}  // namespace

hipError_t launch_draft_stats(const FusedStats& fs, int64_t n_target, int64_t V, int64_t* nparts, hipStream_t stream) {
  const int64_t nd = fs.B * fs.gamma, nch = stat_chunks(V);
  *nparts = nch;
  if (nd == 0 || fs.draft == nullptr) return hipSuccess;
  if (nch > fs.pstride) return hipErrorNotSupported;
  Ws ws{};
  ws.cmax = fs.cmax;
  ws.csum = fs.csum;
  ws.cidx = fs.cidx;
  ws.zx = fs.zx;
  ws.pstride = fs.pstride;
  ws.nparts = ws.nparts_d = nch;
  const dim3 grid(blocks_for(nd * nch, kWavesPerBlock)), blk(kWavesPerBlock * 64);
  if ((V & 3) == 0)
    hipLaunchKernelGGL((stats_kernel<true, false>), grid, blk, 0, stream, nullptr, fs.draft, fs.tokens,
                       n_target, n_target, n_target + nd, fs.gamma, V, fs.inv_t, ws, (int64_t)0);
  else
    hipLaunchKernelGGL((stats_kernel<false, false>), grid, blk, 0, stream, nullptr, fs.draft, fs.tokens,
                       n_target, n_target, n_target + nd, fs.gamma, V, fs.inv_t, ws, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_reject_after_fused(const RejectArgs& a, int64_t nparts, int64_t nparts_draft, hipStream_t stream) {
  const Layout L = make_layout(a.B, a.gamma, a.V);
  return launch_decide(a, bind(a.workspace, L, nparts, nparts_draft), stream);
}

size_t tree_workspace_bytes(int64_t B, int64_t M, int64_t V) { return make_layout(B, M - 1, V).total; }

hipError_t launch_tree_mask(const int32_t* parents, int64_t B, int64_t M, uint64_t* out_mask, int32_t* out_depth,
                            float* out_additive, hipStream_t stream) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(blocks_for(B, kWavesPerBlock)), dim3(kWavesPerBlock * 64), 0, stream,
                     parents, B, (int)M, out_mask, out_depth, out_additive);
  return hipGetLastError();
}

bool tree_fused_stats(const TreeArgs& t, FusedStats* fs) {
  const Layout L = make_layout(t.B, t.M - 1, t.V);
  if (t.B * t.M > kMaxFusedRows || L.pstride < kMaxFusedParts) return false;
  const Ws ws = bind(t.workspace, L, 0);
  *fs = FusedStats{};
  fs->cmax = ws.cmax;
  fs->csum = ws.csum;
  fs->cidx = ws.cidx;
  fs->zx = ws.zx;
  fs->pstride = L.pstride;
  fs->draft = nullptr;
  fs->tokens = nullptr;
  fs->B = t.B;
  fs->gamma = t.M - 1;
  fs->inv_t = 1.0f;
  fs->greedy = true;
  return true;
}

hipError_t launch_tree_greedy(const TreeArgs& t, int64_t nparts, hipStream_t stream) {
  const Layout L = make_layout(t.B, t.M - 1, t.V);
  const dim3 blk(kWavesPerBlock * 64);
  Ws ws;
  if (nparts <= 0) {  // argmax partials from the statistics pass over the given logits
    ws = bind(t.workspace, L, stat_chunks(t.V));
    const int64_t rows = t.B * t.M;
    const dim3 g1(blocks_for(rows * stat_chunks(t.V), kWavesPerBlock));
    if ((t.V & 3) == 0)
      hipLaunchKernelGGL((stats_kernel<true, true>), g1, blk, 0, stream, t.logits, nullptr, nullptr, rows, 0, rows,
                         (int64_t)0, t.V, 1.0f, ws, (int64_t)0);
    else
      hipLaunchKernelGGL((stats_kernel<false, true>), g1, blk, 0, stream, t.logits, nullptr, nullptr, rows, 0, rows,
                         (int64_t)0, t.V, 1.0f, ws, (int64_t)0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    ws = bind(t.workspace, L, nparts);
  }
  hipLaunchKernelGGL(tree_greedy_kernel, dim3((unsigned)t.B), dim3(kTreeWaves * 64), 0, stream, t.parents,
                     t.node_tokens, (int)t.M, t.V, t.out_tokens, t.out_num, t.out_nodes, ws);
  return hipGetLastError();
}

hipError_t launch_reject_sample(const RejectArgs& a, hipStream_t stream) {
  const Layout L = make_layout(a.B, a.gamma, a.V);
  const Ws ws = bind(a.workspace, L, stat_chunks(a.V));
  const bool greedy = a.temperature == 0.0f;
  const bool vec = (a.V & 3) == 0;
  const float inv_t = greedy ? 1.0f : (float)(1.0 / (double)a.temperature);
  const int64_t n_target = a.B * (a.gamma + 1);
  const int64_t n_rows = n_target + ((!greedy && a.draft_kind == 0) ? a.B * a.gamma : 0);
  const dim3 blk(kWavesPerBlock * 64);
  const dim3 g1(blocks_for(n_rows * stat_chunks(a.V), kWavesPerBlock));
  const bool warp = warp_active(a);
  if (!greedy && !warp && a.V <= kSmallV) {  // one wave per sequence does the whole rule
    const dim3 gs(blocks_for(a.B, kWavesPerBlock));
    if (vec)
      hipLaunchKernelGGL(small_rule_kernel<true>, gs, blk, 0, stream, a.target, a.draft, a.draft_kind, a.tokens,
                         a.uniforms, a.B, a.gamma, a.V, inv_t, a.out_tokens, a.out_num, a.out_probs);
    else
      hipLaunchKernelGGL(small_rule_kernel<false>, gs, blk, 0, stream, a.target, a.draft, a.draft_kind, a.tokens,
                         a.uniforms, a.B, a.gamma, a.V, inv_t, a.out_tokens, a.out_num, a.out_probs);
    return hipGetLastError();
  }
  if (warp) {  // the per-row cuts and the warped rows' statistics (no statistics pass)
    const WarpStats so{ws.cmax, ws.csum, ws.zx, ws.pstride, stat_chunks(a.V), a.tokens, a.gamma, a.B, ws.done};
    const hipError_t ew = launch_warp_cuts(a.target, a.draft, n_target, n_rows, a.V, inv_t, a.top_k, a.top_p,
                                           ws.wkey, ws.widx, so, stream);
    if (ew != hipSuccess) return ew;
    return launch_decide(a, ws, stream);
  }
#define SPECDEC_STATS(V4, GR)                                                                                        \
  hipLaunchKernelGGL((stats_kernel<V4, GR>), g1, blk, 0, stream, a.target, a.draft, a.tokens, n_target, 0, n_rows, \
                     a.gamma, a.V, inv_t, ws, greedy ? (int64_t)0 : a.B)
  if (greedy) {
    if (vec) SPECDEC_STATS(true, true); else SPECDEC_STATS(false, true);
  } else {
    if (vec) SPECDEC_STATS(true, false); else SPECDEC_STATS(false, false);
  }
#undef SPECDEC_STATS
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decide(a, ws, stream);
}

}  // namespace specdec
