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
// Data flow (three launches on the caller's stream, no host synchronisation):
//   1. row_stats: one wave per (row, 1024-entry vocabulary chunk) of every
//      target row and (for draft logits) every draft row.  T > 0: chunk max
//      m_c of a = z * (1/T) and s_c = sum exp(a - m_c) (fp32 terms, fp64 wave
//      sum).  T == 0: chunk max value and its lowest index.
//   2. decide: one wave per sequence.  Merges the chunk partials of its rows
//      with m = max m_c, Z = sum s_c exp(m_c - m) in fp64, forms p_i(x_i) and
//      q_i(x_i) (fp64, rounded once to fp32), evaluates every accept test,
//      finds the first rejection k and writes the kept tokens.  Greedy steps
//      finish here.
//   3. draw: one wave per (sequence, chunk) of the one row pair where the step
//      ends: fp32 weights r_v = max(0, p_v - q_v) (or p_v for the bonus), fp64
//      chunk totals.  The last wave to finish for a sequence (device-scope
//      counter) locates the chunk holding u*S from the fp64 running totals,
//      rescans that chunk with an fp64 prefix sum and writes the token.
// p, q, (p - q)+ and p/q are fp32 values, as the first source asks for T > 0
// (section 4, failure mode 1); normalisers and running sums are fp64.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kChunk = 1024;       // vocabulary entries per wave work item
constexpr int kPerLane = kChunk / 64;
constexpr int kWavesPerBlock = 4;
constexpr float kQFloor = 1e-12f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int64_t num_chunks(int64_t V) { return (V + kChunk - 1) / kChunk; }

// Workspace layout, all arrays 16-byte aligned.
struct Layout {
  int64_t rows, nch;
  size_t off_cmax, off_csum, off_cidx;      // per (row, chunk)
  size_t off_kb, off_cnt, off_norm;         // per sequence
  size_t off_sres, off_sp;                  // per (sequence, chunk)
  size_t total;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline Layout make_layout(int64_t B, int64_t gamma, int64_t V) {
  Layout L;
  L.nch = num_chunks(V);
  L.rows = B * (2 * gamma + 1);
  size_t o = 0;
  const size_t rc = (size_t)L.rows * L.nch;
  L.off_cmax = o; o = align16(o + rc * sizeof(float));
  L.off_csum = o; o = align16(o + rc * sizeof(double));
  L.off_cidx = o; o = align16(o + rc * sizeof(int32_t));
  L.off_kb = o;   o = align16(o + (size_t)B * sizeof(int32_t));
  L.off_cnt = o;  o = align16(o + (size_t)B * sizeof(uint32_t));
  L.off_norm = o; o = align16(o + (size_t)B * 4 * sizeof(double));
  L.off_sres = o; o = align16(o + (size_t)B * L.nch * sizeof(double));
  L.off_sp = o;   o = align16(o + (size_t)B * L.nch * sizeof(double));
  L.total = o;
  return L;
}

struct Ws {
  float* cmax;
  double* csum;
  int32_t* cidx;
  int32_t* kb;
  uint32_t* cnt;
  double* norm;  // [B][4]: m_p, Z_p, m_q, Z_q of the row where the step ends
  double* sres;
  double* sp;
};

inline Ws bind(void* base, const Layout& L) {
  char* b = (char*)base;
  return Ws{(float*)(b + L.off_cmax), (double*)(b + L.off_csum), (int32_t*)(b + L.off_cidx), (int32_t*)(b + L.off_kb),
            (uint32_t*)(b + L.off_cnt), (double*)(b + L.off_norm), (double*)(b + L.off_sres), (double*)(b + L.off_sp)};
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes).
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
__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
// Larger value wins; equal values go to the lower index.
__device__ __forceinline__ void wave_argmax(float& val, int& idx) {
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
// Inclusive prefix sum over lanes.
__device__ __forceinline__ double wave_inclusive_scan(double x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Loads this lane's 16 entries of a 1024-entry chunk of one row; entries
// past V read as `fill`.  Entry e of the lane sits at chunk offset
// (e / 4) * 256 + lane * 4 + e % 4 (16-byte loads, 1 KB per instruction).
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t V, int64_t c0, int lane, float fill,
                                           float (&x)[kPerLane]) {
#pragma unroll
  for (int j = 0; j < kPerLane / 4; ++j) {
    const int64_t v = c0 + j * 256 + lane * 4;
    if (VEC && v + 3 < V) {
      const f32x4 t = __builtin_nontemporal_load((const f32x4*)(row + v));
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
__device__ __forceinline__ double coherent_load(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int64_t entry_index(int64_t c0, int lane, int e) {
  return c0 + (e / 4) * 256 + lane * 4 + (e & 3);
}

// ---------------------------------------------------------------------------
// 1. Chunk partials of every target row (rows [0, B*(gamma+1))) and, for draft
//    logits at T > 0, every draft row (rows [B*(gamma+1), B*(2*gamma+1))).
template <bool VEC, bool GREEDY>
__global__ __launch_bounds__(kWavesPerBlock * 64) void row_stats_kernel(const float* __restrict__ target,
                                                                         const float* __restrict__ draft,
                                                                         int64_t n_target_rows, int64_t n_rows,
                                                                         int64_t V, float inv_t, Ws ws) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = num_chunks(V);
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= n_rows * nch) return;
  const int64_t r = item / nch, c = item - r * nch;
  const float* row = r < n_target_rows ? target + (size_t)r * V : draft + (size_t)(r - n_target_rows) * V;
  const int64_t c0 = c * kChunk;
  float x[kPerLane];
  load_chunk<VEC>(row, V, c0, lane, -INFINITY, x);
  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const int idx = (int)entry_index(c0, lane, e);
      if (idx < V && (x[e] > bv || (x[e] == bv && idx < bi))) {
        bv = x[e];
        bi = idx;
      }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
      ws.cmax[item] = bv;
      ws.cidx[item] = bi;
    }
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      x[e] = x[e] * inv_t;
      mx = fmaxf(mx, x[e]);
    }
    mx = wave_max(mx);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) s += expf(x[e] - mx);
    const double tot = wave_sum((double)s);
    if (lane == 0) {
      ws.cmax[item] = mx;
      ws.csum[item] = tot;
    }
  }
}

// Merges the chunk partials of one row: m = max m_c, Z = sum s_c exp(m_c - m).
__device__ void merge_row(const Ws& ws, int64_t row, int64_t nch, int lane, double& m, double& Z) {
  double mx = -INFINITY;
  for (int64_t c = lane; c < nch; c += 64) mx = fmax(mx, (double)ws.cmax[row * nch + c]);
  mx = wave_max_d(mx);
  double s = 0.0;
  for (int64_t c = lane; c < nch; c += 64) s += ws.csum[row * nch + c] * exp((double)ws.cmax[row * nch + c] - mx);
  m = mx;
  Z = wave_sum(s);
}

__device__ __forceinline__ int clamp_token(int32_t t, int64_t V) { return t < 0 ? 0 : (t >= V ? (int)(V - 1) : t); }

// 2. One wave per sequence.
template <bool GREEDY>
__global__ __launch_bounds__(64) void decide_kernel(const float* __restrict__ target, const float* __restrict__ draft,
                                                    int draft_kind, const int32_t* __restrict__ tokens,
                                                    const float* __restrict__ uniforms, int64_t B, int64_t gamma,
                                                    int64_t V, float inv_t, int32_t* __restrict__ out_tokens,
                                                    int32_t* __restrict__ out_num, float* __restrict__ out_probs,
                                                    Ws ws) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t nch = num_chunks(V);
  const int64_t g1 = gamma + 1;
  const int64_t trow0 = b * g1;                  // target rows of this sequence
  const int64_t drow0 = B * g1 + b * gamma;      // draft rows of this sequence
  int k = (int)gamma;
  if (GREEDY) {
    int gk = 0;
    for (int64_t i = 0; i <= gamma; ++i) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int64_t c = lane; c < nch; c += 64) {
        const float v = ws.cmax[(trow0 + i) * nch + c];
        const int idx = ws.cidx[(trow0 + i) * nch + c];
        if (v > bv || (v == bv && idx < bi)) {
          bv = v;
          bi = idx;
        }
      }
      wave_argmax(bv, bi);
      if (bi < 0 || bi >= V) bi = 0;  // all-NaN row: any in-range id
      if (i == gamma || clamp_token(tokens[b * gamma + i], V) != bi) {
        k = (int)i;
        gk = bi;
        break;
      }
    }
    for (int64_t j = lane; j < g1; j += 64)
      out_tokens[b * g1 + j] = j < k ? clamp_token(tokens[b * gamma + j], V) : (j == k ? gk : -1);
    if (lane == 0) out_num[b] = k + 1;
    return;
  }
  // Accept tests of every drafted row (they do not depend on each other).
  for (int64_t i = 0; i < gamma; ++i) {
    const int x = clamp_token(tokens[b * gamma + i], V);
    double mp, Zp;
    merge_row(ws, trow0 + i, nch, lane, mp, Zp);
    const float ap = target[(size_t)(trow0 + i) * V + x] * inv_t;
    const float p = (float)(exp((double)ap - mp) / Zp);
    float q;
    if (draft_kind == 1) {
      q = draft[(size_t)(b * gamma + i) * V + x];
    } else {
      double mq, Zq;
      merge_row(ws, drow0 + i, nch, lane, mq, Zq);
      const float aq = draft[(size_t)(b * gamma + i) * V + x] * inv_t;
      q = (float)(exp((double)aq - mq) / Zq);
    }
    const float ratio = p / (q > kQFloor ? q : kQFloor);
    const float thr = ratio < 1.0f ? ratio : 1.0f;
    const bool keep = uniforms[(b * g1 + i) * 2 + 0] < thr;
    if (lane == 0 && out_probs) {
      out_probs[(b * gamma + i) * 2 + 0] = p;
      out_probs[(b * gamma + i) * 2 + 1] = q;
    }
    if (!keep && k == (int)gamma) k = (int)i;
  }
  // Normalisers of the row where the step ends.
  double mp, Zp, mq = 0.0, Zq = 1.0;
  merge_row(ws, trow0 + k, nch, lane, mp, Zp);
  if (k < gamma && draft_kind == 0) merge_row(ws, drow0 + k, nch, lane, mq, Zq);
  for (int64_t j = lane; j < g1; j += 64)
    out_tokens[b * g1 + j] = j < k ? clamp_token(tokens[b * gamma + j], V) : -1;
  if (lane == 0) {
    out_num[b] = k + 1;
    ws.kb[b] = k;
    ws.cnt[b] = 0u;
    ws.norm[b * 4 + 0] = mp;
    ws.norm[b * 4 + 1] = Zp;
    ws.norm[b * 4 + 2] = mq;
    ws.norm[b * 4 + 3] = Zq;
  }
}

// Weights of the draw at one entry: p_v and r_v = max(0, p_v - q_v) in fp32.
struct DrawRow {
  const float* zp;  // target logits of the row
  const float* zq;  // draft logits or probabilities of the row (null for the bonus)
  float mp, ip, mq, iq, inv_t;
  bool q_probs;
};

__device__ __forceinline__ void weights(const DrawRow& R, float zp, float zq, float& p, float& r) {
  p = expf(zp * R.inv_t - R.mp) * R.ip;
  if (R.zq) {
    const float q = R.q_probs ? zq : expf(zq * R.inv_t - R.mq) * R.iq;
    const float dlt = p - q;
    r = dlt > 0.0f ? dlt : 0.0f;
  } else {
    r = p;
  }
}

// 3. One wave per (sequence, chunk); the last wave of a sequence selects the token.
template <bool VEC>
__global__ __launch_bounds__(kWavesPerBlock * 64) void draw_kernel(const float* __restrict__ target,
                                                                    const float* __restrict__ draft, int draft_kind,
                                                                    const float* __restrict__ uniforms, int64_t B,
                                                                    int64_t gamma, int64_t V, float inv_t,
                                                                    int32_t* __restrict__ out_tokens, Ws ws) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = num_chunks(V);
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= B * nch) return;
  const int64_t b = item / nch, c = item - b * nch;
  const int64_t g1 = gamma + 1;
  const int k = ws.kb[b];
  DrawRow R;
  R.zp = target + (size_t)(b * g1 + k) * V;
  R.zq = k < gamma ? draft + (size_t)(b * gamma + k) * V : nullptr;
  R.mp = (float)ws.norm[b * 4 + 0];
  R.ip = (float)(1.0 / ws.norm[b * 4 + 1]);
  R.mq = (float)ws.norm[b * 4 + 2];
  R.iq = (float)(1.0 / ws.norm[b * 4 + 3]);
  R.inv_t = inv_t;
  R.q_probs = draft_kind == 1;

  const int64_t c0 = c * kChunk;
  float zp[kPerLane], zq[kPerLane];
  load_chunk<VEC>(R.zp, V, c0, lane, -INFINITY, zp);
  if (R.zq) load_chunk<VEC>(R.zq, V, c0, lane, R.q_probs ? 0.0f : -INFINITY, zq);
  double sr = 0.0, sp = 0.0;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) {
    float p, r;
    weights(R, zp[e], R.zq ? zq[e] : 0.0f, p, r);
    sr += (double)r;
    sp += (double)p;
  }
  sr = wave_sum(sr);
  sp = wave_sum(sp);
  uint32_t prev = 0;
  if (lane == 0) {
    ws.sres[item] = sr;
    ws.sp[item] = sp;
    __threadfence();
    prev = atomicAdd(&ws.cnt[b], 1u);
  }
  prev = __shfl(prev, 0);
  if (prev != (uint32_t)(nch - 1)) return;
  __threadfence();

  // Last wave for this sequence: choose the weights (residual, or p when the
  // residual has no mass or the step ends on the bonus row).
  // Partials written by other waves are read with device-scope loads.
  const double* part = ws.sres + b * nch;
  double tot = 0.0;
  if (R.zq) {
    for (int64_t j = 0; j < nch; ++j) tot += coherent_load(part + j);
  }
  const bool use_p = !(tot > 0.0);
  if (use_p) {
    part = ws.sp + b * nch;
    tot = 0.0;
    for (int64_t j = 0; j < nch; ++j) tot += coherent_load(part + j);
  }
  const float u = uniforms[(b * g1 + k) * 2 + 1];
  const double t = (double)u * tot;
  // Chunk whose running total passes t; if rounding leaves none, the last
  // chunk with mass.
  int64_t cs = -1, clast = 0;
  double before = 0.0, run = 0.0;
  for (int64_t j = 0; j < nch; ++j) {
    const double pj = coherent_load(part + j);
    const double nxt = run + pj;
    if (pj > 0.0) clast = j;
    if (cs < 0 && t < nxt) {
      cs = j;
      before = run;
    }
    run = nxt;
  }
  if (cs < 0) {
    cs = clast;
    before = run - coherent_load(part + clast);
  }
  // Rescan that chunk with an fp64 running sum in vocabulary order.  Lane l
  // takes the 16 consecutive entries starting at cs*1024 + 16*l.
  const int64_t s0 = cs * kChunk + 16 * lane;
  double w[16];
  double lsum = 0.0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t v = s0 + e;
    float p = 0.f, r = 0.f;
    if (v < V) weights(R, R.zp[v], R.zq ? R.zq[v] : 0.0f, p, r);
    w[e] = use_p ? (double)p : (double)r;
    lsum += w[e];
  }
  const double incl = wave_inclusive_scan(lsum, lane);
  double C = before + (incl - lsum);
  int hit = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t v = s0 + e;
    C += w[e];
    if (v < V && w[e] > 0.0) {
      lastpos = (int)v;
      if (hit == 0x7fffffff && t < C) hit = (int)v;
    }
  }
  hit = wave_min_i(hit);
  lastpos = wave_max_i(lastpos);
  if (lane == 0) {
    int tok = hit != 0x7fffffff ? hit : lastpos;
    if (tok < 0) tok = 0;  // no positive weight anywhere (non-finite inputs)
    out_tokens[b * g1 + k] = tok;
  }
}

inline unsigned blocks_for(int64_t items) { return (unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock); }

}  // namespace

size_t reject_workspace_bytes(int64_t B, int64_t gamma, int64_t V) { return make_layout(B, gamma, V).total; }

hipError_t launch_reject_sample(const RejectArgs& a, hipStream_t stream) {
  const Layout L = make_layout(a.B, a.gamma, a.V);
  const Ws ws = bind(a.workspace, L);
  const bool greedy = a.temperature == 0.0f;
  const bool vec = (a.V & 3) == 0;
  const float inv_t = greedy ? 1.0f : (float)(1.0 / (double)a.temperature);
  const int64_t n_target = a.B * (a.gamma + 1);
  const int64_t n_rows = n_target + ((!greedy && a.draft_kind == 0) ? a.B * a.gamma : 0);
  const int64_t nch = num_chunks(a.V);
  const dim3 blk(kWavesPerBlock * 64);
  const dim3 g1(blocks_for(n_rows * nch));
#define SPECDEC_STATS(V4, GR) \
  hipLaunchKernelGGL((row_stats_kernel<V4, GR>), g1, blk, 0, stream, a.target, a.draft, n_target, n_rows, a.V, inv_t, ws)
  if (greedy) {
    if (vec) SPECDEC_STATS(true, true); else SPECDEC_STATS(false, true);
  } else {
    if (vec) SPECDEC_STATS(true, false); else SPECDEC_STATS(false, false);
  }
#undef SPECDEC_STATS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (greedy) {
    hipLaunchKernelGGL((decide_kernel<true>), dim3((unsigned)a.B), dim3(64), 0, stream, a.target, a.draft,
                       a.draft_kind, a.tokens, a.uniforms, a.B, a.gamma, a.V, inv_t, a.out_tokens, a.out_num,
                       a.out_probs, ws);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decide_kernel<false>), dim3((unsigned)a.B), dim3(64), 0, stream, a.target, a.draft, a.draft_kind,
                     a.tokens, a.uniforms, a.B, a.gamma, a.V, inv_t, a.out_tokens, a.out_num, a.out_probs, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g3(blocks_for(a.B * nch));
  if (vec)
    hipLaunchKernelGGL((draw_kernel<true>), g3, blk, 0, stream, a.target, a.draft, a.draft_kind, a.uniforms, a.B,
                       a.gamma, a.V, inv_t, a.out_tokens, ws);
  else
    hipLaunchKernelGGL((draw_kernel<false>), g3, blk, 0, stream, a.target, a.draft, a.draft_kind, a.uniforms, a.B,
                       a.gamma, a.V, inv_t, a.out_tokens, ws);
  return hipGetLastError();
}

}  // namespace specdec
