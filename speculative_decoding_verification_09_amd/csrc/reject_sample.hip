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
// Launches on the caller's stream (no host synchronisation, no inter-wave
// signalling inside a launch: kernel boundaries order every step):
//   1. stats: one wave per (row, 2048-entry vocabulary chunk) of every target
//      row and, for draft logits at T > 0, every draft row.  T > 0: chunk max
//      m_c of a = z * (1/T) and s_c = sum exp(a - m_c) (fp32 terms summed in
//      fp64).  T == 0: chunk max value and its lowest index.
//   2. merge: one wave per row: m = max m_c, Z = sum s_c exp(m_c - m) (fp64),
//      and p_i(x_i) or q_i(x_i) of the drafted token (fp64, rounded once to fp32).
//   3. draw sums: one wave per (sequence, 1024-entry chunk).  Each wave takes
//      every accept test of its sequence at once (lane i <-> row i) and finds
//      the first rejection k with a ballot, then sums its chunk of the draw
//      weights of row k: r_v = max(0, p_v - q_v) and p_v (fp32 values, fp64 sums).
//   4. select: one wave per sequence finds the chunk holding u*S with an fp64
//      prefix sum over the chunk totals, rescans that chunk with an fp64
//      running sum in vocabulary order and writes the token.
//   Greedy steps run 1 and then one wave per sequence that merges the argmax
//   partials and applies the greedy rule.
// p, q, (p - q)+ and p/q are fp32 values, as the first source asks for T > 0
// (section 4, failure mode 1); normalisers and running sums are fp64.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kStatChunk = 2048;        // vocabulary entries per statistics work item (one wave)
constexpr int kDrawChunk = 1024;        // vocabulary entries per draw work item (one wave)
constexpr int kWavesPerBlock = 4;
constexpr int kRowBatch = 8;            // rows whose partials are loaded together
constexpr float kQFloor = 1e-12f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int64_t stat_chunks(int64_t V) { return (V + kStatChunk - 1) / kStatChunk; }
__host__ __device__ inline int64_t draw_chunks(int64_t V) { return (V + kDrawChunk - 1) / kDrawChunk; }
__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Workspace layout, every array 16-byte aligned.
struct Layout {
  size_t off_cmax, off_csum, off_cidx;  // per (row, chunk)
  size_t off_rm, off_rz, off_px;        // per row
  size_t off_kb;                        // per sequence
  size_t off_sres, off_sp;              // per (sequence, draw chunk)
  size_t total;
};

__host__ __device__ inline Layout make_layout(int64_t B, int64_t gamma, int64_t V) {
  Layout L;
  const int64_t nch = stat_chunks(V), ndc = draw_chunks(V);
  const size_t rc = (size_t)(B * (2 * gamma + 1)) * nch;
  size_t o = 0;
  L.off_cmax = o; o = align16(o + rc * sizeof(float));
  L.off_csum = o; o = align16(o + rc * sizeof(double));
  L.off_cidx = o; o = align16(o + rc * sizeof(int32_t));
  const size_t rows = (size_t)(B * (2 * gamma + 1));
  L.off_rm = o;   o = align16(o + rows * sizeof(double));
  L.off_rz = o;   o = align16(o + rows * sizeof(double));
  L.off_px = o;   o = align16(o + rows * sizeof(float));
  L.off_kb = o;   o = align16(o + (size_t)B * sizeof(int32_t));
  L.off_sres = o; o = align16(o + (size_t)B * ndc * sizeof(double));
  L.off_sp = o;   o = align16(o + (size_t)B * ndc * sizeof(double));
  L.total = o;
  return L;
}

struct Ws {
  float* cmax;
  double* csum;
  int32_t* cidx;
  double* rm;   // per row: max of a = z / T
  double* rz;   // per row: sum exp(a - m)
  float* px;    // per drafted row: p_i(x_i) (target rows) or q_i(x_i) (draft rows)
  int32_t* kb;  // per sequence: row where the step ends
  double* sres;
  double* sp;
};

inline Ws bind(void* base, const Layout& L) {
  char* b = (char*)base;
  return Ws{(float*)(b + L.off_cmax), (double*)(b + L.off_csum), (int32_t*)(b + L.off_cidx),
            (double*)(b + L.off_rm),  (double*)(b + L.off_rz),   (float*)(b + L.off_px),
            (int32_t*)(b + L.off_kb), (double*)(b + L.off_sres), (double*)(b + L.off_sp)};
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

// Loads lane's PL entries of a (64*PL)-entry chunk, coalesced: entry 4*j + e
// of the lane is chunk offset 256*j + 4*lane + e.  Entries past V read as fill.
template <bool VEC, int PL>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t V, int64_t c0, int lane, float fill,
                                           float (&x)[PL]) {
#pragma unroll
  for (int j = 0; j < PL / 4; ++j) {
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
__device__ __forceinline__ int64_t entry_index(int64_t c0, int lane, int e) {
  return c0 + 256 * (e >> 2) + 4 * lane + (e & 3);
}

__device__ __forceinline__ int clamp_token(int32_t t, int64_t V) { return t < 0 ? 0 : (t >= V ? (int)(V - 1) : t); }

// ---------------------------------------------------------------------------
// 1. Chunk partials.  Target rows are [0, B*(gamma+1)) (row b*(gamma+1) + i),
//    draft rows [B*(gamma+1), B*(2*gamma+1)) (row B*(gamma+1) + b*gamma + i).
template <bool VEC, bool GREEDY>
__global__ __launch_bounds__(kWavesPerBlock * 64) void stats_kernel(const float* __restrict__ target,
                                                                     const float* __restrict__ draft,
                                                                     int64_t n_target_rows, int64_t n_rows,
                                                                     int64_t gamma, int64_t V, float inv_t, Ws ws) {
  constexpr int PL = kStatChunk / 64;
  const int lane = threadIdx.x & 63;
  const int64_t nch = stat_chunks(V);
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= n_rows * nch) return;
  const int64_t r = item / nch, c = item - r * nch;
  const float* row = r < n_target_rows ? target + (size_t)r * V : draft + (size_t)(r - n_target_rows) * V;
  const int64_t c0 = c * kStatChunk;
  float x[PL];
  load_chunk<VEC, PL>(row, V, c0, lane, -INFINITY, x);
  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < PL; ++e) {
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
    for (int e = 0; e < PL; ++e) {
      x[e] = x[e] * inv_t;
      mx = fmaxf(mx, x[e]);
    }
    mx = wave_max(mx);
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < PL; ++e) s += (double)expf(x[e] - mx);
    s = wave_sum(s);
    if (lane == 0) {
      ws.cmax[item] = mx;
      ws.csum[item] = s;
    }
  }
}

// 2. Row merge (T > 0): one wave per row.  m = max m_c, Z = sum s_c exp(m_c - m)
//    (fp64), and for drafted rows the probability of the drafted token,
//    p_i(x_i) or q_i(x_i) = exp(a_x - m) / Z (fp64, rounded once to fp32).
__global__ __launch_bounds__(kWavesPerBlock * 64) void merge_kernel(const float* __restrict__ target,
                                                                     const float* __restrict__ draft,
                                                                     const int32_t* __restrict__ tokens,
                                                                     int64_t n_target_rows, int64_t n_rows,
                                                                     int64_t gamma, int64_t V, float inv_t, Ws ws) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int64_t nch = stat_chunks(V);
  // The drafted token of this row, gathered while the partials load.
  const bool is_target = r < n_target_rows;
  const int64_t g1 = gamma + 1;
  const int64_t b = is_target ? r / g1 : (r - n_target_rows) / gamma;
  const int64_t i = is_target ? r - b * g1 : (r - n_target_rows) - b * gamma;
  const bool drafted = i < gamma;
  float zx = 0.0f;
  if (drafted) {
    const int x = clamp_token(tokens[b * gamma + i], V);
    zx = is_target ? target[(size_t)r * V + x] : draft[(size_t)(r - n_target_rows) * V + x];
  }
  const size_t base = (size_t)r * nch;
  float m = -INFINITY;
  for (int64_t c = lane; c < nch; c += 64) m = fmaxf(m, ws.cmax[base + c]);
  m = wave_max(m);
  double z = 0.0;
  for (int64_t c = lane; c < nch; c += 64) {
    const double sc = ws.csum[base + c];
    if (sc > 0.0) z += sc * exp((double)ws.cmax[base + c] - (double)m);
  }
  z = wave_sum(z);
  if (lane == 0) {
    ws.rm[r] = (double)m;
    ws.rz[r] = z;
    ws.px[r] = drafted ? (float)(exp((double)(zx * inv_t) - (double)m) / z) : 0.0f;
  }
}

// Weights of the draw at one entry: p_v and r_v = max(0, p_v - q_v), fp32.
struct DrawRow {
  const float* zp;  // target logits of the row
  const float* zq;  // draft logits or probabilities of the row (null on the bonus row)
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

// The accept tests of sequence b, lane i <-> drafted row i: every test at
// once, first rejection by ballot.  Returns k (gamma if all are kept).
__device__ __forceinline__ int first_rejection(const float* __restrict__ draft, int draft_kind,
                                               const int32_t* __restrict__ tokens,
                                               const float* __restrict__ uniforms, int64_t b, int64_t B,
                                               int64_t gamma, int64_t V, int lane, const Ws& ws, float& p_x,
                                               float& q_x) {
  const int64_t g1 = gamma + 1;
  const bool drafted = lane < gamma;
  p_x = 0.0f;
  q_x = 0.0f;
  bool reject = false;
  if (drafted) {
    p_x = ws.px[b * g1 + lane];
    if (draft_kind == 1) {
      const int x = clamp_token(tokens[b * gamma + lane], V);
      q_x = draft[(size_t)(b * gamma + lane) * V + x];
    } else {
      q_x = ws.px[B * g1 + b * gamma + lane];
    }
    const float ratio = p_x / (q_x > kQFloor ? q_x : kQFloor);
    const float thr = ratio < 1.0f ? ratio : 1.0f;
    reject = !(uniforms[(b * g1 + lane) * 2 + 0] < thr);
  }
  const uint64_t rej = ballot(reject);
  return rej ? (int)__builtin_ctzll(rej) : (int)gamma;
}

__device__ __forceinline__ DrawRow draw_row(const float* __restrict__ target, const float* __restrict__ draft,
                                            int draft_kind, int64_t b, int64_t B, int64_t gamma, int64_t V, int k,
                                            float inv_t, const Ws& ws) {
  const int64_t g1 = gamma + 1;
  DrawRow R;
  R.zp = target + (size_t)(b * g1 + k) * V;
  R.zq = k < gamma ? draft + (size_t)(b * gamma + k) * V : nullptr;
  R.mp = (float)ws.rm[b * g1 + k];
  R.ip = (float)(1.0 / ws.rz[b * g1 + k]);
  const bool ql = draft_kind == 0 && k < gamma;
  R.mq = ql ? (float)ws.rm[B * g1 + b * gamma + k] : 0.0f;
  R.iq = ql ? (float)(1.0 / ws.rz[B * g1 + b * gamma + k]) : 1.0f;
  R.inv_t = inv_t;
  R.q_probs = draft_kind == 1;
  return R;
}

// 3. Draw sums (T > 0): one wave per (sequence, chunk).  Every wave takes
//    the accept tests of its sequence (cheap: one value per drafted row) and
//    sums its chunk of the weights of the row where the step ends.  The
//    chunk-0 wave writes the kept prefix, the count and the probabilities.
template <bool VEC>
__global__ __launch_bounds__(kWavesPerBlock * 64) void draw_sum_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int draft_kind,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int64_t B, int64_t gamma, int64_t V,
    float inv_t, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num, float* __restrict__ out_probs,
    Ws ws) {
  constexpr int PL = kDrawChunk / 64;
  const int lane = threadIdx.x & 63;
  const int64_t ndc = draw_chunks(V);
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= B * ndc) return;
  const int64_t b = item / ndc, c = item - b * ndc;
  const int64_t g1 = gamma + 1;
  float p_x, q_x;
  const int k = first_rejection(draft, draft_kind, tokens, uniforms, b, B, gamma, V, lane, ws, p_x, q_x);
  if (c == 0) {
    if (lane < g1 && lane != k) out_tokens[b * g1 + lane] = lane < k ? clamp_token(tokens[b * gamma + lane], V) : -1;
    if (lane == 0) {
      out_num[b] = k + 1;
      ws.kb[b] = k;
    }
    if (lane < gamma && out_probs) {
      out_probs[(b * gamma + lane) * 2 + 0] = p_x;
      out_probs[(b * gamma + lane) * 2 + 1] = q_x;
    }
  }
  const DrawRow R = draw_row(target, draft, draft_kind, b, B, gamma, V, k, inv_t, ws);
  const int64_t c0 = c * kDrawChunk;
  float zp[PL], zq[PL];
  load_chunk<VEC, PL>(R.zp, V, c0, lane, -INFINITY, zp);
  if (R.zq) load_chunk<VEC, PL>(R.zq, V, c0, lane, R.q_probs ? 0.0f : -INFINITY, zq);
  double sr = 0.0, sp = 0.0;
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    float p, r;
    weights(R, zp[e], R.zq ? zq[e] : 0.0f, p, r);
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

// 4. Select (T > 0): one wave per sequence.  Chooses the residual, or p when
//    the residual has no mass or the step ends on the bonus row; finds the
//    chunk holding u*S with an fp64 prefix sum over the chunk totals, rescans
//    that chunk with an fp64 running sum in vocabulary order and writes the token.
template <bool VEC>
__global__ __launch_bounds__(kWavesPerBlock * 64) void select_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int draft_kind,
    const float* __restrict__ uniforms, int64_t B, int64_t gamma, int64_t V, float inv_t,
    int32_t* __restrict__ out_tokens, Ws ws) {
  constexpr int PL = kDrawChunk / 64;
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (b >= B) return;
  const int64_t ndc = draw_chunks(V);
  const int64_t g1 = gamma + 1;
  const int k = ws.kb[b];
  const DrawRow R = draw_row(target, draft, draft_kind, b, B, gamma, V, k, inv_t, ws);
  const double* part = ws.sres + b * ndc;
  double tot = 0.0;
  if (R.zq) {
    for (int64_t j0 = 0; j0 < ndc; j0 += 64) tot += wave_sum(j0 + lane < ndc ? part[j0 + lane] : 0.0);
  }
  const bool use_p = !(tot > 0.0);
  if (use_p) {
    part = ws.sp + b * ndc;
    tot = 0.0;
    for (int64_t j0 = 0; j0 < ndc; j0 += 64) tot += wave_sum(j0 + lane < ndc ? part[j0 + lane] : 0.0);
  }
  const float u = uniforms[(b * g1 + k) * 2 + 1];
  const double t = (double)u * tot;
  // First chunk whose running total passes t (or, if rounding leaves none,
  // the last chunk with mass).
  int64_t cs = -1, clast = 0;
  double before = 0.0, run = 0.0;
  for (int64_t j0 = 0; j0 < ndc && cs < 0; j0 += 64) {
    const double pj = j0 + lane < ndc ? part[j0 + lane] : 0.0;
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
  // Rescan: lane l takes the PL consecutive entries starting at cs*kDrawChunk + PL*l.
  const int64_t s0 = cs * kDrawChunk + (int64_t)PL * lane;
  float w[PL];
  double lsum = 0.0;
#pragma unroll
  for (int j = 0; j < PL / 4; ++j) {
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
        if (R.zq) aq[e] = v + e < V ? R.zq[v + e] : (R.q_probs ? 0.0f : -INFINITY);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float p, r;
      weights(R, ap[e], R.zq ? aq[e] : 0.0f, p, r);
      w[4 * j + e] = use_p ? p : r;
      lsum += (double)w[4 * j + e];
    }
  }
  const double incl = wave_inclusive_scan(lsum, lane);
  double C = before + (incl - lsum);
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < PL; ++e) {
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

// 2'. Greedy (T == 0): one wave per sequence; lane i holds row i's argmax.
__global__ __launch_bounds__(kWavesPerBlock * 64) void greedy_kernel(const int32_t* __restrict__ tokens, int64_t B,
                                                                      int64_t gamma, int64_t V,
                                                                      int32_t* __restrict__ out_tokens,
                                                                      int32_t* __restrict__ out_num, Ws ws) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (b >= B) return;
  const int64_t nch = stat_chunks(V);
  const int64_t g1 = gamma + 1;
  int mine = 0;
  for (int r0 = 0; r0 < g1; r0 += kRowBatch) {
    float cv[kRowBatch];
    int ci[kRowBatch];
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      cv[j] = -INFINITY;
      ci[j] = 0x7fffffff;
      if (r0 + j < g1) {
        const size_t base = (size_t)(b * g1 + r0 + j) * nch;
        for (int64_t c = lane; c < nch; c += 64) {
          const float v = ws.cmax[base + c];
          const int i = ws.cidx[base + c];
          if (v > cv[j] || (v == cv[j] && i < ci[j])) {
            cv[j] = v;
            ci[j] = i;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      if (r0 + j >= g1) break;
      wave_argmax(cv[j], ci[j]);
      if (lane == r0 + j) mine = (ci[j] >= 0 && ci[j] < V) ? ci[j] : 0;  // all-NaN row: any in-range id
    }
  }
  const bool drafted = lane < gamma;
  const int xi = drafted ? clamp_token(tokens[b * gamma + lane], V) : 0;
  const uint64_t miss = ballot(drafted && xi != mine);
  const int k = miss ? (int)__builtin_ctzll(miss) : (int)gamma;
  const int gk = __shfl(mine, k);
  if (lane < g1) out_tokens[b * g1 + lane] = lane < k ? xi : (lane == k ? gk : -1);  // gamma + 1 <= 64 lanes
  if (lane == 0) out_num[b] = k + 1;
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
  const int64_t nch = stat_chunks(a.V);
  const dim3 blk(kWavesPerBlock * 64);
  const dim3 g1(blocks_for(n_rows * nch));
#define SPECDEC_STATS(V4, GR)                                                                                      \
  hipLaunchKernelGGL((stats_kernel<V4, GR>), g1, blk, 0, stream, a.target, a.draft, n_target, n_rows, a.gamma, a.V, \
                     inv_t, ws)
  if (greedy) {
    if (vec) SPECDEC_STATS(true, true); else SPECDEC_STATS(false, true);
  } else {
    if (vec) SPECDEC_STATS(true, false); else SPECDEC_STATS(false, false);
  }
#undef SPECDEC_STATS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (greedy) {
    hipLaunchKernelGGL(greedy_kernel, dim3(blocks_for(a.B)), blk, 0, stream, a.tokens, a.B, a.gamma, a.V,
                       a.out_tokens, a.out_num, ws);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(merge_kernel, dim3(blocks_for(n_rows)), blk, 0, stream, a.target, a.draft, a.tokens, n_target,
                     n_rows, a.gamma, a.V, inv_t, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g3(blocks_for(a.B * draw_chunks(a.V)));
  if (vec)
    hipLaunchKernelGGL((draw_sum_kernel<true>), g3, blk, 0, stream, a.target, a.draft, a.draft_kind, a.tokens,
                       a.uniforms, a.B, a.gamma, a.V, inv_t, a.out_tokens, a.out_num, a.out_probs, ws);
  else
    hipLaunchKernelGGL((draw_sum_kernel<false>), g3, blk, 0, stream, a.target, a.draft, a.draft_kind, a.tokens,
                       a.uniforms, a.B, a.gamma, a.V, inv_t, a.out_tokens, a.out_num, a.out_probs, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g4(blocks_for(a.B));
  if (vec)
    hipLaunchKernelGGL((select_kernel<true>), g4, blk, 0, stream, a.target, a.draft, a.draft_kind, a.uniforms, a.B,
                       a.gamma, a.V, inv_t, a.out_tokens, ws);
  else
    hipLaunchKernelGGL((select_kernel<false>), g4, blk, 0, stream, a.target, a.draft, a.draft_kind, a.uniforms, a.B,
                       a.gamma, a.V, inv_t, a.out_tokens, ws);
  return hipGetLastError();
}

}  // namespace specdec
