// C ABI of the verification step: argument checks, then launches on the
// caller's stream.  Every check runs before any HIP call, so invalid
// arguments never reach the device.  The declarations, with the meaning and
// layout of every argument, are in include/specdec.h.
#include <math.h>

#include <atomic>

#include "../../include/specdec.h"
#include "internal.h"

namespace {

constexpr int kVersion = 10300;  // 1.3.0

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Where a step's scoring scratch starts in its workspace: after the sampling
// arrays, rounded up to 256 bytes.
size_t stats_scratch_offset(size_t sampling_bytes) { return (sampling_bytes + 255) & ~(size_t)255; }

// Largest sizes the kernels index with 32-bit arithmetic in places.
constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxRows = (int64_t)1 << 26;

int check_logits_shape(int64_t N, int64_t d, int64_t V, int weight_layout) {
  if (weight_layout != SPECDEC_WEIGHTS_ROW_MAJOR && weight_layout != SPECDEC_WEIGHTS_PACKED) return SPECDEC_ERR_ARG;
  if (N < 1 || N > kMaxRows || d < 8 || d % 8 != 0 || d > kMaxDim || V < 1 || V > kMaxDim) return SPECDEC_ERR_SHAPE;
  if (weight_layout == SPECDEC_WEIGHTS_PACKED && d % 32 != 0) return SPECDEC_ERR_SHAPE;
  if ((size_t)N * (size_t)V > ((size_t)1 << 40) || (size_t)V * (size_t)d > ((size_t)1 << 40)) return SPECDEC_ERR_SHAPE;
  return SPECDEC_OK;
}

// y_optional: Y may be NULL (a greedy step whose scoring kernel takes the
// argmax itself and stores no scores).
int check_logits_args(const void* X, const void* W, const void* Y, int64_t N, int64_t d, int64_t V, int out_dtype,
                      int weight_layout, bool y_optional = false) {
  if (!X || !W || (!Y && !y_optional)) return SPECDEC_ERR_NULL;
  const int st = check_logits_shape(N, d, V, weight_layout);
  if (st != SPECDEC_OK) return st;
  if (out_dtype != SPECDEC_OUT_F32 && out_dtype != SPECDEC_OUT_BF16) return SPECDEC_ERR_ARG;
  if (!aligned16(X) || !aligned16(W)) return SPECDEC_ERR_ALIGN;
  if (V % 4 == 0) {
    const size_t es = out_dtype == SPECDEC_OUT_F32 ? 16 : 8;
    if (((uintptr_t)Y % es) != 0) return SPECDEC_ERR_ALIGN;
  } else if (((uintptr_t)Y % (out_dtype == SPECDEC_OUT_F32 ? 4 : 2)) != 0) {
    return SPECDEC_ERR_ALIGN;
  }
  return SPECDEC_OK;
}

int check_reject_args(const float* target, const float* draft, int draft_kind, const int32_t* tokens, float T,
                      const float* uniforms, int64_t B, int64_t gamma, int64_t V, const int32_t* out_tokens,
                      const int32_t* out_num, const float* out_probs, const void* ws, size_t ws_bytes,
                      bool target_optional = false) {
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA || V < 1 || V > kMaxDim)
    return SPECDEC_ERR_SHAPE;
  if ((size_t)B * (size_t)(gamma + 1) * (size_t)V > ((size_t)1 << 40)) return SPECDEC_ERR_SHAPE;
  if (draft_kind != SPECDEC_DRAFT_LOGITS && draft_kind != SPECDEC_DRAFT_PROBS && draft_kind != SPECDEC_DRAFT_ONEHOT)
    return SPECDEC_ERR_ARG;
  if (isnan(T) || T < 0.0f || isinf(T)) return SPECDEC_ERR_TEMPERATURE;
  const bool greedy = T == 0.0f;
  if ((!target && !target_optional) || !out_tokens || !out_num) return SPECDEC_ERR_NULL;
  if (gamma > 0 && !tokens) return SPECDEC_ERR_NULL;
  if (!greedy && !uniforms) return SPECDEC_ERR_NULL;
  if (!greedy && gamma > 0 && draft_kind != SPECDEC_DRAFT_ONEHOT && !draft) return SPECDEC_ERR_NULL;
  if (!aligned16(target) || (draft && !aligned16(draft))) return SPECDEC_ERR_ALIGN;
  if (((uintptr_t)out_tokens & 3) || ((uintptr_t)out_num & 3) || (tokens && ((uintptr_t)tokens & 3)) ||
      (uniforms && ((uintptr_t)uniforms & 3)) || (out_probs && ((uintptr_t)out_probs & 3)))
    return SPECDEC_ERR_ALIGN;
  const size_t need = specdec::reject_workspace_bytes(B, gamma, V);
  if (!ws || ws_bytes < need) return SPECDEC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SPECDEC_ERR_ALIGN;
  return SPECDEC_OK;
}

specdec::RejectArgs reject_args(const float* target, const float* draft, int draft_kind, const int32_t* tokens,
                                float T, const float* uniforms, int64_t B, int64_t gamma, int64_t V,
                                int32_t* out_tokens, int32_t* out_num, float* out_probs, void* ws, size_t ws_bytes) {
  specdec::RejectArgs a;
  a.target = target;
  a.draft = draft;
  a.draft_kind = draft_kind;
  a.tokens = tokens;
  a.temperature = T;
  a.uniforms = uniforms;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.out_tokens = out_tokens;
  a.out_num = out_num;
  a.out_probs = T == 0.0f ? nullptr : out_probs;
  a.workspace = ws;
  a.workspace_bytes = ws_bytes;
  a.top_k = 0;
  a.top_p = 1.0f;
  return a;
}

// top_k >= 0 (0: off); 0 < top_p <= 1.  The cut kernel ranks entries by a
// composite of key and index and sums fixed-point masses, both exact for
// V <= 2^23.
int check_warp_args(int64_t top_k, float top_p, int64_t V) {
  if (top_k < 0 || !(top_p > 0.0f && top_p <= 1.0f)) return SPECDEC_ERR_ARG;
  if (((top_k > 0 && top_k < V) || top_p < 1.0f) && V > ((int64_t)1 << 23)) return SPECDEC_ERR_SHAPE;
  return SPECDEC_OK;
}

// Partials per row that the scoring kernel of a step of this shape forms
// itself (0: a separate statistics pass reads the logits back).  required: the
// step keeps no logits, so the epilogue is taken wherever it can be formed.
int64_t step_fused_parts(int64_t B, int64_t gamma, int64_t d, int64_t V, int weight_layout, bool required) {
  if (weight_layout != SPECDEC_WEIGHTS_PACKED) return 0;
  const int64_t pstride = specdec::reject_fusable_stride(B, gamma, V);
  return pstride > 0 ? specdec::gemm_stats_parts(B * (gamma + 1), d, V, pstride, required) : 0;
}

}  // namespace

extern "C" {

const char* specdec_status_string(int status) {
  switch (status) {
    case SPECDEC_OK: return "ok";
    case SPECDEC_ERR_NULL: return "a required pointer is NULL";
    case SPECDEC_ERR_SHAPE: return "a size is out of range";
    case SPECDEC_ERR_ALIGN: return "a pointer is not aligned as required";
    case SPECDEC_ERR_TEMPERATURE: return "temperature must be finite and >= 0";
    case SPECDEC_ERR_WORKSPACE: return "workspace is NULL or too small";
    case SPECDEC_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case SPECDEC_ERR_ARG: return "an enumerated argument has an unknown value";
    case SPECDEC_ERR_SCRATCH:
      return "the shape needs more workspace than the library's static device buffer holds (use the entry point "
             "that takes a workspace)";
    case SPECDEC_ERR_DEVICE: return "the HIP runtime could not report the current device or its buffer";
    default: return "unknown status";
  }
}

int specdec_version(void) { return kVersion; }

size_t specdec_workspace_bytes(int64_t B, int64_t gamma, int64_t V) {
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA || V < 1 || V > kMaxDim) return 0;
  return specdec::reject_workspace_bytes(B, gamma, V);
}

size_t specdec_packed_weight_bytes(int64_t V, int64_t d) {
  if (V < 1 || V > kMaxDim || d < 32 || d % 32 != 0 || d > kMaxDim) return 0;
  if ((size_t)V * (size_t)d > ((size_t)1 << 40)) return 0;
  return (size_t)specdec::packed_weight_elems(V, d) * sizeof(uint16_t);
}

int specdec_pack_weights(const void* W, void* W_packed, int64_t V, int64_t d, void* stream) {
  if (!W || !W_packed) return SPECDEC_ERR_NULL;
  if (specdec_packed_weight_bytes(V, d) == 0) return SPECDEC_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(W_packed)) return SPECDEC_ERR_ALIGN;
  const hipError_t e =
      specdec::launch_pack_weights((const uint16_t*)W, (uint16_t*)W_packed, V, d, (hipStream_t)stream);
  return e == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

size_t specdec_logits_workspace_bytes(int64_t N, int64_t d, int64_t V, int weight_layout) {
  if (check_logits_shape(N, d, V, weight_layout) != SPECDEC_OK) return 0;
  return specdec::gemm_workspace_bytes(N, d, V, weight_layout == SPECDEC_WEIGHTS_PACKED);
}

size_t specdec_step_workspace_bytes(int64_t B, int64_t gamma, int64_t d, int64_t V, int weight_layout) {
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA || V < 1 || V > kMaxDim) return 0;
  const int64_t N = B * (gamma + 1);
  if (check_logits_shape(N, d, V, weight_layout) != SPECDEC_OK) return 0;
  const bool packed = weight_layout == SPECDEC_WEIGHTS_PACKED;
  // The fused path keeps the scoring kernel's scratch after the sampling
  // arrays; the unfused one runs the two passes one after the other.
  const size_t r = stats_scratch_offset(specdec::reject_workspace_bytes(B, gamma, V)) +
                   (packed ? specdec::gemm_stats_scratch_bytes(N, d, V) : 0);
  const size_t g = specdec::gemm_workspace_bytes(N, d, V, packed);
  return r > g ? r : g;
}

int specdec_step_options(int64_t B, int64_t gamma, int64_t d, int64_t V, int weight_layout) {
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA || V < 1 || V > kMaxDim) return 0;
  if (check_logits_shape(B * (gamma + 1), d, V, weight_layout) != SPECDEC_OK) return 0;
  int flags = 0;
  if (step_fused_parts(B, gamma, d, V, weight_layout, false) > 0) flags |= SPECDEC_STEP_FUSED_STATISTICS;
  if (step_fused_parts(B, gamma, d, V, weight_layout, true) > 0) flags |= SPECDEC_STEP_GREEDY_WITHOUT_LOGITS;
  return flags;
}

const char* specdec_scoring_kernel(int64_t N, int64_t d, int64_t V, int weight_layout) {
  if (check_logits_shape(N, d, V, weight_layout) != SPECDEC_OK) return "";
  return specdec::scoring_kernel_name(N, d, V, weight_layout == SPECDEC_WEIGHTS_PACKED);
}

int specdec_verify_logits(const void* X, const void* W, void* Y, int64_t N, int64_t d, int64_t V, int out_dtype,
                          int weight_layout, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_logits_args(X, W, Y, N, d, V, out_dtype, weight_layout);
  if (st != SPECDEC_OK) return st;
  const bool packed = weight_layout == SPECDEC_WEIGHTS_PACKED;
  const size_t need = specdec::gemm_workspace_bytes(N, d, V, packed);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SPECDEC_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return SPECDEC_ERR_ALIGN;
  const hipError_t e = specdec::launch_skinny_gemm((const uint16_t*)X, (const uint16_t*)W, Y, N, d, V,
                                                   out_dtype == SPECDEC_OUT_BF16, packed, workspace,
                                                   (hipStream_t)stream);
  return e == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

int specdec_reject_sample(const float* target_logits, const float* draft, int draft_kind,
                          const int32_t* draft_tokens, float temperature, const float* uniforms, int64_t B,
                          int64_t gamma, int64_t V, int32_t* out_tokens, int32_t* out_num_emitted,
                          float* out_probs, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_reject_args(target_logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma, V,
                                   out_tokens, out_num_emitted, out_probs, workspace, workspace_bytes);
  if (st != SPECDEC_OK) return st;
  const specdec::RejectArgs a = reject_args(target_logits, draft, draft_kind, draft_tokens, temperature, uniforms, B,
                                            gamma, V, out_tokens, out_num_emitted, out_probs, workspace,
                                            workspace_bytes);
  const hipError_t e = specdec::launch_reject_sample(a, (hipStream_t)stream);
  return e == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

int specdec_reject_sample_warped(const float* target_logits, const float* draft, int draft_kind,
                                 const int32_t* draft_tokens, float temperature, int64_t top_k, float top_p,
                                 const float* uniforms, int64_t B, int64_t gamma, int64_t V, int32_t* out_tokens,
                                 int32_t* out_num_emitted, float* out_probs, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  int st = check_reject_args(target_logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma, V,
                             out_tokens, out_num_emitted, out_probs, workspace, workspace_bytes);
  if (st != SPECDEC_OK) return st;
  st = check_warp_args(top_k, top_p, V);
  if (st != SPECDEC_OK) return st;
  specdec::RejectArgs a = reject_args(target_logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma,
                                      V, out_tokens, out_num_emitted, out_probs, workspace, workspace_bytes);
  a.top_k = top_k;
  a.top_p = top_p;
  const hipError_t e = specdec::launch_reject_sample(a, (hipStream_t)stream);
  return e == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

int specdec_verify_step_warped(const void* X, const void* W, int weight_layout, const float* draft, int draft_kind,
                               const int32_t* draft_tokens, float temperature, int64_t top_k, float top_p,
                               const float* uniforms, int64_t B, int64_t gamma, int64_t d, int64_t V, float* logits,
                               int32_t* out_tokens, int32_t* out_num_emitted, float* out_probs, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA) return SPECDEC_ERR_SHAPE;
  const int64_t N = B * (gamma + 1);
  int st = check_logits_args(X, W, logits, N, d, V, SPECDEC_OUT_F32, weight_layout);
  if (st != SPECDEC_OK) return st;
  st = check_reject_args(logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma, V, out_tokens,
                         out_num_emitted, out_probs, workspace, workspace_bytes);
  if (st != SPECDEC_OK) return st;
  st = check_warp_args(top_k, top_p, V);
  if (st != SPECDEC_OK) return st;
  if (workspace_bytes < specdec_step_workspace_bytes(B, gamma, d, V, weight_layout)) return SPECDEC_ERR_WORKSPACE;
  specdec::RejectArgs a = reject_args(logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma, V,
                                      out_tokens, out_num_emitted, out_probs, workspace, workspace_bytes);
  a.top_k = top_k;
  a.top_p = top_p;
  if (!specdec::warp_active(a))  // nothing to warp (T == 0, or both settings off): the plain step
    return specdec_verify_step(X, W, weight_layout, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma,
                               d, V, logits, out_tokens, out_num_emitted, out_probs, workspace, workspace_bytes,
                               stream);
  // The cuts need whole rows, so the scores are written first and the
  // statistics pass reads them back.
  if (specdec_verify_logits(X, W, logits, N, d, V, SPECDEC_OUT_F32, weight_layout, workspace, workspace_bytes,
                            stream) != SPECDEC_OK)
    return SPECDEC_ERR_LAUNCH;
  return specdec::launch_reject_sample(a, (hipStream_t)stream) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

int specdec_verify_step(const void* X, const void* W, int weight_layout, const float* draft, int draft_kind,
                        const int32_t* draft_tokens, float temperature, const float* uniforms, int64_t B,
                        int64_t gamma, int64_t d, int64_t V, float* logits, int32_t* out_tokens,
                        int32_t* out_num_emitted, float* out_probs, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA) return SPECDEC_ERR_SHAPE;
  const int64_t N = B * (gamma + 1);
  // No logits: allowed for a greedy step whose scoring kernel takes the argmax
  // itself (checked once the sizes are known to be valid).
  const bool no_logits = logits == nullptr;
  int st = check_logits_args(X, W, logits, N, d, V, SPECDEC_OUT_F32, weight_layout, no_logits);
  if (st != SPECDEC_OK) return st;
  st = check_reject_args(logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma, V, out_tokens,
                         out_num_emitted, out_probs, workspace, workspace_bytes, no_logits);
  if (st != SPECDEC_OK) return st;
  if (no_logits && (temperature != 0.0f || step_fused_parts(B, gamma, d, V, weight_layout, true) == 0))
    return SPECDEC_ERR_NULL;
  if (workspace_bytes < specdec_step_workspace_bytes(B, gamma, d, V, weight_layout)) return SPECDEC_ERR_WORKSPACE;
  const specdec::RejectArgs a = reject_args(logits, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma,
                                            V, out_tokens, out_num_emitted, out_probs, workspace, workspace_bytes);
  const hipStream_t s = (hipStream_t)stream;
  // Packed weights: the scoring kernel also forms the softmax (or argmax)
  // partials of every target row, so no separate statistics pass reads the
  // logits again.
  specdec::FusedStats fs;
  if (weight_layout == SPECDEC_WEIGHTS_PACKED && specdec::reject_fused_stats(a, &fs) &&
      specdec::gemm_stats_parts(N, d, V, fs.pstride, no_logits) > 0) {
    int64_t nparts = 0, nparts_draft = 0;
    void* scratch = (char*)workspace + stats_scratch_offset(specdec::reject_workspace_bytes(B, gamma, V));
    if (specdec::launch_gemm_with_stats((const uint16_t*)X, (const uint16_t*)W, logits, N, d, V, fs, &nparts,
                                        &nparts_draft, scratch, s, no_logits) != hipSuccess)
      return SPECDEC_ERR_LAUNCH;
    return specdec::launch_reject_after_fused(a, nparts, nparts_draft, s) == hipSuccess ? SPECDEC_OK
                                                                                         : SPECDEC_ERR_LAUNCH;
  }
  // The scoring pass finishes (stream order) before the sampling kernels reuse the workspace.
  if (specdec_verify_logits(X, W, logits, N, d, V, SPECDEC_OUT_F32, weight_layout, workspace, workspace_bytes,
                            stream) != SPECDEC_OK)
    return SPECDEC_ERR_LAUNCH;
  return specdec::launch_reject_sample(a, s) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// The static device buffer of specdec_verify_step_noalloc: file-scope device
// memory, one copy on every GPU the library runs on, zero when the code object
// is loaded and held until the process ends.  In host code `scratch` names a
// host-side stand-in; its device address on the current device comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// the kernels.
constexpr size_t kStaticScratchBytes = SPECDEC_NOALLOC_MAX_WORKSPACE;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // per device, null until looked up

// The current device's address of `scratch` (looked up on the first call on
// that device), or null when the runtime cannot give it.
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Two host threads may both look it up: they get the same address.
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int specdec_verify_step_noalloc(const void* X, const void* W, int weight_layout, const float* draft, int draft_kind,
                                const int32_t* draft_tokens, float temperature, const float* uniforms, int64_t B,
                                int64_t gamma, int64_t d, int64_t V, float* logits, int32_t* out_tokens,
                                int32_t* out_num_emitted, float* out_probs, void* stream) {
  // Sizes first, without touching the device: a shape whose workspace does
  // not fit the static buffer is refused before anything else.
  if (B < 1 || B > kMaxRows || gamma < 0 || gamma > SPECDEC_MAX_GAMMA) return SPECDEC_ERR_SHAPE;
  const size_t need = specdec_step_workspace_bytes(B, gamma, d, V, weight_layout);
  if (need == 0) {
    const int st = check_logits_shape(B * (gamma + 1), d, V, weight_layout);
    return st != SPECDEC_OK ? st : SPECDEC_ERR_SHAPE;
  }
  if (need > kStaticScratchBytes) return SPECDEC_ERR_SCRATCH;
  void* ws = static_scratch();
  if (ws == nullptr) return SPECDEC_ERR_DEVICE;
  return specdec_verify_step(X, W, weight_layout, draft, draft_kind, draft_tokens, temperature, uniforms, B, gamma, d,
                             V, logits, out_tokens, out_num_emitted, out_probs, ws, kStaticScratchBytes, stream);
}

size_t specdec_tree_workspace_bytes(int64_t B, int64_t M, int64_t V) {
  if (B < 1 || B > kMaxRows || M < 1 || M > SPECDEC_MAX_TREE_NODES || V < 1 || V > kMaxDim) return 0;
  return specdec::tree_workspace_bytes(B, M, V);
}

int specdec_tree_mask(const int32_t* parents, int64_t B, int64_t M, uint64_t* out_mask, int32_t* out_depth,
                      float* out_additive, void* stream) {
  if (!parents || !out_mask || !out_depth) return SPECDEC_ERR_NULL;
  if (B < 1 || B > kMaxRows || M < 1 || M > SPECDEC_MAX_TREE_NODES) return SPECDEC_ERR_SHAPE;
  if (((uintptr_t)parents & 3) || ((uintptr_t)out_mask & 7) || ((uintptr_t)out_depth & 3) ||
      ((uintptr_t)out_additive & 3))
    return SPECDEC_ERR_ALIGN;
  return specdec::launch_tree_mask(parents, B, M, out_mask, out_depth, out_additive, (hipStream_t)stream) ==
                 hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

namespace {
int check_tree_args(const void* logits, const int32_t* parents, const int32_t* node_tokens, int64_t B, int64_t M,
                    int64_t V, const int32_t* out_tokens, const int32_t* out_num, const int32_t* out_nodes,
                    const void* ws, size_t ws_bytes) {
  if (!logits || !parents || !node_tokens || !out_tokens || !out_num || !out_nodes) return SPECDEC_ERR_NULL;
  if (B < 1 || B > kMaxRows || M < 1 || M > SPECDEC_MAX_TREE_NODES || V < 1 || V > kMaxDim) return SPECDEC_ERR_SHAPE;
  if ((size_t)B * (size_t)M * (size_t)V > ((size_t)1 << 40)) return SPECDEC_ERR_SHAPE;
  if (!aligned16(logits) || ((uintptr_t)parents & 3) || ((uintptr_t)node_tokens & 3) || ((uintptr_t)out_tokens & 3) ||
      ((uintptr_t)out_num & 3) || ((uintptr_t)out_nodes & 3))
    return SPECDEC_ERR_ALIGN;
  if (!ws || ws_bytes < specdec::tree_workspace_bytes(B, M, V)) return SPECDEC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SPECDEC_ERR_ALIGN;
  return SPECDEC_OK;
}

specdec::TreeArgs tree_args(const float* logits, const int32_t* parents, const int32_t* node_tokens, int64_t B,
                            int64_t M, int64_t V, int32_t* out_tokens, int32_t* out_num, int32_t* out_nodes,
                            void* ws) {
  specdec::TreeArgs t;
  t.logits = logits;
  t.parents = parents;
  t.node_tokens = node_tokens;
  t.B = B;
  t.M = M;
  t.V = V;
  t.out_tokens = out_tokens;
  t.out_num = out_num;
  t.out_nodes = out_nodes;
  t.workspace = ws;
  return t;
}
}  // namespace

int specdec_tree_verify_greedy(const float* target_logits, const int32_t* parents, const int32_t* node_tokens,
                               int64_t B, int64_t M, int64_t V, int32_t* out_tokens, int32_t* out_num_emitted,
                               int32_t* out_nodes, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_tree_args(target_logits, parents, node_tokens, B, M, V, out_tokens, out_num_emitted, out_nodes,
                                 workspace, workspace_bytes);
  if (st != SPECDEC_OK) return st;
  const specdec::TreeArgs t =
      tree_args(target_logits, parents, node_tokens, B, M, V, out_tokens, out_num_emitted, out_nodes, workspace);
  return specdec::launch_tree_greedy(t, 0, (hipStream_t)stream) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

size_t specdec_tree_step_workspace_bytes(int64_t B, int64_t M, int64_t d, int64_t V, int weight_layout) {
  if (B < 1 || B > kMaxRows || M < 1 || M > SPECDEC_MAX_TREE_NODES || V < 1 || V > kMaxDim) return 0;
  if (check_logits_shape(B * M, d, V, weight_layout) != SPECDEC_OK) return 0;
  const bool packed = weight_layout == SPECDEC_WEIGHTS_PACKED;
  const size_t r = stats_scratch_offset(specdec::tree_workspace_bytes(B, M, V)) +
                   (packed ? specdec::gemm_stats_scratch_bytes(B * M, d, V) : 0);
  const size_t g = specdec::gemm_workspace_bytes(B * M, d, V, packed);
  return r > g ? r : g;
}

int specdec_tree_verify_step(const void* X, const void* W, int weight_layout, const int32_t* parents,
                             const int32_t* node_tokens, int64_t B, int64_t M, int64_t d, int64_t V, float* logits,
                             int32_t* out_tokens, int32_t* out_num_emitted, int32_t* out_nodes, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (B < 1 || B > kMaxRows || M < 1 || M > SPECDEC_MAX_TREE_NODES) return SPECDEC_ERR_SHAPE;
  const int64_t N = B * M;
  const bool no_logits = logits == nullptr;  // allowed where the scoring kernel takes the argmax itself
  int st = check_logits_args(X, W, logits, N, d, V, SPECDEC_OUT_F32, weight_layout, no_logits);
  if (st != SPECDEC_OK) return st;
  // The tree checks want a logits pointer; without logits, X stands in for it (it is not read there).
  st = check_tree_args(no_logits ? X : logits, parents, node_tokens, B, M, V, out_tokens, out_num_emitted, out_nodes,
                       workspace, workspace_bytes);
  if (st != SPECDEC_OK) return st;
  if (workspace_bytes < specdec_tree_step_workspace_bytes(B, M, d, V, weight_layout)) return SPECDEC_ERR_WORKSPACE;
  const specdec::TreeArgs t =
      tree_args(logits, parents, node_tokens, B, M, V, out_tokens, out_num_emitted, out_nodes, workspace);
  const hipStream_t s = (hipStream_t)stream;
  specdec::FusedStats fs;
  const bool fused = weight_layout == SPECDEC_WEIGHTS_PACKED && specdec::tree_fused_stats(t, &fs) &&
                     specdec::gemm_stats_parts(N, d, V, fs.pstride, no_logits) > 0;
  if (no_logits && !fused) return SPECDEC_ERR_NULL;
  if (fused) {
    int64_t nparts = 0, nparts_draft = 0;
    void* scratch = (char*)workspace + stats_scratch_offset(specdec::tree_workspace_bytes(B, M, V));
    if (specdec::launch_gemm_with_stats((const uint16_t*)X, (const uint16_t*)W, logits, N, d, V, fs, &nparts,
                                        &nparts_draft, scratch, s, no_logits) != hipSuccess)
      return SPECDEC_ERR_LAUNCH;
    return specdec::launch_tree_greedy(t, nparts, s) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
  }
  if (specdec_verify_logits(X, W, logits, N, d, V, SPECDEC_OUT_F32, weight_layout, workspace, workspace_bytes,
                            stream) != SPECDEC_OK)
    return SPECDEC_ERR_LAUNCH;
  return specdec::launch_tree_greedy(t, 0, s) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

/* ---- paged KV cache ---- */

namespace {
int check_kv(const void* kpool, const void* vpool, const int32_t* tables, const int32_t* lens, const int32_t* stack,
             const int32_t* top, const int32_t* status, int64_t R, int64_t num_blocks, int64_t heads,
             int64_t block_size, int64_t head_dim, int64_t elem, int64_t max_blocks, bool need_pools) {
  if ((need_pools && (!kpool || !vpool)) || !tables || !lens || !stack || !top || !status) return SPECDEC_ERR_NULL;
  if (R < 1 || R > kMaxRows || num_blocks < 1 || num_blocks > ((int64_t)1 << 30) || heads < 1 || heads > 4096 ||
      block_size < 1 || block_size > 4096 || head_dim < 1 || head_dim > 65536 || max_blocks < 1 ||
      max_blocks > ((int64_t)1 << 24) || (elem != 2 && elem != 4))
    return SPECDEC_ERR_SHAPE;
  if ((head_dim * elem) % 16 != 0) return SPECDEC_ERR_SHAPE;
  if ((size_t)R * (size_t)max_blocks > ((size_t)1 << 31) ||
      (size_t)num_blocks * heads * block_size * head_dim * elem > ((size_t)1 << 44))
    return SPECDEC_ERR_SHAPE;
  if ((need_pools && (!aligned16(kpool) || !aligned16(vpool))) || ((uintptr_t)tables & 3) || ((uintptr_t)lens & 3) ||
      ((uintptr_t)stack & 3) || ((uintptr_t)top & 3) || ((uintptr_t)status & 3))
    return SPECDEC_ERR_ALIGN;
  return SPECDEC_OK;
}

specdec::KvArgs kv_args(void* kpool, void* vpool, int32_t* tables, int32_t* lens, int32_t* stack, int32_t* top,
                        int32_t* status, int64_t R, int64_t num_blocks, int64_t heads, int64_t block_size,
                        int64_t head_dim, int64_t elem, int64_t max_blocks) {
  specdec::KvArgs a;
  a.kpool = kpool;
  a.vpool = vpool;
  a.tables = tables;
  a.lens = lens;
  a.stack = stack;
  a.top = top;
  a.status = status;
  a.R = R;
  a.num_blocks = num_blocks;
  a.heads = heads;
  a.block_size = block_size;
  a.head_dim = head_dim;
  a.elem = elem;
  a.max_blocks = max_blocks;
  return a;
}
}  // namespace

int specdec_kv_init(int32_t* free_stack, int32_t* free_top, int32_t* seq_lens, int64_t R, int64_t num_blocks,
                    void* stream) {
  if (!free_stack || !free_top || !seq_lens) return SPECDEC_ERR_NULL;
  if (R < 1 || R > kMaxRows || num_blocks < 1 || num_blocks > ((int64_t)1 << 30)) return SPECDEC_ERR_SHAPE;
  if (((uintptr_t)free_stack & 3) || ((uintptr_t)free_top & 3) || ((uintptr_t)seq_lens & 3)) return SPECDEC_ERR_ALIGN;
  return specdec::launch_kv_init(free_stack, free_top, seq_lens, R, num_blocks, (hipStream_t)stream) == hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

size_t specdec_kv_workspace_bytes(int64_t R) {
  if (R < 1 || R > kMaxRows) return 0;
  return ((size_t)R * sizeof(int32_t) + 15) & ~(size_t)15;
}

int specdec_kv_append(void* k_pool, void* v_pool, int32_t* block_tables, int32_t* seq_lens, int32_t* free_stack,
                      int32_t* free_top, int32_t* status, const void* k_new, const void* v_new, int64_t R,
                      int64_t n_new, int64_t num_blocks, int64_t heads, int64_t block_size, int64_t head_dim,
                      int64_t elem_bytes, int64_t max_blocks, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_kv(k_pool, v_pool, block_tables, seq_lens, free_stack, free_top, status, R, num_blocks, heads,
                    block_size, head_dim, elem_bytes, max_blocks, true);
  if (st != SPECDEC_OK) return st;
  if (!k_new || !v_new) return SPECDEC_ERR_NULL;
  if (n_new < 1 || n_new > ((int64_t)1 << 20)) return SPECDEC_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new)) return SPECDEC_ERR_ALIGN;
  if (!workspace || workspace_bytes < specdec_kv_workspace_bytes(R)) return SPECDEC_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 3)) return SPECDEC_ERR_ALIGN;
  const specdec::KvArgs a = kv_args(k_pool, v_pool, block_tables, seq_lens, free_stack, free_top, status, R,
                                    num_blocks, heads, block_size, head_dim, elem_bytes, max_blocks);
  return specdec::launch_kv_append(a, k_new, v_new, n_new, (int32_t*)workspace, (hipStream_t)stream) == hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

int specdec_kv_rollback(int32_t* block_tables, int32_t* seq_lens, int32_t* free_stack, int32_t* free_top,
                        int32_t* status, const int32_t* keep_lens, int64_t R, int64_t num_blocks, int64_t block_size,
                        int64_t max_blocks, void* stream) {
  int st = check_kv(nullptr, nullptr, block_tables, seq_lens, free_stack, free_top, status, R, num_blocks, 1,
                    block_size, 4, 4, max_blocks, false);
  if (st != SPECDEC_OK) return st;
  if (!keep_lens) return SPECDEC_ERR_NULL;
  if (((uintptr_t)keep_lens & 3)) return SPECDEC_ERR_ALIGN;
  const specdec::KvArgs a = kv_args(nullptr, nullptr, block_tables, seq_lens, free_stack, free_top, status, R,
                                    num_blocks, 1, block_size, 4, 4, max_blocks);
  return specdec::launch_kv_rollback(a, keep_lens, nullptr, 0, (hipStream_t)stream) == hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

int specdec_kv_rollback_after_verify(int32_t* block_tables, int32_t* seq_lens, int32_t* free_stack,
                                     int32_t* free_top, int32_t* status, const int32_t* num_emitted, int64_t gamma,
                                     int64_t R, int64_t num_blocks, int64_t block_size, int64_t max_blocks,
                                     void* stream) {
  int st = check_kv(nullptr, nullptr, block_tables, seq_lens, free_stack, free_top, status, R, num_blocks, 1,
                    block_size, 4, 4, max_blocks, false);
  if (st != SPECDEC_OK) return st;
  if (!num_emitted) return SPECDEC_ERR_NULL;
  if (gamma < 0 || gamma > SPECDEC_MAX_GAMMA) return SPECDEC_ERR_SHAPE;
  if (((uintptr_t)num_emitted & 3)) return SPECDEC_ERR_ALIGN;
  const specdec::KvArgs a = kv_args(nullptr, nullptr, block_tables, seq_lens, free_stack, free_top, status, R,
                                    num_blocks, 1, block_size, 4, 4, max_blocks);
  return specdec::launch_kv_rollback(a, nullptr, num_emitted, gamma, (hipStream_t)stream) == hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

int specdec_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                      int64_t R, int64_t num_blocks, int64_t heads, int64_t block_size, int64_t head_dim,
                      int64_t elem_bytes, int64_t max_blocks, int64_t max_len, void* k_out, void* v_out,
                      void* stream) {
  // The stack pointers are not used here: pass the tables for the null checks.
  int st = check_kv(k_pool, v_pool, block_tables, seq_lens, (const int32_t*)block_tables, (const int32_t*)seq_lens,
                    (const int32_t*)seq_lens, R, num_blocks, heads, block_size, head_dim, elem_bytes, max_blocks, true);
  if (st != SPECDEC_OK) return st;
  if (!k_out || !v_out) return SPECDEC_ERR_NULL;
  if (max_len < 1 || max_len > ((int64_t)1 << 24)) return SPECDEC_ERR_SHAPE;
  if (max_len * (head_dim * elem_bytes / 16) > ((int64_t)1 << 30)) return SPECDEC_ERR_SHAPE;  // 32-bit unit index
  if (!aligned16(k_out) || !aligned16(v_out)) return SPECDEC_ERR_ALIGN;
  const specdec::KvArgs a = kv_args((void*)k_pool, (void*)v_pool, (int32_t*)block_tables, (int32_t*)seq_lens, nullptr,
                                    nullptr, nullptr, R, num_blocks, heads, block_size, head_dim, elem_bytes,
                                    max_blocks);
  return specdec::launch_kv_gather(a, max_len, k_out, v_out, (hipStream_t)stream) == hipSuccess ? SPECDEC_OK
                                                                                                : SPECDEC_ERR_LAUNCH;
}

}  // extern "C"
