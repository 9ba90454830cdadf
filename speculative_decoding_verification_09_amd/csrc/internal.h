// Internal interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specdec {

// Y[n, v] = sum_k X[n, k] W[v, k]; X [N, d] bf16; W [V, d] bf16 row-major or
// in the packed tile layout; Y fp32 or bf16.
hipError_t launch_skinny_gemm(const uint16_t* X, const uint16_t* W, void* Y, int64_t N, int64_t d, int64_t V,
                              bool out_bf16, bool packed, hipStream_t stream);

namespace gemm {
// The sweep kernel (packed W, at most 8 positions, X held in LDS whole).
bool sweep_applies(int64_t N, int64_t d);
hipError_t launch_sweep(const uint16_t* X, const uint16_t* Wp, void* Y, int64_t N, int64_t d, int64_t V, bool out_bf16,
                        hipStream_t stream);
}  // namespace gemm

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
};

size_t reject_workspace_bytes(int64_t B, int64_t gamma, int64_t V);
hipError_t launch_reject_sample(const RejectArgs& a, hipStream_t stream);

}  // namespace specdec
