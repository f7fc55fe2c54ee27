// Host-side launch interface between the C ABI (attn_api.cpp) and the kernels
// (attn_kernels.hip). Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn {

struct Problem {
  int B, S, Hq, Hkv, d;
  float scale;
  const int32_t* seqlens;  // device int32[B] or nullptr
  int causal;              // 1: keys j <= i only; 0: every key of the valid prefix
};

hipError_t launch_fwd(const Problem& pr, const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t stream);
hipError_t launch_preprocess(const Problem& pr, const void* o, const void* d_o, float* delta, hipStream_t stream);
hipError_t launch_bwd_dkdv(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, void* dk, void* dv, hipStream_t stream);
hipError_t launch_bwd_dq(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, void* dq, hipStream_t stream);

// Largest grid any launch for this problem would use (checked against the
// hardware's 2^31-1 workgroup limit by the API layer).
int64_t max_grid(const Problem& pr);

}  // namespace attn
