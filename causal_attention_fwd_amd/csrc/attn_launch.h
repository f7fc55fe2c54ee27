// Host-side launch interface between the C ABI (attn_api.cpp) and the kernels
// (attn_kernels.hip). Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Element strides of a [B, S, H, d] tensor (d contiguous).
struct Strides {
  int64_t b, s, h;
};

struct Problem {
  int B, S, Hq, Hkv, d;
  float scale;
  const int32_t* seqlens;  // device int32[B] or nullptr
  int causal;              // 1: keys j <= i only; 0: every key of the valid prefix
  float rope_base;         // > 0: rotary embedding base (q, k rotated); 0: none
  Strides sq, skv, so;     // Q (and q_rot); K, V, dK, dV (and k_rot); O, dO, dQ
};

hipError_t launch_fwd(const Problem& pr, const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t stream);
hipError_t launch_rope(const Problem& pr, const void* q, const void* k, void* q_rot, void* k_rot,
                       hipStream_t stream);
hipError_t launch_preprocess(const Problem& pr, const void* o, const void* d_o, float* delta, hipStream_t stream);
// workspace: bwd_workspace_bytes(pr) bytes (may be null when that is 0)
hipError_t launch_bwd_dkdv(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, void* dk, void* dv, void* workspace,
                           hipStream_t stream);
hipError_t launch_bwd_dq(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, void* dq, hipStream_t stream);
// The dQ pass computing D = rowsum(dO * O) itself (written to delta) instead
// of reading it: the backward preprocess folded into the dQ pass.
hipError_t launch_bwd_dq_with_delta(const Problem& pr, const void* q, const void* k, const void* v,
                                    const void* o, const void* d_o, const float* lse, float* delta, void* dq,
                                    hipStream_t stream);

// Largest grid any launch for this problem would use (checked against the
// hardware's 2^31-1 workgroup limit by the API layer).
int64_t max_grid(const Problem& pr);

// Workgroups per 128-key block of the dK/dV pass, on average (1: no split).
// When the key blocks alone would leave CUs idle, the (head, query tile)
// iterations of the blocks are shared by several workgroups (dealt by
// dkdv_part_base) whose fp32 partial sums are added by a reduce pass.
int dkdv_parts(const Problem& pr);

// With a split, each (sequence, kv head) unit's parts * nkb workgroups are
// dealt to its nkb key blocks in proportion to the blocks' (head, query tile)
// iterations, at least one each: under the causal mask block k meets
// ceil(S/64) - 2k query tiles, so the first blocks get more workgroups and
// every workgroup about the same number of iterations. Returns the index of
// key block kb's first workgroup within the unit (kb = nkb gives the total);
// bidirectional blocks all have the same work and the deal is even. Shared by
// the planner (workspace size), the dK/dV pass and its reduce pass.
__host__ __device__ inline int dkdv_part_base(int kb, int nkb, int parts, int S, int causal) {
  const int64_t n64 = ((int64_t)S + 63) / 64;
  const int64_t before = causal ? (int64_t)kb * n64 - (int64_t)kb * (kb - 1) : kb;
  const int64_t all = causal ? (int64_t)nkb * n64 - (int64_t)nkb * (nkb - 1) : nkb;
  return kb + (int)((int64_t)(parts - 1) * nkb * before / all);
}

// 128-key blocks of the dK/dV pass, and the largest number of parts a block
// is split into: the number of partial-sum slices the split's workspace holds.
int dkdv_blocks(const Problem& pr);
int dkdv_max_parts(const Problem& pr);

// Device workspace the backward needs: the split dK/dV pass's fp32 partial
// sums (2 * dkdv_max_parts * B * S * Hkv * d floats), 0 without a split.
size_t bwd_workspace_bytes(const Problem& pr);

// Decode: Sq new queries per sequence against a [B, Smax, Hkv, d] key/value cache.
struct DecodeProblem {
  int B, Sq, Smax, Hq, Hkv, d;
  float scale;
  const int32_t* cache_lens;  // device int32[B] or nullptr (= Smax)
  float rope_base;            // > 0: new queries rotated at their positions; 0: none
  Strides sq, skv, so;        // q [B,Sq,Hq,d]; k and v caches [B,Smax,Hkv,d]; o [B,Sq,Hq,d]
};

// LDS pipeline stages of the decode split kernel (K and V tiles per stage).
constexpr int kDecodeStages = 2;

// How the decode work is dealt out: `waves` one-wave workgroups share the
// valid 64-key tiles of all (sequence, kv head) units evenly; each writes one
// partial (O, LSE) per unit it touches, and a merge pass combines them by
// log-sum-exp. Workspace: a header, per-unit wave bounds, the partials.
struct DecodePlan {
  int waves;
  int rb, ru;  // 32-row blocks per kv head; partial rows per slot
  size_t off_uinfo, off_lse, off_o;
  size_t workspace_bytes;
};
DecodePlan plan_decode(const DecodeProblem& pr);
hipError_t launch_decode(const DecodeProblem& pr, const DecodePlan& plan, const void* q, const void* k_cache,
                         const void* v_cache, void* o, float* lse, void* workspace, hipStream_t stream);

// The allocation-free decode entry point keeps its workspace in a static
// device array of this many bytes, one per GPU.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
// Device address of the current GPU's scratch array (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t decode_scratch(void** out);

}  // namespace attn
