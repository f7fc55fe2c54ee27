// C ABI of the attention library: host-side validation, then launches on the
// caller's stream. No allocation, no synchronisation, no global state.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "attn.h"
#include "attn_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Longest sequence (and cache) accepted: positions and block counts are
// 32-bit ints on the device and in the launch arithmetic, rounded up there.
constexpr int32_t kMaxLen = 1 << 30;

// A stride triple (sequence, position, head) in elements; all zero means the
// dense [B, S, H, d] layout. Returns false for a negative stride or one that
// is not a multiple of 8 elements (rows must stay 16-byte aligned).
bool resolve_strides(const int64_t (&in)[3], int S, int H, int d, attn::Strides* out) {
  if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
    *out = attn::Strides{(int64_t)S * H * d, (int64_t)H * d, d};
    return true;
  }
  for (int i = 0; i < 3; ++i)
    if (in[i] < 0 || (in[i] & 7) != 0) return false;
  *out = attn::Strides{in[0], in[1], in[2]};
  return true;
}

attn_status check_shape(const attn_shape* s, attn::Problem* pr) {
  if (!s) return ATTN_ERR_INVALID_ARG;
  if (s->batch < 1 || s->seqlen < 1 || s->heads_q < 1 || s->heads_kv < 1) return ATTN_ERR_INVALID_ARG;
  if (s->heads_q % s->heads_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (!(isfinite(s->scale) && s->scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (s->seqlen > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  if (s->causal != 0 && s->causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!(isfinite(s->rope_base) && s->rope_base >= 0.f)) return ATTN_ERR_INVALID_ARG;
  if (s->seqlens && (reinterpret_cast<uintptr_t>(s->seqlens) & 3u) != 0) return ATTN_ERR_MISALIGNED;
  attn::Strides sq, skv, so;
  if (!resolve_strides(s->q_stride, s->seqlen, s->heads_q, s->head_dim, &sq) ||
      !resolve_strides(s->kv_stride, s->seqlen, s->heads_kv, s->head_dim, &skv) ||
      !resolve_strides(s->o_stride, s->seqlen, s->heads_q, s->head_dim, &so))
    return ATTN_ERR_MISALIGNED;
  // tiles are fetched through buffer resources with 32-bit byte offsets that
  // span up to 128 rows of one sequence: 128 * position stride * 2 < 2^31
  constexpr int64_t kMaxRowStride = (int64_t)1 << 22;
  if ((int64_t)s->heads_q * s->head_dim > kMaxRowStride || sq.s > kMaxRowStride || skv.s > kMaxRowStride ||
      so.s > kMaxRowStride)
    return ATTN_ERR_UNSUPPORTED;
  pr->B = s->batch;
  pr->S = s->seqlen;
  pr->Hq = s->heads_q;
  pr->Hkv = s->heads_kv;
  pr->d = s->head_dim;
  pr->scale = s->scale;
  pr->seqlens = s->seqlens;
  pr->causal = s->causal;
  pr->rope_base = s->rope_base;
  pr->sq = sq;
  pr->skv = skv;
  pr->so = so;
  if (attn::max_grid(*pr) > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status check_decode_shape(const attn_decode_shape* s, attn::DecodeProblem* pr) {
  if (!s) return ATTN_ERR_INVALID_ARG;
  if (s->batch < 1 || s->q_len < 1 || s->cache_len < 1 || s->heads_q < 1 || s->heads_kv < 1)
    return ATTN_ERR_INVALID_ARG;
  if (s->heads_q % s->heads_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (!(isfinite(s->scale) && s->scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (s->cache_len > kMaxLen || s->q_len > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  if (!(isfinite(s->rope_base) && s->rope_base >= 0.f)) return ATTN_ERR_INVALID_ARG;
  if (s->cache_lens && (reinterpret_cast<uintptr_t>(s->cache_lens) & 3u) != 0) return ATTN_ERR_MISALIGNED;
  // 32-bit tile offsets (as for the training path) and grid size
  if ((int64_t)s->heads_kv * s->head_dim > (int64_t)1 << 22) return ATTN_ERR_UNSUPPORTED;
  pr->B = s->batch;
  pr->Sq = s->q_len;
  pr->Smax = s->cache_len;
  pr->Hq = s->heads_q;
  pr->Hkv = s->heads_kv;
  pr->d = s->head_dim;
  pr->scale = s->scale;
  pr->cache_lens = s->cache_lens;
  pr->rope_base = s->rope_base;
  if (!resolve_strides(s->q_stride, s->q_len, s->heads_q, s->head_dim, &pr->sq) ||
      !resolve_strides(s->kv_stride, s->cache_len, s->heads_kv, s->head_dim, &pr->skv) ||
      !resolve_strides(s->o_stride, s->q_len, s->heads_q, s->head_dim, &pr->so))
    return ATTN_ERR_MISALIGNED;
  if (pr->skv.s > ((int64_t)1 << 22)) return ATTN_ERR_UNSUPPORTED;  // 32-bit tile offsets
  // the count of valid 64-key tiles over all units (one per kv head and
  // 32-row block of its query rows) is a 32-bit int on the device
  const int64_t row_blocks = ((int64_t)s->q_len * (s->heads_q / s->heads_kv) + 31) / 32;
  if ((int64_t)s->batch * s->heads_kv * row_blocks * ((s->cache_len + 63) / 64) > 0x7fffffffLL)
    return ATTN_ERR_UNSUPPORTED;
  if (((int64_t)s->batch * s->heads_q * s->q_len + 3) / 4 > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return ATTN_ERR_INVALID_ARG;
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// The workspace rule of the backward entry points: at least
// attn_bwd_workspace_bytes() bytes, 16-byte aligned when any are needed.
attn_status check_workspace(const attn::Problem& pr, const void* workspace, size_t workspace_bytes) {
  const size_t need = attn::bwd_workspace_bytes(pr);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (need > 0 && (!workspace || !aligned16(workspace))) return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd(const attn_shape* shape, const void* q, const void* k, const void* v, void* o, float* lse,
                     hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, lse});
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_fwd(pr, q, k, v, o, lse, stream));
}

attn_status attn_bwd_preprocess(const attn_shape* shape, const void* o, const void* d_o, float* delta,
                                hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({o, d_o, delta});
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_preprocess(pr, o, d_o, delta, stream));
}

attn_status attn_rope(const attn_shape* shape, const void* q, const void* k, void* q_rot, void* k_rot,
                      hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  if (!(pr.rope_base > 0.f)) return ATTN_ERR_INVALID_ARG;
  st = check_ptrs({q, k, q_rot, k_rot});
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_rope(pr, q, k, q_rot, k_rot, stream));
}

size_t attn_bwd_workspace_bytes(const attn_shape* shape) {
  attn::Problem pr;
  if (check_shape(shape, &pr) != ATTN_OK) return 0;
  return attn::bwd_workspace_bytes(pr);
}

attn_status attn_bwd_dkdv(const attn_shape* shape, const void* q, const void* k, const void* v, const void* d_o,
                          const float* lse, const float* delta, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, d_o, lse, delta, dk, dv});
  if (st != ATTN_OK) return st;
  st = check_workspace(pr, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dkdv(pr, q, k, v, d_o, lse, delta, dk, dv, workspace, stream));
}

attn_status attn_bwd_dq(const attn_shape* shape, const void* q, const void* k, const void* v, const void* d_o,
                        const float* lse, const float* delta, void* dq, hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, d_o, lse, delta, dq});
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dq(pr, q, k, v, d_o, lse, delta, dq, stream));
}

attn_status attn_bwd(const attn_shape* shape, const void* q, const void* k, const void* v, const void* d_o,
                     const float* lse, const float* delta, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, d_o, lse, delta, dq, dk, dv});
  if (st != ATTN_OK) return st;
  st = check_workspace(pr, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  st = from_hip(attn::launch_bwd_dkdv(pr, q, k, v, d_o, lse, delta, dk, dv, workspace, stream));
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dq(pr, q, k, v, d_o, lse, delta, dq, stream));
}

attn_status attn_bwd_fused(const attn_shape* shape, const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, float* delta, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, d_o, lse, delta, dq, dk, dv});
  if (st != ATTN_OK) return st;
  st = check_workspace(pr, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  // dQ first: it computes D, which the dK/dV pass then reads
  st = from_hip(attn::launch_bwd_dq_with_delta(pr, q, k, v, o, d_o, lse, delta, dq, stream));
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dkdv(pr, q, k, v, d_o, lse, delta, dk, dv, workspace, stream));
}

attn_status attn_bwd_dq_delta(const attn_shape* shape, const void* q, const void* k, const void* v, const void* o,
                              const void* d_o, const float* lse, float* delta, void* dq, hipStream_t stream) {
  attn::Problem pr;
  attn_status st = check_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, d_o, lse, delta, dq});
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dq_with_delta(pr, q, k, v, o, d_o, lse, delta, dq, stream));
}

size_t attn_decode_workspace_bytes(const attn_decode_shape* shape) {
  attn::DecodeProblem pr;
  if (check_decode_shape(shape, &pr) != ATTN_OK) return 0;
  return attn::plan_decode(pr).workspace_bytes;
}

attn_status attn_decode(const attn_decode_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                        void* o, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  attn::DecodeProblem pr;
  attn_status st = check_decode_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k_cache, v_cache, o, lse});
  if (st != ATTN_OK) return st;
  const attn::DecodePlan plan = attn::plan_decode(pr);
  if (workspace_bytes < plan.workspace_bytes || !workspace || !aligned16(workspace)) return ATTN_ERR_WORKSPACE;
  return from_hip(attn::launch_decode(pr, plan, q, k_cache, v_cache, o, lse, workspace, stream));
}

attn_status attn_decode_noalloc(const attn_decode_shape* shape, const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse, hipStream_t stream) {
  attn::DecodeProblem pr;
  attn_status st = check_decode_shape(shape, &pr);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k_cache, v_cache, o, lse});
  if (st != ATTN_OK) return st;
  const attn::DecodePlan plan = attn::plan_decode(pr);
  if (plan.workspace_bytes > attn::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
  void* scratch = nullptr;
  st = from_hip(attn::decode_scratch(&scratch));
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_decode(pr, plan, q, k_cache, v_cache, o, lse, scratch, stream));
}

const char* attn_status_string(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG:
      return "ATTN_ERR_INVALID_ARG: null pointer, non-positive size, Hq % Hkv != 0, scale not finite and > 0, "
             "causal not 0 or 1, or rope_base negative or not finite";
    case ATTN_ERR_UNSUPPORTED:
      return "ATTN_ERR_UNSUPPORTED: head_dim must be 64 or 128, lengths at most 2^30, heads * head_dim and "
             "every position stride at most 2^22 elements, and no launch above 2^31 - 1 blocks";
    case ATTN_ERR_MISALIGNED:
      return "ATTN_ERR_MISALIGNED: tensor pointers must be 16-byte aligned (lengths 4-byte) and strides "
             "non-negative multiples of 8 elements";
    case ATTN_ERR_WORKSPACE:
      return "ATTN_ERR_WORKSPACE: workspace missing, misaligned or smaller than required (attn_decode_noalloc: "
             "the problem needs more than its 32 MiB static scratch)";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: the HIP runtime reported a launch error";
  }
  return "ATTN_ERR_UNKNOWN";
}

}  // extern "C"
