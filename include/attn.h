/*
 * attn.h - C ABI of the MI355X (gfx950) fused causal attention library.
 *
 * Operation. Causal (or, with causal = 0, bidirectional) scaled-dot-product
 * softmax attention for transformer training, forward and full backward, with
 * grouped-query heads. The pages
 * this follows describe it as fused flash attention, forward and backward,
 * whose probabilities never reach memory, stored in bf16 and accumulated in
 * fp32 ("Axis", Zyora Labs page, feature list), with query heads sharing kv
 * heads ("AxiomLM" PyPI page, "Key Features": grouped-query attention). For a
 * sequence b with valid prefix length L_b, query head h and kv head
 * g = h / (Hq / Hkv):
 *
 *   s_ij  = scale * <Q[b,i,h,:], K[b,j,g,:]>      valid when j <= i < L_b
 *   LSE_i = ln sum_{j <= i} exp(s_ij)              (-inf when i >= L_b)
 *   P_ij  = exp(s_ij - LSE_i)
 *   O_i   = sum_j P_ij V[b,j,g,:]                  (0 when i >= L_b)
 *   D_i   = <dO_i, O_i>
 *   dS_ij = P_ij (<dO_i, V_j> - D_i)
 *   dQ_i  = scale sum_j dS_ij K_j
 *   dK_j  = scale sum_{h in group g} sum_i dS_ij Q_i
 *   dV_j  = sum_{h in group g} sum_i P_ij dO_i
 *
 * With causal = 0 ("Axis" Rust/cuTile page, "Sudoku as an acceptance test":
 * bidirectional multi-head attention) every "j <= i" above reads "j < L_b".
 *
 * The S x S matrices (scores, P, dS) are never written to device memory:
 * every call needs O(B * S * H * d) memory only.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or synchronises; work is enqueued on `stream` (0 =
 *    the null stream) in call order. Buffers must stay alive until the stream
 *    has run the work.
 *  - Layouts are row-major: Q, O, dO, dQ are [B, S, Hq, d]; K, V, dK, dV
 *    are [B, S, Hkv, d]; all bf16 (bfloat16 bit patterns), dense unless the
 *    shape gives strides. LSE and D are fp32 [B, Hq, S], always dense.
 *  - Outputs are fully overwritten, including padded rows (zeros, LSE = -inf);
 *    gradients are not accumulated into existing contents.
 *  - Every tensor pointer must be 16-byte aligned (seqlens: 4-byte aligned).
 *  - Arguments are validated on the host before any HIP call; an invalid call
 *    returns an error code and enqueues nothing. A launch error reported by
 *    the HIP runtime returns ATTN_ERR_HIP. There is no global error state and
 *    the functions are thread-safe.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, Hq % Hkv != 0,
                                non-finite or non-positive scale, causal not 0/1,
                                negative or non-finite rope_base */
  ATTN_ERR_UNSUPPORTED = 2,  /* head_dim not in {64, 128}; a sequence or cache
                                length above 2^30; heads_q * head_dim
                                (decode: heads_kv * head_dim) above 2^22, or a
                                position stride above 2^22 (tile offsets are
                                32-bit); or a launch beyond 2^31 - 1 blocks */
  ATTN_ERR_MISALIGNED = 3,   /* a pointer is not 16-byte aligned, or a stride is
                                negative or not a multiple of 8 elements */
  ATTN_ERR_WORKSPACE = 4,    /* workspace smaller than attn_bwd_workspace_bytes() */
  ATTN_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} attn_status;

typedef struct attn_shape {
  int32_t batch;       /* B >= 1 */
  int32_t seqlen;      /* 1 <= S <= 2^30 (query and key lengths are equal) */
  int32_t heads_q;     /* Hq >= 1, a multiple of heads_kv */
  int32_t heads_kv;    /* Hkv >= 1 */
  int32_t head_dim;    /* d: 64 or 128 */
  float scale;         /* softmax scale, finite and > 0 (typically 1/sqrt(d)) */
  int32_t causal;      /* 1: causal (query i sees keys j <= i); 0: bidirectional
                          (every query sees every key of the valid prefix) */
  /* Optional DEVICE int32[B]: valid prefix length L_b of each sequence (right
     padding). NULL means every sequence has length S. Values are clamped into
     [0, S] on the device; positions i >= L_b take no part in any sum, may hold
     any bits (including NaN), and receive zero outputs/gradients. */
  const int32_t* seqlens;
  /* Rotary position embedding base, or 0 for none (finite and >= 0, else
     ATTN_ERR_INVALID_ARG). When > 0, the q and k handed to attn_fwd and the
     backward entry points are the ROTATED tensors written by attn_rope, and
     the backward entry points return dq and dk with respect to the unrotated
     q and k (the rotation's adjoint is applied as they are written).
     attn_fwd and attn_bwd_preprocess do not depend on it. */
  float rope_base;
  /* Optional strides, in elements, of the (sequence, position, head)
     dimensions; the head dimension d is always contiguous. All three zero
     means the dense layout above. q_stride: Q (and q_rot in attn_rope);
     kv_stride: K, V, dK, dV (and k_rot); o_stride: O, dO, dQ. Each must be a
     non-negative multiple of 8 (ATTN_ERR_MISALIGNED otherwise) and the
     position stride at most 2^22 (ATTN_ERR_UNSUPPORTED). They let Q, K, V be
     views into one fused projection output, for instance. Outputs written
     through strides that make rows overlap race; the caller keeps them
     disjoint. */
  int64_t q_stride[3];
  int64_t kv_stride[3];
  int64_t o_stride[3];
} attn_shape;

/*
 * Rotary position embedding ("AxiomLM" PyPI page, "Key Features": RoPE in its
 * modern architecture suite; "8. Standalone Modern Architectural Modules":
 * frequencies precomputed for the head size, applied to q [B,S,Hq,d] and k
 * [B,S,Hkv,d] ahead of attention). Pair (2i, 2i+1) of every head at token
 * position p (0 .. S-1) is rotated by a = p * theta_i, theta_i =
 * rope_base^(-2i/d):
 *   r_2i = x_2i cos a - x_2i+1 sin a,   r_2i+1 = x_2i sin a + x_2i+1 cos a.
 * q_rot [B,S,Hq,d] and k_rot [B,S,Hkv,d] bf16 (rounded once from fp32). The
 * caller keeps them for the backward pass (they replace q and k there).
 * Requires shape->rope_base > 0 (ATTN_ERR_INVALID_ARG otherwise). Padded
 * positions are rotated too; no attention pass reads them.
 */
attn_status attn_rope(const attn_shape* shape, const void* q, const void* k, void* q_rot, void* k_rot,
                      hipStream_t stream);

/*
 * Forward ("Axis", Zyora Labs page, feature list: the fused flash-attention
 * forward whose probabilities never reach memory, bf16 storage, fp32
 * accumulation): O = softmax(scale * Q K^T + causal/padding mask) V, and the
 * fp32 natural-log row normaliser LSE that the backward recomputes P from.
 * Q [B,S,Hq,d], K/V [B,S,Hkv,d], O [B,S,Hq,d] bf16; LSE [B,Hq,S] fp32.
 * Deterministic (bitwise repeatable).
 */
attn_status attn_fwd(const attn_shape* shape, const void* q, const void* k, const void* v,
                     void* o, float* lse, hipStream_t stream);

/*
 * Backward preprocess (the row term D of the softmax gradient used by the
 * fused backward of the "Axis" Zyora Labs page, feature list; the pages give
 * no formula, D is the standard one for the exact gradient of softmax
 * attention): D[b,h,i] = sum_c dO[b,i,h,c] * O[b,i,h,c] accumulated in fp32
 * from the bf16 inputs (0 on padded rows). O, dO [B,S,Hq,d] bf16; D [B,Hq,S]
 * fp32.
 */
attn_status attn_bwd_preprocess(const attn_shape* shape, const void* o, const void* d_o,
                                float* delta, hipStream_t stream);

/*
 * Bytes of device workspace attn_bwd, attn_bwd_dkdv and attn_bwd_fused need
 * for `shape`: O(B*S*Hkv*d) at most, never O(S^2) (the "Axis" Zyora Labs page,
 * feature list: memory stays flat as the sequence grows). It is 0 unless the
 * shape has too few 128-key blocks (B * ceil(S/128) * Hkv < 256) to give every
 * CU work; then each (sequence, kv head) gets parts * ceil(S/128) workgroups,
 * parts <= 8, dealt to its key blocks by their work under the causal mask (at
 * most 2 * parts - 1 to one block), and their fp32 partial dK and dV sums
 * (2 * P * B * S * Hkv * d floats, P the largest count of any block) are added
 * by a reduce pass. Depends only on batch, seqlen, heads, head_dim and the
 * causal flag. Returns 0 for a NULL or invalid shape.
 */
size_t attn_bwd_workspace_bytes(const attn_shape* shape);

/*
 * Backward ("Axis", Zyora Labs page, feature list: the fused flash-attention
 * backward; grouped kv heads per the "AxiomLM" PyPI page, "Key Features"):
 * dQ, dK, dV from Q, K, V, dO, the forward's LSE and the preprocess's D. The probabilities are recomputed from LSE tile by tile.
 * dQ [B,S,Hq,d], dK/dV [B,S,Hkv,d] bf16 (dK/dV summed over each kv head's
 * query-head group). `workspace` may be NULL when attn_bwd_workspace_bytes()
 * is 0; otherwise it must be 16-byte aligned and hold at least that many
 * bytes. Deterministic (bitwise repeatable).
 */
attn_status attn_bwd(const attn_shape* shape, const void* q, const void* k, const void* v,
                     const void* d_o, const float* lse, const float* delta,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * The two passes attn_bwd runs, exported separately (same operation and
 * citation as attn_bwd). They read the same inputs,
 * write disjoint outputs and do not depend on each other, so a caller may run
 * them in either order or concurrently on two streams; attn_bwd enqueues
 * attn_bwd_dkdv then attn_bwd_dq on one stream.
 *   attn_bwd_dkdv: dK, dV [B,S,Hkv,d] bf16 (one pass per key block over the
 *                  query rows of every head in the kv head's group; with a
 *                  nonzero attn_bwd_workspace_bytes() the blocks are split and
 *                  a reduce pass follows, using the workspace).
 *   attn_bwd_dq:   dQ [B,S,Hq,d] bf16 (one pass per query block over its keys;
 *                  no workspace).
 * Same validation, layouts and error codes as attn_bwd. Two concurrent
 * attn_bwd_dkdv calls need distinct workspaces.
 */
attn_status attn_bwd_dkdv(const attn_shape* shape, const void* q, const void* k, const void* v,
                          const void* d_o, const float* lse, const float* delta,
                          void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);
attn_status attn_bwd_dq(const attn_shape* shape, const void* q, const void* k, const void* v,
                        const void* d_o, const float* lse, const float* delta,
                        void* dq, hipStream_t stream);

/*
 * Backward with the preprocess folded in (same operation and citation as
 * attn_bwd_preprocess followed by attn_bwd): the dQ pass computes D = rowsum(dO * O)
 * from the O and dO rows it loads (fp32 from the bf16 inputs, 0 on padded
 * rows), writes it to `delta` [B,Hq,S] fp32 (an output here) and uses it; the
 * dK/dV pass then reads it. Same results as attn_bwd_preprocess followed by
 * attn_bwd up to the fp32 summation order of D, one launch fewer and one pass
 * over O and dO fewer. O shares the o_stride triple with dO and dQ. Same
 * validation, workspace rule and error codes as attn_bwd. Deterministic.
 */
attn_status attn_bwd_fused(const attn_shape* shape, const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, float* delta, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The first launch of attn_bwd_fused on its own: the dQ pass of the fused
 * flash-attention backward ("Axis", Zyora Labs page, feature list; D is the
 * standard row term of the exact softmax gradient, as in attn_bwd_preprocess)
 * with the preprocess folded in. It computes
 * D = rowsum(dO * O) from the O and dO rows it loads (fp32 from the bf16
 * inputs, 0 on padded rows), writes it to `delta` [B,Hq,S] fp32 (an output
 * here) and forms dQ [B,S,Hq,d] bf16 with it. attn_bwd_dq_delta followed on
 * the same stream by attn_bwd_dkdv, which then reads that D, enqueues exactly
 * the launches of attn_bwd_fused; a caller splits the two to time them or to
 * place other work between them. O shares the o_stride triple with dO and dQ.
 * Same validation and error codes as attn_bwd_dq; no workspace.
 * Deterministic.
 */
attn_status attn_bwd_dq_delta(const attn_shape* shape, const void* q, const void* k, const void* v, const void* o,
                              const void* d_o, const float* lse, float* delta, void* dq, hipStream_t stream);

/*
 * Decode: attention of Sq new queries per sequence against a key/value cache
 * (inference). "AxiomLM" (PyPI page), "Key Features" and "Zero-Overhead
 * Inference & Streaming Generation": a state-cached key/value decode engine,
 * with grouped kv heads ("Benchmarks": 4-head GQA shrinks the cache).
 * Sequence b holds L_b valid cache positions; the last Sq of them belong to
 * the new queries (their keys/values are already in the cache), so query t
 * sits at position p = L_b - Sq + t and attends to cached keys j <= p:
 *   LSE_t = ln sum_{j <= p} exp(scale <q_t, k_j>),
 *   O_t   = sum_{j <= p} exp(scale <q_t, k_j> - LSE_t) v_j,
 * with O_t = 0 and LSE_t = -inf when p < 0 (the query sees no key).
 * With rope_base > 0 the cache holds keys already rotated at their positions
 * (see attn_rope) and each new query is rotated at its position p before use
 * (the rotated query is rounded to bf16, like any stored tensor).
 */
typedef struct attn_decode_shape {
  int32_t batch;       /* B >= 1 */
  int32_t q_len;       /* 1 <= Sq <= 2^30 new queries per sequence (the Sq * Hq / Hkv
                          query rows of a kv head run in blocks of 32) */
  int32_t cache_len;   /* 1 <= Smax <= 2^30: cache capacity (positions) per sequence */
  int32_t heads_q;     /* Hq >= 1, a multiple of heads_kv */
  int32_t heads_kv;    /* Hkv >= 1 */
  int32_t head_dim;    /* d: 64 or 128 */
  float scale;         /* finite and > 0 */
  /* Optional DEVICE int32[B]: valid cache length L_b of each sequence, clamped
     into [0, Smax] on the device; NULL means L_b = Smax. Positions >= L_b may
     hold any bits (including NaN). */
  const int32_t* cache_lens;
  /* Rotary embedding base for the new queries, or 0 for none (finite and
     >= 0, else ATTN_ERR_INVALID_ARG). */
  float rope_base;
  /* Optional element strides of the (sequence, position, head) dimensions,
     as in attn_shape (all zero: dense; multiples of 8, else
     ATTN_ERR_MISALIGNED; cache position stride at most 2^22). q_stride: q;
     kv_stride: both caches, e.g. {Hkv*Smax*d, d, Smax*d} for a cache stored
     head-major as [B, Hkv, Smax, d]; o_stride: o. */
  int64_t q_stride[3];
  int64_t kv_stride[3];
  int64_t o_stride[3];
} attn_decode_shape;

/*
 * Bytes of device workspace attn_decode needs. A unit is one (sequence, kv
 * head, block of up to 32 of the kv head's R = Sq * Hq / Hkv query rows);
 * U = B * Hkv * ceil(R / 32). The valid 64-key tiles of all units are shared
 * evenly by W <= 1024 waves (fewer when there are fewer tiles); each wave
 * leaves one partial result, (d + 1) floats per row, for each unit it
 * touches, so the workspace holds (W + U - 1) * min(R, 32) * (d + 1) floats
 * plus an 8-byte record per unit and a small header; it does not grow with
 * Smax once W is capped.
 * Returns 0 for a NULL or invalid shape.
 */
size_t attn_decode_workspace_bytes(const attn_decode_shape* shape);

/*
 * q [B,Sq,Hq,d], k_cache/v_cache [B,Smax,Hkv,d] (any strides the shape
 * gives), o [B,Sq,Hq,d] bf16; lse
 * [B,Hq,Sq] fp32; workspace: caller-owned device memory of at least
 * attn_decode_workspace_bytes() bytes, 16-byte aligned (ATTN_ERR_WORKSPACE
 * otherwise), overwritten by the call and free again when the stream has run
 * it. Two launches (partials, then their merge); deterministic for a given
 * shape and cache lengths.
 */
attn_status attn_decode(const attn_decode_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                        void* o, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc. Same operation,
 * layouts, validation and results as attn_decode (bit for bit: the same
 * kernels and work split); the partial results live in a static device array
 * of ATTN_DECODE_SCRATCH_BYTES (32 MiB) that the library holds on each GPU it
 * runs on until the process ends (its address is looked up on the first call
 * on each device). A problem whose attn_decode_workspace_bytes() exceeds that
 * returns ATTN_ERR_WORKSPACE and enqueues nothing. Every call on one GPU uses
 * the same array: calls that may overlap on one GPU (several streams, several
 * host threads without ordering) race and must be serialised by the caller.
 * Nothing in the array has to start at zero; each call writes what it reads.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
attn_status attn_decode_noalloc(const attn_decode_shape* shape, const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse, hipStream_t stream);

/* Static, human-readable name of a status code and the conditions that return
   it (never NULL). Not an operation of the pages: the error convention of this
   library (validation on the host before any launch). */
const char* attn_status_string(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
