/* Plain-C client of include/attn.h (no HIP compiler, no GPU work): prints the
   struct layouts the Python binding mirrors, and the status codes of calls that
   host validation must refuse before any HIP call. */
#include <stddef.h>
#include <stdio.h>

#include "attn.h"

int main(void) {
  printf("attn_shape %zu rope_base %zu q_stride %zu kv_stride %zu o_stride %zu seqlens %zu\n",
         sizeof(attn_shape), offsetof(attn_shape, rope_base), offsetof(attn_shape, q_stride),
         offsetof(attn_shape, kv_stride), offsetof(attn_shape, o_stride), offsetof(attn_shape, seqlens));
  printf("attn_decode_shape %zu cache_lens %zu rope_base %zu dq_stride %zu dkv_stride %zu do_stride %zu\n",
         sizeof(attn_decode_shape), offsetof(attn_decode_shape, cache_lens), offsetof(attn_decode_shape, rope_base),
         offsetof(attn_decode_shape, q_stride), offsetof(attn_decode_shape, kv_stride),
         offsetof(attn_decode_shape, o_stride));
  attn_shape s = {0};
  s.batch = 1;
  s.seqlen = 64;
  s.heads_q = 2;
  s.heads_kv = 1;
  s.head_dim = 96; /* unsupported */
  s.scale = 0.125f;
  s.causal = 1;
  printf("fwd_bad_dim %d\n", (int)attn_fwd(&s, 0, 0, 0, 0, 0, 0));
  s.head_dim = 64;
  printf("fwd_null_ptr %d\n", (int)attn_fwd(&s, 0, 0, 0, 0, 0, 0));
  s.q_stride[0] = 8;
  s.q_stride[1] = 8;
  s.q_stride[2] = 4; /* not a multiple of 8 */
  printf("fwd_bad_stride %d\n", (int)attn_fwd(&s, 0, 0, 0, 0, 0, 0));
  printf("status_1 %s\n", attn_status_string(ATTN_ERR_INVALID_ARG));
  return 0;
}
