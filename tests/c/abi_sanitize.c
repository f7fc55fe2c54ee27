/* Host-only driver of the C ABI validation layer, built with AddressSanitizer
   and UndefinedBehaviorSanitizer together with attn_api.cpp, attn_plan.cpp and
   the stub launchers of launch_stub.cpp (no GPU, no HIP compiler). Every call
   either passes validation (and requests its launches from the stubs) or
   returns the expected error code without requesting any; extreme sizes
   exercise the overflow guards. Prints "abi_sanitize ok" and exits 0 when
   every expectation holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

extern int g_stub_launches;

static int failures = 0;

static void expect(const char* what, attn_status got, attn_status want, int launches_before, int launches_want) {
  int launched = g_stub_launches - launches_before;
  if (got != want || launched != launches_want) {
    printf("FAIL %s: status %d (want %d), launches %d (want %d)\n", what, (int)got, (int)want, launched,
           launches_want);
    ++failures;
  }
}

/* 16-byte aligned stand-ins for device pointers (the stubs never dereference them) */
static _Alignas(16) unsigned char arena[16 * 32];
#define P(i) ((void*)(arena + 16 * (i)))

static attn_shape base_shape(void) {
  attn_shape s;
  memset(&s, 0, sizeof(s));
  s.batch = 2;
  s.seqlen = 300;
  s.heads_q = 8;
  s.heads_kv = 2;
  s.head_dim = 64;
  s.scale = 0.125f;
  s.causal = 1;
  return s;
}

static attn_decode_shape base_decode(void) {
  attn_decode_shape s;
  memset(&s, 0, sizeof(s));
  s.batch = 3;
  s.q_len = 2;
  s.cache_len = 1000;
  s.heads_q = 8;
  s.heads_kv = 2;
  s.head_dim = 128;
  s.scale = 0.088f;
  return s;
}

#define CALL_FWD(s) attn_fwd(&(s), P(1), P(2), P(3), P(4), (float*)P(5), 0)
/* the backward gets a workspace of exactly the size it asks for (a placeholder
   address: the stubs never dereference it) */
#define CALL_BWD(s) \
  attn_bwd(&(s), P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(8), P(9), P(10), P(15), \
           attn_bwd_workspace_bytes(&(s)), 0)

int main(void) {
  int n;
  attn_shape s = base_shape();

  /* valid calls: one launch each (attn_bwd and attn_bwd_fused: two) */
  n = g_stub_launches; expect("fwd", CALL_FWD(s), ATTN_OK, n, 1);
  n = g_stub_launches; expect("pre", attn_bwd_preprocess(&s, P(4), P(6), (float*)P(7), 0), ATTN_OK, n, 1);
  n = g_stub_launches; expect("bwd", CALL_BWD(s), ATTN_OK, n, 2);
  n = g_stub_launches;
  expect("dkdv", attn_bwd_dkdv(&s, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(9), P(10), P(15),
                               attn_bwd_workspace_bytes(&s), 0), ATTN_OK, n, 1);
  /* this shape has few key blocks: the split needs a workspace, refused when short or missing */
  if (attn_bwd_workspace_bytes(&s) == 0) { printf("FAIL small shape needs no workspace\n"); ++failures; }
  n = g_stub_launches;
  expect("dkdv short ws", attn_bwd_dkdv(&s, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(9), P(10), P(15),
                                        attn_bwd_workspace_bytes(&s) - 1, 0), ATTN_ERR_WORKSPACE, n, 0);
  n = g_stub_launches;
  expect("bwd null ws", attn_bwd(&s, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(8), P(9), P(10), NULL,
                                 attn_bwd_workspace_bytes(&s), 0), ATTN_ERR_WORKSPACE, n, 0);
  n = g_stub_launches;
  expect("bwd misaligned ws", attn_bwd(&s, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(8), P(9), P(10),
                                       (void*)(arena + 4), attn_bwd_workspace_bytes(&s), 0), ATTN_ERR_WORKSPACE, n, 0);
  {
    /* many key blocks: no split, no workspace */
    attn_shape big = base_shape();
    big.batch = 16; big.seqlen = 4096; big.heads_q = 32; big.heads_kv = 8;
    if (attn_bwd_workspace_bytes(&big) != 0) { printf("FAIL large shape asks for a workspace\n"); ++failures; }
    n = g_stub_launches;
    expect("bwd no ws needed", attn_bwd(&big, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(8), P(9), P(10),
                                        NULL, 0, 0), ATTN_OK, n, 2);
  }
  n = g_stub_launches;
  expect("dq", attn_bwd_dq(&s, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(8), 0), ATTN_OK, n, 1);
  n = g_stub_launches;
  expect("fused", attn_bwd_fused(&s, P(1), P(2), P(3), P(4), P(6), (float*)P(5), (float*)P(7), P(8), P(9), P(10),
                                 P(15), attn_bwd_workspace_bytes(&s), 0), ATTN_OK, n, 2);
  n = g_stub_launches;
  expect("dq delta", attn_bwd_dq_delta(&s, P(1), P(2), P(3), P(4), P(6), (float*)P(5), (float*)P(7), P(8), 0),
         ATTN_OK, n, 1);
  n = g_stub_launches;
  expect("dq delta null o", attn_bwd_dq_delta(&s, P(1), P(2), P(3), NULL, P(6), (float*)P(5), (float*)P(7), P(8), 0),
         ATTN_ERR_INVALID_ARG, n, 0);
  s.rope_base = 10000.f;
  n = g_stub_launches; expect("rope", attn_rope(&s, P(1), P(2), P(11), P(12), 0), ATTN_OK, n, 1);
  s.rope_base = 0.f;
  n = g_stub_launches; expect("rope without base", attn_rope(&s, P(1), P(2), P(11), P(12), 0),
                              ATTN_ERR_INVALID_ARG, n, 0);
  s.causal = 0;
  n = g_stub_launches; expect("bidirectional", CALL_FWD(s), ATTN_OK, n, 1);
  s.seqlens = (const int32_t*)P(13);
  n = g_stub_launches; expect("padded", CALL_BWD(s), ATTN_OK, n, 2);
  s.seqlens = (const int32_t*)(arena + 2);
  n = g_stub_launches; expect("misaligned seqlens", CALL_FWD(s), ATTN_ERR_MISALIGNED, n, 0);

  /* invalid shapes: nothing launched */
  struct { const char* what; int field; long long value; attn_status want; } bad[] = {
      {"batch 0", 0, 0, ATTN_ERR_INVALID_ARG},        {"seqlen -1", 1, -1, ATTN_ERR_INVALID_ARG},
      {"heads_q 0", 2, 0, ATTN_ERR_INVALID_ARG},      {"heads_kv 3", 3, 3, ATTN_ERR_INVALID_ARG},
      {"head_dim 96", 4, 96, ATTN_ERR_UNSUPPORTED},   {"head_dim 0", 4, 0, ATTN_ERR_UNSUPPORTED},
      {"causal 2", 5, 2, ATTN_ERR_INVALID_ARG},       {"heads_q huge", 2, 1 << 20, ATTN_ERR_UNSUPPORTED},
      {"batch max", 0, 0x7fffffff, ATTN_ERR_UNSUPPORTED}, {"seqlen max", 1, 0x7fffffff, ATTN_ERR_UNSUPPORTED},
  };
  for (unsigned i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
    attn_shape t = base_shape();
    if (bad[i].field == 0) t.batch = (int32_t)bad[i].value;
    if (bad[i].field == 1) t.seqlen = (int32_t)bad[i].value;
    if (bad[i].field == 2) { t.heads_q = (int32_t)bad[i].value; t.heads_kv = 1; }
    if (bad[i].field == 3) t.heads_kv = (int32_t)bad[i].value;
    if (bad[i].field == 4) t.head_dim = (int32_t)bad[i].value;
    if (bad[i].field == 5) t.causal = (int32_t)bad[i].value;
    n = g_stub_launches; expect(bad[i].what, CALL_FWD(t), bad[i].want, n, 0);
    n = g_stub_launches; expect(bad[i].what, CALL_BWD(t), bad[i].want, n, 0);
    (void)attn_bwd_workspace_bytes(&t);
  }
  {
    attn_shape t = base_shape();
    float bad_scales[] = {0.f, -1.f, 1.f / 0.f, 0.f / 0.f};
    for (unsigned i = 0; i < 4; ++i) {
      t.scale = bad_scales[i];
      n = g_stub_launches; expect("bad scale", CALL_FWD(t), ATTN_ERR_INVALID_ARG, n, 0);
    }
    t = base_shape();
    t.rope_base = -1.f;
    n = g_stub_launches; expect("negative rope base", CALL_BWD(t), ATTN_ERR_INVALID_ARG, n, 0);
  }
  /* strides */
  {
    attn_shape t = base_shape();
    t.q_stride[0] = 300 * 8 * 64; t.q_stride[1] = 8 * 64; t.q_stride[2] = 64;
    n = g_stub_launches; expect("dense strides given", CALL_FWD(t), ATTN_OK, n, 1);
    t.q_stride[2] = 60;
    n = g_stub_launches; expect("stride not multiple of 8", CALL_FWD(t), ATTN_ERR_MISALIGNED, n, 0);
    t.q_stride[2] = -64;
    n = g_stub_launches; expect("negative stride", CALL_FWD(t), ATTN_ERR_MISALIGNED, n, 0);
    t = base_shape();
    t.kv_stride[0] = 8; t.kv_stride[1] = ((int64_t)1 << 22) + 8; t.kv_stride[2] = 8;
    n = g_stub_launches; expect("position stride too large", CALL_BWD(t), ATTN_ERR_UNSUPPORTED, n, 0);
    t.kv_stride[1] = (int64_t)1 << 62;
    n = g_stub_launches; expect("huge stride", CALL_BWD(t), ATTN_ERR_UNSUPPORTED, n, 0);
  }
  /* pointers */
  {
    attn_shape t = base_shape();
    n = g_stub_launches;
    expect("null q", attn_fwd(&t, NULL, P(2), P(3), P(4), (float*)P(5), 0), ATTN_ERR_INVALID_ARG, n, 0);
    n = g_stub_launches;
    expect("misaligned o", attn_fwd(&t, P(1), P(2), P(3), (void*)(arena + 8), (float*)P(5), 0),
           ATTN_ERR_MISALIGNED, n, 0);
    n = g_stub_launches; expect("null shape", attn_fwd(NULL, P(1), P(2), P(3), P(4), (float*)P(5), 0),
                                ATTN_ERR_INVALID_ARG, n, 0);
    n = g_stub_launches;
    expect("null dv", attn_bwd(&t, P(1), P(2), P(3), P(6), (float*)P(5), (float*)P(7), P(8), P(9), NULL, NULL, 0, 0),
           ATTN_ERR_INVALID_ARG, n, 0);
  }

  /* decode */
  {
    attn_decode_shape d = base_decode();
    size_t ws = attn_decode_workspace_bytes(&d);
    if (ws == 0) { printf("FAIL decode workspace 0\n"); ++failures; }
    n = g_stub_launches;
    expect("decode", attn_decode(&d, P(1), P(2), P(3), P(4), (float*)P(5), P(14), ws, 0), ATTN_OK, n, 1);
    n = g_stub_launches;
    expect("decode small ws", attn_decode(&d, P(1), P(2), P(3), P(4), (float*)P(5), P(14), ws - 1, 0),
           ATTN_ERR_WORKSPACE, n, 0);
    n = g_stub_launches;
    expect("decode null ws", attn_decode(&d, P(1), P(2), P(3), P(4), (float*)P(5), NULL, ws, 0),
           ATTN_ERR_WORKSPACE, n, 0);
    attn_decode_shape e = d;
    e.batch = 0x7fffffff; e.cache_len = 0x7fffffff; e.q_len = 0x7fffffff;
    n = g_stub_launches;
    expect("decode huge", attn_decode(&e, P(1), P(2), P(3), P(4), (float*)P(5), P(14), (size_t)-1, 0),
           ATTN_ERR_UNSUPPORTED, n, 0);
    if (attn_decode_workspace_bytes(&e) != 0) { printf("FAIL decode huge workspace\n"); ++failures; }
    e = d; e.heads_kv = 3;
    if (attn_decode_workspace_bytes(&e) != 0) { printf("FAIL decode bad heads workspace\n"); ++failures; }
    e = d; e.head_dim = 32;
    n = g_stub_launches;
    expect("decode head_dim", attn_decode(&e, P(1), P(2), P(3), P(4), (float*)P(5), P(14), ws, 0),
           ATTN_ERR_UNSUPPORTED, n, 0);
    e = d; e.cache_lens = (const int32_t*)(arena + 1);
    n = g_stub_launches;
    expect("decode misaligned lens", attn_decode(&e, P(1), P(2), P(3), P(4), (float*)P(5), P(14), ws, 0),
           ATTN_ERR_MISALIGNED, n, 0);
    if (attn_decode_workspace_bytes(NULL) != 0) { printf("FAIL decode null shape\n"); ++failures; }
    /* the allocation-free variant: same validation, scratch limit instead of a workspace */
    n = g_stub_launches;
    expect("decode noalloc", attn_decode_noalloc(&d, P(1), P(2), P(3), P(4), (float*)P(5), 0), ATTN_OK, n, 1);
    e = d; e.batch = 64; e.q_len = 64; e.cache_len = 64; e.heads_q = 64; e.heads_kv = 64;
    n = g_stub_launches;
    expect("decode noalloc beyond scratch", attn_decode_noalloc(&e, P(1), P(2), P(3), P(4), (float*)P(5), 0),
           ATTN_ERR_WORKSPACE, n, 0);
    n = g_stub_launches;
    expect("decode noalloc null o", attn_decode_noalloc(&d, P(1), P(2), P(3), NULL, (float*)P(5), 0),
           ATTN_ERR_INVALID_ARG, n, 0);
  }

  /* status strings: every code has a non-empty static string */
  for (int c = 0; c <= 7; ++c) {
    const char* str = attn_status_string((attn_status)c);
    if (!str || !str[0]) { printf("FAIL status string %d\n", c); ++failures; }
  }
  if (attn_bwd_workspace_bytes(NULL) != 0) { printf("FAIL bwd workspace null shape\n"); ++failures; }

  if (failures) {
    printf("abi_sanitize: %d failures\n", failures);
    return 1;
  }
  printf("abi_sanitize ok (%d launches requested)\n", g_stub_launches);
  return 0;
}
