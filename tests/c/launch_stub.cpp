// Host-only stand-ins for the kernel launchers (attn_launch.h), for the
// sanitizer build of the C ABI layer: no GPU and no HIP compiler. Each records
// that a launch was requested and checks the arguments the real launchers
// would pass to a kernel, so a validation bug that lets a bad call through
// shows up as a failed check or a sanitizer report rather than a GPU fault.
#include <stdio.h>
#include <stdlib.h>

#include "attn_launch.h"

extern "C" {
int g_stub_launches = 0;
}

namespace {

void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "stub launcher: %s\n", what);
    abort();
  }
}

void check_problem(const attn::Problem& pr) {
  require(pr.B >= 1 && pr.S >= 1 && pr.Hq >= 1 && pr.Hkv >= 1, "sizes");
  require(pr.Hq % pr.Hkv == 0, "group size");
  require(pr.d == 64 || pr.d == 128, "head dim");
  require(pr.causal == 0 || pr.causal == 1, "causal flag");
  require(pr.scale > 0.f, "scale");
  for (const attn::Strides* st : {&pr.sq, &pr.skv, &pr.so}) {
    require(st->b >= 0 && st->s >= 0 && st->h >= 0, "negative stride");
    require(st->b % 8 == 0 && st->s % 8 == 0 && st->h % 8 == 0, "stride not a multiple of 8");
    require(st->s <= (int64_t)1 << 22, "position stride");
  }
  require(attn::max_grid(pr) <= 0x7fffffffLL, "grid");
}

void check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) require(p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0, "pointer");
}

hipError_t done() {
  ++g_stub_launches;
  return hipSuccess;
}

}  // namespace

namespace attn {

hipError_t launch_fwd(const Problem& pr, const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t) {
  check_problem(pr);
  check_ptrs({q, k, v, o, lse});
  return done();
}

hipError_t launch_rope(const Problem& pr, const void* q, const void* k, void* q_rot, void* k_rot, hipStream_t) {
  check_problem(pr);
  require(pr.rope_base > 0.f, "rope base");
  check_ptrs({q, k, q_rot, k_rot});
  return done();
}

hipError_t launch_preprocess(const Problem& pr, const void* o, const void* d_o, float* delta, hipStream_t) {
  check_problem(pr);
  check_ptrs({o, d_o, delta});
  return done();
}

hipError_t launch_bwd_dkdv(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, void* dk, void* dv, void* workspace, hipStream_t) {
  check_problem(pr);
  check_ptrs({q, k, v, d_o, lse, delta, dk, dv});
  if (bwd_workspace_bytes(pr) > 0) check_ptrs({workspace});
  return done();
}

hipError_t launch_bwd_dq(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, void* dq, hipStream_t) {
  check_problem(pr);
  check_ptrs({q, k, v, d_o, lse, delta, dq});
  return done();
}

hipError_t launch_bwd_dq_with_delta(const Problem& pr, const void* q, const void* k, const void* v, const void* o,
                                    const void* d_o, const float* lse, float* delta, void* dq, hipStream_t) {
  check_problem(pr);
  check_ptrs({q, k, v, o, d_o, lse, delta, dq});
  return done();
}

hipError_t launch_decode(const DecodeProblem& pr, const DecodePlan& plan, const void* q, const void* k_cache,
                         const void* v_cache, void* o, float* lse, void* workspace, hipStream_t) {
  require(pr.B >= 1 && pr.Sq >= 1 && pr.Smax >= 1 && pr.Hq % pr.Hkv == 0, "decode sizes");
  require(plan.waves >= 1 && plan.workspace_bytes > plan.off_o, "decode plan");
  check_ptrs({q, k_cache, v_cache, o, lse, workspace});
  return done();
}

hipError_t decode_scratch(void** out) {
  // stands in for the device address of the static scratch array
  alignas(256) static unsigned char fake[256];
  *out = fake;
  return hipSuccess;
}

}  // namespace attn
