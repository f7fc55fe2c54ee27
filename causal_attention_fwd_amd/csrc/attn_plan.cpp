// Host-side planning shared by the C ABI and the launchers: the largest grid a
// problem launches (checked against the hardware limit before any launch) and
// the decode work split with its workspace layout. Plain C++ (no device code),
// so a host-only build (the sanitizer test) links the same planning logic.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "attn_launch.h"

namespace attn {

int64_t max_grid(const Problem& pr) {
  // smallest blocks: 64 query rows (forward/dQ), 64 key rows (dK/dV), 16 rows (preprocess)
  const int64_t nb = ((int64_t)pr.S + 63) / 64;
  int64_t m = nb * pr.B * pr.Hq;
  const int64_t pre = ((int64_t)pr.B * pr.S * pr.Hq + 15) / 16;
  // RoPE pre-pass: one workgroup per (sequence, position)
  const int64_t rope = (int64_t)pr.B * pr.S;
  m = m > pre ? m : pre;
  return m > rope ? m : rope;
}

int dkdv_parts(const Problem& pr) {
  constexpr int64_t kCUs = 256, kMaxParts = 8;
  // the dK/dV pass runs one 8-wave (d = 64) or 4-wave (d = 128) workgroup per
  // CU over 128-key blocks
  const int64_t units = ((int64_t)pr.S + 127) / 128 * pr.B * pr.Hkv;
  if (units >= kCUs) return 1;
  const int64_t want = (kCUs + units - 1) / units;
  // at most a quarter of the longest block's (head, query tile) iterations:
  // the uneven deal gives that block at most 2 * parts - 1 workgroups, so each
  // still gets more than two (one per wave group)
  const int64_t iters0 = ((int64_t)pr.S + 63) / 64 * (pr.Hq / pr.Hkv);
  const int64_t cap = std::max<int64_t>(1, iters0 / 4);
  return (int)std::min(std::min(want, cap), kMaxParts);
}

int dkdv_blocks(const Problem& pr) { return (int)(((int64_t)pr.S + 127) / 128); }

int dkdv_max_parts(const Problem& pr) {
  const int parts = dkdv_parts(pr);
  if (parts <= 1) return 1;
  // the first block has the most work, but the rounding of the deal can give
  // a later one a part more: take the largest count
  const int nkb = dkdv_blocks(pr);
  int most = 1;
  for (int kb = 0; kb < nkb; ++kb)
    most = std::max(most, dkdv_part_base(kb + 1, nkb, parts, pr.S, pr.causal) -
                              dkdv_part_base(kb, nkb, parts, pr.S, pr.causal));
  return most;
}

size_t bwd_workspace_bytes(const Problem& pr) {
  if (dkdv_parts(pr) <= 1) return 0;
  return (size_t)2 * dkdv_max_parts(pr) * pr.B * pr.S * pr.Hkv * pr.d * sizeof(float);
}

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

// Workspace layout: [hdr: 256 B][uinfo: int2 per unit][partial LSE][partial O],
// each part 256-byte aligned.
DecodePlan plan_decode(const DecodeProblem& pr) {
  // one wave per decode workgroup; as many waves as fit on the 256 CUs at
  // once (LDS decides: kDecodeStages stages of a 64-key K and V tile), but no
  // more than there are tiles
  constexpr int kCUs = 256;
  const int per_cu = (pr.d == 64 ? 8 : 4) / kDecodeStages;
  const int64_t rows = (int64_t)(pr.Hq / pr.Hkv) * pr.Sq;  // query rows per kv head
  DecodePlan plan;
  plan.rb = (int)((rows + 31) / 32);
  plan.ru = plan.rb == 1 ? (int)rows : 32;
  const int64_t units = (int64_t)pr.B * pr.Hkv * plan.rb;
  const int64_t tmax = units * (((int64_t)pr.Smax + 63) / 64);
  plan.waves = (int)std::min<int64_t>((int64_t)kCUs * per_cu, tmax);
  const int64_t slots = plan.waves + units - 1;
  const int64_t R = plan.ru;
  plan.off_uinfo = 256;
  plan.off_lse = plan.off_uinfo + align256((size_t)units * 8);
  plan.off_o = plan.off_lse + align256((size_t)(slots * R) * sizeof(float));
  plan.workspace_bytes = plan.off_o + (size_t)(slots * R) * pr.d * sizeof(float);
  return plan;
}

}  // namespace attn
