"""The split dK/dV pass's workgroups per 128-key block, from the rule the
planner documents (not from the library): each (sequence, kv head) gets
parts * nkb workgroups, parts = min(ceil(256 / blocks), a quarter of the first
block's (head, query tile) iterations, 8); every block gets one, and the rest
go in proportion to the blocks' query tiles (ceil(S/64) - 2*kb under the
causal mask, all equal without it). All ones when there is no split."""


def dealt_parts(B, S, Hq, Hkv, causal):
    nkb = (S + 127) // 128
    units = nkb * B * Hkv
    if units >= 256:
        return [1] * nkb
    parts = min((256 + units - 1) // units, max(1, (S + 63) // 64 * (Hq // Hkv) // 4), 8)
    n64 = (S + 63) // 64
    w = [n64 - 2 * kb if causal else 1 for kb in range(nkb)]
    extra = (parts - 1) * nkb
    cum, first = 0, []
    for kb in range(nkb + 1):
        first.append(kb + extra * cum // sum(w))
        if kb < nkb:
            cum += w[kb]
    return [first[kb + 1] - first[kb] for kb in range(nkb)]
