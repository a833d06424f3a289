"""The host's launch plans, restated for the tests (no GPU needed): how many
work items a chunked dQ launch has, which fixes its workspace size."""


def chunk_prefix(m, t):
    return sum(-(-x // t) for x in range(1, m + 1))


def dq_chunk_items(B, Lq, Lk, Hl, causal):
    """Work items of a chunked dQ launch (0: whole walks), as the host plans
    them: 128-row query blocks over batch x local heads, 64-key tiles; the
    causal block qb cut into ceil((qb + 1) / t) parts, a bidirectional block
    into c parts; the cut ranked by its critical path in tiles (one round of
    512 workgroups: the longest item; more: the average load plus half an
    item), 2 tiles of start-up per round, 1/64 tile per item and 3 for the
    extra launch, taken when it beats the whole walks by 10 %."""
    nqb, nhb = -(-Lq // 128), B * Hl
    W, nkt = nqb * nhb, -(-Lk // 64)
    if W >= 2048:
        return 0
    total = nhb * (nqb * (nqb - 1) + nkt) if causal else W * nkt
    avg = total / 512
    rounds = lambda n, per: -(-n // per)
    if (W < 512) if causal else (W <= 256):
        whole = max((nkt + 1) // 2, avg) + 2 * rounds(W, 256)
    else:
        whole = max(nkt, avg) + 2 * rounds(W, 512)
    best, items_best = 0.9 * whole, 0
    cuts = ([(nhb * chunk_prefix(nqb, t), min(2 * t, nkt)) for t in range(1, nqb)] if causal else
            [(W * c, -(-nkt // c)) for c in range(2, nkt + 1) if W * c <= 2048])
    for items, longest in cuts:
        if items > 2048:
            continue
        path = longest if items <= 512 else max(longest, avg + 0.5 * longest)
        cost = path + 2 * rounds(items, 512) + items / 64 + 3
        if cost < best:
            best, items_best = cost, items
    return items_best


def dkdv_chunk_t(B, L, Hk, causal):
    """Part length t of a balanced dK/dV split (0: halves or no split): causal
    bf16 launches of at most 128 key-block columns (batch x local K/V heads x
    128-token key blocks) cut key block kb into ceil((nkb - kb) / t) parts,
    with the smallest t whose parts fit the halves' two slots per column,
    taken when 2t is at most 0.8 of nkb."""
    nkb, nkhb = -(-L // 128), B * Hk
    ncol = nkb * nkhb
    if not causal or ncol >= 512 or 2 * ncol > 256:
        return 0
    for t in range(1, nkb):
        if nkhb * chunk_prefix(nkb, t) <= 2 * ncol:
            return t if 10 * t <= 4 * nkb else 0
    return 0


def fwd_groups(B, Lq, Hq, causal):
    """Wave groups that share each query block's key walk in a dense bf16
    forward launch of W = ceil(Lq / 256) x B x Hq blocks: four below 192 causal
    blocks or up to 64 bidirectional ones, two below 384 causal or up to 128
    bidirectional ones, else one walk per block."""
    W = -(-Lq // 256) * B * Hq
    if W < 192 if causal else W <= 64:
        return 4
    if W < 384 if causal else W <= 128:
        return 2
    return 1


def dkdv_whole_walks(B, L, Hk, causal):
    """True when a dense bf16 dK/dV launch gives every key-block column one
    workgroup walking all its query tiles: causal launches of at least 512
    columns (batch x local K/V heads x 128-token key blocks), bidirectional
    ones of more than 128 (below those the walks are split)."""
    ncol = B * Hk * -(-L // 128)
    return ncol >= 512 if causal else ncol > 128
