"""The absorbed decode's split-KV work plan, restated in Python for the tests.

The library plans on the host from the sequence lengths: the keys of all
sequences, one sequence after another, each preceded by ``SEGMENT_COST``
placeholder keys, form one long work order; workgroup g takes positions
[g R, (g + 1) R) of it (R, the quota, a multiple of 32 giving about one
workgroup per CU, at most ``max_quota``); where such a range cuts a sequence
the cut moves to the nearest multiple of 32 keys of that sequence.  The
decode over an E4M3 cache works on tiles of 64 keys: its quota and cuts are
multiples of 64 (``tile=64``).  Sequence b,
whose first key sits at r_b in the work order, collects one partial result per
workgroup that touches it.

The tests use this to place inputs inside a segment (not in its first tile)
and to check the library's workspace size against the plan.
"""
TILE = 32
SEGMENT_COST = 256                 # placeholder keys ahead of each sequence
TARGET_GROUPS = 256                # about one workgroup per CU
MAX_CHUNK_BLOCKS = 512             # block ids one segment may stage


def max_quota(tile=TILE):
    return ((MAX_CHUNK_BLOCKS - 2) * 16 - tile) // tile * tile


MAX_QUOTA = max_quota()


def plan(lens, tile=TILE):
    """(quota, groups, segments) where segments[b] lists the (k0, k1, slot)
    key ranges of sequence b, in order."""
    total = sum(L + SEGMENT_COST for L in lens if L > 0)
    quota = tile * max(1, -(-total // (tile * TARGET_GROUPS)))
    quota = min(quota, max_quota(tile))
    groups = -(-total // quota)
    segs = []
    st = 0
    for L in lens:
        if L <= 0:
            segs.append([])
            continue
        r0 = st + SEGMENT_COST

        def cut(x):
            if x <= 0:
                return 0
            if x >= L:
                return L
            return min(L, (x + tile // 2) // tile * tile)

        mine = []
        for g in range(r0 // quota, (r0 + L - 1) // quota + 1):
            k0, k1 = cut(g * quota - r0), cut((g + 1) * quota - r0)
            mine.append((k0, k1, g - r0 // quota))
        segs.append(mine)
        st = r0 + L
    return quota, groups, segs


def max_slots(lens, tile=TILE):
    _, _, segs = plan(lens, tile)
    return max([1] + [len(s) for s in segs])


def workspace_bytes(lens, heads, kv_lora_rank, tile=TILE):
    """Workspace the plan needs: the absorbed query [B, H, r_kv] bf16, then
    one partial entry per (workgroup g, sequence b) segment at index g + b
    (so groups + B entries): outputs [., H, r_kv] fp16 and (max, sum) pairs
    [., H, 2] fp32, each region rounded up to 256 bytes."""
    a = lambda x: (x + 255) // 256 * 256
    _, groups, _ = plan(lens, tile)
    B, P = len(lens), groups + len(lens)
    return a(B * heads * kv_lora_rank * 2) + a(P * heads * kv_lora_rank * 2) + a(P * heads * 2 * 4)


def entries(lens, tile=TILE):
    """Partial-buffer entry of every segment: (b, slot) -> g + b.  Distinct
    for distinct segments, all below groups + B."""
    quota, groups, segs = plan(lens, tile)
    out = {}
    st = 0
    for b, L in enumerate(lens):
        r0 = st + SEGMENT_COST
        for _, _, slot in segs[b]:
            out[(b, slot)] = r0 // quota + slot + b
        st = r0 + L
    return out, groups + len(lens)
