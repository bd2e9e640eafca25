"""The work-chunk rule of the host-side plan, written once here for the tests.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages say only that planning inspects the sequence lengths and cache
metadata, picks a schedule and prepares the workspace, and that a plan is
reused while the geometry is unchanged (article "FlashInfer", section
"Plan and run"), and that a fixed schedule can leave GPU work uneven (same
article, section "Purpose and scope"). The exact rule below is this library's
reading; the C++ planner implements the same rule independently and the tests
require the two to agree item for item.

Rule (all integer arithmetic; ceil(a / b) for b > 0):

1.  Rows. Query rows are GQA-packed: row r of request b is query token r // G
    and query head g * G + r % G of KV head g. A tile holds ``rows_per_tile``
    consecutive rows (decode: rows_per_tile = G, one tile per request; prefill:
    128 rows). Request b has tiles_b = ceil(Q_b * G / rows_per_tile).
2.  KV extent of a tile. kv_end = L_b, or with the bottom-right causal mask
    kv_end = clamp(L_b - Q_b + t_last + 1, 0, L_b), where t_last is the query
    token of the tile's last row. With a sliding window of W >= 0 keys to the
    left (``window_left``; W < 0: none) the extent starts at
    kv_lo = max(0, L_b - Q_b + t_first - W) (t_first: the query token of the
    tile's first row), else kv_lo = 0. The tile's pages run from
    p_lo = floor(kv_lo / P) to p_hi = ceil(kv_end / P);
    pages = max(0, p_hi - p_lo).
3.  work = Hkv * sum over (b, tile) of pages.  target = num_cus * wg_per_cu.
    c_min = max(1, ceil(min_chunk_tokens / P)).
    c = max(c_min, ceil(work / target))   (c = c_min when work = 0).
4.  Each (b, tile, g) group splits into n_chunks = max(1, ceil(pages / c))
    chunks; chunk j covers pages [p_lo + j*c, min(p_lo + (j+1)*c, p_hi)) and
    KV tokens [min((p_lo + j*c)*P, kv_end), min((p_lo + (j+1)*c)*P, kv_end)).
    A group with one chunk writes its final output; a group with more chunks
    writes partial states into consecutive partial slots, assigned to split
    groups in (b, tile, g) order, chunk j at slot_begin + j; those groups are
    listed, in the same order, as merge groups.
5.  Items are executed longest first: sorted by descending KV token count,
    ties broken by ascending (b, tile, g, j).
6.  ``group_all``: every group writes partial states and is a merge group, also
    a group of one chunk (slots and merge groups as in 4, for every group). The
    cascade plans both of its levels this way (``cascade_spec``).

The cascade (docs index "Cascade Attention": a shared prefix evaluated once,
then merged with each request's suffix; article "FlashInfer", section
"Attention states") is planned as two parts. Level 0 is one "request" whose
query tokens are the batch's decode tokens (Q = batch) over the prefix
(L = prefix length), unmasked, 128-row tiles; level 1 is the batch decode over
the suffixes. Both with ``group_all``. Suffix group (b, g) also merges the
level-0 states of its G rows: packed rows b*G .. b*G + G - 1 of KV head g at
level 0, i.e. tile t = (b*G) // 128 from row (b*G) % 128 on (rows past 127 are
the next tile's first rows), whose n0 chunk slots start at (t * Hkv + g) * n0
(n0: the chunks of every level-0 group, which all have the same extent).
``cascade_spec`` takes the two levels' schedules explicitly; with no schedule
the library uses the decode default for level 1 and the prefill default with
wg_per_cu = 1 (one level-0 item per CU) for level 0.
"""

from __future__ import annotations

from dataclasses import dataclass, field


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class PlanSpec:
    chunk_pages: int
    rows_per_tile: int
    # (b, g, tile, page_begin, page_end, kv_begin, kv_end, slot) in execution order
    items: list = field(default_factory=list)
    # (b, tile, g, slot_begin, num_chunks) in (b, tile, g) order
    merge_groups: list = field(default_factory=list)
    num_slots: int = 0


def plan_spec(qo_lens, kv_lens, page_size: int, num_kv_heads: int, group_size: int,
              rows_per_tile: int, causal: bool, num_cus: int, wg_per_cu: int,
              min_chunk_tokens: int, window_left: int = -1, group_all: bool = False) -> PlanSpec:
    """Apply the rule in the module docstring. ``qo_lens`` / ``kv_lens`` per request."""
    P, G = int(page_size), int(group_size)
    B = len(kv_lens)
    tiles = []   # (b, tile, kv_end, p_lo, pages)
    for b in range(B):
        Q, L = int(qo_lens[b]), int(kv_lens[b])
        n_rows = Q * G
        for tile in range(_ceil_div(n_rows, rows_per_tile)):
            first_row = tile * rows_per_tile
            last_row = min((tile + 1) * rows_per_tile, n_rows) - 1
            t_first, t_last = first_row // G, last_row // G
            kv_end = min(max(L - Q + t_last + 1, 0), L) if causal else L
            kv_lo = max(0, L - Q + t_first - window_left) if window_left >= 0 else 0
            p_lo = kv_lo // P
            tiles.append((b, tile, kv_end, p_lo, max(0, _ceil_div(kv_end, P) - p_lo)))
    work = num_kv_heads * sum(t[4] for t in tiles)
    target = num_cus * wg_per_cu
    c_min = max(1, _ceil_div(min_chunk_tokens, P))
    c = max(c_min, _ceil_div(work, target))

    spec = PlanSpec(chunk_pages=c, rows_per_tile=rows_per_tile)
    raw = []      # (kv_count, b, tile, g, j, item)
    slot = 0
    for (b, tile, kv_end, p_lo, pages) in tiles:     # (b, tile) order
        n_chunks = max(1, _ceil_div(pages, c))
        grouped = n_chunks > 1 or group_all
        for g in range(num_kv_heads):                # then g
            slot_begin = slot if grouped else -1
            if grouped:
                spec.merge_groups.append((b, tile, g, slot_begin, n_chunks))
                slot += n_chunks
            for j in range(n_chunks):
                p0, p1 = p_lo + j * c, p_lo + min((j + 1) * c, pages)
                k0, k1 = min(p0 * P, kv_end), min((p_lo + (j + 1) * c) * P, kv_end)
                item = (b, g, tile, p0, p1, k0, k1, slot_begin + j if grouped else -1)
                raw.append((k1 - k0, b, tile, g, j, item))
    raw.sort(key=lambda r: (-r[0], r[1], r[2], r[3], r[4]))
    spec.items = [r[5] for r in raw]
    spec.num_slots = slot
    return spec


def cascade_spec(prefix_len: int, suffix_lens, page_size: int, num_kv_heads: int,
                 group_size: int, sched_prefix, sched_suffix):
    """(level-0 PlanSpec, level-1 PlanSpec, base) of the cascade rule in the module
    docstring; base[i] = (base_slot_begin, base_num_chunks, base_row) of the i-th
    level-1 merge group. ``sched_*`` = (num_cus, wg_per_cu, min_chunk_tokens)."""
    B, G, H = len(suffix_lens), int(group_size), int(num_kv_heads)
    level0 = plan_spec([B], [prefix_len], page_size, H, G, 128, False, *sched_prefix,
                       group_all=True)
    level1 = plan_spec([1] * B, list(suffix_lens), page_size, H, G, G, False, *sched_suffix,
                       group_all=True)
    n0 = level0.merge_groups[0][4] if level0.merge_groups else 0
    base = []
    for (b, _tile, g, _sb, _n) in level1.merge_groups:
        t = (b * G) // 128
        base.append(((t * H + g) * n0, n0, (b * G) % 128))
    return level0, level1, base


def pod_order(items_a, items_b) -> list:
    """Launch order of a grid that runs two plans' items (the mixed prefill + decode
    launch): entry i >= 0 is items_a[i], entry -j-1 is items_b[j].

    Rule (this library's; the pages only name the fused prefill + decode kernel):
    each list keeps its own order; an item costs kv_end - kv_begin + 1; the next
    entry is taken from the list whose emitted cost, as a fraction of that list's
    total, is smaller, and from ``items_a`` on ties.
    """
    from fractions import Fraction
    cost_a = [int(it[6]) - int(it[5]) + 1 for it in items_a]
    cost_b = [int(it[6]) - int(it[5]) + 1 for it in items_b]
    tot_a, tot_b = sum(cost_a), sum(cost_b)
    i = j = 0
    frac_a = frac_b = Fraction(0)
    order = []
    while i < len(items_a) or j < len(items_b):
        if j == len(items_b) or (i < len(items_a) and frac_a <= frac_b):
            frac_a += Fraction(cost_a[i], tot_a)
            order.append(i)
            i += 1
        else:
            frac_b += Fraction(cost_b[j], tot_b)
            order.append(-j - 1)
            j += 1
    return order
