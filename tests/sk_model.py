"""Python emulation of the stream-K decode kernel's schedule arithmetic.

It follows the kernel's own integer steps, not the host planner's: the prefix
sums of per-sequence units (blocks plus the segment cost, times the head
groups), the search for a workgroup's first sequence, the piece loop that
skips segments of which a workgroup holds only virtual units, the partial
slot of a piece (2 w + side, side 0 when the piece starts at the workgroup's
first unit) and the slot list a merge reads (piece j of a segment belongs to
workgroup w_first + j). The planner's work items are computed independently
by the host code, so comparing the two checks the kernel's arithmetic
against the plan; the trace build's device records are compared with this
emulation on the GPU.
"""

from __future__ import annotations


def heads_per_wg(hkv: int) -> int:
    return 8 if hkv % 8 == 0 else 4 if hkv % 4 == 0 else 2 if hkv % 2 == 0 else 1


def emulate(lens, bs: int, hkv: int, max_blocks: int, cost: int, W: int):
    """Per-workgroup piece lists and the merge list of every shared segment.

    Returns (C, pieces, merges): pieces[w] is a list of (sequence, head
    group, first block, end block, slot or -1 when direct, pieces of the
    segment, first unit); merges maps (sequence, head group) of a segment
    with several pieces to (first unit of the segment, workgroup of its first
    piece, slots read in piece order)."""
    hw = heads_per_wg(hkv)
    n_hg = hkv // hw
    nbs = [max(0, min(-(-int(x) // bs), max_blocks)) for x in lens]
    pre = [0]
    for nb in nbs:
        pre.append(pre[-1] + (nb + cost) * n_hg)
    U = pre[-1]
    C = -(-U // W)
    pieces = [[] for _ in range(W)]
    merges = {}
    for w in range(W):
        u = w * C
        u_end = min(U, u + C)
        if u >= u_end:
            continue
        # Last s with pre[s] <= u.
        s, hi = 0, len(lens) - 1
        while s < hi:
            mid = (s + hi + 1) // 2
            if pre[mid] <= u:
                s = mid
            else:
                hi = mid - 1
        while u < u_end:
            if u >= pre[s + 1]:
                s += 1
            nb = nbs[s]
            seg_units = nb + cost
            hg = (u - pre[s]) // seg_units
            seg_start = pre[s] + hg * seg_units
            seg_end = seg_start + seg_units
            real_end = seg_start + (nb if nb > 0 else 1)
            if u >= real_end:
                u = min(seg_end, u_end)
                continue
            b_lo = u - seg_start
            piece_end = min(u_end, real_end)
            b_hi = min(piece_end - seg_start, nb)
            w_first = seg_start // C
            n_pieces = (real_end - 1) // C - w_first + 1
            direct = n_pieces == 1
            slot = -1 if direct else 2 * w + (0 if u == w * C else 1)
            pieces[w].append((s, hg, b_lo, b_hi, slot, n_pieces, u))
            if not direct and (s, hg) not in merges:
                wf = seg_start // C
                slots = [2 * (wf + j) + (1 if j == 0 and seg_start != (wf + j) * C else 0)
                         for j in range(n_pieces)]
                merges[(s, hg)] = (seg_start, wf, slots)
            u = min(seg_end, u_end)
    return C, pieces, merges


def work_items(pieces, hkv: int):
    """The emulated pieces as the planner's work items (one per KV head of
    the head group), in launch order."""
    hw = heads_per_wg(hkv)
    items = []
    for w, lst in enumerate(pieces):
        for s, hg, b_lo, b_hi, _slot, _n, _u in lst:
            items += [(s, hg * hw + k, w, b_lo, b_hi) for k in range(hw)]
    return items
