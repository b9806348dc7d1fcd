"""The stream-K kernel's schedule arithmetic, emulated on the CPU
(tests/sk_model.py), against the host planner's work items and the
invariants the in-launch merge relies on: every piece of a shared segment
publishes to its own partial slot, no two pieces of a launch share a slot,
and the slot list a merge reads is exactly the slots the segment's pieces
published. No GPU; the device's own records are compared with the same
emulation in tests/test_gpu_trace.py."""

import numpy as np
import pytest

from paged_kv_cache_178_amd import binding as B
from tests import sk_model


def desc(num_seqs, hq, hkv, bs, max_blocks):
    d = B.Desc()
    d.dtype = B.NP_BF16
    d.num_seqs = d.n_q_total = num_seqs
    d.num_q_heads, d.num_kv_heads, d.head_dim, d.block_size = hq, hkv, 64, bs
    d.n_blocks = 10 ** 6
    d.max_blocks_per_seq = max_blocks
    d.q_stride[0], d.q_stride[1] = hq * 64, 64
    d.kv_stride[0], d.kv_stride[1], d.kv_stride[2] = bs * hkv * 64, hkv * 64, 64
    d.out_stride[0], d.out_stride[1] = hq * 64, 64
    d.bt_stride = max_blocks
    return d


def check_invariants(pieces, merges):
    published = {}
    slots = set()
    for w, lst in enumerate(pieces):
        for s, hg, b_lo, b_hi, slot, n_pieces, u in lst:
            assert b_hi >= b_lo
            if slot < 0:
                assert n_pieces == 1
                continue
            assert slot // 2 == w, "a piece publishes to one of its own workgroup's slots"
            assert slot not in slots, f"slot {slot} written twice"
            slots.add(slot)
            published.setdefault((s, hg), []).append((w, slot))
    assert set(published) == set(merges)
    for seg, lst in published.items():
        _start, _wf, want = merges[seg]
        assert len(lst) == len(want), "arrivals must equal the segment's pieces"
        assert [slot for _w, slot in sorted(lst)] == want


def random_case(seed):
    rng = np.random.default_rng(7000 + seed)
    num_seqs = int(rng.integers(1, 90))
    bs = int(rng.choice([1, 4, 16, 64]))
    max_blocks = int(rng.integers(1, 300))
    lens = np.where(rng.random(num_seqs) < 0.25,
                    rng.integers(1, max_blocks * bs + 1, size=num_seqs),
                    rng.integers(1, max(2, max_blocks * bs // 8) + 1, size=num_seqs))
    lens = np.minimum(lens, max_blocks * bs).astype(np.int32)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    opts = B.PlanOpts(schedule=2)
    cost = 4
    if seed % 3:
        opts.num_cus = int(rng.integers(1, 300))
        opts.wgs_per_cu = int(rng.integers(1, 5))
        opts.min_blocks_per_split = int(rng.integers(1, 20))
        opts.segment_cost = cost = int(rng.integers(1, 12))
    return lens, bs, hkv, max_blocks, cost, opts


@pytest.mark.parametrize("chunk", range(10))
def test_emulation_matches_plan(chunk):
    """3000 random shapes: the kernel's arithmetic names exactly the plan's
    pieces, in the same order, with a consistent merge."""
    for seed in range(chunk * 300, (chunk + 1) * 300):
        lens, bs, hkv, max_blocks, cost, opts = random_case(seed)
        d = desc(len(lens), hkv * 2, hkv, bs, max_blocks)
        plan = B.np_plan(d, lens, None, opts)
        (W, _, _), _, _ = plan.launch_shape()
        C, pieces, merges = sk_model.emulate(lens, bs, hkv, max_blocks, cost, W)
        assert C == plan.blocks_per_split, seed
        assert sk_model.work_items(pieces, hkv) == plan.work_items(), seed
        n_max = max([p[5] for lst in pieces for p in lst], default=1)
        assert n_max == plan.max_splits, seed
        check_invariants(pieces, merges)


def test_wrong_side_rule_is_caught():
    """A planted mistake in the slot rule (every piece on side 0) makes two
    pieces of one workgroup share a slot, which the invariants reject."""
    # 7 blocks per sequence, cost 1: segments of 8 units, 5 workgroups of 5
    # units; workgroup 1 ends segment 0 and starts segment 1.
    lens = np.array([100, 100, 100], np.int32)
    C, pieces, merges = sk_model.emulate(lens, 16, 4, 8, 1, 5)
    assert [p[4] % 2 for p in pieces[1]] == [0, 1]
    bad = [[(s, hg, a, b, (2 * w if slot >= 0 else -1), n, u) for s, hg, a, b, slot, n, u in lst]
           for w, lst in enumerate(pieces)]
    check_invariants(pieces, merges)
    with pytest.raises(AssertionError):
        check_invariants(bad, merges)
