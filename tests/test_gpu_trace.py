"""What the decode kernels actually read, from the trace build
(libnp_paged_trace.so): every workgroup records the pieces or the split it
took, the partial slot it published to, its arrival ticket and, for the
workgroup that merged, the slots it read. The records are compared bit for
bit with the host plan's work items and with the CPU emulation of the
stream-K arithmetic (tests/sk_model.py), and the outputs with the oracle
("Day 23: the real triton.jit paged-attention kernel", section "Why it
matters": which tile did a program actually read)."""

import numpy as np
import pytest
import torch

from paged_kv_cache_178_amd import binding
from paged_kv_cache_178_amd import workloads as wl
from tests import helpers as H
from tests import sk_model

pytestmark = pytest.mark.gpu

SK_WORDS, SK_PIECES, SK_MERGE0, SK_MERGE_WORDS = 2048, 32, 8 + 8 * 32, 8 + 768
SK_STAMP0 = SK_MERGE0 + 2 * SK_MERGE_WORDS
UNI_WORDS = 32


def sk_stamps_in_order(r):
    """The stream-K record's timestamps (np_trace.h: start, schedule known,
    each piece's start and publish, pieces done, each merge, end) are all
    taken and never go back in time (s_memrealtime is one clock for the
    whole device)."""
    def t(at):
        lo, hi = int(r[SK_STAMP0 + at]) & 0xFFFFFFFF, int(r[SK_STAMP0 + at + 1]) & 0xFFFFFFFF
        return (hi << 32) | lo
    seq = [t(0), t(2)]
    if t(4) == 0:   # a workgroup whose unit range is empty stops after the schedule
        return int(r[0]) == 0 and int(r[1]) == 0 and 0 < t(0) <= t(2) <= t(6)
    for i in range(min(int(r[0]), SK_PIECES)):
        seq += [t(8 + 4 * i), t(10 + 4 * i)]
    seq.append(t(4))
    for j in range(int(r[1])):
        seq += [t(8 + 4 * SK_PIECES + 4 * j), t(10 + 4 * SK_PIECES + 4 * j)]
    seq.append(t(6))
    return all(x > 0 for x in seq) and all(a <= b for a, b in zip(seq, seq[1:]))


def run_traced(inp, opts, words):
    lib = binding.trace_library()
    dev = H.to_device(inp)
    out = torch.empty_like(dev["q"])
    desc = binding.make_desc(dev["q"], dev["k_pool"], dev["block_table"], out=out,
                             scale=inp.scale)
    plan = binding.np_plan(desc, inp.context_lens, None, opts, lib=lib)
    grid, _, _ = plan.launch_shape()
    n_wg = grid[0] * grid[1] * grid[2]
    trace = torch.zeros(n_wg * words, dtype=torch.int32, device="cuda")
    ws = binding.workspace_for(plan, "cuda")
    print(f"[trace] {inp.name} seqs={inp.num_seqs} schedule={plan.schedule} grid={grid}",
          flush=True)
    st = lib.np_debug_set_trace(trace.data_ptr(), trace.numel() * 4)
    assert st == 0
    try:
        binding.np_paged_attention_decode(desc, plan, dev["q"], dev["k_pool"], dev["v_pool"],
                                          dev["block_table"], dev["context_lens"], out, ws)
        torch.cuda.synchronize()
    finally:
        lib.np_debug_set_trace(None, 0)
    H.assert_close(out, H.oracle_out(inp), inp.dtype, inp.name)
    return plan, trace.view(n_wg, words).cpu().numpy()


SK_CASES = [dict(num_cus=1, wgs_per_cu=1),
            dict(num_cus=300, wgs_per_cu=8, min_blocks_per_split=1, segment_cost=1),
            dict(num_cus=37, wgs_per_cu=3, min_blocks_per_split=1, segment_cost=11),
            dict()]


@pytest.mark.parametrize("case", list(range(len(SK_CASES))) + ["batching", "hkv4", "hkv2"],
                         ids=["one_wg", "unit_per_wg", "virtual_only", "auto", "batching",
                              "four_heads_per_wg", "two_heads_per_wg"])
def test_stream_k_trace_matches_plan(case):
    lens = [1, 16, 17, 900, 4096, 33, 2000, 15]
    if case == "batching":
        inp, shape = wl.continuous_batching(), {}
    elif case == "hkv4":     # a workgroup serves 4 KV heads
        inp, shape = wl.custom(43, lens, hq=16, hkv=4, d=64, dtype="bf16"), {}
    elif case == "hkv2":     # 2 KV heads, many small pieces
        inp = wl.custom(44, lens, hq=8, hkv=2, d=64, dtype="bf16")
        shape = SK_CASES[2]
    else:
        inp = wl.custom(41, [1, 16, 17, 900, 4096, 33, 2000, 15], hq=32, hkv=8, d=64,
                        dtype="bf16")
        shape = SK_CASES[case]
    opts = binding.PlanOpts(schedule=2, **shape)
    plan, rec = run_traced(inp, opts, SK_WORDS)
    W = rec.shape[0]
    cost = shape.get("segment_cost", 0) or 4
    C, want, merges = sk_model.emulate(inp.context_lens.numpy(), inp.block_size,
                                       inp.num_kv_heads, inp.block_table.shape[1], cost, W)
    assert sk_model.work_items(want, inp.num_kv_heads) == plan.work_items()
    n_hg = inp.num_kv_heads // sk_model.heads_per_wg(inp.num_kv_heads)
    U = sum((min(-(-int(x) // inp.block_size), inp.block_table.shape[1]) + cost) * n_hg
            for x in inp.context_lens.tolist())
    tickets, merged = {}, {}
    for w in range(W):
        r = rec[w]
        assert r[3] == 0, f"workgroup {w}: trace overflow"
        assert (r[4], r[5]) == (U, C), w
        assert sk_stamps_in_order(r), f"workgroup {w}: timestamps"

        n = int(r[0])
        got = [tuple(int(x) for x in r[8 + 8 * i: 8 + 8 * i + 7]) for i in range(n)]
        # (sequence, head group, first, end, slot, pieces, ticket, first unit)
        assert [g[:6] + (int(r[8 + 8 * i + 7]),) for i, g in enumerate(got)] == want[w], w
        for i, g in enumerate(got):
            if g[4] >= 0:
                tickets.setdefault((g[0], g[1]), []).append((g[6], w))
            else:
                assert g[6] == -1
        for j in range(int(r[1])):
            m = r[SK_MERGE0 + SK_MERGE_WORDS * j:]
            key = (int(m[0]), int(m[1]))
            assert key not in merged, f"segment {key} merged twice"
            n_p = int(m[2])
            merged[key] = (w, (int(m[3]), int(m[4]), [int(x) for x in m[8:8 + n_p]]))
    assert set(merged) == set(merges)
    for key, (w, got_merge) in merged.items():
        assert got_merge == merges[key], key
        t = sorted(tickets[key])
        n_p = len(merges[key][2])
        assert [x[0] for x in t] == list(range(n_p)), f"tickets of {key}: {t}"
        assert t[-1][1] == w, "the merge is done by the last arrival"


@pytest.mark.parametrize("maker", [lambda: wl.llama_decode(4096),
                                   lambda: wl.custom(48, [4096, 700, 3000, 17], hq=32, hkv=8,
                                                     d=64, dtype="bf16")],
                         ids=["llama_4096", "ragged"])
def test_uniform_trace_matches_plan(maker):
    inp = maker()
    plan, rec = run_traced(inp, binding.PlanOpts(schedule=1), UNI_WORDS)
    items = [tuple(int(x) for x in r[2:7]) for r in rec if (r[0] & 1) and r[8] > 0]
    assert items == plan.work_items()
    by_head = {}
    for r in rec:
        if not (r[0] & 1) or r[8] == 0:
            continue
        by_head.setdefault((int(r[2]), int(r[3])), []).append(r)
    for key, rs in by_head.items():
        splits = int(rs[0][8])
        assert len(rs) == splits
        if splits == 1:
            assert rs[0][0] & 4 and rs[0][7] == -1
            continue
        assert sorted(int(r[7]) for r in rs) == list(range(splits)), key
        mergers = [r for r in rs if r[0] & 2]
        assert len(mergers) == 1 and mergers[0][7] == splits - 1, key
