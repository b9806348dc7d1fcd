"""GPU parity of the contiguous-cache mode (NULL block table) through the C ABI.

A NULL table makes logical block j of sequence s physical block
s * max_blocks_per_seq + j, i.e. dense [num_seqs, capacity, Hkv, d] caches: the
split-KV decode over one contiguous KV tensor and the fused prefill of "I Wrote
the Three Attention Kernels That Run LLM Inference" (sections "2. Split-KV
flash-decoding", "1. Fused prefill attention"; shapes of its "Benchmark
method": B = 4, H = 16, D = 64, fp16). The oracle gets the explicit identity
table. Tolerances: atol = rtol = 1e-2 for fp16/bf16, 1e-5 for fp32.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_178_amd import binding as B
from paged_kv_cache_178_amd import workloads as wl
from tests import helpers as H

pytestmark = pytest.mark.gpu


def dense_decode(inp, opts=None, out=None):
    """Decode through make_desc_contiguous with a NULL table."""
    dev = H.to_device(inp)
    k = wl.dense_view(dev["k_pool"], inp.num_seqs)
    v = wl.dense_view(dev["v_pool"], inp.num_seqs)
    out = torch.empty_like(dev["q"]) if out is None else out
    desc = B.make_desc_contiguous(dev["q"], k, out=out, scale=inp.scale)
    assert B.np_check_paged_inputs(desc, dev["q"], k, v, None, dev["context_lens"], out,
                                   None, inp.context_lens) == 0
    plan = B.np_plan(desc, inp.context_lens, None, opts)
    ws = B.workspace_for(plan, "cuda")
    B.np_paged_attention_decode(desc, plan, dev["q"], k, v, None, dev["context_lens"], out, ws)
    torch.cuda.synchronize()
    return out, plan


@pytest.mark.parametrize("opts", [dict(), dict(schedule=1), dict(schedule=2),
                                  dict(force_blocks_per_split=1),
                                  dict(force_blocks_per_split=5, combine_mode=1)],
                         ids=["auto", "uniform", "stream_k", "split_per_block", "separate"])
def test_splitkv_shape_decode(opts):
    inp = wl.splitkv_decode(1024)
    print(f"[contiguous decode] {inp.name} opts={opts}", flush=True)
    got, _ = dense_decode(inp, B.PlanOpts(**opts))
    H.assert_close(got, H.oracle_out(inp), "f16", inp.name)


@pytest.mark.parametrize("splits", wl.SPLITKV_SPLITS)
def test_splitkv_num_splits_sweep_matches(splits):
    """The pages' num_splits values (as blocks per split, page-aligned) all
    give the oracle's output at N = 2048."""
    inp = wl.splitkv_decode(2048)
    nb = 2048 // 16
    bps = max(1, -(-nb // splits))
    print(f"[contiguous decode] {inp.name} splits={splits} bps={bps}", flush=True)
    got, plan = dense_decode(inp, B.PlanOpts(force_blocks_per_split=bps))
    assert plan.max_splits == -(-nb // bps)
    H.assert_close(got, H.oracle_out(inp), "f16", f"splits={splits}")


def test_contiguous_equals_identity_table_bit_exact():
    """Same kernel, same schedule: a NULL table and the explicit identity
    table give the same bits."""
    inp = wl.custom(60, [1000, 1024, 17, 512], hq=16, hkv=16, d=64, dtype="f16",
                    max_blocks=64, identity=True)
    for opts in (dict(schedule=1), dict(schedule=2)):
        print(f"[contiguous decode] identity table vs NULL, opts={opts}", flush=True)
        got, _ = dense_decode(inp, B.PlanOpts(**opts))
        ref = H.gpu_decode(inp, opts=B.PlanOpts(**opts))
        assert torch.equal(got, ref)
        H.assert_close(got, H.oracle_out(inp), "f16", "ragged contiguous")


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 64), ("f32", 8, 2, 128),
                                            ("f16", 12, 4, 48)])
def test_contiguous_other_shapes(dtype, hq, hkv, d):
    inp = wl.custom(61, [300, 77, 1], hq=hq, hkv=hkv, d=d, dtype=dtype, max_blocks=20,
                    identity=True)
    print(f"[contiguous decode] {dtype} hq={hq} hkv={hkv} d={d}", flush=True)
    got, _ = dense_decode(inp)
    H.assert_close(got, H.oracle_out(inp), dtype, "contiguous")


def test_fused_prefill_contiguous():
    """Whole-prompt causal prefill (past = 0) over dense caches."""
    inp = wl.fused_prefill(320, num_seqs=2)
    dev = H.to_device(inp)
    k = wl.dense_view(dev["k_pool"], inp.num_seqs)
    v = wl.dense_view(dev["v_pool"], inp.num_seqs)
    out = torch.empty_like(dev["q"])
    desc = B.make_desc_contiguous(dev["q"], k, out=out, scale=inp.scale)
    plan = B.np_plan(desc, inp.context_lens, inp.q_start)
    ws = B.workspace_for(plan, "cuda")
    print(f"[contiguous prefill] {inp.name}", flush=True)
    B.np_paged_attention_prefill(desc, plan, dev["q"], k, v, None, dev["context_lens"],
                                 dev["q_start"], out, ws)
    torch.cuda.synchronize()
    H.assert_close(out, H.oracle_out(inp, prefill=True), "f16", inp.name)


def test_append_contiguous_bit_exact():
    """The cache write with a NULL table stores row t of sequence s at token t
    of the dense cache."""
    num_seqs, cap, hkv, d = 3, 64, 4, 64
    g = torch.Generator().manual_seed(62)
    k = torch.randn((num_seqs * cap // 16, 16, hkv, d), generator=g).to(torch.float16)
    v = torch.randn((num_seqs * cap // 16, 16, hkv, d), generator=g).to(torch.float16)
    lens = np.array([40, 64, 5], np.int32)
    chunk = np.array([7, 20, 5], np.int32)
    new_start = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    n = int(new_start[-1])
    kn = torch.randn((n, hkv, d), generator=g).to(torch.float16)
    vn = torch.randn((n, hkv, d), generator=g).to(torch.float16)
    table = np.arange(num_seqs * cap // 16, dtype=np.int32).reshape(num_seqs, cap // 16)
    want_k, want_v = oracle.append_kv(k.numpy(), v.numpy(), table, lens, new_start,
                                      kn.numpy(), vn.numpy())
    kd, vd = k.cuda(), v.cuda()
    kdense, vdense = wl.dense_view(kd, num_seqs), wl.dense_view(vd, num_seqs)
    q_dummy = torch.zeros((n, 4, d), dtype=torch.float16, device="cuda")
    desc = B.make_desc_contiguous(q_dummy, kdense, n_q_total=n)
    plan = B.np_plan(desc, lens, new_start)
    print("[contiguous append] 3 sequences", flush=True)
    B.np_paged_kv_append(desc, plan, kn.cuda(), vn.cuda(), None,
                         torch.from_numpy(lens).cuda(), torch.from_numpy(new_start).cuda(),
                         kdense, vdense)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().view(torch.int16).numpy(), want_k)
    assert np.array_equal(vd.cpu().view(torch.int16).numpy(), want_v)


@pytest.mark.parametrize("opts", [dict(), dict(force_blocks_per_split=128)],
                         ids=["default", "8_splits"])
def test_splitkv_full_size_16k(opts):
    """The largest context of the split-KV sweep, in the plans the benchmark
    times (the planner's default and the best forced split), against the full
    oracle."""
    inp = wl.splitkv_decode(16384)
    print(f"[contiguous decode] {inp.name} opts={opts}", flush=True)
    got, _ = dense_decode(inp, B.PlanOpts(**opts))
    H.assert_close(got, H.oracle_out(inp), "f16", inp.name)


def test_fused_prefill_full_size_sampled():
    """The benchmark's 4 x 4096 whole-prompt prefill; sampled rows checked one
    by one (row t of sequence s is the decode of query t over keys 0..t)."""
    inp = wl.fused_prefill(4096)
    dev = H.to_device(inp)
    k = wl.dense_view(dev["k_pool"], inp.num_seqs)
    v = wl.dense_view(dev["v_pool"], inp.num_seqs)
    out = torch.empty_like(dev["q"])
    desc = B.make_desc_contiguous(dev["q"], k, out=out, scale=inp.scale)
    plan = B.np_plan(desc, inp.context_lens, inp.q_start)
    print(f"[contiguous prefill] {inp.name}", flush=True)
    B.np_paged_attention_prefill(desc, plan, dev["q"], k, v, None, dev["context_lens"],
                                 dev["q_start"], out, B.workspace_for(plan, "cuda"))
    torch.cuda.synchronize()
    got = out.cpu()
    rng = np.random.default_rng(63)
    n = 4096
    for s in range(inp.num_seqs):
        for t in sorted({0, 1, 63, 64, n // 2, n - 1, *rng.integers(n, size=4).tolist()}):
            r = s * n + t
            b0 = int(inp.block_table[s, 0])
            nb_t = t // 16 + 1
            ref = oracle.paged_attention(inp.q[r:r + 1], inp.k_pool[b0:b0 + nb_t],
                                         inp.v_pool[b0:b0 + nb_t],
                                         torch.arange(nb_t, dtype=torch.int32)[None],
                                         torch.tensor([t + 1], dtype=torch.int32),
                                         scale=inp.scale)
            H.assert_close(got[r:r + 1], ref, "f16", f"seq {s} row {t}")
