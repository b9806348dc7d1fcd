"""Helpers shared by the GPU parity tests."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_cache_178_amd import binding
from paged_kv_cache_178_amd.workloads import PagedInputs

TOL = {"f32": (1e-5, 1e-5), "f16": (1e-2, 1e-2), "bf16": (1e-2, 1e-2)}


def to_device(inp: PagedInputs, device="cuda"):
    return dict(q=inp.q.to(device), k_pool=inp.k_pool.to(device), v_pool=inp.v_pool.to(device),
                block_table=inp.block_table.to(device), context_lens=inp.context_lens.to(device),
                q_start=inp.q_start.to(device))


def oracle_out(inp: PagedInputs, prefill=False):
    return oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                  inp.context_lens, q_start=inp.q_start if prefill else None,
                                  scale=inp.scale)


def gpu_decode(inp: PagedInputs, dev=None, opts=None, out=None):
    dev = dev or to_device(inp)
    o = binding.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                       dev["context_lens"], out=out, scale=inp.scale,
                       context_lens_host=inp.context_lens, opts=opts, check_tables=True)
    torch.cuda.synchronize()
    return o


def gpu_prefill(inp: PagedInputs, dev=None):
    dev = dev or to_device(inp)
    o = binding.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                        dev["context_lens"], dev["q_start"], scale=inp.scale,
                        context_lens_host=inp.context_lens, q_start_host=inp.q_start,
                        check_tables=True)
    torch.cuda.synchronize()
    return o


def assert_close(gpu, ref, dtype: str, what=""):
    """Element-wise |gpu - ref| <= atol + rtol |ref| (NaN fails), in float64."""
    atol, rtol = TOL[dtype]
    g = gpu.detach().to("cpu", torch.float64).numpy()
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
            f"(atol={atol}, rtol={rtol}); first at {tuple(idx)}: gpu={g[tuple(idx)]!r} "
            f"ref={ref[tuple(idx)]!r}; max abs err {np.nanmax(err):.3e}")
    return float(err.max())


def referenced_slots(inp: PagedInputs) -> np.ndarray:
    """[n_blocks, block_size] bool: slots some sequence's history reads."""
    used = np.zeros(inp.k_pool.shape[:2], dtype=bool)
    bt = inp.block_table.numpy()
    for s, length in enumerate(inp.context_lens.tolist()):
        for t in range(length):
            used[bt[s, t // inp.block_size], t % inp.block_size] = True
    return used


def poisoned(inp: PagedInputs) -> PagedInputs:
    """Copy with NaN in every pool slot no history references (tails
    included). Table entries past each history are already -1."""
    used = torch.from_numpy(referenced_slots(inp))
    k = inp.k_pool.clone()
    v = inp.v_pool.clone()
    k[~used] = float("nan")
    v[~used] = float("nan")
    return PagedInputs(**{**inp.__dict__, "k_pool": k, "v_pool": v})
