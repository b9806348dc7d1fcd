"""Seeded synthetic inputs for paged attention.

This module only draws random inputs; it computes no attention and shares no
arithmetic with either the HIP path or the oracle. Both sides receive the same
tensors from it.

The five workloads follow the shapes the pages use: the Llama-3.2-1B decode
shape of "Day 20: the number the Triton kernel has to beat" (section "What I
added today": shapes, not weights, set the read cost) and the awkward,
ragged and prefill shapes the kernel design of "Day 23: the real triton.jit
paged-attention kernel" (section "What I learned", item 1) says are the ones
worth testing.

Recipe (fixed here, stated once):

* ``numpy.random.Generator(PCG64(seed))``; draw order: context lengths, block
  tables, q, K pool, V pool, K spikes.
* q, K, V ~ N(0, 1) drawn in float32 over every pool slot, then rounded to the
  workload dtype (round to nearest even).
* Pool size: twice the blocks the histories need unless the workload fixes it.
  Each table holds the next ``ceil(L/B)`` entries of one random permutation of
  the pool, sequences in order; unused table entries are -1.
* K spikes (awkward workload): per sequence ``max(1, round(0.01 L))`` token
  positions drawn without replacement, K at those positions multiplied by 4 in
  float32 before rounding.
* Contiguous caches (``identity=True``): no permutation is drawn; sequence s
  owns blocks ``s * max_blocks .. (s + 1) * max_blocks - 1`` in order, so the
  pool is a dense ``[num_seqs, max_blocks * B, Hkv, d]`` tensor and the table
  is the identity (the split-KV decode and fused prefill shapes of "I Wrote
  the Three Attention Kernels That Run LLM Inference", section "Benchmark
  method": B = 4, H = 16, D = 64, fp16).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class PagedInputs:
    name: str
    seed: int
    dtype: str                      # "f32" | "f16" | "bf16"
    q: torch.Tensor                 # [n_q_total, Hq, d]
    k_pool: torch.Tensor            # [n_blocks, B, Hkv, d]
    v_pool: torch.Tensor
    block_table: torch.Tensor       # int32 [num_seqs, max_blocks], -1 unused
    context_lens: torch.Tensor      # int32 [num_seqs]
    q_start: torch.Tensor           # int32 [num_seqs + 1]
    scale: float

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pool.shape[2])

    @property
    def block_size(self) -> int:
        return int(self.k_pool.shape[1])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes: valid tokens only, every KV head."""
        elt = self.k_pool.element_size()
        return 2 * self.num_kv_heads * self.head_dim * elt * int(self.context_lens.sum())


def make_paged(name: str, seed, lens, n_q, hq: int, hkv: int, d: int, block_size: int,
               dtype: str, n_blocks: int | None = None, max_blocks: int | None = None,
               spike_frac: float = 0.0, scale: float | None = None,
               lens_rng=None, identity: bool = False) -> PagedInputs:
    """Draw one workload. ``lens`` is a list of context lengths, or a callable
    ``rng -> lens`` drawn first from the workload's generator; ``n_q`` is the
    number of query rows per sequence (an int or a list)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if callable(lens):
        lens = lens(rng)
    lens = [int(x) for x in lens]
    num_seqs = len(lens)
    n_q = [int(n_q)] * num_seqs if np.isscalar(n_q) else [int(x) for x in n_q]
    need = [-(-length // block_size) for length in lens]
    if max_blocks is None:
        max_blocks = max(need)
    if identity:
        n_blocks = num_seqs * max_blocks
        table = np.arange(n_blocks, dtype=np.int32).reshape(num_seqs, max_blocks)
    else:
        if n_blocks is None:
            n_blocks = 2 * sum(need)
        perm = rng.permutation(n_blocks)
        table = np.full((num_seqs, max_blocks), -1, dtype=np.int32)
        cursor = 0
        for s in range(num_seqs):
            table[s, : need[s]] = perm[cursor: cursor + need[s]]
            cursor += need[s]
    assert sum(need) <= n_blocks and max(need) <= max_blocks
    n_q_total = sum(n_q)
    q = rng.standard_normal((n_q_total, hq, d), dtype=np.float32)
    k = rng.standard_normal((n_blocks, block_size, hkv, d), dtype=np.float32)
    v = rng.standard_normal((n_blocks, block_size, hkv, d), dtype=np.float32)
    if spike_frac > 0.0:
        for s in range(num_seqs):
            count = max(1, int(round(spike_frac * lens[s])))
            for t in rng.choice(lens[s], size=count, replace=False):
                k[table[s, t // block_size], t % block_size, :, :] *= 4.0
    tdt = DTYPES[dtype]
    q_start = np.zeros(num_seqs + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(n_q)
    return PagedInputs(
        name=name, seed=int(seed) if np.isscalar(seed) else -1, dtype=dtype,
        q=torch.from_numpy(q).to(tdt), k_pool=torch.from_numpy(k).to(tdt),
        v_pool=torch.from_numpy(v).to(tdt),
        block_table=torch.from_numpy(table),
        context_lens=torch.tensor(lens, dtype=torch.int32),
        q_start=torch.from_numpy(q_start),
        scale=(1.0 / math.sqrt(d)) if scale is None else float(scale))


# The five workloads. Seeds are the workload numbers 1..5.

LLAMA_HISTORIES = (16, 64, 256, 1024, 4096)


def tiny_fp32() -> PagedInputs:
    """1 sequence, Hq=4, Hkv=2, d=64, B=16, 64 tokens in 4 blocks of a
    16-block pool, fp32, scale 1/8, one query token."""
    return make_paged("tiny_fp32", 1, [64], 1, 4, 2, 64, 16, "f32", n_blocks=16,
                      scale=1.0 / 8.0)


def llama_decode(history: int, seed_base: int = 2) -> PagedInputs:
    """Llama-3.2-1B head shape (Hq=32, Hkv=8, d=64), B=16, one sequence, one
    query token, bf16. Child seeds are spawned in the sweep order 16..4096."""
    idx = LLAMA_HISTORIES.index(history) if history in LLAMA_HISTORIES else None
    if idx is None:
        seed = np.random.SeedSequence([seed_base, history])
    else:
        seed = np.random.SeedSequence(seed_base).spawn(len(LLAMA_HISTORIES))[idx]
    return make_paged(f"llama_decode_L{history}", seed, [history], 1, 32, 8, 64, 16, "bf16")


def awkward_fp16() -> PagedInputs:
    """Hq=12, Hkv=4 (group 3), d=48, B=16, histories 13/100/1037, fp16, K x4 on
    1% of tokens."""
    return make_paged("awkward_fp16", 3, [13, 100, 1037], 1, 12, 4, 48, 16, "f16",
                      spike_frac=0.01)


def continuous_batching(seed: int = 4, num_seqs: int = 64) -> PagedInputs:
    """64 sequences, lengths uniform on [128, 8192], Llama head shape, bf16,
    shared pool of 40000 blocks, table width 512."""
    return make_paged("continuous_batching", seed,
                      lambda rng: rng.integers(128, 8192, size=num_seqs, endpoint=True),
                      1, 32, 8, 64, 16, "bf16", n_blocks=40000, max_blocks=512)


def chunked_prefill(seed: int = 5, num_seqs: int = 4, cached: int = 2048,
                    chunk: int = 512) -> PagedInputs:
    """num_seqs sequences of ``cached`` cached tokens plus a ``chunk``-token
    chunk of new queries (causal over past + chunk), Llama head shape, bf16."""
    return make_paged("chunked_prefill", seed, [cached + chunk] * num_seqs, chunk,
                      32, 8, 64, 16, "bf16")


SPLITKV_CONTEXTS = (1024, 2048, 4096, 8192, 16384)
SPLITKV_SPLITS = (1, 8, 16, 32, 64, 128)


def splitkv_decode(n_ctx: int, seed: int = 6) -> PagedInputs:
    """Contiguous-cache decode sweep shape: 4 sequences of n_ctx tokens, Hq =
    Hkv = 16, d = 64, fp16, one query row each."""
    return make_paged(f"splitkv_N{n_ctx}", seed, [n_ctx] * 4, 1, 16, 16, 64, 16, "f16",
                      identity=True)


def fused_prefill(n_ctx: int, seed: int = 7, num_seqs: int = 4) -> PagedInputs:
    """Contiguous-cache prefill of a whole prompt: num_seqs sequences of n_ctx
    tokens, all of them queries (past = 0), Hq = Hkv = 16, d = 64, fp16."""
    return make_paged(f"fused_prefill_N{n_ctx}", seed, [n_ctx] * num_seqs, n_ctx, 16, 16, 64,
                      16, "f16", identity=True)


def dense_view(pool: torch.Tensor, num_seqs: int) -> torch.Tensor:
    """The dense [num_seqs, capacity, Hkv, d] view of an identity-table pool."""
    nb, bs, hkv, d = pool.shape
    return pool.view(num_seqs, (nb // num_seqs) * bs, hkv, d)


def custom(seed: int, lens, n_q=1, hq=8, hkv=2, d=64, block_size=16, dtype="bf16",
           n_blocks=None, max_blocks=None, spike_frac=0.0, scale=None,
           identity=False) -> PagedInputs:
    """Any other shape, same recipe (used by edge-case tests)."""
    return make_paged(f"custom_s{seed}", seed, lens, n_q, hq, hkv, d, block_size, dtype,
                      n_blocks=n_blocks, max_blocks=max_blocks, spike_frac=spike_frac,
                      scale=scale, identity=identity)
