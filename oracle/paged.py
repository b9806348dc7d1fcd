"""Plain float64 oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE. This module is the correctness reference that the HIP
path is compared against. It is slow on purpose: every step is written out
the way the pages state it, with numpy float64 and no blocking, fusion or
reordering beyond what the definition itself says. Only ``tests/``, the smoke
check and the benchmark's CPU-baseline leg may use it. It shares no code with
the HIP library or its binding.

Sources (pages by title, then section):

* "I Wrote the Three Attention Kernels That Run LLM Inference -- in Portable
  Triton, on a Free Colab T4", section "What is attention, really?": the
  definition softmax(Q K^T / sqrt(d)) V.
* Same page, section "3. Paged KV-cache attention": a key at logical position
  p lives in physical page ``block_table[b, p // PAGE_SIZE]`` at offset
  ``p % PAGE_SIZE`` inside that page; the read is GQA-aware.
* Same page, section "2. Split-KV flash-decoding": each split reduces its own
  slice of K/V; the splits are merged with weights ``exp(lse - max lse)``
  and the weighted outputs are divided by the sum of the weights.
* "Day 20: the number the Triton kernel has to beat", section "What I added
  today": two CPU reads of the same cache, a gather that rebuilds the
  contiguous history and then runs ordinary masked attention, and a fused read
  that attends block by block over the scattered blocks; the two must agree.
* "What a Kernel Is, and Why Everyone Is Writing New Ones", section
  "Technical Details": online softmax keeps a running max and sum and is exact.
* "Day 23: the real triton.jit paged-attention kernel", section "What I added
  today": ``past`` is a host-side integer; query position i of a chunk sees
  keys up to ``past + i``.
* "Day 20: the number the Triton kernel has to beat", section
  "What I learned": the cache write grows the table and scatters the new
  tokens' K/V into their slots; the read then attends over them.

Readings taken where the pages are silent (each is listed in the design notes):

* GQA grouping is contiguous: query head h reads KV head ``h // (Hq // Hkv)``.
* ``context_lens[s]`` counts every cached token of sequence s including the
  current query tokens, so ``past = context_lens[s] - n_q``.
* The default scale is ``1 / sqrt(head_dim)`` over the real head_dim.

Every function here is pinned by the CPU test suite against brute force,
closed forms, a library special case and hand-derived fixtures; none is
"parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.int64)


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   allowed: np.ndarray) -> np.ndarray:
    """softmax(scale * q k^T) v for one head, masked.

    q [n, d], k [T, d], v [T, d], allowed [n, T] boolean (every row must allow
    at least one key). Returns [n, d] float64.

    Definition from "I Wrote the Three Attention Kernels ...", section "What is
    attention, really?". Masked scores are -inf, so their weight is exactly 0.
    """
    s = scale * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def gather_history(pool: np.ndarray, table_row: np.ndarray, length: int) -> np.ndarray:
    """Rebuild one sequence's contiguous history from its block table.

    pool [n_blocks, block_size, Hkv, d]; table_row [max_blocks] physical block
    ids. Logical token t is slot ``t % block_size`` of physical block
    ``table_row[t // block_size]`` ("I Wrote the Three Attention Kernels ...",
    section "3. Paged KV-cache attention"). Returns [length, Hkv, d].

    This is the gather read of "Day 20: the number the Triton kernel has to
    beat", section "What I added today".
    """
    block_size = pool.shape[1]
    n_used = -(-length // block_size)
    blocks = pool[table_row[:n_used]]                       # [n_used, B, Hkv, d]
    flat = blocks.reshape(n_used * block_size, *pool.shape[2:])
    return flat[:length]


def _default_q_start(num_seqs: int) -> np.ndarray:
    return np.arange(num_seqs + 1, dtype=np.int64)


def kv_head_for(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head h: contiguous groups of Hq // Hkv heads."""
    return h // (hq // hkv)


def visible_keys(length: int, n_q: int) -> np.ndarray:
    """[n_q, length] mask: query row i sits at position past + i and sees the
    keys t <= past + i, past = length - n_q ("Day 23 ...", section "What I
    added today": past is a host-side integer)."""
    past = length - n_q
    return np.arange(length)[None, :] <= past + np.arange(n_q)[:, None]


def paged_attention(q, k_pool, v_pool, block_table, context_lens, q_start=None,
                    scale: float | None = None) -> np.ndarray:
    """Attention over a paged cache, by gather then dense masked softmax.

    q           [n_q_total, Hq, d]; rows of sequence s are
                ``q_start[s]:q_start[s+1]`` (decode: one row per sequence,
                ``q_start = 0..num_seqs``).
    k_pool      [n_blocks, block_size, Hkv, d]; v_pool the same.
    block_table [num_seqs, max_blocks] int.
    context_lens[num_seqs] int: cached tokens of each sequence, the current
                query tokens included.
    Returns out [n_q_total, Hq, d] float64.

    Query row i of sequence s, head h attends to the keys t with
    ``0 <= t <= past_s + i``, ``past_s = context_lens[s] - n_q_s``, of KV head
    ``h // (Hq // Hkv)``.
    """
    q = _f64(q)
    k_pool = _f64(k_pool)
    v_pool = _f64(v_pool)
    block_table = _i64(block_table)
    context_lens = _i64(context_lens)
    num_seqs = context_lens.shape[0]
    q_start = _default_q_start(num_seqs) if q_start is None else _i64(q_start)
    n_q_total, hq, d = q.shape
    hkv = k_pool.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((n_q_total, hq, d), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        keys = gather_history(k_pool, block_table[s], length)     # [L, Hkv, d]
        vals = gather_history(v_pool, block_table[s], length)
        allowed = visible_keys(length, r1 - r0)                   # [n_q, L]
        for h in range(hq):
            kvh = kv_head_for(h, hq, hkv)
            out[r0:r1, h, :] = attention_rows(q[r0:r1, h, :], keys[:, kvh, :],
                                              vals[:, kvh, :], scale, allowed)
    return out


def paged_attention_blockwise(q, k_pool, v_pool, block_table, context_lens,
                              q_start=None, scale: float | None = None) -> np.ndarray:
    """Second formulation: online softmax block by block over the table.

    Walks each sequence's physical blocks in table order and keeps, per query
    row and head, a running max m, a running sum l and an unnormalised
    accumulator acc. For each block it takes the new max, rescales the old sum
    and accumulator by exp(m_old - m_new), adds the block's exp(s - m_new)
    weights and their weighted V rows, and divides by l at the end ("What a
    Kernel Is ...", section "Technical Details"; "Day 20 ...", section "What I
    added today", the fused read). Used only to cross-check
    :func:`paged_attention`.
    """
    q = _f64(q)
    k_pool = _f64(k_pool)
    v_pool = _f64(v_pool)
    block_table = _i64(block_table)
    context_lens = _i64(context_lens)
    num_seqs = context_lens.shape[0]
    q_start = _default_q_start(num_seqs) if q_start is None else _i64(q_start)
    n_q_total, hq, d = q.shape
    block_size, hkv = k_pool.shape[1], k_pool.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((n_q_total, hq, d), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        n_q = r1 - r0
        past = length - n_q
        last_pos = past + np.arange(n_q)                 # last visible key per row
        n_blocks_used = -(-length // block_size)
        for h in range(hq):
            kvh = kv_head_for(h, hq, hkv)
            qh = q[r0:r1, h, :]
            m = np.full(n_q, -np.inf)
            l = np.zeros(n_q)
            acc = np.zeros((n_q, d))
            for j in range(n_blocks_used):
                phys = int(block_table[s, j])
                t0 = j * block_size
                t1 = min(t0 + block_size, length)
                kb = k_pool[phys, : t1 - t0, kvh, :]
                vb = v_pool[phys, : t1 - t0, kvh, :]
                sc = scale * (qh @ kb.T)                      # [n_q, t1-t0]
                vis = np.arange(t0, t1)[None, :] <= last_pos[:, None]
                sc = np.where(vis, sc, -np.inf)
                m_new = np.maximum(m, sc.max(axis=1))
                live = np.isfinite(m_new)
                alpha = np.where(live, np.exp(np.where(live, m - m_new, 0.0)), 1.0)
                p = np.where(vis, np.exp(sc - np.where(live, m_new, 0.0)[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ vb
                m = m_new
            out[r0:r1, h, :] = acc / l[:, None]
    return out


def split_partials(q_row: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                   scale: float, bounds) -> list[tuple[float, np.ndarray]]:
    """Per-split (lse, normalised output) for one query row and one head.

    keys/vals [L, d] (already gathered); bounds a list of (t0, t1) ranges that
    partition 0..L. Each split reduces its own slice ("I Wrote the Three
    Attention Kernels ...", section "2. Split-KV flash-decoding"): it returns
    ``lse = log sum exp(s_t)`` over its keys and ``out = softmax(s) v`` over
    its keys.
    """
    q_row = _f64(q_row)
    keys = _f64(keys)
    vals = _f64(vals)
    parts = []
    for t0, t1 in bounds:
        sc = scale * (keys[t0:t1] @ q_row)
        m = sc.max()
        w = np.exp(sc - m)
        lse = m + math.log(w.sum())
        parts.append((lse, (w / w.sum()) @ vals[t0:t1]))
    return parts


def combine_splits_lse(parts: list[tuple[float, np.ndarray]]) -> np.ndarray:
    """Merge split results by their log-sum-exp.

    ``w_j = exp(lse_j - max_k lse_k)``; ``out = sum_j w_j out_j / sum_j w_j``
    ("I Wrote the Three Attention Kernels ...", section "2. Split-KV
    flash-decoding", the cross-SM combine).
    """
    lse = np.array([p[0] for p in parts], dtype=np.float64)
    outs = np.stack([p[1] for p in parts]).astype(np.float64)
    w = np.exp(lse - lse.max())
    return (outs * w[:, None]).sum(axis=0) / w.sum()


def _raw_bits(x) -> np.ndarray:
    """The stored elements of a pool or of new rows as raw integers of the
    same width (torch CPU tensor or numpy array), so that a copy can be
    compared bit for bit whatever the element type."""
    if hasattr(x, "detach"):
        import torch

        t = x.detach().to("cpu").contiguous()
        width = {2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]
        return t.view(width).numpy().copy()
    a = np.ascontiguousarray(x)
    return a.view({2: np.int16, 4: np.int32, 8: np.int64}[a.itemsize]).copy()


def append_kv(k_pool, v_pool, block_table, context_lens, new_start, k_new, v_new):
    """Write new tokens' K/V rows into the pools.

    Sequence s gets rows ``new_start[s] .. new_start[s+1] - 1`` of k_new and
    v_new ([rows, Hkv, d]); they are its last tokens, at positions
    ``past_s + i`` with ``past_s = context_lens[s] - n_s`` (the lengths already
    count them: append, then attend). Token t goes to slot ``t % B`` of
    physical block ``block_table[s, t // B]`` ("3. Paged KV-cache attention"
    gives the addressing; "Day 20 ...", "What I learned", gives the write: the
    table is extended first, then the new K/V are stored in their slots).
    Every other slot keeps its contents.

    Returns (k, v): copies of the pools as raw-bit integer arrays with the
    pools' shapes, so a GPU result can be compared bit for bit.
    """
    k = _raw_bits(k_pool)
    v = _raw_bits(v_pool)
    kn = _raw_bits(k_new)
    vn = _raw_bits(v_new)
    table = _i64(block_table)
    lens = _i64(context_lens)
    starts = _i64(new_start)
    block_size = k.shape[1]
    for s in range(len(lens)):
        n = int(starts[s + 1] - starts[s])
        past = int(lens[s]) - n
        for i in range(n):
            t = past + i
            blk = int(table[s, t // block_size])
            k[blk, t % block_size] = kn[starts[s] + i]
            v[blk, t % block_size] = vn[starts[s] + i]
    return k, v
