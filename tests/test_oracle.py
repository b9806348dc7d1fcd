"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:

* hand-derived fixtures under ``tests/golden/`` (exact values, cited);
* a pure-Python brute force of the definition on tiny inputs, written with
  explicit integer division for the page/slot lookup and exp(s)/sum(exp(s))
  without a max shift, summed with ``math.fsum``;
* a library special case: torch float64 ``scaled_dot_product_attention`` on a
  contiguous history that the test scatters into pages itself;
* closed forms (one key returns its V row; equal scores return the mean of V;
  a dominant key returns its V row);
* invariants (permuting physical blocks changes nothing bit for bit; the
  split/LSE combine equals the unsplit result; the block-by-block online
  softmax equals the gather form; NaN in memory the table does not reference
  never reaches the output);
* planted mistakes: each plausible bug inserted into the oracle makes at least
  one of the pins above fail.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import paged as opa
from tests.golden.load import load


# ----------------------------------------------------------------- helpers


def random_case(seed, num_seqs=None, block_size=None, hkv=None, group=None, d=None,
                prefill=False, max_len=9):
    rng = np.random.default_rng(seed)
    num_seqs = num_seqs or int(rng.integers(1, 4))
    block_size = block_size or int(rng.choice([1, 2, 4]))
    hkv = hkv or int(rng.integers(1, 3))
    group = group or int(rng.integers(1, 4))
    d = d or int(rng.integers(1, 9))
    hq = hkv * group
    lens = [int(rng.integers(1, max_len + 1)) for _ in range(num_seqs)]
    if prefill:
        n_q = [int(rng.integers(1, length + 1)) for length in lens]
    else:
        n_q = [1] * num_seqs
    need = [-(-length // block_size) for length in lens]
    n_blocks = sum(need) + int(rng.integers(0, 4))
    perm = rng.permutation(n_blocks)
    max_blocks = max(need) + int(rng.integers(0, 2))
    table = np.full((num_seqs, max_blocks), -1, dtype=np.int64)
    c = 0
    for s in range(num_seqs):
        table[s, : need[s]] = perm[c: c + need[s]]
        c += need[s]
    q_start = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int64)
    q = rng.standard_normal((int(q_start[-1]), hq, d))
    kp = rng.standard_normal((n_blocks, block_size, hkv, d))
    vp = rng.standard_normal((n_blocks, block_size, hkv, d))
    scale = float(rng.uniform(0.2, 1.5)) if rng.integers(0, 2) else None
    return dict(q=q, k_pool=kp, v_pool=vp, block_table=table,
                context_lens=np.array(lens, dtype=np.int64), q_start=q_start, scale=scale)


def brute_force(case):
    """Pure-Python definition: out = sum_t exp(s_t) v_t / sum_u exp(s_u)."""
    q, kp, vp = case["q"], case["k_pool"], case["v_pool"]
    table, lens, q_start = case["block_table"], case["context_lens"], case["q_start"]
    n_rows, hq, d = q.shape
    block_size, hkv = kp.shape[1], kp.shape[2]
    scale = case["scale"] if case["scale"] is not None else 1.0 / math.sqrt(d)
    out = np.zeros_like(q)
    for s in range(len(lens)):
        length = int(lens[s])
        rows = range(int(q_start[s]), int(q_start[s + 1]))
        n_q = len(rows)
        for i, r in enumerate(rows):
            position = length - n_q + i
            for h in range(hq):
                kvh = h * hkv // hq
                weights, values = [], []
                for t in range(position + 1):
                    blk = int(table[s][t // block_size])
                    slot = t % block_size
                    dot = math.fsum(float(q[r, h, c]) * float(kp[blk, slot, kvh, c])
                                    for c in range(d))
                    weights.append(math.exp(scale * dot))
                    values.append([float(vp[blk, slot, kvh, c]) for c in range(d)])
                total = math.fsum(weights)
                for c in range(d):
                    out[r, h, c] = math.fsum(w * v[c] for w, v in zip(weights, values)) / total
    return out


def run(case, fn=None):
    fn = fn or oracle.paged_attention
    return fn(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
              case["context_lens"], q_start=case["q_start"], scale=case["scale"])


# ---------------------------------------------------------- hand fixtures


def golden_case(mode):
    g = load("hand_paged_gqa.json")
    sub = g[mode]
    n_rows = sub["q"].shape[0]
    q_start = sub["q_start"].astype(np.int64) if "q_start" in sub else np.arange(n_rows + 1)
    return dict(q=sub["q"], k_pool=g["k_pool"], v_pool=g["v_pool"],
                block_table=g["block_table"].astype(np.int64),
                context_lens=g["context_lens"].astype(np.int64), q_start=q_start,
                scale=g["scale"]), sub["out"]


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_golden_hand_derived(mode):
    case, expect = golden_case(mode)
    np.testing.assert_allclose(run(case), expect, rtol=0, atol=1e-12)
    np.testing.assert_allclose(run(case, oracle.paged_attention_blockwise), expect,
                               rtol=0, atol=1e-12)


def test_golden_split_combine():
    g = load("hand_split_combine.json")
    bounds = [tuple(int(x) for x in b) for b in g["bounds"]]
    parts = oracle.split_partials(g["q"], g["keys"], g["vals"], g["scale"], bounds)
    for (lse, out_s), lse_x, out_x in zip(parts, g["lse"], g["outs"]):
        assert abs(lse - lse_x) < 1e-12
        np.testing.assert_allclose(out_s, out_x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.combine_splits_lse(parts), g["out"], rtol=0, atol=1e-12)


# ------------------------------------------------------------- brute force


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("prefill", [False, True])
def test_brute_force_tiny(seed, prefill):
    case = random_case(1000 * int(prefill) + seed, prefill=prefill)
    np.testing.assert_allclose(run(case), brute_force(case), rtol=1e-12, atol=1e-13)


# ------------------------------------------------ library special case (SDPA)


@pytest.mark.parametrize("seed,group,prefill", [(0, 1, False), (1, 2, False), (2, 3, False),
                                                (3, 4, True), (4, 2, True)])
def test_torch_sdpa_special_case(seed, group, prefill):
    """Contiguous history -> scattered by the test -> oracle == torch SDPA."""
    rng = np.random.default_rng(seed + 77)
    hkv, d, block_size, length = 2, 16, 4, 37
    hq = hkv * group
    n_q = 9 if prefill else 1
    k_hist = rng.standard_normal((length, hkv, d))
    v_hist = rng.standard_normal((length, hkv, d))
    q = rng.standard_normal((n_q, hq, d))
    nb = -(-length // block_size)
    n_blocks = 3 * nb
    table = rng.permutation(n_blocks)[:nb]
    kp = rng.standard_normal((n_blocks, block_size, hkv, d))   # garbage elsewhere
    vp = rng.standard_normal((n_blocks, block_size, hkv, d))
    for t in range(length):
        kp[table[t // block_size], t % block_size] = k_hist[t]
        vp[table[t // block_size], t % block_size] = v_hist[t]
    got = oracle.paged_attention(q, kp, vp, table[None, :], np.array([length]),
                                 q_start=np.array([0, n_q]))
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, n_q, d]
    kt = torch.from_numpy(k_hist).permute(1, 0, 2).repeat_interleave(group, 0)
    vt = torch.from_numpy(v_hist).permute(1, 0, 2).repeat_interleave(group, 0)
    mask = torch.ones(n_q, length, dtype=torch.bool).tril(diagonal=length - n_q)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- closed forms


def test_single_key_returns_its_value_exactly():
    case = random_case(5, num_seqs=1, block_size=4)
    case["context_lens"] = np.array([1])
    case["q_start"] = np.array([0, 1])
    case["q"] = case["q"][:1]
    blk = case["block_table"][0, 0]
    out = run(case)
    hq, hkv = out.shape[1], case["k_pool"].shape[2]
    for h in range(hq):
        np.testing.assert_array_equal(out[0, h], case["v_pool"][blk, 0, h * hkv // hq])


@pytest.mark.parametrize("prefill", [False, True])
def test_equal_scores_give_mean_of_visible_values(prefill):
    case = random_case(6, num_seqs=3, block_size=4, hkv=2, group=3, d=5,
                       prefill=prefill, max_len=30)
    case["q"] = np.zeros_like(case["q"])
    out = run(case)
    kp_block = case["block_table"]
    for s, length in enumerate(case["context_lens"]):
        hist = np.stack([case["v_pool"][kp_block[s, t // 4], t % 4] for t in range(length)])
        r0, r1 = case["q_start"][s], case["q_start"][s + 1]
        for i, r in enumerate(range(r0, r1)):
            visible = length - (r1 - r0) + i + 1
            mean = hist[:visible].mean(axis=0)                    # [Hkv, d]
            for h in range(out.shape[1]):
                np.testing.assert_allclose(out[r, h], mean[h // 3], rtol=0, atol=1e-14)


def test_dominant_key_returns_its_value_everywhere():
    """For every position t*, a key aligned with q and 60 units of scaled score
    above the rest pulls the output onto V[t*]: every logical position is
    reachable and the mapping t -> (block, slot) is the one stated."""
    rng = np.random.default_rng(8)
    hkv, group, d, block_size, length = 1, 2, 4, 4, 11
    hq = hkv * group
    nb = -(-length // block_size)
    table = rng.permutation(2 * nb)[:nb]
    q = np.zeros((1, hq, d))
    q[0, :, 0] = 1.0
    for t_star in range(length):
        kp = 0.01 * rng.standard_normal((2 * nb, block_size, hkv, d))
        vp = rng.standard_normal((2 * nb, block_size, hkv, d))
        kp[table[t_star // block_size], t_star % block_size, 0, 0] = 120.0
        out = oracle.paged_attention(q, kp, vp, table[None], np.array([length]))
        want = vp[table[t_star // block_size], t_star % block_size, 0]
        for h in range(hq):
            np.testing.assert_allclose(out[0, h], want, rtol=0, atol=1e-12)


# --------------------------------------------------------------- invariants


@pytest.mark.parametrize("seed", range(4))
def test_block_permutation_is_bit_exact(seed):
    case = random_case(200 + seed, prefill=bool(seed % 2), max_len=20)
    base = run(case)
    rng = np.random.default_rng(seed)
    n_blocks = case["k_pool"].shape[0]
    perm = rng.permutation(n_blocks)          # new position of old block b: perm[b]
    kp = np.empty_like(case["k_pool"])
    vp = np.empty_like(case["v_pool"])
    kp[perm] = case["k_pool"]
    vp[perm] = case["v_pool"]
    table = np.where(case["block_table"] >= 0, perm[case["block_table"]], -1)
    moved = dict(case, k_pool=kp, v_pool=vp, block_table=table)
    np.testing.assert_array_equal(run(moved), base)


def test_identity_table_equals_contiguous_attention():
    rng = np.random.default_rng(3)
    hkv, group, d, block_size, length = 2, 2, 8, 4, 14
    nb = -(-length // block_size)
    kp = rng.standard_normal((nb, block_size, hkv, d))
    vp = rng.standard_normal((nb, block_size, hkv, d))
    q = rng.standard_normal((1, hkv * group, d))
    out = oracle.paged_attention(q, kp, vp, np.arange(nb)[None], np.array([length]))
    k_hist = kp.reshape(-1, hkv, d)[:length]
    v_hist = vp.reshape(-1, hkv, d)[:length]
    allowed = np.ones((1, length), dtype=bool)
    for h in range(hkv * group):
        ref = oracle.attention_rows(q[:, h], k_hist[:, h // group], v_hist[:, h // group],
                                    1.0 / math.sqrt(d), allowed)
        np.testing.assert_array_equal(out[:, h], ref)


@pytest.mark.parametrize("seed", range(6))
def test_split_combine_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    length, d = int(rng.integers(2, 200)), 16
    keys = rng.standard_normal((length, d)) * 2
    vals = rng.standard_normal((length, d))
    qr = rng.standard_normal(d)
    cuts = sorted(set(rng.integers(1, length, size=int(rng.integers(1, 6))).tolist()))
    bounds = list(zip([0] + cuts, cuts + [length]))
    combined = oracle.combine_splits_lse(oracle.split_partials(qr, keys, vals, 0.25, bounds))
    whole = oracle.attention_rows(qr[None], keys, vals, 0.25, np.ones((1, length), bool))[0]
    np.testing.assert_allclose(combined, whole, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(8))
def test_blockwise_equals_gather(seed):
    case = random_case(300 + seed, prefill=bool(seed % 2), max_len=40)
    np.testing.assert_allclose(run(case, oracle.paged_attention_blockwise), run(case),
                               rtol=1e-12, atol=1e-12)


def test_unreferenced_nan_never_reaches_output():
    case = random_case(9, num_seqs=3, block_size=4, prefill=True, max_len=30)
    base = run(case)
    kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
    used = np.zeros(kp.shape[:2], dtype=bool)
    for s, length in enumerate(case["context_lens"]):
        for t in range(length):
            used[case["block_table"][s, t // 4], t % 4] = True
    kp[~used] = np.nan
    vp[~used] = np.nan
    got = run(dict(case, k_pool=kp, v_pool=vp))
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got, base)


# ---------------------------------------------------------- planted mistakes


def _pins_pass():
    """True when every pin used below passes for the current oracle."""
    try:
        for mode in ("decode", "prefill"):
            case, expect = golden_case(mode)
            if not np.allclose(run(case), expect, rtol=0, atol=1e-9):
                return False
        for seed in (0, 1, 2, 1001, 1002, 1003):
            case = random_case(seed, prefill=seed > 1000, hkv=2, group=2)
            if not np.allclose(run(case), brute_force(case), rtol=1e-9, atol=1e-9):
                return False
    except Exception:
        return False
    return True


def _bad_gather_ignores_table(pool, table_row, length):
    n = -(-length // pool.shape[1])
    return pool[:n].reshape(-1, *pool.shape[2:])[:length]


def _bad_gather_off_by_one(pool, table_row, length):
    n = -(-length // pool.shape[1])
    rows = pool[table_row[:n]].reshape(-1, *pool.shape[2:])
    return np.roll(rows, 1, axis=0)[:length]


def _bad_gather_transposed(pool, table_row, length):
    n = -(-length // pool.shape[1])
    blocks = pool[table_row[:n]]
    return np.ascontiguousarray(blocks.transpose(0, 2, 1, 3)).reshape(
        n * pool.shape[1], *pool.shape[2:])[:length]


def _bad_attention_no_scale(q, k, v, scale, allowed):
    return _good_attention(q, k, v, 1.0, allowed)


def _bad_attention_sign(q, k, v, scale, allowed):
    return _good_attention(q, k, v, -scale, allowed)


def _bad_attention_wrong_axis(q, k, v, scale, allowed):
    s = np.where(allowed, scale * (q @ k.T), -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=0, keepdims=True)
    return p @ v


def _bad_attention_transposed_v(q, k, v, scale, allowed):
    w = _good_attention(q, k, np.eye(k.shape[0]), scale, allowed)
    return w @ v[::-1]


_good_attention = opa.attention_rows

MUTANTS = {
    "gqa_modulo": ("kv_head_for", lambda h, hq, hkv: h % hkv),
    "causal_strict": ("visible_keys", lambda length, n_q:
                      np.arange(length)[None, :] < (length - n_q) + np.arange(n_q)[:, None]),
    "causal_no_past": ("visible_keys", lambda length, n_q:
                       np.arange(length)[None, :] <= np.arange(n_q)[:, None]),
    "gather_ignores_table": ("gather_history", _bad_gather_ignores_table),
    "gather_off_by_one": ("gather_history", _bad_gather_off_by_one),
    "gather_transposed": ("gather_history", _bad_gather_transposed),
    "no_scale": ("attention_rows", _bad_attention_no_scale),
    "sign_flip": ("attention_rows", _bad_attention_sign),
    "softmax_wrong_axis": ("attention_rows", _bad_attention_wrong_axis),
    "values_reversed": ("attention_rows", _bad_attention_transposed_v),
}


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(opa, attr, bad)
    assert not _pins_pass(), f"planted mistake {name} slipped past every pin"
