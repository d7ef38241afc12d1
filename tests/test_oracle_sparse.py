"""Pins of the block-sparse top-k oracle (alice-llm 2.0.0,
sparse_attention/llama3_bridge.rs, `llama3_sparse_attention`: proxy block-max
scores from the first query head of each KV head, top-k blocks per (query,
KV head), attention over the kept blocks merged by log-sum-exp) against
things other than itself: the dense oracle (the page's dense-fallback parity
for topk = 0 and topk >= the number of blocks), exact rational arithmetic for
the proxy scores and the top-k choice, the pure-Python dense brute force over
the kept keys, and the page's log-sum-exp combination of per-block parts."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import random_batch

CASES = [
    dict(dtype="bf16", hq=8, hkv=2, d=64, page_size=16, q_counts=(1, 6, 1), max_len=700),
    dict(dtype="bf16", hq=4, hkv=1, d=32, page_size=4, q_counts=(3, 1), max_len=300, causal=False),
    dict(dtype="f16", hq=6, hkv=3, d=64, page_size=8, q_counts=(1, 1, 2), max_len=500, window=150),
    dict(dtype="f32", hq=4, hkv=2, d=16, page_size=16, q_counts=(2, 1), max_len=400),
]


def _values(b, arr):
    return oracle.widen(arr, b.dtype)


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("block", [16, 64])
def test_dense_fallback_equals_dense_oracle_bitwise(i, block):
    """topk = 0, and topk at least the number of candidate blocks, keep every
    block: the page's dense-fallback parity, here bit for bit."""
    b = random_batch(8000 + i, **CASES[i])
    ref_o, ref_l = oracle.attention(b)
    nmax = -(-int(b.seq_lens.max()) // block)
    for topk in (0, nmax, nmax + 5):
        sel = oracle.sparse_select(b, block, topk)
        o, l = oracle.sparse_attention(b, sel, block)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l), topk


def _exact_block_scores(b, block):
    """Exact rational proxy scores (max over visible keys of q_first . k) and
    their f32 error bound per (query, KV head, block)."""
    q, k = _values(b, b.q), _values(b, b.k)
    G = b.hq // b.hkv
    out = {}
    for s in range(b.num_seqs):
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            lo, hi = oracle.visible_range(b, i, s)
            for h in range(b.hkv):
                qv = [Fraction(float(x)) for x in q[i, h * G]]
                for t in range(lo, hi + 1):
                    kv = k[b.block_table[s, t // b.page_size], t % b.page_size, h]
                    prods = [a * Fraction(float(c)) for a, c in zip(qv, kv)]
                    exact = sum(prods)
                    bound = b.d * 2.0 ** -23 * float(sum(abs(p) for p in prods)) + 1e-30
                    r = t // block
                    cur = out.get((i, h, r))
                    if cur is None or exact > cur[0]:
                        out[(i, h, r)] = (exact, bound)
    return out


@pytest.mark.parametrize("i", range(len(CASES)))
def test_proxy_scores_match_exact_arithmetic(i):
    """Each block score is within the f32 summation bound of the exact largest
    dot product of the group's first query head with a visible key of the
    block; blocks without a visible key score -inf."""
    b = random_batch(8100 + i, **CASES[i])
    block = 16
    sc = oracle.sparse_proxy_scores(b, block)
    exact = _exact_block_scores(b, block)
    for (qi, h, r) in np.ndindex(*sc.shape):
        e = exact.get((qi, h, r))
        if e is None:
            assert sc[qi, h, r] == -np.inf, (qi, h, r)
        else:
            assert abs(float(sc[qi, h, r]) - float(e[0])) <= e[1], (qi, h, r, sc[qi, h, r], float(e[0]))


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("topk", [1, 2, 3])
def test_topk_choice_matches_exact_ranking(i, topk):
    """The kept blocks are the topk best by exact score (ties to the lower
    index) wherever the exact gap at the cut exceeds the f32 error; the list
    is increasing, -1 padded, and never longer than the candidates."""
    b = random_batch(8200 + i, **CASES[i])
    block = 16
    sel = oracle.sparse_select(b, block, topk)
    exact = _exact_block_scores(b, block)
    checked = 0
    for s in range(b.num_seqs):
        for qi in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            lo, hi = oracle.visible_range(b, qi, s)
            cand = list(range(lo // block, hi // block + 1))
            for h in range(b.hkv):
                got = [x for x in sel[qi, h] if x >= 0]
                assert got == sorted(got) and len(got) == min(topk, len(cand))
                assert all(x < 0 for x in sel[qi, h, len(got):])
                if len(cand) <= topk:
                    assert got == cand
                    continue
                ranked = sorted(cand, key=lambda r: (-exact[(qi, h, r)][0], r))
                gap = exact[(qi, h, ranked[topk - 1])][0] - exact[(qi, h, ranked[topk])][0]
                err = exact[(qi, h, ranked[topk - 1])][1] + exact[(qi, h, ranked[topk])][1]
                if float(gap) > 2 * err:
                    assert got == sorted(ranked[:topk]), (qi, h)
                    checked += 1
    assert checked > 0


@pytest.mark.parametrize("i", range(3))
def test_sparse_equals_brute_force_over_kept_keys(i):
    """Attention over the kept blocks equals the pure-Python dense brute force
    over exactly the visible keys of those blocks (renumbered, no mask)."""
    b = random_batch(8300 + i, **CASES[i])
    block = 16
    sel = oracle.sparse_select(b, block, 2)
    out, lse = oracle.sparse_attention(b, sel, block)
    q, k, v = _values(b, b.q), _values(b, b.k), _values(b, b.v)
    G = b.hq // b.hkv
    for s in range(b.num_seqs):
        for qi in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            lo, hi = oracle.visible_range(b, qi, s)
            for h in range(b.hkv):
                kept = set(int(x) for x in sel[qi, h] if x >= 0)
                keys = [t for t in range(lo, hi + 1) if t // block in kept]
                kk = [[list(k[b.block_table[s, t // b.page_size], t % b.page_size, h])] for t in keys]
                vv = [[list(v[b.block_table[s, t // b.page_size], t % b.page_size, h])] for t in keys]
                qq = [[list(q[qi, h * G + g]) for g in range(G)]]
                ro, rl = brute.dense_attention(qq, kk, vv, [len(keys) - 1], G, 1, b.scale, False, 0)
                np.testing.assert_allclose(out[qi, h * G:(h + 1) * G], np.array(ro[0]), rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(lse[qi, h * G:(h + 1) * G], np.array(rl[0]), rtol=1e-12, atol=1e-12)


def test_lse_combine_of_per_block_parts():
    """The result over several kept blocks is the log-sum-exp combination of
    the results over each block alone (alice-llm `lse_combine`)."""
    b = random_batch(8400, dtype="bf16", hq=8, hkv=2, d=64, page_size=16, q_counts=(1, 4), max_len=600)
    block = 32
    sel = oracle.sparse_select(b, block, 3)
    out, lse = oracle.sparse_attention(b, sel, block)
    parts = []
    for j in range(sel.shape[2]):
        one = np.full_like(sel, -1)
        one[:, :, 0] = sel[:, :, j]
        parts.append(oracle.sparse_attention(b, one, block) if (sel[:, :, j] >= 0).all() else None)
    assert all(p is not None for p in parts)
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    O = sum(np.exp(p[1] - L)[..., None] * p[0] for p in parts)
    np.testing.assert_allclose(lse, L, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, O, rtol=0, atol=1e-12)


def test_planted_block_is_kept():
    """A block whose keys are a large multiple of the proxy query wins the
    top-1 choice of every row of its KV head that sees it."""
    b = random_batch(8500, dtype="f32", hq=4, hkv=1, d=16, page_size=8, q_counts=(1,), max_len=200, poison=False)
    block, s, qi = 16, 0, 0
    L = int(b.seq_lens[0])
    r_star = (L // block) // 2
    k = b.k.copy()
    for t in range(r_star * block, min(L, (r_star + 1) * block)):
        k[b.block_table[s, t // b.page_size], t % b.page_size, 0] = 50.0 * b.q[qi, 0]
    import dataclasses
    b2 = dataclasses.replace(b, k=k)
    sel = oracle.sparse_select(b2, block, 1)
    assert sel[qi, 0, 0] == r_star
