"""Pins for the fp64 oracle: each test checks it against something other than
itself -- an independent brute force, a library routine, a closed form, an
invariant of the definition, or the fixture a page defines.

Definition pinned: boostr 0.2.0-beta.2 attention/flash_standard.rs
(`standard_attention_fwd`, `build_attention_mask`, `expand_kv`) on the paged
layout with absolute positions of ruDNN 0.1.107 paged_attention/mod.rs
(`DevicePlan::attention`, `DevicePlan::mla`).
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import f32_to_bf16_bits, f32_to_f16_bits, random_batch, random_mla_batch, PagedBatch
from tests.dense_view import dense_sequence, scatter_into_pool, widen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_batch(b):
    """Brute force over the dense per-sequence view of a paged batch."""
    q = widen(b.q, b.dtype)
    k = widen(b.k, b.dtype)
    v = widen(b.v, b.dtype)
    outs, lses = [], []
    for s in range(b.num_seqs):
        lo, hi = int(b.cu_q[s]), int(b.cu_q[s + 1])
        if hi == lo:
            continue
        L = int(b.seq_lens[s])
        kd = dense_sequence(k, b.block_table, s, L, b.page_size).tolist()
        vd = dense_sequence(v, b.block_table, s, L, b.page_size).tolist()
        o, l = brute.dense_attention(q[lo:hi].tolist(), kd, vd, b.q_pos[lo:hi].tolist(), b.hq, b.hkv,
                                     b.scale, b.causal, b.window)
        outs.append(np.array(o))
        lses.append(np.array(l))
    return np.concatenate(outs), np.concatenate(lses)


CASES = [
    dict(dtype="f32", hq=4, hkv=1, d=8, page_size=4, q_counts=(1, 3), causal=True, window=0),
    dict(dtype="bf16", hq=4, hkv=2, d=16, page_size=3, q_counts=(2, 1, 4), causal=True, window=5),
    dict(dtype="f32", hq=2, hkv=2, d=8, page_size=1, q_counts=(1, 2), causal=False, window=0),
    dict(dtype="bf16", hq=6, hkv=3, d=8, page_size=16, q_counts=(3, 1), causal=False, window=7),
    dict(dtype="f32", hq=8, hkv=2, d=12, page_size=5, q_counts=(1, 1, 1), causal=True, window=1),
    dict(dtype="bf16", hq=3, hkv=1, d=8, page_size=2, q_counts=(5,), causal=True, window=2, dv=4),
    dict(dtype="f16", hq=4, hkv=2, d=16, page_size=4, q_counts=(1, 3, 2), causal=True, window=6),
    dict(dtype="f16", hq=2, hkv=1, d=8, page_size=1, q_counts=(2, 1), causal=False, window=0, dv=4),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_oracle_matches_pure_python_brute_force(i):
    b = random_batch(100 + i, max_len=40, **CASES[i])
    out, lse = oracle.attention(b)
    ref_o, ref_l = _brute_batch(b)
    assert out.shape == ref_o.shape
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-12, atol=1e-12)


def test_oracle_matches_torch_sdpa_float64():
    """Library routine: torch's scaled_dot_product_attention in float64 on
    the dense per-sequence view with an explicit boolean visibility mask and
    explicitly repeated KV heads."""
    torch = pytest.importorskip("torch")
    b = random_batch(7, dtype="bf16", hq=8, hkv=2, d=64, page_size=16, q_counts=(1, 9, 1, 33),
                     max_len=200, causal=True, window=50)
    out, _ = oracle.attention(b)
    q = widen(b.q, b.dtype)
    k = widen(b.k, b.dtype)
    v = widen(b.v, b.dtype)
    G = b.hq // b.hkv
    for s in range(b.num_seqs):
        lo, hi = int(b.cu_q[s]), int(b.cu_q[s + 1])
        L = int(b.seq_lens[s])
        kd = torch.from_numpy(dense_sequence(k, b.block_table, s, L, b.page_size))   # [L, hkv, d]
        vd = torch.from_numpy(dense_sequence(v, b.block_table, s, L, b.page_size))
        kd = kd.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()            # [hq, L, d]
        vd = vd.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
        qq = torch.from_numpy(q[lo:hi]).permute(1, 0, 2).contiguous()                # [hq, n, d]
        pos = torch.from_numpy(b.q_pos[lo:hi].astype(np.int64))[:, None]
        t = torch.arange(L)[None, :]
        allowed = (t <= pos) & (t > pos - b.window)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kd, vd, attn_mask=allowed, scale=b.scale)
        np.testing.assert_allclose(out[lo:hi], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_p4_fixture_paged_matches_dense():
    """alice-llm `fixture_gqa`: paged through 4-token pages vs the dense brute
    force, non-causal (the page's own bar is rel 1e-4 in f32; fp64 agrees to
    rounding)."""
    fx = json.load(open(os.path.join(GOLDEN, "p4_fixture_gqa.json")))
    tq, hq, hkv, d, L, ps = (fx[k] for k in ("tq", "hq", "hkv", "head_dim", "seq_len", "page_size"))
    q = np.sin(np.arange(tq * hq * d, dtype=np.float32) * np.float32(fx["q_freq"])).reshape(tq, hq, d)
    k = np.cos(np.arange(L * hkv * d, dtype=np.float32) * np.float32(fx["k_freq"])).reshape(L, hkv, d)
    v = np.sin(np.arange(L * hkv * d, dtype=np.float32) * np.float32(fx["v_freq"])).reshape(L, hkv, d)
    perm = np.random.default_rng(0).permutation(L // ps + 2)
    kp, bt = scatter_into_pool([k], ps, perm, 2, np.float32(np.nan))
    vp, _ = scatter_into_pool([v], ps, perm, 2, np.float32(np.nan))
    b = PagedBatch("p4", "f32", np.array([L], np.int32), np.array([0, tq], np.int32),
                   np.array([L - 1] * tq, np.int32), bt, ps, kp.shape[0], hq, hkv, d, d,
                   1.0 / math.sqrt(d), False, 0, q, kp, vp)
    out, _ = oracle.attention(b)
    ref, _ = brute.dense_attention(q.astype(np.float64).tolist(), k.astype(np.float64).tolist(),
                                   v.astype(np.float64).tolist(), [L - 1] * tq, hq, hkv, 1.0 / math.sqrt(d),
                                   False, 0)
    ref = np.array(ref)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    rel = np.abs(out - ref) / np.maximum(np.abs(ref), 1e-6)
    assert rel.max() < fx["page_rel_tolerance"]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_window_one_returns_own_value_bitwise(dtype):
    """W = 1: each query sees only its own key, so the softmax has one weight
    e^0 = 1 and the output is that key's value row exactly."""
    b = random_batch(11, dtype=dtype, hq=8, hkv=2, d=32, page_size=16, q_counts=(1, 4, 1, 17), max_len=100,
                     causal=True, window=1)
    out, lse = oracle.attention(b)
    v = widen(b.v, dtype)
    k = widen(b.k, dtype)
    q = widen(b.q, dtype)
    G = b.hq // b.hkv
    for s in range(b.num_seqs):
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            p = int(b.q_pos[i])
            page, slot = b.block_table[s, p // b.page_size], p % b.page_size
            for h in range(b.hq):
                assert np.array_equal(out[i, h], v[page, slot, h // G])
                dot = math.fsum(q[i, h] * k[page, slot, h // G])
                assert abs(lse[i, h] - b.scale * dot) <= 1e-12 * max(1.0, abs(b.scale * dot))


def test_first_position_causal_returns_first_value():
    """Causal query at position 0 sees only key 0."""
    b = random_batch(12, dtype="bf16", hq=4, hkv=4, d=16, page_size=4, q_counts=(1,), histories=[0],
                     causal=True, window=0)
    out, _ = oracle.attention(b)
    v = widen(b.v, "bf16")
    assert np.array_equal(out[0], v[b.block_table[0, 0], 0])


def test_page_permutation_and_extra_pages_bitwise_invariant():
    """Output depends only on logical order: moving pages to other physical
    slots (and adding NaN pages) changes nothing, bit for bit."""
    b = random_batch(13, dtype="bf16", hq=8, hkv=2, d=32, page_size=8, q_counts=(1, 6, 2), max_len=120,
                     causal=True, window=30)
    out, lse = oracle.attention(b)
    rng = np.random.default_rng(99)
    extra = 5
    perm = rng.permutation(b.num_pages + extra)             # old physical page -> new physical page
    k2 = np.full((b.num_pages + extra,) + b.k.shape[1:], 0x7FC0, dtype=np.uint16)
    v2 = np.full((b.num_pages + extra,) + b.v.shape[1:], 0x7FC0, dtype=np.uint16)
    k2[perm[:b.num_pages]] = b.k
    v2[perm[:b.num_pages]] = b.v
    bt2 = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1).astype(np.int32)
    b2 = dataclasses.replace(b, k=k2, v=v2, block_table=bt2, num_pages=b.num_pages + extra)
    out2, lse2 = oracle.attention(b2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_gqa_equals_explicit_kv_head_repetition():
    """boostr `expand_kv`: GQA over Hkv heads equals MHA over a pool whose
    head h is a copy of KV head floor(h / G)."""
    b = random_batch(14, dtype="f32", hq=8, hkv=2, d=16, page_size=4, q_counts=(2, 1, 3), max_len=60,
                     causal=True, window=0)
    out, lse = oracle.attention(b)
    G = b.hq // b.hkv
    k_rep = np.repeat(b.k, G, axis=2)
    v_rep = np.repeat(b.v, G, axis=2)
    b2 = dataclasses.replace(b, k=k_rep, v=v_rep, hkv=b.hq)
    out2, lse2 = oracle.attention(b2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_constant_values_give_that_constant():
    b = random_batch(15, dtype="f32", hq=4, hkv=2, d=16, page_size=4, q_counts=(1, 5), max_len=80,
                     causal=True, window=9, poison=False)
    b = dataclasses.replace(b, v=np.full_like(b.v, 0.625))
    out, _ = oracle.attention(b)
    np.testing.assert_allclose(out, 0.625, rtol=1e-12, atol=0)


def _closed_form_visible_count(p, L, causal, window):
    hi = p if causal else L - 1
    lo = max(0, p - window + 1) if window > 0 else 0
    return hi - lo + 1, lo, hi


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 7), (False, 0), (False, 5)])
def test_vanishing_scale_counts_visible_keys(causal, window):
    """scale -> 0: every visible weight is e^0 = 1 in double precision, so
    lse = ln |T| and the output is the plain mean of the visible value rows;
    |T| has a closed form in (p, L, causal, W)."""
    b = random_batch(16, dtype="bf16", hq=4, hkv=1, d=8, page_size=4, q_counts=(1, 3, 6), max_len=50,
                     causal=causal, window=window, scale=1e-30)
    out, lse = oracle.attention(b)
    v = widen(b.v, "bf16")
    for s in range(b.num_seqs):
        L = int(b.seq_lens[s])
        vd = dense_sequence(v, b.block_table, s, L, b.page_size)
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            n, lo, hi = _closed_form_visible_count(int(b.q_pos[i]), L, causal, window)
            assert np.allclose(lse[i], math.log(n), rtol=0, atol=1e-12)
            np.testing.assert_allclose(out[i], np.broadcast_to(vd[lo:hi + 1, 0].mean(axis=0), out[i].shape),
                                       rtol=1e-12, atol=1e-12)


def test_logsumexp_combines_over_disjoint_key_ranges():
    """Splitting the visible keys into two disjoint ranges and recombining
    their (out, lse) by log-sum-exp weights reproduces the full result: the
    identity the split-KV merge relies on (alice-llm `lse_combine`)."""
    b = random_batch(17, dtype="f32", hq=4, hkv=2, d=16, page_size=4, q_counts=(1,), histories=[70],
                     causal=True, window=0, poison=False)
    L = int(b.seq_lens[0])
    W = 29
    full_o, full_l = oracle.attention(b)
    near_o, near_l = oracle.attention(dataclasses.replace(b, window=W))               # keys [L-W, L)
    far = dataclasses.replace(b, seq_lens=np.array([L - W], np.int32), q_pos=np.array([L - W - 1], np.int32))
    far_o, far_l = oracle.attention(far)                                               # keys [0, L-W)
    # the far sub-problem uses the same keys in the same pages
    tot = np.logaddexp(near_l, far_l)
    np.testing.assert_allclose(tot, full_l, rtol=1e-13, atol=1e-13)
    comb = (np.exp(near_l - tot)[..., None] * near_o + np.exp(far_l - tot)[..., None] * far_o)
    np.testing.assert_allclose(comb, full_o, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_mla_equals_mqa_over_concatenated_key(dtype):
    """ruDNN `DevicePlan::mla` passes the latent as key and value and adds a
    position term to the score: that is single-KV-head attention whose key is
    [latent | kpos] (width R+P), whose query is [q_abs | q_rope] and whose
    value is the latent (width R)."""
    m = random_mla_batch(18, heads=4, r=32, p=8, page_size=8, q_counts=(1, 3, 1), max_len=60, dtype=dtype)
    out, lse = oracle.mla(m)
    k = np.concatenate([m.latent, m.kpos], axis=-1)
    q = np.concatenate([m.q_abs, m.q_rope], axis=-1)
    b = PagedBatch("mqa", dtype, m.seq_lens, m.cu_q, m.q_pos, m.block_table, m.page_size, m.num_pages,
                   m.heads, 1, m.r + m.p, m.r, m.scale, m.causal, m.window, q, k, m.latent)
    out2, lse2 = oracle.attention(b)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-13)


def test_mla_without_position_terms_is_mqa_with_k_equal_v():
    m = random_mla_batch(19, heads=4, r=16, p=4, page_size=4, q_counts=(2, 1), max_len=30)
    m = dataclasses.replace(m, q_rope=np.zeros_like(m.q_rope), kpos=np.zeros_like(m.kpos))
    out, _ = oracle.mla(m)
    b = PagedBatch("mqa0", "bf16", m.seq_lens, m.cu_q, m.q_pos, m.block_table, m.page_size, m.num_pages,
                   m.heads, 1, m.r, m.r, m.scale, m.causal, m.window, m.q_abs, m.latent, m.latent)
    out2, _ = oracle.attention(b)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-13)


def test_rows_subset_matches_full_evaluation():
    b = random_batch(20, dtype="bf16", hq=8, hkv=2, d=16, page_size=16, q_counts=(1, 8, 2), max_len=90)
    out, lse = oracle.attention(b)
    rows = np.array([0, 5, 17, 40, b.num_queries * b.hq - 1], dtype=np.int64)
    o2, l2 = oracle.attention(b, rows=rows)
    assert np.array_equal(o2, out.reshape(-1, b.dv)[rows]) and np.array_equal(l2, lse.reshape(-1)[rows])


def test_oracle_never_reads_invisible_nan_data():
    """Unreferenced pages and tail slots are NaN in random batches; no output
    may be NaN."""
    b = random_batch(21, dtype="bf16", hq=4, hkv=2, d=16, page_size=8, q_counts=(1, 7, 1), max_len=70,
                     causal=True, window=13, poison=True)
    out, lse = oracle.attention(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, np.inf, -0.0], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0);
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: rounds to even (1+2^-6)
    assert list(bits[:3]) == [0x3F80, 0x3F80, 0x3F82]
    assert bits[3] == 0xC020 and bits[5] == 0x7F80 and bits[6] == 0x8000


def test_f16_rounding_is_round_to_nearest_even():
    """IEEE binary16: 10 fraction bits, so ulp(1) = 2^-10; the smallest
    subnormal is 2^-24; values from 65520 up overflow to infinity."""
    x = np.array([1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -2.5, 65504.0, 65520.0, 2.0 ** -25, 3 * 2.0 ** -25,
                  -0.0, np.inf], dtype=np.float32)
    bits = f32_to_f16_bits(x)
    assert [int(v) for v in bits] == [0x3C00, 0x3C00, 0x3C02, 0xC100, 0x7BFF, 0x7C00, 0x0000, 0x0002, 0x8000,
                                      0x7C00]


def test_oracle_f16_widening_is_ieee_binary16():
    """The oracle's own binary16 decoding against the IEEE definition: hand
    values (sign, exponent bias 15, subnormals m 2^-24, infinities, NaN), then
    all 65536 patterns against numpy's float16 (a library routine)."""
    table = {0x0000: 0.0, 0x8000: -0.0, 0x3C00: 1.0, 0xC000: -2.0, 0x3555: 0.333251953125, 0x7BFF: 65504.0,
             0x0400: 2.0 ** -14, 0x03FF: 1023 * 2.0 ** -24, 0x0001: 2.0 ** -24, 0x8001: -(2.0 ** -24),
             0x7C00: math.inf, 0xFC00: -math.inf, 0x3BFF: 1 - 2.0 ** -11, 0x4248: 3.140625}
    got = oracle.widen(np.array(list(table), dtype=np.uint16), "f16")
    for (bits, want), g in zip(table.items(), got):
        assert g == want and math.copysign(1, g) == math.copysign(1, want), hex(bits)
    assert np.isnan(oracle.widen(np.array([0x7E00, 0xFC01, 0x7C01], dtype=np.uint16), "f16")).all()
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(every, "f16")
    ref = every.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan]) and np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("dtype,page_size", [("bf16", 16), ("f32", 1), ("bf16", 64), ("f16", 8)])
def test_append_places_rows_at_their_positions(dtype, page_size):
    """Paged append (ruDNN paged_attention `DevicePlan::append`): read back in
    logical order through the dense view (numpy indexing, not the oracle's
    loop), position q_pos[i] of each sequence holds query i's new rows, every
    other position and every unreferenced page is unchanged."""
    b = random_batch(70, dtype=dtype, hq=8, hkv=2, d=64, page_size=page_size, q_counts=(1, 5, 0, 3),
                     histories=[40, 0, 7, 129])
    rng = np.random.default_rng(71)
    store = np.float32 if dtype == "f32" else np.uint16
    k_new = rng.integers(0, 1 << 15, size=(b.num_queries, b.hkv, b.d)).astype(store)
    v_new = rng.integers(0, 1 << 15, size=(b.num_queries, b.hkv, b.dv)).astype(store)
    k2, v2 = oracle.append_kv(b.seq_lens, b.cu_q, b.q_pos, b.block_table, b.page_size, k_new, v_new, b.k, b.v)
    touched = np.zeros(b.k.shape[:2], bool)
    for s in range(b.num_seqs):
        L = int(b.seq_lens[s])
        before_k = dense_sequence(b.k, b.block_table, s, L, b.page_size)
        after_k = dense_sequence(k2, b.block_table, s, L, b.page_size)
        after_v = dense_sequence(v2, b.block_table, s, L, b.page_size)
        mine = np.zeros(L, bool)
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            p = int(b.q_pos[i])
            mine[p] = True
            assert np.array_equal(after_k[p], k_new[i]) and np.array_equal(after_v[p], v_new[i])
        same = ~mine
        assert np.array_equal(after_k[same].view(np.uint8), before_k[same].view(np.uint8))
        t = np.arange(L)[mine]
        touched[b.block_table[s, t // b.page_size], t % b.page_size] = True
    # nothing outside the written slots changed (NaN-poisoned rows compared bitwise)
    assert np.array_equal(k2[~touched].view(np.uint8), b.k[~touched].view(np.uint8))
    assert np.array_equal(v2[~touched].view(np.uint8), b.v[~touched].view(np.uint8))


def test_append_then_window_one_attention_returns_the_new_values():
    """After appending, attention with a one-key window reads each query's own
    new V row through the C oracle's paged gather (an independent route from
    page number and slot to row)."""
    b = random_batch(72, dtype="bf16", hq=8, hkv=2, d=64, page_size=16, q_counts=(1, 4, 2), histories=[33, 0, 500],
                     window=1)
    rng = np.random.default_rng(73)
    v_new = f32_to_bf16_bits(rng.standard_normal((b.num_queries, b.hkv, b.dv)).astype(np.float32))
    k_new = f32_to_bf16_bits(rng.standard_normal((b.num_queries, b.hkv, b.d)).astype(np.float32))
    k2, v2 = oracle.append_kv(b.seq_lens, b.cu_q, b.q_pos, b.block_table, b.page_size, k_new, v_new, b.k, b.v)
    out, lse = oracle.attention(dataclasses.replace(b, k=k2, v=v2))
    G = b.hq // b.hkv
    want = widen(v_new, "bf16")[:, np.arange(b.hq) // G]
    assert np.array_equal(out, want) and np.all(lse == lse)
