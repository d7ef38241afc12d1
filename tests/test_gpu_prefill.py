"""GPU parity of chunked prefill and of mixed decode + prefill batches in one
launch (HIP kernels through the C ABI) against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import config_bf16_chunked_prefill, config_bf16_mixed_batch, random_batch
from tests.gpu_harness import GqaRun, assert_close, to_f64

pytestmark = pytest.mark.gpu


def _all_rows(b, **kw):
    run = GqaRun(b, **kw)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.attention(b)
    assert_close(out, ref_o, b.dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3 if b.dtype == "bf16" else 1e-4)
    return run


PREFILL_CASES = [
    dict(hq=32, hkv=8, d=128, page_size=16, q_counts=(300, 1, 77), max_len=900),
    dict(hq=64, hkv=8, d=128, page_size=64, q_counts=(1, 130, 1, 1), max_len=3000, window=257),
    dict(hq=8, hkv=8, d=128, page_size=16, q_counts=(200,), histories=[0]),
    dict(hq=16, hkv=1, d=128, page_size=16, q_counts=(40, 9), max_len=400),
    dict(hq=8, hkv=2, d=64, page_size=32, q_counts=(150, 5), max_len=700, causal=False),
    dict(hq=4, hkv=2, d=64, page_size=16, q_counts=(65, 66), max_len=500, window=31),
    dict(hq=32, hkv=8, d=128, page_size=1, q_counts=(70,), max_len=200),
    dict(hq=32, hkv=8, d=128, page_size=16, q_counts=(513,), histories=[4096 - 513]),
    dict(hq=32, hkv=8, d=128, page_size=16, q_counts=(33, 1, 2, 3, 4, 5), max_len=300, causal=False, window=100),
    # sequences without queries (one without keys) around a chunk and a decode row
    dict(hq=32, hkv=8, d=128, page_size=16, q_counts=(0, 97, 0, 1, 0), histories=[40, 200, 0, 1000, 3]),
]


@pytest.mark.parametrize("i", range(len(PREFILL_CASES)))
def test_random_prefill_and_mixed_parity(i):
    b = random_batch(2000 + i, dtype="bf16", **PREFILL_CASES[i])
    run = _all_rows(b)
    assert run.info["prefill_items"] > 0


@pytest.mark.parametrize("case", [
    dict(dtype="f32", hq=8, hkv=2, d=64, page_size=16, q_counts=(20, 1), max_len=300),
    dict(dtype="bf16", hq=4, hkv=1, d=256, page_size=16, q_counts=(12,), max_len=200, window=20),
])
def test_prefill_f32_and_d256_short_chunks(case):
    """f32 data runs prefill tiles query by query (no MFMA tile); head size
    256 runs the two-pass MFMA tile on a chunk shorter than one tile."""
    b = random_batch(2100, **case)
    _all_rows(b)


@pytest.mark.timeout(900)
def test_chunked_prefill_full_size_every_row():
    """The chunked-prefill workload (8 sequences, 512-query chunks after 0..4096
    cached keys, Hq 32, Hkv 8, D 128, page 16): every output element and
    every lse against the oracle."""
    b = config_bf16_chunked_prefill()
    run = _all_rows(b)
    assert run.info["prefill_items"] > 0 and run.info["decode_items"] == 0


@pytest.mark.timeout(900)
def test_mixed_batch_full_size_every_row_one_launch():
    """The mixed workload in one launch (64 decode rows of 1024..32768 keys and
    4 chunks of 1024 queries, Hq 64, Hkv 8, page 64, window 4096): every
    output element and every lse against the oracle."""
    b = config_bf16_mixed_batch()
    run = _all_rows(b)
    assert run.info["prefill_items"] > 0 and run.info["decode_items"] > 0 and run.info["launches"] >= 1


def test_prefill_window_one_returns_own_value_bitwise():
    b = random_batch(2200, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(150, 1, 40), max_len=600,
                     window=1)
    run = GqaRun(b)
    run()
    out, _ = run.result()
    v = to_f64(run.v)
    G = b.hq // b.hkv
    for s in range(b.num_seqs):
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            p = int(b.q_pos[i])
            row = v[b.block_table[s, p // b.page_size], p % b.page_size]
            for h in range(b.hq):
                assert np.array_equal(out[i, h], row[h // G]), (i, h)


def test_prefill_page_permutation_bitwise_and_deterministic():
    b = random_batch(2300, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(180, 1, 60), max_len=1500)
    r1 = GqaRun(b)
    r1()
    o1, l1 = r1.result()
    r1()
    o1b, l1b = r1.result()
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    rng = np.random.default_rng(6)
    extra = 5
    perm = rng.permutation(b.num_pages + extra)
    k2 = np.full((b.num_pages + extra,) + b.k.shape[1:], 0x7FC0, dtype=np.uint16)
    v2 = np.full((b.num_pages + extra,) + b.v.shape[1:], 0x7FC0, dtype=np.uint16)
    k2[perm[:b.num_pages]] = b.k
    v2[perm[:b.num_pages]] = b.v
    bt2 = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1).astype(np.int32)
    r2 = GqaRun(dataclasses.replace(b, k=k2, v=v2, block_table=bt2, num_pages=b.num_pages + extra))
    r2()
    o2, l2 = r2.result()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_prefill_sequence_order_does_not_change_rows():
    """Per-query outputs do not depend on where a sequence sits in the batch."""
    b = random_batch(2400, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 90, 1, 33), max_len=800)
    r1 = GqaRun(b)
    r1()
    o1, _ = r1.result()
    order = [3, 1, 0, 2]
    counts = np.diff(b.cu_q)
    cu = np.concatenate([[0], np.cumsum(counts[order])]).astype(np.int32)
    qidx = np.concatenate([np.arange(b.cu_q[s], b.cu_q[s + 1]) for s in order])
    b2 = dataclasses.replace(b, seq_lens=b.seq_lens[order], cu_q=cu, q_pos=b.q_pos[qidx],
                             block_table=b.block_table[order], q=b.q[qidx])
    r2 = GqaRun(b2)
    r2()
    o2, _ = r2.result()
    assert np.array_equal(o1[qidx], o2)


GROUP_CASES = [  # group sizes that are not powers of two (Hq / Hkv)
    dict(hq=24, hkv=8, d=128, page_size=16, q_counts=(1, 90, 1, 3), max_len=1500),          # G = 3
    dict(hq=40, hkv=8, d=128, page_size=64, q_counts=(2, 1, 70), max_len=2500, window=300),  # G = 5
    dict(hq=12, hkv=2, d=64, page_size=16, q_counts=(1, 1, 130), max_len=900),              # G = 6
    dict(hq=28, hkv=4, d=128, page_size=32, q_counts=(1, 60, 1), max_len=3000),            # G = 7
    dict(hq=48, hkv=4, d=128, page_size=16, q_counts=(1, 1, 40), max_len=2000, causal=False),  # G = 12
    dict(hq=14, hkv=2, d=128, page_size=16, q_counts=(1, 1), max_len=5000),                # G = 7, decode only
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("i", range(len(GROUP_CASES)))
def test_group_sizes_beyond_powers_of_two(i, dtype):
    """Hq / Hkv of 3, 5, 6, 7 and 12: decode rows (split and whole) and MFMA
    prefill tiles whose 256 rows hold floor(256 / G) queries."""
    b = random_batch(2500 + i, dtype=dtype, **GROUP_CASES[i])
    for split_tokens in (0, 128):
        run = GqaRun(b, split_tokens=split_tokens)
        run()
        out, lse = run.result()
        ref_o, ref_l = oracle.attention(b)
        assert_close(out, ref_o, dtype)
        np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)


def test_group_size_seven_f32_and_window_one_bitwise():
    """f32 tiles (query by query) at G = 7, and one visible key returning its
    own value row bit for bit at G = 5 in a mixed launch."""
    b = random_batch(2600, dtype="f32", hq=28, hkv=4, d=64, page_size=16, q_counts=(1, 20, 2), max_len=700)
    _all_rows(b)
    b = random_batch(2601, dtype="bf16", hq=40, hkv=8, d=128, page_size=16, q_counts=(1, 50, 1), max_len=900,
                     window=1)
    run = GqaRun(b)
    run()
    out, _ = run.result()
    v = to_f64(run.v)
    for s in range(b.num_seqs):
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            p = int(b.q_pos[i])
            row = v[b.block_table[s, p // b.page_size], p % b.page_size]
            for h in range(b.hq):
                assert np.array_equal(out[i, h], row[h // 5]), (i, h)

