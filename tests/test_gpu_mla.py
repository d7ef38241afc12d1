"""GPU parity of absorbed-MLA decode (HIP kernels through the C ABI) against
the fp64 oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import config_bf16_mla_decode, random_mla_batch
from tests.gpu_harness import MlaRun, assert_close, to_f64

pytestmark = pytest.mark.gpu


def _parity(m, **kw):
    run = MlaRun(m, **kw)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.mla(m)
    assert_close(out, ref_o, "bf16")
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)
    return run


MLA_CASES = [
    dict(page_size=64, q_counts=(1, 1, 1), max_len=3000),
    dict(page_size=16, q_counts=(1, 1), max_len=700),
    dict(page_size=64, q_counts=(1, 1), histories=[0, 1]),
    dict(page_size=64, q_counts=(5, 1), max_len=2000, window=300),
    dict(page_size=32, q_counts=(3,), max_len=900, causal=False),
    dict(page_size=1, q_counts=(1, 2), max_len=100),
]


@pytest.mark.parametrize("i", range(len(MLA_CASES)))
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_random_mla_parity(i, split_tokens):
    m = random_mla_batch(3000 + i, **MLA_CASES[i])
    _parity(m, split_tokens=split_tokens)


MLA_HEAD_CASES = [
    (128, dict(page_size=64, q_counts=(1, 1, 1), max_len=3000)),               # a full head count on one GPU
    (32, dict(page_size=16, q_counts=(1, 1), max_len=900)),
    (20, dict(page_size=64, q_counts=(1, 9, 1), max_len=1500)),                # partial last group, a chunk
    (8, dict(page_size=64, q_counts=(1, 6), max_len=1500, window=300)),
    (1, dict(page_size=32, q_counts=(3, 1), max_len=700, causal=False)),
    (48, dict(page_size=64, q_counts=(0, 12, 1), histories=[50, 600, 90])),
    (48, dict(page_size=64, q_counts=(1, 1, 1), max_len=2500)),                # decode only: groups in pairs, odd count
    (40, dict(page_size=16, q_counts=(1, 2), max_len=1800, window=700)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("split_tokens", [0, 64])
@pytest.mark.parametrize("i", range(len(MLA_HEAD_CASES)))
def test_mla_head_counts_parity(i, split_tokens, dtype):
    """Head counts other than 16: the heads run in groups of 16 (the MFMA
    columns), the last group partial, and decode-only plans pair the groups
    (an odd count leaves the last item's second group past the end); every
    output element is written (the output starts as NaN) and matches the
    oracle."""
    heads, kw = MLA_HEAD_CASES[i]
    m = random_mla_batch(3200 + i, heads=heads, dtype=dtype, **kw)
    run = MlaRun(m, split_tokens=split_tokens)
    run.out.fill_(float("nan"))
    run.lse.fill_(float("nan"))
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.mla(m)
    assert_close(out, ref_o, dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)


def test_mla_decode_full_size_all_rows():
    m = config_bf16_mla_decode()
    run = _parity(m)
    assert run.info["decode_items"] >= 64 and run.info["split_rows"] > 0


MLA_SHAPE_CASES = [
    ("f32", 16, 512, 64, dict(page_size=64, q_counts=(1, 1, 7), max_len=1200)),
    ("f32", 128, 512, 64, dict(page_size=16, q_counts=(1, 3), max_len=600)),
    ("bf16", 16, 256, 32, dict(page_size=64, q_counts=(1, 9, 1), max_len=1500)),      # a smaller latent
    ("f16", 40, 128, 32, dict(page_size=32, q_counts=(2, 1), max_len=900, window=200)),
    ("bf16", 5, 100, 7, dict(page_size=1, q_counts=(1, 4), max_len=150, causal=False)),  # odd widths
    ("f32", 20, 1024, 256, dict(page_size=64, q_counts=(1, 1, 6), max_len=700)),       # the widest rows
]


@pytest.mark.parametrize("split_tokens", [0, 64])
@pytest.mark.parametrize("i", range(len(MLA_SHAPE_CASES)))
def test_mla_other_shapes_and_f32(i, split_tokens):
    """f32 data and latent / rotary widths other than 512 / 64 (the vector
    kernel), decode rows and chunks, split and unsplit: every element and
    lse against the oracle, output and lse starting as NaN."""
    dtype, heads, r, p, kw = MLA_SHAPE_CASES[i]
    m = random_mla_batch(3300 + i, heads=heads, r=r, p=p, dtype=dtype, **kw)
    run = MlaRun(m, split_tokens=split_tokens)
    run.out.fill_(float("nan"))
    run.lse.fill_(float("nan"))
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.mla(m)
    assert_close(out, ref_o, dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-4 if dtype == "f32" else 1e-3)


@pytest.mark.timeout(600)
def test_mla_decode_h128_full_size_all_rows():
    """The MLA decode shape with 128 query heads (eight head groups reading
    the same latent rows): every output element and lse against the oracle."""
    from synth import config_bf16_mla_decode_h128
    m = config_bf16_mla_decode_h128()
    run = _parity(m)
    assert run.info["decode_items"] >= 64 * 8 and run.info["split_rows"] > 0


def test_mla_window_one_returns_own_latent_bitwise():
    m = random_mla_batch(3100, page_size=64, q_counts=(1, 1, 2), max_len=1500, window=1)
    run = MlaRun(m)
    run()
    out, _ = run.result()
    lat = to_f64(run.latent)
    for s in range(m.num_seqs):
        for i in range(int(m.cu_q[s]), int(m.cu_q[s + 1])):
            p = int(m.q_pos[i])
            row = lat[m.block_table[s, p // m.page_size], p % m.page_size, 0]
            for h in range(m.heads):
                assert np.array_equal(out[i, h], row), (i, h)


def test_mla_page_permutation_bitwise_and_deterministic():
    m = random_mla_batch(3200, page_size=64, q_counts=(1, 1, 1), max_len=4000)
    r1 = MlaRun(m)
    r1()
    o1, l1 = r1.result()
    r1()
    o1b, l1b = r1.result()
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    rng = np.random.default_rng(8)
    extra = 3
    perm = rng.permutation(m.num_pages + extra)

    def move(t):
        t2 = np.full((m.num_pages + extra,) + t.shape[1:], 0x7FC0, dtype=np.uint16)
        t2[perm[:m.num_pages]] = t
        return t2

    bt2 = np.where(m.block_table >= 0, perm[np.maximum(m.block_table, 0)], -1).astype(np.int32)
    r2 = MlaRun(dataclasses.replace(m, latent=move(m.latent), kpos=move(m.kpos), block_table=bt2,
                                    num_pages=m.num_pages + extra))
    r2()
    o2, l2 = r2.result()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("max_splits", [64, 1])
def test_mla_64k_key_row(max_splits):
    """One MLA row over 65536 keys: split to the 64-piece limit, or unsplit
    (one workgroup walks 4096 tiles, reloading its page-number window 64
    times)."""
    m = random_mla_batch(3100, page_size=64, q_counts=(1,), histories=[65535], max_splits=max_splits)
    _parity(m)


MLA_PREFILL_CASES = [
    dict(page_size=64, q_counts=(64, 1, 17), max_len=1500),
    dict(page_size=16, q_counts=(33,), histories=[0]),
    dict(page_size=64, q_counts=(40, 5), max_len=2000, window=300),
    dict(page_size=32, q_counts=(9, 1), max_len=900, causal=False),
    dict(page_size=1, q_counts=(7,), max_len=100),
    dict(page_size=64, q_counts=(0, 12, 0, 1, 3), histories=[50, 600, 0, 20, 90]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("i", range(len(MLA_PREFILL_CASES)))
def test_mla_chunked_prefill_parity(i, dtype):
    """Sequences with more than four queries run as chunked-prefill items (two
    queries per workgroup sharing the latent tiles), next to decode items."""
    m = random_mla_batch(3600 + i, dtype=dtype, **MLA_PREFILL_CASES[i])
    run = MlaRun(m)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.mla(m)
    assert_close(out, ref_o, dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)
    assert run.info["prefill_items"] > 0


def test_mla_chunked_prefill_window_one_bitwise():
    m = random_mla_batch(3700, page_size=64, q_counts=(30, 1, 9), max_len=1500, window=1)
    run = MlaRun(m)
    run()
    out, _ = run.result()
    lat = to_f64(run.latent)
    for s in range(m.num_seqs):
        for i in range(int(m.cu_q[s]), int(m.cu_q[s + 1])):
            p = int(m.q_pos[i])
            row = lat[m.block_table[s, p // m.page_size], p % m.page_size, 0]
            for h in range(m.heads):
                assert np.array_equal(out[i, h], row), (i, h)


@pytest.mark.timeout(900)
def test_mla_chunked_prefill_full_size_every_row():
    """The MLA chunked-prefill workload (8 chunks of 256 queries after
    histories of up to 4096 keys): every output element and every lse
    against the oracle."""
    from synth import config_bf16_mla_chunked_prefill
    m = config_bf16_mla_chunked_prefill()
    run = MlaRun(m)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.mla(m)
    assert_close(out, ref_o, "bf16")
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)
    assert run.info["prefill_items"] > 0 and run.info["decode_items"] == 0
