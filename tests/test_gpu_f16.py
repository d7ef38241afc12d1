"""GPU parity of the IEEE binary16 (f16) path -- split-KV decode, chunked
prefill and mixed launches, absorbed MLA, the split merge and the paged append
-- through the C ABI against the fp64 oracle (ruDNN paged_attention's tensor
check admits F16 beside F32 and BF16).

Bar: |gpu - oracle| <= 2.5e-3 + 1.25e-3 |oracle| (the bf16 bar scaled by 2^-3
for f16's three more significand bits); lse within 1e-3; window-one rows
bit for bit."""
import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import f32_to_f16_bits, random_batch, random_mla_batch
from tests.dense_view import widen
from tests.gpu_harness import GqaRun, MlaRun, assert_close, to_f64, to_torch

pytestmark = pytest.mark.gpu


def _check(run, ref_o, ref_l, rows=None):
    out, lse = run.result()
    if rows is not None:
        out, lse = out.reshape(-1, out.shape[-1])[rows], lse.reshape(-1)[rows]
    assert_close(out, ref_o, "f16")
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)
    assert np.isfinite(out).all()


DECODE_CASES = [
    dict(hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1, 2, 1), max_len=3000),
    dict(hq=64, hkv=8, d=128, page_size=64, q_counts=(1, 1, 3), max_len=5000, window=700),
    dict(hq=16, hkv=16, d=128, page_size=16, q_counts=(1, 4), max_len=900),
    dict(hq=16, hkv=1, d=128, page_size=16, q_counts=(1, 1), max_len=2100),
    dict(hq=8, hkv=4, d=64, page_size=32, q_counts=(1, 2, 1), max_len=1500, causal=False),
    dict(hq=8, hkv=1, d=256, page_size=16, q_counts=(1, 1), max_len=1200, window=33),
    dict(hq=4, hkv=2, d=128, page_size=1, q_counts=(1, 1), max_len=300),
    dict(hq=12, hkv=6, d=128, page_size=16, q_counts=(1, 1, 1), max_len=2500),
]


@pytest.mark.parametrize("i", range(len(DECODE_CASES)))
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_f16_decode_parity(i, split_tokens):
    b = random_batch(5000 + i, dtype="f16", **DECODE_CASES[i])
    run = GqaRun(b, split_tokens=split_tokens)
    run()
    _check(run, *oracle.attention(b))


def test_f16_decode_batch_full_size_all_rows():
    """The decode-batch shape (32 sequences of 512..8192 keys, Hq 32, Hkv 8,
    D 128, 16-key pages) in f16, every row, with split rows merged."""
    rng = np.random.default_rng(5100)
    hist = rng.integers(511, 8191 + 1, size=32)
    b = random_batch(5101, dtype="f16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1,) * 32, histories=hist)
    run = GqaRun(b)
    run()
    _check(run, *oracle.attention(b))
    assert run.info["split_rows"] > 0


PREFILL_CASES = [
    dict(hq=32, hkv=8, d=128, page_size=16, q_counts=(300, 1, 77), max_len=900),
    dict(hq=64, hkv=8, d=128, page_size=64, q_counts=(1, 130, 1, 1), max_len=3000, window=257),
    dict(hq=16, hkv=1, d=128, page_size=16, q_counts=(40, 9), max_len=400),
    dict(hq=8, hkv=2, d=64, page_size=32, q_counts=(150, 5), max_len=700, causal=False),
    dict(hq=32, hkv=8, d=128, page_size=1, q_counts=(70,), max_len=200),
    dict(hq=4, hkv=1, d=256, page_size=16, q_counts=(12,), max_len=200, window=20),
]


@pytest.mark.parametrize("i", range(len(PREFILL_CASES)))
def test_f16_prefill_and_mixed_parity(i):
    b = random_batch(5200 + i, dtype="f16", **PREFILL_CASES[i])
    run = GqaRun(b)
    run()
    _check(run, *oracle.attention(b))
    assert run.info["prefill_items"] > 0


@pytest.mark.timeout(900)
def test_f16_chunked_prefill_full_size_every_row():
    """The chunked-prefill shape (8 sequences, 512-query chunks after 0..4096
    cached keys, Hq 32, Hkv 8, D 128) in f16: every output element and every
    lse against the oracle."""
    rng = np.random.default_rng(5300)
    hist = rng.integers(0, 4096 + 1, size=8)
    b = random_batch(5301, dtype="f16", hq=32, hkv=8, d=128, page_size=16, q_counts=(512,) * 8, histories=hist)
    run = GqaRun(b)
    run()
    _check(run, *oracle.attention(b))
    assert run.info["prefill_items"] > 0


@pytest.mark.parametrize("q_counts,page_size", [((1, 1, 2, 1), 16), ((150, 1, 40), 16), ((3, 90), 64)])
def test_f16_window_one_returns_own_value_bitwise(q_counts, page_size):
    """One visible key: weight 1, so the output row is the key's value row
    exactly (decode items and MFMA prefill tiles)."""
    b = random_batch(5400, dtype="f16", hq=32, hkv=8, d=128, page_size=page_size, q_counts=q_counts,
                     max_len=1500, window=1)
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


MLA_CASES = [
    dict(page_size=64, q_counts=(1, 1, 1), max_len=3000),
    dict(page_size=16, q_counts=(1, 1), max_len=700),
    dict(page_size=64, q_counts=(5, 1), max_len=2000, window=300),
    dict(page_size=32, q_counts=(3,), max_len=900, causal=False),
]


@pytest.mark.parametrize("i", range(len(MLA_CASES)))
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_f16_mla_parity(i, split_tokens):
    m = random_mla_batch(5500 + i, dtype="f16", **MLA_CASES[i])
    run = MlaRun(m, split_tokens=split_tokens)
    run()
    _check(run, *oracle.mla(m))


def test_f16_mla_window_one_returns_own_latent_bitwise():
    m = random_mla_batch(5600, dtype="f16", page_size=64, q_counts=(1, 1, 2), max_len=1500, window=1)
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


def test_f16_append_then_attend():
    """f16 rows appended bit for bit (whole pools against the oracle's loop),
    then a one-key-window forward call returns each query's new V row."""
    import torch
    b = random_batch(5700, dtype="f16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 2, 130),
                     max_len=2000, window=1)
    rng = np.random.default_rng(5701)
    k_new = f32_to_f16_bits(rng.standard_normal((b.num_queries, b.hkv, b.d)).astype(np.float32))
    v_new = f32_to_f16_bits(rng.standard_normal((b.num_queries, b.hkv, b.dv)).astype(np.float32))
    run = GqaRun(b)
    pa.pa_append_kv(run.plan, to_torch(k_new, "f16"), to_torch(v_new, "f16"), run.k, run.v)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.append_kv(b.seq_lens, b.cu_q, b.q_pos, b.block_table, b.page_size, k_new, v_new, b.k, b.v)
    assert np.array_equal(run.k.view(torch.int16).cpu().numpy().view(np.uint16), ref_k)
    assert np.array_equal(run.v.view(torch.int16).cpu().numpy().view(np.uint16), ref_v)
    run()
    out, _ = run.result()
    G = b.hq // b.hkv
    assert np.array_equal(out, widen(v_new, "f16")[:, np.arange(b.hq) // G])


def test_f16_mismatched_tensor_type_is_refused():
    """An f16 call within the f16 bar; the same call with a bf16 view of the
    K pool is refused by the binding before reaching the library."""
    import torch
    b = random_batch(5800, dtype="f16", hq=16, hkv=4, d=64, page_size=16, q_counts=(1, 9), max_len=600)
    run = GqaRun(b)
    run()
    _check(run, *oracle.attention(b))
    with pytest.raises(ValueError):
        pa.pa_attention_fwd(run.plan, run.q, run.k.view(torch.bfloat16), run.v, run.out, run.lse, scale=b.scale,
                            workspace=run.workspace)
