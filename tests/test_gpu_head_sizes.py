"""GPU parity for K and V rows of different widths (ruDNN paged_attention:
K [pages, page_size, Hkv, D], V [pages, page_size, Hkv, Dv], output
[queries, Hq, Dv]): D = 192 with Dv = 128, the shape of a 128-wide
no-position key part plus a 64-wide rotary part, and D = Dv = 256.  Decode
items, split merges and prefill tiles against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import random_batch
from tests.gpu_harness import GqaRun, assert_close, to_f64

pytestmark = pytest.mark.gpu


def _parity(b, **kw):
    run = GqaRun(b, **kw)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.attention(b)
    assert out.shape == ref_o.shape == (b.num_queries, b.hq, b.dv)
    assert_close(out, ref_o, b.dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-4 if b.dtype == "f32" else 1e-3)
    return run


CASES = [
    dict(dtype="bf16", hq=32, hkv=8, page_size=16, q_counts=(1, 1, 1, 2, 1), max_len=3000),
    dict(dtype="bf16", hq=128, hkv=128, page_size=64, q_counts=(1, 3), max_len=2000),
    dict(dtype="bf16", hq=16, hkv=1, page_size=16, q_counts=(1, 1), max_len=2100, window=300),
    dict(dtype="f16", hq=16, hkv=2, page_size=32, q_counts=(1, 2, 1), max_len=1500, causal=False),
    dict(dtype="f16", hq=8, hkv=8, page_size=1, q_counts=(1, 1), max_len=300),
    dict(dtype="f32", hq=8, hkv=2, page_size=16, q_counts=(1, 1, 1), max_len=1200),
    dict(dtype="f32", hq=16, hkv=1, page_size=64, q_counts=(2,), max_len=700, window=65),
]


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_d192_dv128_decode_parity(i, split_tokens):
    b = random_batch(6000 + i, d=192, dv=128, **CASES[i])
    _parity(b, split_tokens=split_tokens)


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", hq=32, hkv=8, page_size=16, q_counts=(40, 1, 9), max_len=400),
    dict(dtype="f16", hq=16, hkv=16, page_size=64, q_counts=(1, 70), max_len=500, window=33),
    dict(dtype="f32", hq=8, hkv=2, page_size=16, q_counts=(12, 1), max_len=200, causal=False),
    # 16-bit tiles on MFMA: MHA (G = 1) chunks over several 256-row tiles, G = 16, G = 8 with a
    # window, page size 1, non-causal, history 0
    dict(dtype="bf16", hq=16, hkv=16, page_size=16, q_counts=(600,), max_len=1000),
    dict(dtype="bf16", hq=16, hkv=1, page_size=64, q_counts=(65, 2), max_len=700),
    dict(dtype="f16", hq=64, hkv=8, page_size=16, q_counts=(100, 3), max_len=900, window=129),
    dict(dtype="bf16", hq=32, hkv=8, page_size=1, q_counts=(70,), max_len=200),
    dict(dtype="bf16", hq=8, hkv=2, page_size=32, q_counts=(150, 5), max_len=700, causal=False),
    dict(dtype="f16", hq=32, hkv=8, page_size=16, q_counts=(200,), histories=[0]),
])
def test_d192_dv128_prefill_and_mixed_parity(case):
    b = random_batch(6100, d=192, dv=128, **case)
    run = _parity(b)
    assert run.info["prefill_items"] > 0


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_d192_dv128_window_one_returns_own_value_bitwise(dtype):
    b = random_batch(6200, dtype=dtype, hq=32, hkv=8, d=192, dv=128, page_size=16, q_counts=(1, 1, 5, 1),
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


def test_d192_dv128_long_rows_split_to_the_limit():
    """Rows of 20-40k keys: every piece of every row merged (the merge reads
    Dv-wide partials)."""
    b = random_batch(6300, dtype="bf16", hq=16, hkv=2, d=192, dv=128, page_size=16, q_counts=(1, 1),
                     histories=[20000, 40000])
    run = _parity(b, max_splits=64)
    assert run.info["split_rows"] > 0


def test_d192_dv128_prefill_window_one_bitwise():
    """MFMA prefill tiles with a one-key window return each query's own V row."""
    b = random_batch(6500, dtype="bf16", hq=32, hkv=8, d=192, dv=128, page_size=16, q_counts=(150, 1, 40),
                     max_len=600, window=1)
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


@pytest.mark.parametrize("case", [
    # D = Dv = 256 on the 32x32x16 tile in two passes of 128 output dims:
    # several tiles and a ragged tail, MHA with a window, G = 8 and 16, page
    # size 1 (per-lane page lookups), non-causal, history 0, f16
    dict(dtype="bf16", hq=32, hkv=8, page_size=16, q_counts=(300, 1, 9), max_len=900),
    dict(dtype="f16", hq=16, hkv=16, page_size=64, q_counts=(1, 270), max_len=700, window=33),
    dict(dtype="bf16", hq=64, hkv=8, page_size=16, q_counts=(100, 3), max_len=800, window=129),
    dict(dtype="bf16", hq=16, hkv=1, page_size=32, q_counts=(65, 2), max_len=500),
    dict(dtype="bf16", hq=32, hkv=8, page_size=1, q_counts=(70,), max_len=200),
    dict(dtype="bf16", hq=8, hkv=2, page_size=32, q_counts=(150, 5), max_len=700, causal=False),
    dict(dtype="f16", hq=32, hkv=8, page_size=16, q_counts=(200,), histories=[0]),
])
def test_d256_prefill_and_mixed_parity(case):
    b = random_batch(6600, d=256, **case)
    run = _parity(b)
    assert run.info["prefill_items"] > 0


@pytest.mark.timeout(900)
def test_d256_chunked_prefill_full_size_every_row():
    """The D = Dv = 256 chunked-prefill workload (8 sequences, 512-query
    chunks after 0..4096 cached keys, Hq 32, Hkv 8, page 16): every output
    element and every lse against the oracle."""
    from synth import config_bf16_chunked_prefill_d256
    b = config_bf16_chunked_prefill_d256()
    run = _parity(b)
    assert run.info["prefill_items"] > 0 and run.info["decode_items"] == 0


def test_d256_prefill_window_one_bitwise():
    """Both 128-dim passes of the D = 256 tiles return each query's own V
    row under a one-key window."""
    b = random_batch(6700, dtype="bf16", hq=32, hkv=8, d=256, page_size=16, q_counts=(150, 1, 40),
                     max_len=600, window=1)
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


def test_head_size_pairs_without_kernels_run_on_the_vector_kernel():
    """(D, Dv) = (128, 64) has no specialised kernel: the vector kernel runs
    it, decode rows and a chunk, against the oracle."""
    b = random_batch(6400, dtype="bf16", hq=8, hkv=2, d=128, dv=64, page_size=16, q_counts=(1, 1, 12), max_len=400)
    _parity(b)


def test_head_sizes_past_1024_are_refused():
    import torch
    b = random_batch(6401, dtype="bf16", hq=2, hkv=1, d=64, page_size=16, q_counts=(1,), max_len=50)
    run = GqaRun(b)
    q = torch.zeros((b.num_queries, b.hq, 1032), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(tuple(run.k.shape[:3]) + (1032,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_attention_fwd(run.plan, q, k, run.v, run.out, run.lse, scale=b.scale, workspace=run.workspace)
    assert e.value.name == "PA_ERR_SHAPE"
    torch.cuda.synchronize()
