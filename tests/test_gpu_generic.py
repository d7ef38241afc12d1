"""GPU parity of the vector-ALU forward that runs every GQA shape the
specialised kernels do not take (ruDNN `execute_attention_into` admits any
Hq % Hkv == 0 and head sizes up to 1024): group sizes 9, 20, 32, 48 and 71
(heads of one KV head in groups of 16, the last one partial), head sizes 80,
96, 512 and 1024, Dv != D, in f32, bf16 and f16, decode rows and prefill
chunks, split and unsplit, against the fp64 oracle; the output and lse
start as NaN so that every element must be written.  The backward of the
shapes without a specialised backward kernel runs on vector kernels too
(group sizes 3, 5, 6, 7, 32, head sizes 80 / 48, 96, 512, MLA in f32 and at
other widths), checked against the oracle's backward."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import random_batch
from tests.gpu_harness import GqaRun, assert_close

pytestmark = pytest.mark.gpu

CASES = [
    dict(dtype="bf16", hq=32, hkv=1, d=128, page_size=16, q_counts=(1, 1, 9), max_len=1200),        # MQA, G = 32
    dict(dtype="bf16", hq=72, hkv=8, d=128, page_size=16, q_counts=(1, 40), max_len=700),           # G = 9
    dict(dtype="f16", hq=71, hkv=1, d=64, page_size=64, q_counts=(2, 1), max_len=900, window=300),  # G = 71
    dict(dtype="f32", hq=40, hkv=2, d=128, page_size=32, q_counts=(1, 5), max_len=600, causal=False),  # G = 20
    dict(dtype="bf16", hq=16, hkv=4, d=96, page_size=16, q_counts=(1, 1, 20), max_len=900),         # D = 96
    dict(dtype="f16", hq=8, hkv=8, d=80, dv=48, page_size=1, q_counts=(3, 1), max_len=120),         # D 80, Dv 48
    dict(dtype="f32", hq=32, hkv=8, d=512, page_size=64, q_counts=(1, 7), max_len=500),             # D = 512
    dict(dtype="bf16", hq=48, hkv=1, d=1024, page_size=16, q_counts=(1, 1), max_len=300),           # D = 1024, G = 48
]


@pytest.mark.parametrize("split_tokens", [0, 64])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_generic_shapes_parity(i, split_tokens):
    b = random_batch(5100 + i, **CASES[i])
    run = GqaRun(b, split_tokens=split_tokens)
    run.out.fill_(float("nan"))
    run.lse.fill_(float("nan"))
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.attention(b)
    assert_close(out, ref_o, b.dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-4 if b.dtype == "f32" else 1e-3)


def test_group_size_32_decode_batch_balanced():
    """An MQA decode batch with 32 query heads per KV head on the balanced
    planner (rows cut into pieces, merges): every row against the oracle."""
    b = random_batch(5200, dtype="bf16", hq=32, hkv=1, d=128, page_size=16, q_counts=(1,) * 24, max_len=6000)
    run = GqaRun(b)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.attention(b)
    assert_close(out, ref_o, "bf16")
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)
    assert run.info["split_rows"] > 0




# ---------------------------------------------------------------------------
# The vector-ALU backward (shapes without a specialised backward kernel)
# ---------------------------------------------------------------------------
from tests.test_gpu_backward import _parity as _bwd_parity  # noqa: E402
from tests.test_gpu_mla_backward import _parity as _mla_bwd_parity  # noqa: E402
from synth import random_mla_batch, with_shared_pages  # noqa: E402

BWD_CASES = [
    dict(dtype="bf16", hq=28, hkv=4, d=128, page_size=16, q_counts=(1, 20, 1), max_len=300),        # G = 7
    dict(dtype="f16", hq=40, hkv=8, d=64, page_size=64, q_counts=(9, 1), max_len=250, window=100),  # G = 5
    dict(dtype="bf16", hq=32, hkv=1, d=128, page_size=16, q_counts=(1, 6), max_len=200),            # G = 32
    dict(dtype="f32", hq=20, hkv=1, d=80, dv=48, page_size=8, q_counts=(3, 1), max_len=150, causal=False),
    dict(dtype="bf16", hq=12, hkv=4, d=96, page_size=1, q_counts=(5,), max_len=60),                 # G = 3, D 96
    dict(dtype="f32", hq=8, hkv=2, d=512, page_size=32, q_counts=(1, 4), max_len=120),              # D 512
]


@pytest.mark.parametrize("i", range(len(BWD_CASES)))
def test_generic_backward_parity(i):
    """dq and the whole dk / dv pools of shapes without a specialised backward
    kernel against the oracle's backward (the pools start as NaN, rows no
    visible key lands on -- whole dV rows of zero in the oracle -- must come
    out zero; a dK element may be zero in the oracle by cancellation alone,
    e.g. a query that sees only its own key, and is then held to the bar)."""
    b = random_batch(5400 + i, **BWD_CASES[i])
    run, got, ref = _bwd_parity(b, 5450 + i)
    unref = np.all(ref[2] == 0, axis=-1)
    assert unref.any()
    for g in (got[1], got[2]):
        assert np.array_equal(g[unref], np.zeros_like(g[unref]))


def test_generic_backward_shared_pages():
    """Two sequences reading one prefix (shared pages): the dK/dV items add
    into f32 sums, G = 6."""
    b = random_batch(5500, dtype="bf16", hq=12, hkv=2, d=64, page_size=16, q_counts=(3, 2), histories=[100, 120])
    b = with_shared_pages(b, [(1, 0, 0, 0), (1, 1, 0, 1)])
    _bwd_parity(b, 5501)


MLA_BWD_CASES = [
    dict(dtype="f32", heads=16, q_counts=(1, 6), max_len=200),                     # f32, the MFMA widths
    dict(dtype="bf16", heads=20, r=256, p=32, page_size=16, q_counts=(7, 1), max_len=150),
    dict(dtype="f16", heads=4, r=100, p=7, page_size=1, q_counts=(2, 1), max_len=60, causal=False),
]


@pytest.mark.parametrize("i", range(len(MLA_BWD_CASES)))
def test_generic_mla_backward_parity(i):
    """MLA backward of f32 data and other latent / rotary widths: dq_abs,
    dq_rope and the whole latent and rotary gradient pools."""
    kw = dict(MLA_BWD_CASES[i])
    kw.setdefault("page_size", 64)
    m = random_mla_batch(5600 + i, **kw)
    _mla_bwd_parity(m, 5650 + i)
