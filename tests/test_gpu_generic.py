"""GPU parity of the vector-ALU forward that runs every GQA shape the
specialised kernels do not take (ruDNN `execute_attention_into` admits any
Hq % Hkv == 0 and head sizes up to 1024): group sizes 9, 20, 32, 48 and 71
(heads of one KV head in groups of 16, the last one partial), head sizes 80,
96, 512 and 1024, Dv != D, in f32, bf16 and f16, decode rows and prefill
chunks, split and unsplit, against the fp64 oracle; the output and lse
start as NaN so that every element must be written."""
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


def test_backward_of_a_group_size_without_kernel_is_refused():
    """The backward runs group sizes 1, 2, 4, 8 and 16: G = 32 is refused
    before anything is launched."""
    b = random_batch(5300, dtype="bf16", hq=32, hkv=1, d=128, page_size=16, q_counts=(1, 3), max_len=100)
    run = GqaRun(b)
    run()
    z = torch.zeros_like(run.out)
    with pytest.raises(pa.PaError) as e:
        pa.pa_attention_bwd(run.plan, run.q, run.k, run.v, run.out, run.lse, z, torch.zeros_like(run.q),
                            torch.zeros_like(run.k), torch.zeros_like(run.v), scale=b.scale)
    assert e.value.name == "PA_ERR_UNSUPPORTED"
