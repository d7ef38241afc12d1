"""pa_attention_fwd_noalloc (split partials in the library's fixed per-GPU
device array, no allocation) against pa_attention_fwd with a caller
workspace: the same kernels, so the outputs must agree bit for bit, and both
within the bf16 bar of the fp64 oracle.  Two calls in a row, the second with
a smaller batch, share the array."""
import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import random_batch
from tests.gpu_harness import GqaRun, assert_close, to_f64


def _noalloc_matches_workspace_forward(b):
    import torch
    run = GqaRun(b, split_tokens=256)
    assert run.info["split_rows"] > 0, run.info  # the partials go through the array
    run()
    ref_out, ref_lse = run.out.clone(), run.lse.clone()
    out = torch.full_like(run.out, float("nan"))
    lse = torch.full_like(run.lse, float("nan"))
    pa.pa_attention_fwd_noalloc(run.plan, run.q, run.k, run.v, out, lse, scale=b.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    o64, l64 = to_f64(out), lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle.attention(b)
    assert_close(o64, ref_o, b.dtype)
    np.testing.assert_allclose(l64, ref_l, rtol=0, atol=1e-3)


@pytest.mark.gpu
def test_noalloc_forward_two_calls_second_smaller():
    big = random_batch(9100, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1, 1, 1, 1, 60),
                       max_len=6000)
    small = random_batch(9101, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1), max_len=1500)
    _noalloc_matches_workspace_forward(big)
    _noalloc_matches_workspace_forward(small)


@pytest.mark.gpu
def test_noalloc_forward_without_split_rows():
    """A plan that splits nothing uses no part of the array."""
    import torch
    b = random_batch(9102, dtype="bf16", hq=16, hkv=4, d=64, page_size=16, q_counts=(1, 30), max_len=400,
                     max_splits=1)
    run = GqaRun(b, max_splits=1)
    assert run.info["split_rows"] == 0
    run()
    out = torch.empty_like(run.out)
    pa.pa_attention_fwd_noalloc(run.plan, run.q, run.k, run.v, out, None, scale=b.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), run.out.view(torch.int16))


def test_noalloc_refuses_plans_beyond_the_array():
    """A plan whose split partials exceed the array is refused before
    anything is launched (host-only plan: no GPU needed)."""
    lib = pa.load_library()
    S, L, ps = 64, 32768, 64
    seq_lens = np.full(S, L, np.int32)
    cu_q = np.arange(S + 1, dtype=np.int32)
    q_pos = seq_lens - 1
    bt = np.arange(S * (L // ps), dtype=np.int32).reshape(S, L // ps)
    plan = pa.pa_plan_create_host(seq_lens, cu_q, q_pos, bt, num_cus=256, page_size=ps, num_pages=S * (L // ps),
                                  num_q_heads=64, num_kv_heads=8, max_splits=64, split_tokens=64)
    need = pa.pa_plan_workspace_bytes(plan, 128)
    scratch = 32 << 20
    assert need > scratch
    rc = lib.pa_attention_fwd_noalloc(plan.handle, pa._binding.PA_BF16, None, None, None, None, None, 128, 128,
                                      ctypes.c_float(0.088), None)
    assert rc == -5, (rc, pa.pa_last_error())  # PA_ERR_WORKSPACE
    assert str(need) in pa.pa_last_error()
