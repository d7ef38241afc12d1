"""GPU parity of the split-KV decode path (HIP kernels through the C ABI)
against the fp64 oracle, plus bitwise properties."""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import config_bf16_decode_batch, config_tiny_f32_decode, random_batch
from tests.gpu_harness import GqaRun, assert_close, to_f64

pytestmark = pytest.mark.gpu


def _parity(b, **kw):
    run = GqaRun(b, **kw)
    run()
    out, lse = run.result()
    ref_o, ref_l = oracle.attention(b)
    assert_close(out, ref_o, b.dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3 if b.dtype == "bf16" else 1e-4)
    return run


@pytest.mark.parametrize("max_splits,split_tokens", [(16, 0), (1, 0), (16, 64)])
def test_tiny_f32_decode_nan_pool(max_splits, split_tokens):
    b = config_tiny_f32_decode()
    run = _parity(b, max_splits=max_splits, split_tokens=split_tokens)
    if split_tokens:
        assert run.info["split_rows"] == 1 and run.info["launches"] == 2


DECODE_CASES = [
    dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1, 2, 1), max_len=3000),
    dict(dtype="bf16", hq=64, hkv=8, d=128, page_size=64, q_counts=(1, 1, 3), max_len=5000, window=700),
    dict(dtype="bf16", hq=16, hkv=16, d=128, page_size=16, q_counts=(1, 4), max_len=900),
    dict(dtype="bf16", hq=16, hkv=1, d=128, page_size=16, q_counts=(1, 1), max_len=2100),
    dict(dtype="bf16", hq=8, hkv=4, d=64, page_size=32, q_counts=(1, 2, 1), max_len=1500, causal=False),
    dict(dtype="bf16", hq=8, hkv=1, d=256, page_size=16, q_counts=(1, 1), max_len=1200, window=33),
    dict(dtype="f32", hq=4, hkv=1, d=64, page_size=16, q_counts=(1, 1, 1), max_len=2000),
    dict(dtype="f32", hq=16, hkv=2, d=128, page_size=64, q_counts=(1, 3), max_len=1800, causal=False, window=100),
    dict(dtype="f32", hq=2, hkv=1, d=256, page_size=16, q_counts=(2,), max_len=700),
    dict(dtype="bf16", hq=4, hkv=2, d=128, page_size=1, q_counts=(1, 1), max_len=300),
    dict(dtype="bf16", hq=8, hkv=2, d=128, page_size=16, q_counts=(1, 1, 1), histories=[0, 1, 2]),
    # KV head counts that are not powers of two: items of two heads (Hkv = 6)
    # and of one head (Hkv = 3)
    dict(dtype="bf16", hq=12, hkv=6, d=128, page_size=16, q_counts=(1, 1, 1), max_len=2500),
    dict(dtype="bf16", hq=24, hkv=3, d=64, page_size=32, q_counts=(1, 2), max_len=1800),
]


@pytest.mark.parametrize("i", range(len(DECODE_CASES)))
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_random_decode_parity(i, split_tokens):
    b = random_batch(1000 + i, **DECODE_CASES[i])
    _parity(b, split_tokens=split_tokens)


def test_bf16_decode_batch_full_size_all_rows():
    b = config_bf16_decode_batch()
    run = _parity(b)
    assert run.info["decode_items"] > 256 and run.info["split_rows"] > 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_one_returns_own_value_bitwise(dtype):
    b = random_batch(31, dtype=dtype, hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 2, 1), max_len=2000,
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


def test_page_permutation_is_bitwise_invariant_and_runs_are_deterministic():
    b = random_batch(32, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1), max_len=3000,
                     window=1500)
    r1 = GqaRun(b)
    r1()
    o1, l1 = r1.result()
    r1()
    o1b, l1b = r1.result()
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    rng = np.random.default_rng(5)
    extra = 7
    perm = rng.permutation(b.num_pages + extra)
    k2 = np.full((b.num_pages + extra,) + b.k.shape[1:], 0x7FC0, dtype=np.uint16)
    v2 = np.full((b.num_pages + extra,) + b.v.shape[1:], 0x7FC0, dtype=np.uint16)
    k2[perm[:b.num_pages]] = b.k
    v2[perm[:b.num_pages]] = b.v
    bt2 = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1).astype(np.int32)
    b2 = dataclasses.replace(b, k=k2, v=v2, block_table=bt2, num_pages=b.num_pages + extra)
    r2 = GqaRun(b2)
    r2()
    o2, l2 = r2.result()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_constant_values_give_that_constant():
    b = random_batch(33, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1), max_len=2500,
                     poison=False)
    b = dataclasses.replace(b, v=np.full_like(b.v, 0x3F20))  # bf16 0.625
    run = GqaRun(b)
    run()
    out, _ = run.result()
    assert np.abs(out - 0.625).max() <= 2e-2 + 1e-2 * 0.625


@pytest.mark.parametrize("max_splits,page_size", [(1, 16), (1, 64), (16, 16)])
def test_long_rows_span_several_page_windows(max_splits, page_size):
    """Rows of ~20k keys: unsplit, each wave of the workgroup walks > 64
    blocks (several windows of preloaded page numbers) and ends on a partial
    block; split, the pieces start and end inside pages."""
    b = random_batch(41, dtype="bf16", hq=8, hkv=2, d=128, page_size=page_size, q_counts=(1, 1, 1),
                     histories=[20000, 16385, 4095], max_splits=max_splits)
    run = _parity(b)
    if max_splits == 1:
        assert run.info["split_rows"] == 0


def test_windowed_long_row_starts_mid_page():
    """A sliding window makes each row start at an arbitrary key: the first
    block of every piece straddles the window start."""
    b = random_batch(42, dtype="bf16", hq=16, hkv=4, d=128, page_size=16, q_counts=(1, 2),
                     histories=[12345, 9999], window=7001)
    _parity(b)


def test_sequences_without_queries():
    """Sequences with no queries (one of them with no keys either) between
    decode rows and a three-query chunk."""
    b = random_batch(50, dtype="bf16", hq=8, hkv=2, d=128, page_size=16, q_counts=(0, 1, 0, 3),
                     histories=[5, 300, 0, 40])
    _parity(b)


def test_batch_without_queries_launches_nothing():
    import torch
    b = random_batch(51, dtype="bf16", hq=8, hkv=2, d=128, page_size=16, q_counts=(0, 0), histories=[5, 0])
    run = GqaRun(b)
    assert run.info["launches"] == 0 and run.info["workgroups"] == 0
    run()
    torch.cuda.synchronize()
    assert run.out.numel() == 0


@pytest.mark.parametrize("hq,hkv,max_splits", [(8, 1, 64), (32, 2, 64), (32, 8, 1)])
def test_128k_key_row(hq, hkv, max_splits):
    """One decode row over 131072 keys (8192 pages): split up to the 64-piece
    limit, or walked unsplit by one workgroup per head group."""
    b = random_batch(52, dtype="bf16", hq=hq, hkv=hkv, d=128, page_size=16, q_counts=(1,), histories=[131071],
                     max_splits=max_splits)
    run = _parity(b)
    assert (run.info["split_rows"] > 0) == (max_splits > 1)


def test_plan_is_bound_to_its_stream_and_freed_in_stream_order():
    """A plan works on the stream it was made on and is refused on another
    (PA_ERR_DEVICE, before any launch); destroying it right after a call on
    its stream leaves that call's result intact (the free is ordered after
    the kernels that read the plan)."""
    import torch
    import paged_kv_attention_gqa_amd as pa
    from tests.gpu_harness import make_plan
    b = random_batch(1900, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1), max_len=3000)
    run = GqaRun(b, split_tokens=256)
    torch.cuda.synchronize()  # inputs were copied on the default stream
    side = torch.cuda.Stream()
    with pytest.raises(pa.PaError) as e:
        pa.pa_attention_fwd(run.plan, run.q, run.k, run.v, run.out, run.lse, scale=b.scale,
                            workspace=run.workspace, stream=side)
    assert e.value.name == "PA_ERR_DEVICE"
    # a plan made on the side stream runs there; it is destroyed before the
    # stream has finished the call
    with torch.cuda.stream(side):
        plan = make_plan(b, split_tokens=256, stream=side)
        pa.pa_attention_fwd(plan, run.q, run.k, run.v, run.out, run.lse, scale=b.scale, workspace=run.workspace,
                            stream=side)
        pa.pa_plan_destroy(plan)
    side.synchronize()
    out, lse = to_f64(run.out), run.lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle.attention(b)
    assert_close(out, ref_o, "bf16")
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)


def test_main_kernel_timing_events():
    """main_events receive the main kernel's own start and end: the interval
    is positive and no longer than the whole call measured around it."""
    import torch
    b = config_bf16_decode_batch()
    run = GqaRun(b)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outer0, outer1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for ev in (start, end):
        ev.record()
    torch.cuda.synchronize()
    outer0.record()
    run(main_events=(start, end))
    outer1.record()
    torch.cuda.synchronize()
    k_ms, call_ms = start.elapsed_time(end), outer0.elapsed_time(outer1)
    assert 0 < k_ms <= call_ms, (k_ms, call_ms)
    out, _ = run.result()
    assert_close(out, oracle.attention(b)[0], "bf16")
