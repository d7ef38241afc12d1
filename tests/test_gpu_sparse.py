"""GPU parity of block-sparse top-k attention (alice-llm 2.0.0,
sparse_attention/llama3_bridge.rs, `llama3_sparse_attention`) through the C
ABI: the kept blocks must equal the oracle's bit for bit (the proxy scores
are f32 sums in a fixed order on both sides), and the outputs must match the
fp64 oracle's attention over those blocks within the data type's bar."""
import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import config_bf16_decode_batch, random_batch
from tests.gpu_harness import assert_close, make_plan, to_f64, to_torch, torch_dtype

pytestmark = pytest.mark.gpu


def run_sparse(b, block, topk):
    import torch
    q, k, v = to_torch(b.q, b.dtype), to_torch(b.k, b.dtype), to_torch(b.v, b.dtype)
    plan = make_plan(b)
    nbytes, width = pa.pa_sparse_workspace_bytes(plan, b.dv, block, topk)
    ws = torch.empty(max(nbytes, 4) // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.empty((b.num_queries, b.hq, b.dv), dtype=torch_dtype(b.dtype), device="cuda")
    lse = torch.empty((b.num_queries, b.hq), dtype=torch.float32, device="cuda")
    sel = torch.full((b.num_queries, b.hkv, width), -7, dtype=torch.int32, device="cuda")
    pa.pa_sparse_attention_fwd(plan, q, k, v, out, lse, scale=b.scale, block_size=block, topk=topk, selection=sel,
                               workspace=ws)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64), sel.cpu().numpy()


def check(b, block, topk):
    out, lse, sel = run_sparse(b, block, topk)
    ref_sel = oracle.sparse_select(b, block, topk)
    assert sel.shape == ref_sel.shape
    bad = np.argwhere(sel != ref_sel)
    assert bad.size == 0, f"selection differs at {bad[:5].tolist()}: gpu {sel[tuple(bad[0])]}, oracle {ref_sel[tuple(bad[0])]}"
    ref_o, ref_l = oracle.sparse_attention(b, ref_sel, block)
    assert_close(out, ref_o, b.dtype)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3 if b.dtype != "f32" else 1e-4)
    return sel


CASES = [
    dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1, 2), max_len=5000),
    dict(dtype="bf16", hq=64, hkv=8, d=128, page_size=64, q_counts=(1, 40, 1), max_len=3000, window=900),
    dict(dtype="f16", hq=16, hkv=4, d=64, page_size=16, q_counts=(3, 1, 1), max_len=2500, causal=False),
    dict(dtype="f32", hq=8, hkv=2, d=64, page_size=16, q_counts=(1, 1), max_len=2000),
    dict(dtype="bf16", hq=28, hkv=4, d=128, page_size=32, q_counts=(1, 2, 1), max_len=4000),    # G = 7
    dict(dtype="bf16", hq=8, hkv=1, d=256, page_size=16, q_counts=(1, 1), max_len=1500),
    dict(dtype="bf16", hq=16, hkv=2, d=192, dv=128, page_size=16, q_counts=(1, 1, 1), max_len=1800),
]


@pytest.mark.parametrize("i", range(len(CASES)))
# 48: a block size that is no power of two (per-key block maxima); 2048:
# blocks wider than one scoring span of 1024 keys (the span is the block)
@pytest.mark.parametrize("block,topk", [(64, 4), (16, 1), (128, 3), (48, 5), (2048, 1)])
def test_sparse_selection_bit_exact_and_output_parity(i, block, topk):
    b = random_batch(9300 + i, **CASES[i])
    if block % b.page_size:
        pytest.skip("block size must be a multiple of the page size")
    check(b, block, topk)


@pytest.mark.parametrize("i", [0, 1, 2])
def test_topk_zero_and_large_topk_keep_every_block(i):
    """topk = 0 and topk beyond every row's candidates keep all blocks: the
    result is dense attention (the page's dense-fallback parity), within the
    bar of the dense oracle."""
    b = random_batch(9400 + i, **CASES[i])
    ref_o, ref_l = oracle.attention(b)
    for topk in (0, 10000):
        out, lse, sel = run_sparse(b, 64, topk)
        assert_close(out, ref_o, b.dtype)
        np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-3)
        assert np.array_equal(sel[:, :, :oracle.sparse_select(b, 64, 0).shape[2]],
                              oracle.sparse_select(b, 64, 0)) if topk == 0 else True


def test_decode_batch_workload_top16_of_64_key_blocks():
    """The bf16 decode-batch workload (32 sequences of 512..8192 keys, Hq 32,
    Hkv 8, D 128, 16-key pages) keeping 16 blocks of 64 keys per (query, KV
    head): every selection bit-exact, every output row within the bar."""
    b = config_bf16_decode_batch()
    sel = check(b, 64, 16)
    kept = (sel >= 0).sum(axis=2)
    cand = np.array([-(-int(L) // 64) for L in b.seq_lens])  # decode rows see their whole context
    assert np.array_equal(kept, np.minimum(cand, 16)[:, None].repeat(b.hkv, axis=1))


def test_bad_block_size_is_refused():
    b = random_batch(9500, dtype="bf16", hq=8, hkv=2, d=64, page_size=16, q_counts=(1,), max_len=300)
    plan = make_plan(b)
    with pytest.raises(pa.PaError) as e:
        pa.pa_sparse_workspace_bytes(plan, b.dv, 24, 2)
    assert e.value.name == "PA_ERR_SHAPE"
