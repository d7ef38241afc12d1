"""GPU parity of the paged K/V append (HIP kernel through the C ABI) against
the oracle's loop: the whole pools after the append must match bit for bit,
including every row no query names (NaN-poisoned pages included)."""
import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import f32_to_bf16_bits, random_batch, random_mla_batch
from tests.dense_view import widen
from tests.gpu_harness import GqaRun, make_plan, to_torch

pytestmark = pytest.mark.gpu


def _new_rows(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _append_and_compare(b, k_pool, v_pool, k_new, v_new, dtype, mla=False):
    import torch
    plan = make_plan(b, mla=mla)
    dk, dv = to_torch(k_pool, dtype), to_torch(v_pool, dtype)
    kn, vn = to_torch(k_new, dtype), to_torch(v_new, dtype)
    pa.pa_append_kv(plan, kn, vn, dk, dv)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.append_kv(b.seq_lens, b.cu_q, b.q_pos, b.block_table, b.page_size, k_new, v_new,
                                    k_pool, v_pool)
    as_bits = (lambda t: t.view(torch.int32) if dtype == "f32" else t.view(torch.int16))
    got_k, got_v = as_bits(dk).cpu().numpy(), as_bits(dv).cpu().numpy()
    want_k, want_v = ref_k.view(got_k.dtype), ref_v.view(got_v.dtype)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


CASES = [
    dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1, 1), max_len=3000),
    dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(300, 0, 1, 77), max_len=900),
    dict(dtype="bf16", hq=16, hkv=1, d=256, page_size=64, q_counts=(5, 130), max_len=2000),
    dict(dtype="f32", hq=8, hkv=2, d=64, page_size=1, q_counts=(3, 1, 20), max_len=300),
    dict(dtype="bf16", hq=8, hkv=4, d=64, page_size=32, q_counts=(65, 66), histories=[0, 31]),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_append_matches_oracle_bitwise(i):
    c = CASES[i]
    b = random_batch(4000 + i, **c)
    rng = np.random.default_rng(4100 + i)
    k_new = _new_rows(rng, (b.num_queries, b.hkv, b.d), c["dtype"])
    v_new = _new_rows(rng, (b.num_queries, b.hkv, b.dv), c["dtype"])
    _append_and_compare(b, b.k, b.v, k_new, v_new, c["dtype"])


def test_mla_latent_and_rotary_append():
    """MLA plans: one shared head, latent rows (512) and rotary rows (64)."""
    m = random_mla_batch(4200, page_size=64, q_counts=(1, 1, 7), max_len=3000)
    rng = np.random.default_rng(4201)
    lat_new = _new_rows(rng, (m.num_queries, 1, m.r), "bf16")
    pos_new = _new_rows(rng, (m.num_queries, 1, m.p), "bf16")
    _append_and_compare(m, m.latent, m.kpos, lat_new, pos_new, "bf16", mla=True)


def test_append_then_attend_reads_the_new_rows():
    """Append, then a one-key-window forward call: every output row is the
    query's own new V row, bit for bit (the append and the attention gather
    agree on where a position lives)."""
    b = random_batch(4300, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 2, 130),
                     max_len=2000, window=1)
    rng = np.random.default_rng(4301)
    k_new = _new_rows(rng, (b.num_queries, b.hkv, b.d), "bf16")
    v_new = _new_rows(rng, (b.num_queries, b.hkv, b.dv), "bf16")
    run = GqaRun(b)
    pa.pa_append_kv(run.plan, to_torch(k_new, "bf16"), to_torch(v_new, "bf16"), run.k, run.v)
    run()
    out, _ = run.result()
    G = b.hq // b.hkv
    assert np.array_equal(out, widen(v_new, "bf16")[:, np.arange(b.hq) // G])


def test_duplicate_slots_are_rejected_before_any_launch():
    import torch
    b = random_batch(4400, dtype="bf16", hq=8, hkv=2, d=64, page_size=16, q_counts=(2,), histories=[10])
    q_pos = b.q_pos.copy()
    q_pos[1] = q_pos[0]  # two queries naming one position
    plan = pa.pa_plan_create(b.seq_lens, b.cu_q, q_pos, b.block_table, page_size=b.page_size,
                             num_pages=b.num_pages, num_q_heads=b.hq, num_kv_heads=b.hkv)
    k, v = to_torch(b.k, "bf16"), to_torch(b.v, "bf16")
    kn = torch.zeros((2, b.hkv, b.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_append_kv(plan, kn, kn.clone(), k, v)
    assert e.value.status == -3
