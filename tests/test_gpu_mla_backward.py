"""GPU parity of the absorbed-MLA backward (pa_mla_bwd through the C ABI)
against the fp64 oracle's MLA backward (ruDNN `mla_backward`; the latent
gradient holds the key and the value terms), after the GPU forward.

Bar: the forward's per-dtype bar on dq_abs, dq_rope and the whole latent and
rotary gradient pools (f32 1e-4 + 1e-4 |ref| as the GQA backward's, bf16
2e-2 + 1e-2 |ref|, f16 2.5e-3 + 1.25e-3 |ref|);
pool rows no visible key lands on must be exactly zero."""
import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import f32_to_bf16_bits, f32_to_f16_bits, random_mla_batch, with_shared_pages
from tests.gpu_harness import MlaRun, to_f64, to_torch, torch_dtype

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2), "f16": (2.5e-3, 1.25e-3)}


def _dout(m, seed):
    x = np.random.default_rng(seed).standard_normal((m.num_queries, m.heads, m.r)).astype(np.float32)
    return x if m.dtype == "f32" else (f32_to_bf16_bits(x) if m.dtype == "bf16" else f32_to_f16_bits(x))


class MlaBwdRun:
    def __init__(self, m, dout):
        import torch
        self.fwd = MlaRun(m)
        self.fwd()
        self.m = m
        self.dout = to_torch(dout, m.dtype)
        dt = torch_dtype(m.dtype)
        self.dqa = torch.empty((m.num_queries, m.heads, m.r), dtype=dt, device="cuda")
        self.dqr = torch.empty((m.num_queries, m.heads, m.p), dtype=dt, device="cuda")
        self.dlat = torch.full_like(self.fwd.latent, float("nan"))  # every element must be written
        self.dkp = torch.full_like(self.fwd.kpos, float("nan"))
        n = pa.pa_plan_bwd_workspace_bytes(self.fwd.plan, m.dtype, m.r, m.p)
        self.ws = torch.empty(max(n, 4) // 4 + 64, dtype=torch.float32, device="cuda") if n else None

    def __call__(self):
        f = self.fwd
        pa.pa_mla_bwd(f.plan, f.q_abs, f.q_rope, f.latent, f.kpos, f.out, f.lse, self.dout, self.dqa, self.dqr,
                      self.dlat, self.dkp, scale=self.m.scale, workspace=self.ws)

    def result(self):
        import torch
        torch.cuda.synchronize()
        return to_f64(self.dqa), to_f64(self.dqr), to_f64(self.dlat), to_f64(self.dkp)


def _close(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside {atol} + {rtol}|ref|, max err "
                           f"{np.nanmax(err):.3g}, first {np.argwhere(bad)[:3].tolist()}")


def _parity(m, seed):
    dout = _dout(m, seed)
    run = MlaBwdRun(m, dout)
    run()
    got = run.result()
    ref = oracle.mla_bwd(m, dout)
    for g, r, what in zip(got, ref, ("dq_abs", "dq_rope", "dlatent", "dkpos")):
        _close(g, r, m.dtype, what)
    return run, got, ref


CASES = [
    dict(page_size=64, q_counts=(1, 1, 1), max_len=900),                              # decode rows
    dict(page_size=16, q_counts=(1, 40, 2), max_len=600),                             # a chunk beside decode rows
    dict(page_size=64, q_counts=(20, 1), max_len=700, window=100),
    dict(page_size=32, q_counts=(9, 1), max_len=500, causal=False),
    dict(page_size=1, q_counts=(7,), max_len=80),
    dict(page_size=64, q_counts=(0, 12, 0, 1, 3), histories=[50, 300, 0, 20, 90]),   # sequences without queries
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_mla_backward_parity(i, dtype):
    m = random_mla_batch(9600 + i, dtype=dtype, **CASES[i])
    run, got, _ = _parity(m, 9700 + i)
    # single writer per pool row: a second call repeats every bit
    run()
    again = run.result()
    for g, h in zip(got, again):
        assert np.array_equal(g, h, equal_nan=True)


@pytest.mark.parametrize("heads,kw", [
    (32, dict(page_size=64, q_counts=(1, 20, 1), max_len=600)),
    (20, dict(page_size=16, q_counts=(9, 1), max_len=500, window=100)),
    (1, dict(page_size=64, q_counts=(1, 3), max_len=300)),
])
def test_mla_backward_head_counts(heads, kw):
    """Head counts other than 16: dQ items per group of 16 heads, and every
    dK/dV block item summing all head groups of its queries."""
    m = random_mla_batch(9900 + heads, heads=heads, dtype="bf16", **kw)
    _parity(m, 9950 + heads)


def test_mla_backward_unreferenced_rows_are_zero():
    """Pool rows that no visible key of any query lands on (extra pages, tail
    slots, keys before a window) get gradient exactly zero."""
    m = random_mla_batch(9800, dtype="bf16", page_size=16, q_counts=(1, 5), max_len=400, window=50)
    run, got, ref = _parity(m, 9801)
    for g, r in ((got[2], ref[2]), (got[3], ref[3])):
        assert np.array_equal(g[r == 0], r[r == 0])


def test_mla_backward_shared_pages():
    """Two sequences reading one prefix page: that page's gradients are
    summed over both readers (f32 sums in the workspace)."""
    m = random_mla_batch(9900, dtype="bf16", page_size=16, q_counts=(3, 2), histories=[40, 60])
    m2 = with_shared_pages(m, [(1, 0, 0, 0)])
    run, _, _ = _parity(m2, 9901)
    assert run.fwd.info["bwd_shared_pages"] == 1


def test_gqa_plan_is_refused_by_mla_backward():
    from synth import random_batch
    from tests.gpu_harness import GqaRun
    b = random_batch(9950, dtype="bf16", hq=16, hkv=1, d=128, page_size=16, q_counts=(1,), max_len=100)
    f = GqaRun(b)
    with pytest.raises(pa.PaError) as e:
        pa.pa_mla_bwd(f.plan, f.q, f.q, f.k, f.k, f.out, f.lse, f.out, f.q, f.q, f.k, f.k, scale=b.scale)
    assert e.value.name == "PA_ERR_INVALID"
