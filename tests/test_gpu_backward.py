"""GPU parity of the paged GQA backward (pa_attention_bwd through the C ABI)
against the fp64 oracle's backward (ruDNN `attention_backward`; formulas of
boostr `standard_attention_bwd`).  The forward runs first on the GPU to give
the output and logsumexp the backward takes.

Bar: the forward's per-dtype bar on dq and on the whole gradient pools
(f32 |d| <= 1e-4 + 1e-4 |ref|, the gradients being sums of thousands of
terms; bf16 2e-2 + 1e-2 |ref|; f16 2.5e-3 + 1.25e-3 |ref|); pool rows no
visible key lands on must be exactly zero."""
import numpy as np
import pytest

import oracle
import paged_kv_attention_gqa_amd as pa
from synth import f32_to_bf16_bits, f32_to_f16_bits, random_batch, with_shared_pages
from tests.gpu_harness import GqaRun, make_plan, to_f64, to_torch, torch_dtype

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2), "f16": (2.5e-3, 1.25e-3)}


def _dout(b, seed):
    x = np.random.default_rng(seed).standard_normal((b.num_queries, b.hq, b.dv)).astype(np.float32)
    return x if b.dtype == "f32" else (f32_to_bf16_bits(x) if b.dtype == "bf16" else f32_to_f16_bits(x))


class BwdRun:
    def __init__(self, b, dout):
        import torch
        self.fwd = GqaRun(b)
        self.fwd()
        self.b = b
        self.dout = to_torch(dout, b.dtype)
        dt = torch_dtype(b.dtype)
        self.dq = torch.empty((b.num_queries, b.hq, b.d), dtype=dt, device="cuda")
        self.dk = torch.full_like(self.fwd.k, float("nan"))  # every element must be written
        self.dv = torch.full_like(self.fwd.v, float("nan"))
        n = pa.pa_plan_bwd_workspace_bytes(self.fwd.plan, b.dtype, b.d, b.dv)
        self.ws = torch.empty(max(n, 4) // 4 + 64, dtype=torch.float32, device="cuda") if n else None

    def __call__(self):
        f = self.fwd
        pa.pa_attention_bwd(f.plan, f.q, f.k, f.v, f.out, f.lse, self.dout, self.dq, self.dk, self.dv,
                            scale=self.b.scale, workspace=self.ws)

    def result(self):
        import torch
        torch.cuda.synchronize()
        return to_f64(self.dq), to_f64(self.dk), to_f64(self.dv)


def _close(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside {atol} + {rtol}|ref|, max err "
                           f"{np.nanmax(err):.3g}, first {np.argwhere(bad)[:3].tolist()}")


def _parity(b, seed):
    dout = _dout(b, seed)
    run = BwdRun(b, dout)
    run()
    dq, dk, dv = run.result()
    rq, rk, rv = oracle.attention_bwd(b, dout)
    _close(dq, rq, b.dtype, "dq")
    _close(dk, rk, b.dtype, "dk")
    _close(dv, rv, b.dtype, "dv")
    return run, (dq, dk, dv), (rq, rk, rv)


def _bits(t):
    import torch
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


CASES = [
    dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(1, 1, 1, 2, 1), max_len=1500),
    dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(100, 1, 37), max_len=400),
    dict(dtype="bf16", hq=64, hkv=8, d=128, page_size=64, q_counts=(1, 70, 1), max_len=900, window=257),
    dict(dtype="bf16", hq=16, hkv=16, d=64, page_size=32, q_counts=(40, 9), max_len=300, causal=False),
    dict(dtype="bf16", hq=16, hkv=1, d=128, page_size=1, q_counts=(12, 1), max_len=150),
    dict(dtype="f16", hq=8, hkv=2, d=256, page_size=16, q_counts=(20, 1), max_len=300, window=33),
    dict(dtype="f16", hq=32, hkv=8, d=192, dv=128, page_size=16, q_counts=(30, 2), max_len=500),
    dict(dtype="f32", hq=8, hkv=2, d=64, page_size=16, q_counts=(20, 1, 3), max_len=300),
    dict(dtype="f32", hq=16, hkv=4, d=128, page_size=64, q_counts=(9,), max_len=700, causal=False, window=100),
    dict(dtype="bf16", hq=8, hkv=2, d=128, page_size=16, q_counts=(0, 33, 0, 1), histories=[40, 100, 0, 5]),
    # 16-bit MFMA backward for the other head sizes
    dict(dtype="bf16", hq=16, hkv=16, d=192, dv=128, page_size=16, q_counts=(70, 1), max_len=400),
    dict(dtype="bf16", hq=8, hkv=2, d=256, page_size=32, q_counts=(40, 3), max_len=300, window=50),
    dict(dtype="f16", hq=16, hkv=2, d=64, page_size=1, q_counts=(33,), max_len=100, causal=False),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_backward_parity(i):
    b = random_batch(7000 + i, **CASES[i])
    _parity(b, 7100 + i)


def test_backward_training_shape_medium():
    """Two 256-query chunks after ~1000 cached keys, Hq 32, Hkv 8, D 128."""
    b = random_batch(7200, dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(256, 256),
                     histories=[900, 1100])
    run, _, _ = _parity(b, 7201)
    info = pa.pa_plan_get_info(run.fwd.plan)
    assert info["bwd_dq_items"] == b.num_queries * b.hkv and info["bwd_kv_items"] > 0


def test_backward_unreferenced_rows_are_zero_and_runs_repeat_bitwise():
    b = random_batch(7300, dtype="bf16", hq=16, hkv=4, d=128, page_size=16, q_counts=(1, 30, 2), max_len=500,
                     window=50, extra_pages=5)
    dout = _dout(b, 7301)
    run = BwdRun(b, dout)
    run()
    first = [t.clone() for t in (run.dq, run.dk, run.dv)]
    run()
    _, rk, rv = oracle.attention_bwd(b, dout)
    for t0, t1 in zip(first, (run.dq, run.dk, run.dv)):
        assert np.array_equal(_bits(t0), _bits(t1))
    dk, dv = to_f64(run.dk), to_f64(run.dv)
    assert np.all(dk[rk == 0] == 0) and np.all(dv[rv == 0] == 0)
    assert np.isfinite(dk).all() and np.isfinite(dv).all()


def test_backward_without_queries_zeroes_the_pools():
    import torch
    b = random_batch(7400, dtype="bf16", hq=8, hkv=2, d=128, page_size=16, q_counts=(0, 0), histories=[20, 3])
    plan = make_plan(b)
    k, v = to_torch(b.k, "bf16"), to_torch(b.v, "bf16")
    dk, dv = torch.full_like(k, 1.0), torch.full_like(v, 1.0)
    empty = torch.empty((0, b.hq, b.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, b.hq), dtype=torch.float32, device="cuda")
    pa.pa_attention_bwd(plan, empty, k, v, empty, lse, empty, empty, dk, dv, scale=b.scale)
    torch.cuda.synchronize()
    assert not dk.float().abs().sum().item() and not dv.float().abs().sum().item()


SHARED_CASES = [
    # two sequences continue a 128-key prefix held by sequence 0's pages
    (dict(dtype="bf16", hq=32, hkv=8, d=128, page_size=16, q_counts=(40, 30, 1), histories=[200, 180, 300]),
     [(s, j, 0, j) for s in (1, 2) for j in range(8)]),
    (dict(dtype="f16", hq=32, hkv=8, d=192, dv=128, page_size=16, q_counts=(20, 9), histories=[100, 90]),
     [(1, j, 0, j) for j in range(5)]),
    # f32 (vector kernels add into the pools), one page read at two positions of a sequence too
    (dict(dtype="f32", hq=8, hkv=2, d=64, page_size=16, q_counts=(12, 5), histories=[70, 80]),
     [(1, 0, 0, 0), (1, 1, 0, 1), (1, 4, 1, 2)]),
    (dict(dtype="bf16", hq=16, hkv=4, d=64, page_size=1, q_counts=(17, 2), histories=[30, 25], window=20),
     [(1, j, 0, j) for j in range(20)]),
]


@pytest.mark.parametrize("i", range(len(SHARED_CASES)))
def test_backward_shared_pages_parity(i):
    """Pages read by two sequences (prefix sharing) or at two positions of one:
    their rows' gradients are f32 sums of every reader's contribution."""
    kw, links = SHARED_CASES[i]
    b = with_shared_pages(random_batch(7500 + i, **kw), links)
    run, _, _ = _parity(b, 7550 + i)
    info = pa.pa_plan_get_info(run.fwd.plan)
    assert info["bwd_shared_pages"] == 1
    es = 4 if b.dtype == "f32" else 2
    extra = 0 if es == 4 else b.num_pages * b.page_size * b.hkv * (b.d + b.dv) * 4
    base = pa.pa_plan_bwd_workspace_bytes(make_plan(random_batch(7500 + i, **kw)), b.dtype, b.d, b.dv)
    assert pa.pa_plan_bwd_workspace_bytes(run.fwd.plan, b.dtype, b.d, b.dv) >= base + extra
