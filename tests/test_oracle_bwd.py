"""Pins for the oracle's backward (ruDNN paged_attention `attention_backward`
/ `mla_backward`; formulas of boostr `standard_attention_bwd`): torch autograd
in float64 on the dense per-sequence view (a library routine, with explicit
KV-head repetition and an explicit mask), central finite differences of the
forward oracle, and invariants of the gradient (the key gradient sums to zero
over the keys of a row; the value gradient sums to the output gradient)."""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from synth import PagedBatch, random_batch, random_mla_batch
from tests.dense_view import dense_sequence, widen


def _dout(b, seed, width=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b.num_queries, b.hq if hasattr(b, "hq") else b.heads, width or b.dv))
    x = x.astype(np.float32)
    if b.dtype == "f32":
        return x
    from synth import f32_to_bf16_bits, f32_to_f16_bits
    return f32_to_bf16_bits(x) if b.dtype == "bf16" else f32_to_f16_bits(x)


def _torch_grads(b, dout):
    """Autograd of sum(dout * out) over dense per-sequence views, scattered back
    into pool-shaped arrays with numpy indexing."""
    torch = pytest.importorskip("torch")
    q = torch.from_numpy(widen(b.q, b.dtype)).requires_grad_(True)
    k = widen(b.k, b.dtype)
    v = widen(b.v, b.dtype)
    g = torch.from_numpy(widen(dout, b.dtype))
    G = b.hq // b.hkv
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dq = np.zeros(q.shape)
    for s in range(b.num_seqs):
        lo, hi = int(b.cu_q[s]), int(b.cu_q[s + 1])
        if hi == lo:
            continue
        L = int(b.seq_lens[s])
        kd = torch.from_numpy(dense_sequence(k, b.block_table, s, L, b.page_size)).requires_grad_(True)
        vd = torch.from_numpy(dense_sequence(v, b.block_table, s, L, b.page_size)).requires_grad_(True)
        qs = q[lo:hi].detach().clone().requires_grad_(True)
        ke = kd.repeat_interleave(G, dim=1).permute(1, 0, 2)  # [hq, L, d]
        ve = vd.repeat_interleave(G, dim=1).permute(1, 0, 2)
        qq = qs.permute(1, 0, 2)                                # [hq, n, d]
        pos = torch.from_numpy(b.q_pos[lo:hi].astype(np.int64))[:, None]
        t = torch.arange(L)[None, :]
        allowed = (t < L) & ((t <= pos) if b.causal else torch.ones_like(t, dtype=torch.bool))
        if b.window:
            allowed = allowed & (t > pos - b.window)
        sc = (qq @ ke.transpose(1, 2)) * b.scale
        sc = sc.masked_fill(~allowed, -math.inf)
        out = torch.softmax(sc, dim=-1) @ ve                   # [hq, n, dv]
        (out.permute(1, 0, 2) * g[lo:hi]).sum().backward()
        dq[lo:hi] = qs.grad.numpy()
        tt = np.arange(L)
        np.add.at(dk, (b.block_table[s, tt // b.page_size], tt % b.page_size), kd.grad.numpy())
        np.add.at(dv, (b.block_table[s, tt // b.page_size], tt % b.page_size), vd.grad.numpy())
    return dq, dk, dv


CASES = [
    dict(dtype="f32", hq=4, hkv=1, d=8, page_size=4, q_counts=(1, 3), causal=True, window=0),
    dict(dtype="bf16", hq=4, hkv=2, d=16, page_size=3, q_counts=(2, 1, 4), causal=True, window=5),
    dict(dtype="f32", hq=2, hkv=2, d=8, page_size=1, q_counts=(1, 2), causal=False, window=0),
    dict(dtype="f16", hq=6, hkv=3, d=8, page_size=16, q_counts=(3, 1), causal=False, window=7),
    dict(dtype="bf16", hq=3, hkv=1, d=8, page_size=2, q_counts=(5,), causal=True, window=2, dv=4),
    dict(dtype="bf16", hq=8, hkv=2, d=12, page_size=5, q_counts=(0, 6, 1), causal=True, window=0, dv=20),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_backward_matches_torch_autograd_float64(i):
    b = random_batch(300 + i, max_len=40, poison=False, **CASES[i])
    dout = _dout(b, 400 + i)
    dq, dk, dv = oracle.attention_bwd(b, dout)
    rq, rk, rv = _torch_grads(b, dout)
    np.testing.assert_allclose(dq, rq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, rv, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_with_shared_pages_matches_torch_autograd_float64(dtype):
    """Prefix sharing (sequence 1 reads sequence 0's first two pages) and one
    page at two positions of sequence 2: a pool row's key and value gradients
    are the sums over every position that reads it (np.add.at over the dense
    views in the reference)."""
    from synth import with_shared_pages
    b = random_batch(350, dtype=dtype, hq=4, hkv=2, d=8, page_size=4, q_counts=(3, 2, 4),
                     histories=[10, 12, 14], poison=True)
    s = with_shared_pages(b, [(1, 0, 0, 0), (1, 1, 0, 1), (2, 3, 2, 1)])
    dout = _dout(s, 351)
    dq, dk, dv = oracle.attention_bwd(s, dout)
    rq, rk, rv = _torch_grads(s, dout)
    np.testing.assert_allclose(dq, rq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, rv, rtol=1e-11, atol=1e-12)
    # the shared rows really take two contributions: differ from the
    # unshared tables' gradients there
    _, uk, _ = oracle.attention_bwd(b, dout)
    p0 = b.block_table[0, 0]
    assert not np.allclose(dk[p0], uk[p0])


def test_backward_matches_central_differences_of_the_forward():
    """d/dx of sum(dout * out) by (f(x + h) - f(x - h)) / 2h on f32 inputs,
    h = 2^-12 (exact in f32 for these values), for elements of q, k and v."""
    b = random_batch(310, dtype="f32", hq=4, hkv=2, d=8, page_size=4, q_counts=(2, 3), max_len=20,
                     causal=True, window=6, poison=False)
    dout = _dout(b, 410)
    dq, dk, dv = oracle.attention_bwd(b, dout)
    g = dout.astype(np.float64)
    h = 2.0 ** -12

    def loss(bb):
        out, _ = oracle.attention(bb)
        return float(np.sum(out * g))

    rng = np.random.default_rng(311)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        arr = getattr(b, name)
        flat = np.flatnonzero(np.abs(grad.reshape(-1)) > 0)
        for idx in rng.choice(flat, size=6, replace=False):
            plus, minus = arr.copy(), arr.copy()
            plus.reshape(-1)[idx] += np.float32(h)
            minus.reshape(-1)[idx] -= np.float32(h)
            fd = (loss(dataclasses.replace(b, **{name: plus})) - loss(dataclasses.replace(b, **{name: minus}))) / (2 * h)
            assert abs(fd - grad.reshape(-1)[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad.reshape(-1)[idx])


def test_backward_gradient_sums():
    """Per row the key-side score gradients dS sum to zero (softmax), so dK
    summed over the whole pool is zero for every KV head and dim; the weights
    sum to one, so dV summed over the pool equals the output gradient summed
    over the rows of that KV head.  Rows of unreferenced pages stay zero."""
    b = random_batch(320, dtype="bf16", hq=8, hkv=2, d=16, page_size=8, q_counts=(1, 7, 3), max_len=70,
                     causal=True, window=13, extra_pages=3)
    dout = _dout(b, 420)
    dq, dk, dv = oracle.attention_bwd(b, dout)
    G = b.hq // b.hkv
    g = widen(dout, b.dtype)
    for kvh in range(b.hkv):
        assert np.abs(dk[:, :, kvh].sum(axis=(0, 1))).max() < 1e-12
        want = g[:, kvh * G:(kvh + 1) * G].sum(axis=(0, 1))
        np.testing.assert_allclose(dv[:, :, kvh].sum(axis=(0, 1)), want, rtol=1e-12, atol=1e-12)
    used = set()
    for s in range(b.num_seqs):
        for t in range(int(b.seq_lens[s])):
            used.add(int(b.block_table[s, t // b.page_size]))
    for page in range(b.num_pages):
        if page not in used:
            assert not dk[page].any() and not dv[page].any()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mla_backward_is_mqa_backward_with_shared_latent(dtype):
    """MLA = single-KV-head attention with key [latent | kpos], query [q_abs |
    q_rope] and value latent; the latent gradient is that attention's key
    gradient (first r columns) plus its value gradient."""
    m = random_mla_batch(330, heads=4, r=16, p=8, page_size=8, q_counts=(1, 3, 1), max_len=50, dtype=dtype)
    dout = _dout(m, 430, width=m.r)
    dqa, dqr, dlat, dkp = oracle.mla_bwd(m, dout)
    k = np.concatenate([m.latent, m.kpos], axis=-1)
    q = np.concatenate([m.q_abs, m.q_rope], axis=-1)
    b = PagedBatch("mqa", dtype, m.seq_lens, m.cu_q, m.q_pos, m.block_table, m.page_size, m.num_pages,
                   m.heads, 1, m.r + m.p, m.r, m.scale, m.causal, m.window, q, k, m.latent)
    dq, dk, dv = oracle.attention_bwd(b, dout)
    np.testing.assert_allclose(dqa, dq[..., :m.r], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dqr, dq[..., m.r:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dkp, dk[..., m.r:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dlat, dk[..., :m.r] + dv, rtol=1e-12, atol=1e-13)
