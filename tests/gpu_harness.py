"""Test/bench helpers: move a synthetic batch to the GPU and run it through
the C ABI (via the ctypes binding).  Marshalling only; no attention math."""
from __future__ import annotations

import numpy as np

import paged_kv_attention_gqa_amd as pa
from synth import bf16_bits_to_f32


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    """Stored values (f32, or bf16 / f16 bit patterns) -> a device tensor of
    that type, bit for bit."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device).view(torch_dtype(dtype))


def to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.float16).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def make_plan(b, *, mla=False, max_splits=None, split_tokens=0, stream=None):
    hq = b.heads if mla else b.hq
    hkv = 1 if mla else b.hkv
    return pa.pa_plan_create(b.seq_lens, b.cu_q, b.q_pos, b.block_table, page_size=b.page_size,
                             num_pages=b.num_pages, num_q_heads=hq, num_kv_heads=hkv, causal=b.causal,
                             window=b.window, max_splits=b.max_splits if max_splits is None else max_splits,
                             mla=mla, split_tokens=split_tokens, stream=stream)


class GqaRun:
    """Device copies of a PagedBatch plus a plan, output, lse and workspace."""

    def __init__(self, b, *, max_splits=None, split_tokens=0, with_lse=True):
        import torch
        self.b = b
        self.q = to_torch(b.q, b.dtype)
        self.k = to_torch(b.k, b.dtype)
        self.v = to_torch(b.v, b.dtype)
        self.plan = make_plan(b, max_splits=max_splits, split_tokens=split_tokens)
        tdt = torch_dtype(b.dtype)
        self.out = torch.empty((b.num_queries, b.hq, b.dv), dtype=tdt, device="cuda")
        self.lse = torch.empty((b.num_queries, b.hq), dtype=torch.float32, device="cuda") if with_lse else None
        nbytes = pa.pa_plan_workspace_bytes(self.plan, b.dv)
        self.workspace = torch.zeros(max(nbytes, 1) // 4 + 64, dtype=torch.float32, device="cuda") if nbytes else None
        self.info = pa.pa_plan_get_info(self.plan)

    def __call__(self, main_events=None):
        pa.pa_attention_fwd(self.plan, self.q, self.k, self.v, self.out, self.lse, scale=self.b.scale,
                            workspace=self.workspace, main_events=main_events)
        return self.out

    def result(self):
        import torch
        torch.cuda.synchronize()
        return to_f64(self.out), (self.lse.cpu().numpy().astype(np.float64) if self.lse is not None else None)


class MlaRun:
    """Device copies of an MlaBatch plus a plan, output, lse and workspace."""

    def __init__(self, m, *, max_splits=None, split_tokens=0, with_lse=True):
        import torch
        self.m = m
        self.q_abs = to_torch(m.q_abs, m.dtype)
        self.q_rope = to_torch(m.q_rope, m.dtype)
        self.latent = to_torch(m.latent, m.dtype)
        self.kpos = to_torch(m.kpos, m.dtype)
        self.plan = make_plan(m, mla=True, max_splits=max_splits, split_tokens=split_tokens)
        self.out = torch.empty((m.num_queries, m.heads, m.r), dtype=torch_dtype(m.dtype), device="cuda")
        self.lse = torch.empty((m.num_queries, m.heads), dtype=torch.float32, device="cuda") if with_lse else None
        nbytes = pa.pa_plan_workspace_bytes(self.plan, m.r)
        self.workspace = torch.zeros(max(nbytes, 1) // 4 + 64, dtype=torch.float32, device="cuda") if nbytes else None
        self.info = pa.pa_plan_get_info(self.plan)

    def __call__(self, main_events=None):
        pa.pa_mla_fwd(self.plan, self.q_abs, self.q_rope, self.latent, self.kpos, self.out, self.lse,
                      scale=self.m.scale, workspace=self.workspace, main_events=main_events)
        return self.out

    def result(self):
        import torch
        torch.cuda.synchronize()
        return to_f64(self.out), (self.lse.cpu().numpy().astype(np.float64) if self.lse is not None else None)


def tolerance(dtype: str):
    """(atol, rtol) of the GPU-vs-oracle bar: f32 max-abs 1e-4; bf16
    |gpu - oracle| <= 2e-2 + 1e-2 |oracle|; f16 the bf16 bar scaled by 2^-3
    for its three more significand bits: 2.5e-3 + 1.25e-3 |oracle|."""
    return {"f32": (1e-4, 0.0), "bf16": (2e-2, 1e-2), "f16": (2.5e-3, 1.25e-3)}[dtype]


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "out"):
    atol, rtol = tolerance(dtype)
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside |d| <= {atol} + {rtol}|ref|; "
                             f"max err {np.nanmax(err):.3g}; first {idx.tolist()}: gpu={gpu[bad][:5]}, "
                             f"ref={ref[bad][:5]}")
