"""fp64 CPU oracle for paged-KV attention (GQA/MHA and absorbed MLA).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the HIP
library and never imports it.

`paged_oracle.c` holds the arithmetic (plain double-precision loops written
from the definition: boostr 0.2.0-beta.2 `standard_attention_fwd` /
`build_attention_mask` / `expand_kv`, with the paged layout and absolute
positions of ruDNN 0.1.107 `DevicePlan::attention` and `DevicePlan::mla`).
The backward (`attention_bwd`, `mla_bwd`: ruDNN `attention_backward` /
`mla_backward`, written out from boostr `standard_attention_bwd`) lives in
the same file.  This module only builds it with gcc and marshals numpy
arrays into it.  `brute.py` is an independent pure-Python brute force for
tiny inputs.  `append_kv` (the cache write before attention) is a plain
numpy loop.  `sparse_proxy_scores`, `sparse_select` and `sparse_attention`
are the block-sparse top-k path of alice-llm 2.0.0
sparse_attention/llama3_bridge.rs (proxy block-max scores and attention
over the kept blocks in the C file, the top-k choice here).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "paged_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libpaged_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                           "-o", tmp, _SRC, "-lm", "-lpthread"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        I = ctypes.c_int
        for name in ("po_attention", "po_mla", "po_widen", "po_attention_bwd", "po_mla_bwd", "po_sparse_proxy",
                     "po_sparse_attention"):
            getattr(lib, name).restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except Exception:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


_DT = {"f32": 0, "bf16": 1, "f16": 2}


def _storage(a: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16  # bf16 and f16: raw 16-bit patterns
    return np.ascontiguousarray(a, dtype=want)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored elements (f32 values, or bf16 / f16 bit patterns) -> float64,
    exactly, through the oracle's own conversion."""
    lib = _load()
    x = _storage(a, dtype)
    out = np.empty(x.size, dtype=np.float64)
    rc = lib.po_widen(ctypes.c_int(_DT[dtype]), _ptr(x), ctypes.c_int64(x.size), _ptr(out))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    return out.reshape(x.shape)


_ERR = {-1: "query outside every sequence", -2: "block-table entry outside the pool",
        -3: "out of memory", -4: "bad geometry"}


def attention(b, rows: Optional[np.ndarray] = None, nthreads: Optional[int] = None
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Paged GQA/MHA attention of batch `b` (fields as in synth.PagedBatch).

    rows: optional flat indices query*hq + head to evaluate; returns
    (out [n, dv], lse [n]).  Without rows returns (out [Q, hq, dv], lse [Q, hq]).
    """
    lib = _load()
    Q = int(b.cu_q[-1])
    n = Q * b.hq if rows is None else int(len(rows))
    out = np.empty((n, b.dv), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    q, k, v = (_storage(x, b.dtype) for x in (b.q, b.k, b.v))
    sl, cu, qp, bt = _i32(b.seq_lens), _i32(b.cu_q), _i32(b.q_pos), _i32(b.block_table)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = lib.po_attention(
        ctypes.c_int(_DT[b.dtype]), _ptr(q), _ptr(k), _ptr(v),
        ctypes.c_int(len(sl)), _ptr(sl), _ptr(cu), _ptr(qp), _ptr(bt), ctypes.c_int(bt.shape[1]),
        ctypes.c_int(b.page_size), ctypes.c_int(b.num_pages), ctypes.c_int(b.hq), ctypes.c_int(b.hkv),
        ctypes.c_int(b.d), ctypes.c_int(b.dv), ctypes.c_double(b.scale), ctypes.c_int(int(b.causal)),
        ctypes.c_int(int(b.window)), _ptr(r), ctypes.c_int64(0 if r is None else len(r)),
        _ptr(out), _ptr(lse), ctypes.c_int(nthreads or default_threads()))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    if rows is None:
        return out.reshape(Q, b.hq, b.dv), lse.reshape(Q, b.hq)
    return out, lse


def mla(b, rows: Optional[np.ndarray] = None, nthreads: Optional[int] = None
        ) -> Tuple[np.ndarray, np.ndarray]:
    """Absorbed MLA of batch `b` (fields as in synth.MlaBatch); same return
    convention as `attention` with dv = R."""
    lib = _load()
    Q = int(b.cu_q[-1])
    n = Q * b.heads if rows is None else int(len(rows))
    out = np.empty((n, b.r), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    qa, qr, lat, kp = (_storage(x, b.dtype) for x in (b.q_abs, b.q_rope, b.latent, b.kpos))
    sl, cu, qp, bt = _i32(b.seq_lens), _i32(b.cu_q), _i32(b.q_pos), _i32(b.block_table)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = lib.po_mla(
        ctypes.c_int(_DT[b.dtype]), _ptr(qa), _ptr(qr), _ptr(lat), _ptr(kp),
        ctypes.c_int(len(sl)), _ptr(sl), _ptr(cu), _ptr(qp), _ptr(bt), ctypes.c_int(bt.shape[1]),
        ctypes.c_int(b.page_size), ctypes.c_int(b.num_pages), ctypes.c_int(b.heads), ctypes.c_int(b.r),
        ctypes.c_int(b.p), ctypes.c_double(b.scale), ctypes.c_int(int(b.causal)), ctypes.c_int(int(b.window)),
        _ptr(r), ctypes.c_int64(0 if r is None else len(r)), _ptr(out), _ptr(lse),
        ctypes.c_int(nthreads or default_threads()))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    if rows is None:
        return out.reshape(Q, b.heads, b.r), lse.reshape(Q, b.heads)
    return out, lse


def attention_bwd(b, dout: np.ndarray, nthreads: Optional[int] = None
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of `attention(b)` for the output gradient `dout` [Q, hq, dv]
    (storage dtype of b), following ruDNN paged_attention
    `attention_backward` with the formulas of boostr `standard_attention_bwd`.
    Returns float64 (dq [Q, hq, d], dk [pages, ps, hkv, d], dv [pages, ps,
    hkv, dv]); pool rows no visible key names are zero."""
    lib = _load()
    Q = int(b.cu_q[-1])
    dq = np.empty((Q, b.hq, b.d), dtype=np.float64)
    dk = np.empty((b.num_pages, b.page_size, b.hkv, b.d), dtype=np.float64)
    dv = np.empty((b.num_pages, b.page_size, b.hkv, b.dv), dtype=np.float64)
    q, k, v, g = (_storage(x, b.dtype) for x in (b.q, b.k, b.v, dout))
    assert g.shape == (Q, b.hq, b.dv)
    sl, cu, qp, bt = _i32(b.seq_lens), _i32(b.cu_q), _i32(b.q_pos), _i32(b.block_table)
    rc = lib.po_attention_bwd(
        ctypes.c_int(_DT[b.dtype]), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        ctypes.c_int(len(sl)), _ptr(sl), _ptr(cu), _ptr(qp), _ptr(bt), ctypes.c_int(bt.shape[1]),
        ctypes.c_int(b.page_size), ctypes.c_int(b.num_pages), ctypes.c_int(b.hq), ctypes.c_int(b.hkv),
        ctypes.c_int(b.d), ctypes.c_int(b.dv), ctypes.c_double(b.scale), ctypes.c_int(int(b.causal)),
        ctypes.c_int(int(b.window)), _ptr(dq), _ptr(dk), _ptr(dv), ctypes.c_int(nthreads or default_threads()))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    return dq, dk, dv


def mla_bwd(b, dout: np.ndarray, nthreads: Optional[int] = None
            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of `mla(b)` for `dout` [Q, heads, r] (ruDNN `mla_backward`):
    float64 (dq_abs [Q, heads, r], dq_rope [Q, heads, p], dlatent [pages, ps,
    1, r] with its key and value terms, dkpos [pages, ps, 1, p])."""
    lib = _load()
    Q = int(b.cu_q[-1])
    dqa = np.empty((Q, b.heads, b.r), dtype=np.float64)
    dqr = np.empty((Q, b.heads, b.p), dtype=np.float64)
    dlat = np.empty((b.num_pages, b.page_size, 1, b.r), dtype=np.float64)
    dkp = np.empty((b.num_pages, b.page_size, 1, b.p), dtype=np.float64)
    qa, qr, lat, kp, g = (_storage(x, b.dtype) for x in (b.q_abs, b.q_rope, b.latent, b.kpos, dout))
    assert g.shape == (Q, b.heads, b.r)
    sl, cu, qp, bt = _i32(b.seq_lens), _i32(b.cu_q), _i32(b.q_pos), _i32(b.block_table)
    rc = lib.po_mla_bwd(
        ctypes.c_int(_DT[b.dtype]), _ptr(qa), _ptr(qr), _ptr(lat), _ptr(kp), _ptr(g),
        ctypes.c_int(len(sl)), _ptr(sl), _ptr(cu), _ptr(qp), _ptr(bt), ctypes.c_int(bt.shape[1]),
        ctypes.c_int(b.page_size), ctypes.c_int(b.num_pages), ctypes.c_int(b.heads), ctypes.c_int(b.r),
        ctypes.c_int(b.p), ctypes.c_double(b.scale), ctypes.c_int(int(b.causal)), ctypes.c_int(int(b.window)),
        _ptr(dqa), _ptr(dqr), _ptr(dlat), _ptr(dkp), ctypes.c_int(nthreads or default_threads()))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    return dqa, dqr, dlat, dkp


def append_kv(seq_lens, cu_q, q_pos, block_table, page_size: int, k_new: np.ndarray, v_new: np.ndarray,
              k_pool: np.ndarray, v_pool: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Paged K/V append, following ruDNN 0.1.107 paged_attention
    `DevicePlan::append`: query i of sequence s at absolute position p writes
    its new rows into pool page block_table[s][p // page_size], slot
    p % page_size.  Returns updated copies of the pools (any storage dtype:
    rows are copied as they are).  A plain loop over the queries."""
    k_out, v_out = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    for s in range(len(seq_lens)):
        for i in range(int(cu_q[s]), int(cu_q[s + 1])):
            p = int(q_pos[i])
            page = int(block_table[s][p // page_size])
            k_out[page, p % page_size] = k_new[i]
            v_out[page, p % page_size] = v_new[i]
    return k_out, v_out


def visible_range(b, i: int, s: int) -> Tuple[int, int]:
    """Keys [lo, hi] query i of sequence s sees (causal, window, t < L)."""
    p, L = int(b.q_pos[i]), int(b.seq_lens[s])
    hi = p if b.causal else L - 1
    lo = max(0, p - b.window + 1) if b.window > 0 else 0
    return lo, hi


def sparse_proxy_scores(b, block_size: int, nthreads: Optional[int] = None) -> np.ndarray:
    """Proxy block scores float32 [Q, hkv, nblk] (nblk = ceil(max L /
    block_size)): the largest f32 dot product of the group's first query
    head with a visible key of the block, summed in increasing dimension
    order; -inf for blocks without a visible key (alice-llm
    `compute_proxy_block_max_scores` with the first query head of each KV
    head as proxy)."""
    lib = _load()
    Q = int(b.cu_q[-1])
    nblk = max(1, -(-int(max(b.seq_lens, default=0)) // block_size))
    scores = np.empty((Q, b.hkv, nblk), dtype=np.float32)
    q, k = (_storage(x, b.dtype) for x in (b.q, b.k))
    sl, cu, qp, bt = _i32(b.seq_lens), _i32(b.cu_q), _i32(b.q_pos), _i32(b.block_table)
    rc = lib.po_sparse_proxy(
        ctypes.c_int(_DT[b.dtype]), _ptr(q), _ptr(k), ctypes.c_int(len(sl)), _ptr(sl), _ptr(cu), _ptr(qp), _ptr(bt),
        ctypes.c_int(bt.shape[1]), ctypes.c_int(b.page_size), ctypes.c_int(b.num_pages), ctypes.c_int(b.hq),
        ctypes.c_int(b.hkv), ctypes.c_int(b.d), ctypes.c_int(int(b.causal)), ctypes.c_int(int(b.window)),
        ctypes.c_int(block_size), _ptr(scores), ctypes.c_int(nblk), ctypes.c_int(nthreads or default_threads()))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    return scores


def sparse_select(b, block_size: int, topk: int, scores: Optional[np.ndarray] = None) -> np.ndarray:
    """Kept blocks int32 [Q, hkv, topk] in increasing order, -1 padded
    (alice-llm `sparse_topk_select_batch`).  The candidates of a row are the
    blocks holding a visible key; topk == 0 or topk >= their number keeps
    them all (the dense fallback), else the topk largest proxy scores, a tie
    going to the lower block index.  With topk == 0 the width is the largest
    candidate count of any row."""
    if scores is None:
        scores = sparse_proxy_scores(b, block_size)
    Q = int(b.cu_q[-1])
    rows = []
    for s in range(b.num_seqs):
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            lo, hi = visible_range(b, i, s)
            cand = list(range(lo // block_size, hi // block_size + 1))
            for h in range(b.hkv):
                if topk == 0 or topk >= len(cand):
                    keep = cand
                else:
                    keep = sorted(sorted(cand, key=lambda r: (-float(scores[i, h, r]), r))[:topk])
                rows.append((i, h, keep))
    width = topk if topk > 0 else max([len(k) for _, _, k in rows], default=1)
    sel = np.full((Q, b.hkv, max(width, 1)), -1, dtype=np.int32)
    for i, h, keep in rows:
        sel[i, h, :len(keep)] = keep
    return sel


def sparse_attention(b, sel: np.ndarray, block_size: int, nthreads: Optional[int] = None
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of batch `b` over the visible keys of the kept blocks `sel`
    [Q, hkv, k] (-1 = none), all query heads of a KV head sharing its
    blocks (alice-llm `kvouter_forward` + `lse_combine`, written as one
    softmax over the union of the kept keys).  Returns (out [Q, hq, dv],
    lse [Q, hq])."""
    lib = _load()
    Q = int(b.cu_q[-1])
    out = np.empty((Q * b.hq, b.dv), dtype=np.float64)
    lse = np.empty(Q * b.hq, dtype=np.float64)
    q, k, v = (_storage(x, b.dtype) for x in (b.q, b.k, b.v))
    sl, cu, qp, bt = _i32(b.seq_lens), _i32(b.cu_q), _i32(b.q_pos), _i32(b.block_table)
    sel = _i32(sel)
    assert sel.shape[:2] == (Q, b.hkv)
    rc = lib.po_sparse_attention(
        ctypes.c_int(_DT[b.dtype]), _ptr(q), _ptr(k), _ptr(v),
        ctypes.c_int(len(sl)), _ptr(sl), _ptr(cu), _ptr(qp), _ptr(bt), ctypes.c_int(bt.shape[1]),
        ctypes.c_int(b.page_size), ctypes.c_int(b.num_pages), ctypes.c_int(b.hq), ctypes.c_int(b.hkv),
        ctypes.c_int(b.d), ctypes.c_int(b.dv), ctypes.c_double(b.scale), ctypes.c_int(int(b.causal)),
        ctypes.c_int(int(b.window)), _ptr(sel), ctypes.c_int(sel.shape[2]), ctypes.c_int(block_size),
        _ptr(out), _ptr(lse), ctypes.c_int(nthreads or default_threads()))
    if rc:
        raise RuntimeError(f"oracle: {_ERR.get(rc, rc)}")
    return out.reshape(Q, b.hq, b.dv), lse.reshape(Q, b.hq)
