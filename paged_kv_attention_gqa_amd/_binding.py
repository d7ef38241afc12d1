"""ctypes binding of libpaged_attn.so: the C ABI of include/paged_attn.h under
the same names.  Argument marshalling only (host metadata arrays, device
pointers and the HIP stream of torch tensors, and the shape checks the C ABI
cannot make because it receives raw pointers); every step of the attention
runs in the library's HIP kernels.  There is no fallback: if the library is
not built, loading fails."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")

PA_OK = 0
PA_F32 = 0
PA_BF16 = 1
PA_F16 = 2
STATUS_NAMES = {0: "PA_OK", -1: "PA_ERR_INVALID", -2: "PA_ERR_SHAPE", -3: "PA_ERR_PLAN", -4: "PA_ERR_UNSUPPORTED",
                -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_OVERLAP", -7: "PA_ERR_RANGE", -8: "PA_ERR_HIP",
                -9: "PA_ERR_DEVICE"}
EXPORTED = ("pa_plan_create", "pa_plan_create_host", "pa_plan_get_work", "pa_plan_destroy", "pa_plan_get_info",
            "pa_plan_workspace_bytes", "pa_attention_fwd", "pa_mla_fwd", "pa_append_kv", "pa_status_string",
            "pa_last_error", "pa_plan_bwd_workspace_bytes", "pa_attention_bwd", "pa_attention_fwd_noalloc",
            "pa_sparse_attention_fwd", "pa_sparse_workspace_bytes", "pa_mla_bwd")


class PaError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.name}: {detail}")


class _PlanDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("seq_lens", ctypes.c_void_p), ("cu_q", ctypes.c_void_p),
                ("q_pos", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("table_width", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("mla", ctypes.c_int32), ("split_tokens", ctypes.c_int32)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("num_queries", ctypes.c_int32), ("decode_items", ctypes.c_int32),
                ("prefill_items", ctypes.c_int32), ("split_rows", ctypes.c_int32),
                ("split_slots", ctypes.c_int32), ("launches", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("heads_per_item", ctypes.c_int32), ("bwd_dq_items", ctypes.c_int32),
                ("bwd_kv_items", ctypes.c_int32), ("bwd_shared_pages", ctypes.c_int32)]


_lib = None


def load_library():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.pa_plan_create.argtypes = [ctypes.POINTER(_PlanDesc), P, ctypes.POINTER(P)]
    lib.pa_plan_create_host.argtypes = [ctypes.POINTER(_PlanDesc), I, ctypes.POINTER(P)]
    IP = ctypes.POINTER(ctypes.c_int32)
    lib.pa_plan_get_work.argtypes = [P, P, IP, P, IP, P, IP]
    lib.pa_plan_destroy.argtypes = [P]
    lib.pa_plan_get_info.argtypes = [P, ctypes.POINTER(_PlanInfo)]
    lib.pa_plan_workspace_bytes.argtypes = [P, I, ctypes.POINTER(S)]
    lib.pa_attention_fwd.argtypes = [P, I, P, P, P, P, P, I, I, F, P, S, P, P]
    lib.pa_attention_fwd_noalloc.argtypes = [P, I, P, P, P, P, P, I, I, F, P]
    lib.pa_sparse_attention_fwd.argtypes = [P, I, P, P, P, P, P, I, I, F, I, I, P, P, S, P]
    lib.pa_sparse_workspace_bytes.argtypes = [P, I, I, I, ctypes.POINTER(S), ctypes.POINTER(I)]
    lib.pa_mla_bwd.argtypes = [P, I, P, P, P, P, P, P, P, P, P, P, P, I, I, F, P, S, P]
    lib.pa_mla_fwd.argtypes = [P, I, P, P, P, P, P, P, I, I, F, P, S, P, P]
    lib.pa_append_kv.argtypes = [P, I, P, P, P, P, I, I, P]
    lib.pa_plan_bwd_workspace_bytes.argtypes = [P, I, I, I, ctypes.POINTER(S)]
    lib.pa_attention_bwd.argtypes = [P, I, P, P, P, P, P, P, P, P, P, I, I, F, P, S, P]
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    for n in ("pa_plan_create", "pa_plan_create_host", "pa_plan_get_work", "pa_plan_destroy", "pa_plan_get_info",
              "pa_plan_workspace_bytes", "pa_attention_fwd", "pa_mla_fwd", "pa_append_kv",
              "pa_plan_bwd_workspace_bytes", "pa_attention_bwd", "pa_attention_fwd_noalloc",
            "pa_sparse_attention_fwd", "pa_sparse_workspace_bytes", "pa_mla_bwd"):
        getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, where: str):
    if rc != PA_OK:
        raise PaError(rc, where, pa_last_error())


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(status).decode()


def pa_last_error() -> str:
    return load_library().pa_last_error().decode()


class Plan:
    """Owning handle of a pa_plan (destroyed by pa_plan_destroy or on GC)."""

    def __init__(self, handle: ctypes.c_void_p, desc: dict):
        self._h = handle
        self.desc = desc

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("plan already destroyed")
        return self._h

    def __del__(self):
        try:
            if self._h is not None and _lib is not None:
                _lib.pa_plan_destroy(self._h)
                self._h = None
        except Exception:
            pass


def _host_i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        # torch's current stream when a device is present, else the null stream
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _plan_desc(seq_lens, cu_q, q_pos, block_table, page_size, num_pages, num_q_heads, num_kv_heads, causal, window,
               max_splits, mla, split_tokens):
    """(descriptor, host arrays it points into, Plan.desc dict)."""
    sl, cu, qp = _host_i32(seq_lens), _host_i32(cu_q), _host_i32(q_pos)
    bt = _host_i32(block_table)
    if bt.ndim != 2:
        raise ValueError("block_table must be 2-D [num_seqs, table_width]")
    if cu.shape[0] != sl.shape[0] + 1 or bt.shape[0] != sl.shape[0]:
        raise ValueError("cu_q must have num_seqs+1 entries and block_table num_seqs rows")
    if sl.shape[0] > 0 and qp.shape[0] != int(cu[-1]):
        raise ValueError("q_pos must have cu_q[-1] entries")
    desc = _PlanDesc(int(sl.shape[0]), sl.ctypes.data, cu.ctypes.data, qp.ctypes.data if qp.size else None,
                     bt.ctypes.data, int(bt.shape[1]), int(page_size), int(num_pages), int(num_q_heads),
                     int(num_kv_heads), int(bool(causal)), int(window), int(max_splits), int(bool(mla)),
                     int(split_tokens))
    info = dict(num_seqs=int(sl.shape[0]), num_queries=int(cu[-1]), table_width=int(bt.shape[1]),
                page_size=int(page_size), num_pages=int(num_pages), num_q_heads=int(num_q_heads),
                num_kv_heads=int(num_kv_heads), causal=bool(causal), window=int(window),
                max_splits=int(max_splits), mla=bool(mla))
    return desc, (sl, cu, qp, bt), info


def pa_plan_create(seq_lens, cu_q, q_pos, block_table, *, page_size: int, num_pages: int, num_q_heads: int,
                   num_kv_heads: int, causal: bool = True, window: int = 0, max_splits: int = 16, mla: bool = False,
                   split_tokens: int = 0, stream=None) -> Plan:
    """Validate and upload a schedule (host arrays); see pa_plan_create in paged_attn.h."""
    lib = load_library()
    desc, keep, info = _plan_desc(seq_lens, cu_q, q_pos, block_table, page_size, num_pages, num_q_heads,
                                  num_kv_heads, causal, window, max_splits, mla, split_tokens)
    h = ctypes.c_void_p()
    _check(lib.pa_plan_create(ctypes.byref(desc), _stream_handle(stream), ctypes.byref(h)), "pa_plan_create")
    del keep
    return Plan(h, info)


def pa_plan_create_host(seq_lens, cu_q, q_pos, block_table, *, num_cus: int, page_size: int, num_pages: int,
                        num_q_heads: int, num_kv_heads: int, causal: bool = True, window: int = 0,
                        max_splits: int = 16, mla: bool = False, split_tokens: int = 0) -> Plan:
    """Work lists for a device of `num_cus` CUs, built on the host only (no
    device access); see pa_plan_create_host in paged_attn.h."""
    lib = load_library()
    desc, keep, info = _plan_desc(seq_lens, cu_q, q_pos, block_table, page_size, num_pages, num_q_heads,
                                  num_kv_heads, causal, window, max_splits, mla, split_tokens)
    h = ctypes.c_void_p()
    _check(lib.pa_plan_create_host(ctypes.byref(desc), int(num_cus), ctypes.byref(h)), "pa_plan_create_host")
    del keep
    return Plan(h, info)


def pa_plan_get_work(plan: Plan):
    """(items [n, 8], wg_first [n_wg + 1], merges [m, 5]) int32 arrays; see
    pa_plan_get_work in paged_attn.h for the columns."""
    lib = load_library()
    ni, nw, nm = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.pa_plan_get_work(plan.handle, None, ctypes.byref(ni), None, ctypes.byref(nw), None, ctypes.byref(nm)),
           "pa_plan_get_work")
    items = np.zeros((ni.value, 8), np.int32)
    wg = np.zeros(nw.value + 1, np.int32)
    merges = np.zeros((nm.value, 5), np.int32)
    _check(lib.pa_plan_get_work(plan.handle, items.ctypes.data, ctypes.byref(ni), wg.ctypes.data, ctypes.byref(nw),
                                merges.ctypes.data, ctypes.byref(nm)), "pa_plan_get_work")
    return items, wg, merges


def pa_plan_destroy(plan: Plan) -> None:
    lib = load_library()
    if plan._h is not None:
        _check(lib.pa_plan_destroy(plan._h), "pa_plan_destroy")
        plan._h = None


def pa_plan_get_info(plan: Plan) -> dict:
    info = _PlanInfo()
    _check(load_library().pa_plan_get_info(plan.handle, ctypes.byref(info)), "pa_plan_get_info")
    return {n: int(getattr(info, n)) for n, _ in _PlanInfo._fields_}


def pa_plan_workspace_bytes(plan: Plan, v_head_dim: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().pa_plan_workspace_bytes(plan.handle, int(v_head_dim), ctypes.byref(n)),
           "pa_plan_workspace_bytes")
    return int(n.value)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float16:
        return PA_F16
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def _dtype_enum(dtype) -> int:
    """Library dtype code of a torch dtype or of "f32" / "bf16" / "f16"."""
    names = {"f32": PA_F32, "bf16": PA_BF16, "f16": PA_F16}
    if isinstance(dtype, str):
        if dtype not in names:
            raise ValueError(f"unsupported dtype {dtype!r}")
        return names[dtype]
    import torch
    codes = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float16: PA_F16}
    if dtype not in codes:
        raise ValueError(f"unsupported dtype {dtype}")
    return codes[dtype]


def _dev(t, name: str, ndim: int):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have rank {ndim}")
    return t.data_ptr()


def _ws(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _event(ev) -> int:
    return ev.cuda_event if hasattr(ev, "cuda_event") else int(ev)


def _events(main_events):
    """(start, end) torch events or raw hipEvent_t handles -> a C array of two
    handles (kept alive by the caller's reference), or None."""
    if main_events is None:
        return None
    start, end = main_events
    return (ctypes.c_void_p * 2)(_event(start), _event(end))


def _fwd_args(plan: Plan, q, k_pool, v_pool, out, lse):
    """Checked device pointers and sizes of a GQA forward call."""
    d = plan.desc
    dt = _dtype_code(q)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool), ("out", out)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    pq, pk, pv, po = _dev(q, "q", 3), _dev(k_pool, "k_pool", 4), _dev(v_pool, "v_pool", 4), _dev(out, "out", 3)
    D, Dv = int(q.shape[2]), int(v_pool.shape[3])
    Q, Hq = d["num_queries"], d["num_q_heads"]
    pool = (d["num_pages"], d["page_size"], d["num_kv_heads"])
    if tuple(q.shape) != (Q, Hq, D):
        raise ValueError(f"q shape {tuple(q.shape)} != {(Q, Hq, D)}")
    if tuple(k_pool.shape) != pool + (D,) or tuple(v_pool.shape) != pool + (Dv,):
        raise ValueError(f"pool shapes {tuple(k_pool.shape)}, {tuple(v_pool.shape)} do not match {pool} x (D, Dv)")
    if tuple(out.shape) != (Q, Hq, Dv):
        raise ValueError(f"out shape {tuple(out.shape)} != {(Q, Hq, Dv)}")
    pl = None
    if lse is not None:
        import torch
        if lse.dtype != torch.float32 or tuple(lse.shape) != (Q, Hq):
            raise ValueError("lse must be float32 [Q, Hq]")
        pl = _dev(lse, "lse", 2)
    return dt, pq, pk, pv, po, pl, D, Dv


def pa_attention_fwd(plan: Plan, q, k_pool, v_pool, out, lse=None, *, scale: float, workspace=None,
                     main_events=None, stream=None) -> None:
    """Paged GQA forward into `out` (see pa_attention_fwd in paged_attn.h).
    main_events: None or (start, end) timing events (torch.cuda.Event that
    have been recorded once, or hipEvent_t handles) that receive the main
    kernel's own start and end."""
    dt, pq, pk, pv, po, pl, D, Dv = _fwd_args(plan, q, k_pool, v_pool, out, lse)
    wp, wn = _ws(workspace)
    ev = _events(main_events)
    _check(load_library().pa_attention_fwd(plan.handle, dt, pq, pk, pv, po, pl, D, Dv, float(scale), wp, wn,
                                           ev, _stream_handle(stream)), "pa_attention_fwd")


def pa_attention_fwd_noalloc(plan: Plan, q, k_pool, v_pool, out, lse=None, *, scale: float, stream=None) -> None:
    """Paged GQA forward that allocates nothing: split partials in the
    library's fixed per-GPU array (see pa_attention_fwd_noalloc in
    paged_attn.h)."""
    dt, pq, pk, pv, po, pl, D, Dv = _fwd_args(plan, q, k_pool, v_pool, out, lse)
    _check(load_library().pa_attention_fwd_noalloc(plan.handle, dt, pq, pk, pv, po, pl, D, Dv, float(scale),
                                                   _stream_handle(stream)), "pa_attention_fwd_noalloc")


def pa_sparse_workspace_bytes(plan: Plan, v_head_dim: int, block_size: int, topk: int):
    """(workspace bytes, selection width) of pa_sparse_attention_fwd."""
    n, w = ctypes.c_size_t(), ctypes.c_int32()
    _check(load_library().pa_sparse_workspace_bytes(plan.handle, int(v_head_dim), int(block_size), int(topk),
                                                    ctypes.byref(n), ctypes.byref(w)), "pa_sparse_workspace_bytes")
    return int(n.value), int(w.value)


def pa_sparse_attention_fwd(plan: Plan, q, k_pool, v_pool, out, lse=None, *, scale: float, block_size: int,
                            topk: int, selection=None, workspace=None, stream=None) -> None:
    """Block-sparse top-k forward into `out` (see pa_sparse_attention_fwd in
    paged_attn.h); selection: None or an int32 device tensor [Q, Hkv, width]."""
    import torch
    dt, pq, pk, pv, po, pl, D, Dv = _fwd_args(plan, q, k_pool, v_pool, out, lse)
    psel = None
    if selection is not None:
        if selection.dtype != torch.int32 or selection.dim() != 3:
            raise ValueError("selection must be an int32 [Q, Hkv, width] tensor")
        psel = _dev(selection, "selection", 3)
    wp, wn = _ws(workspace)
    _check(load_library().pa_sparse_attention_fwd(plan.handle, dt, pq, pk, pv, po, pl, D, Dv, float(scale),
                                                  int(block_size), int(topk), psel, wp, wn, _stream_handle(stream)),
           "pa_sparse_attention_fwd")


def pa_plan_bwd_workspace_bytes(plan: Plan, dtype, head_dim: int, v_head_dim: int) -> int:
    """Workspace bytes pa_attention_bwd needs; dtype is a torch dtype or
    "f32" / "bf16" / "f16"."""
    n = ctypes.c_size_t()
    _check(load_library().pa_plan_bwd_workspace_bytes(plan.handle, _dtype_enum(dtype), int(head_dim), int(v_head_dim),
                                                      ctypes.byref(n)), "pa_plan_bwd_workspace_bytes")
    return int(n.value)


def pa_attention_bwd(plan: Plan, q, k_pool, v_pool, out, lse, dout, dq, dk_pool, dv_pool, *, scale: float,
                     workspace=None, stream=None) -> None:
    """Paged GQA backward into dq, dk_pool, dv_pool (see pa_attention_bwd in
    paged_attn.h); out and lse are the forward's."""
    import torch
    d = plan.desc
    dt = _dtype_code(q)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool), ("out", out), ("dout", dout), ("dq", dq),
                    ("dk_pool", dk_pool), ("dv_pool", dv_pool)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    D, Dv = int(q.shape[2]), int(v_pool.shape[3])
    Q, Hq = d["num_queries"], d["num_q_heads"]
    pool = (d["num_pages"], d["page_size"], d["num_kv_heads"])
    for name, t, shape in (("q", q, (Q, Hq, D)), ("out", out, (Q, Hq, Dv)), ("dout", dout, (Q, Hq, Dv)),
                           ("dq", dq, (Q, Hq, D)), ("k_pool", k_pool, pool + (D,)), ("v_pool", v_pool, pool + (Dv,)),
                           ("dk_pool", dk_pool, pool + (D,)), ("dv_pool", dv_pool, pool + (Dv,))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Q, Hq):
        raise ValueError("lse must be float32 [Q, Hq]")
    wp, wn = _ws(workspace)
    _check(load_library().pa_attention_bwd(
        plan.handle, dt, _dev(q, "q", 3), _dev(k_pool, "k_pool", 4), _dev(v_pool, "v_pool", 4), _dev(out, "out", 3),
        _dev(lse, "lse", 2), _dev(dout, "dout", 3), _dev(dq, "dq", 3), _dev(dk_pool, "dk_pool", 4),
        _dev(dv_pool, "dv_pool", 4), D, Dv, float(scale), wp, wn, _stream_handle(stream)), "pa_attention_bwd")


def pa_mla_bwd(plan: Plan, q_abs, q_rope, latent, kpos, out, lse, dout, dq_abs, dq_rope, dlatent, dkpos, *,
               scale: float, workspace=None, stream=None) -> None:
    """Absorbed-MLA backward into dq_abs, dq_rope, dlatent, dkpos (see
    pa_mla_bwd in paged_attn.h); out and lse are the forward's."""
    import torch
    d = plan.desc
    dt = _dtype_code(q_abs)
    R, P = int(q_abs.shape[2]), int(q_rope.shape[2])
    Q, H = d["num_queries"], d["num_q_heads"]
    pool = (d["num_pages"], d["page_size"], 1)
    for name, t, shape in (("q_abs", q_abs, (Q, H, R)), ("q_rope", q_rope, (Q, H, P)), ("out", out, (Q, H, R)),
                           ("dout", dout, (Q, H, R)), ("dq_abs", dq_abs, (Q, H, R)), ("dq_rope", dq_rope, (Q, H, P)),
                           ("latent", latent, pool + (R,)), ("kpos", kpos, pool + (P,)),
                           ("dlatent", dlatent, pool + (R,)), ("dkpos", dkpos, pool + (P,))):
        if t.dtype != q_abs.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q_abs dtype {q_abs.dtype}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Q, H):
        raise ValueError("lse must be float32 [Q, H]")
    wp, wn = _ws(workspace)
    _check(load_library().pa_mla_bwd(
        plan.handle, dt, _dev(q_abs, "q_abs", 3), _dev(q_rope, "q_rope", 3), _dev(latent, "latent", 4),
        _dev(kpos, "kpos", 4), _dev(out, "out", 3), _dev(lse, "lse", 2), _dev(dout, "dout", 3),
        _dev(dq_abs, "dq_abs", 3), _dev(dq_rope, "dq_rope", 3), _dev(dlatent, "dlatent", 4), _dev(dkpos, "dkpos", 4),
        R, P, float(scale), wp, wn, _stream_handle(stream)), "pa_mla_bwd")


def pa_mla_fwd(plan: Plan, q_abs, q_rope, latent, kpos, out, lse=None, *, scale: float, workspace=None,
               main_events=None, stream=None) -> None:
    """Absorbed-MLA forward into `out` (see pa_mla_fwd in paged_attn.h);
    main_events as for pa_attention_fwd."""
    d = plan.desc
    dt = _dtype_code(q_abs)
    for name, t in (("q_rope", q_rope), ("latent", latent), ("kpos", kpos), ("out", out)):
        if t.dtype != q_abs.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q_abs dtype {q_abs.dtype}")
    pa_, pr, pl_, pk, po = (_dev(q_abs, "q_abs", 3), _dev(q_rope, "q_rope", 3), _dev(latent, "latent", 4),
                            _dev(kpos, "kpos", 4), _dev(out, "out", 3))
    R, P = int(q_abs.shape[2]), int(q_rope.shape[2])
    Q, H = d["num_queries"], d["num_q_heads"]
    pool = (d["num_pages"], d["page_size"], 1)
    if tuple(q_abs.shape) != (Q, H, R) or tuple(q_rope.shape) != (Q, H, P):
        raise ValueError("q_abs / q_rope shapes do not match the plan")
    if tuple(latent.shape) != pool + (R,) or tuple(kpos.shape) != pool + (P,):
        raise ValueError("MLA latent cache must have one shared head and match the plan's pool")
    if tuple(out.shape) != (Q, H, R):
        raise ValueError("out shape does not match [Q, H, R]")
    plse = None
    if lse is not None:
        import torch
        if lse.dtype != torch.float32 or tuple(lse.shape) != (Q, H):
            raise ValueError("lse must be float32 [Q, H]")
        plse = _dev(lse, "lse", 2)
    wp, wn = _ws(workspace)
    ev = _events(main_events)
    _check(load_library().pa_mla_fwd(plan.handle, dt, pa_, pr, pl_, pk, po, plse, R, P, float(scale), wp, wn,
                                     ev, _stream_handle(stream)), "pa_mla_fwd")


def pa_append_kv(plan: Plan, k_new, v_new, k_pool, v_pool, *, stream=None) -> None:
    """Write the new K/V rows of every query into its pool slot (see
    pa_append_kv in paged_attn.h)."""
    d = plan.desc
    dt = _dtype_code(k_pool)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("v_pool", v_pool)):
        if t.dtype != k_pool.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from k_pool dtype {k_pool.dtype}")
    pk, pv = _dev(k_pool, "k_pool", 4), _dev(v_pool, "v_pool", 4)
    Q, heads = d["num_queries"], d["num_kv_heads"]
    D, Dv = int(k_pool.shape[3]), int(v_pool.shape[3])
    pool = (d["num_pages"], d["page_size"], heads)
    if tuple(k_pool.shape[:3]) != pool or tuple(v_pool.shape[:3]) != pool:
        raise ValueError(f"pool shapes {tuple(k_pool.shape)}, {tuple(v_pool.shape)} do not match {pool} x (D, Dv)")
    if tuple(k_new.shape) != (Q, heads, D) or tuple(v_new.shape) != (Q, heads, Dv):
        raise ValueError(f"new-row shapes {tuple(k_new.shape)}, {tuple(v_new.shape)} != {(Q, heads, D)}, {(Q, heads, Dv)}")
    pkn, pvn = _dev(k_new, "k_new", 3), _dev(v_new, "v_new", 3)
    _check(load_library().pa_append_kv(plan.handle, dt, pkn, pvn, pk, pv, D, Dv, _stream_handle(stream)),
           "pa_append_kv")
