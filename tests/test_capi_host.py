"""Host-side checks of the C-ABI library that need no GPU: every symbol the
header declares is exported, and malformed schedules are rejected before any
HIP call, with the status classes of the header (error-before-launch, as
ruDNN `execute_attention_into` does)."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_attention_gqa_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "paged_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = pa.load_library()
    declared = _declared_functions()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in paged_attn.h but not exported"
    assert set(declared) == set(pa.EXPORTED)


def test_status_strings():
    for code in pa.STATUS_NAMES:
        assert pa.pa_status_string(code)
    assert pa.pa_status_string(123) == "unknown status"


def _good():
    return dict(seq_lens=np.array([20, 7], np.int32), cu_q=np.array([0, 1, 3], np.int32),
                q_pos=np.array([19, 5, 6], np.int32), block_table=np.array([[0, 2], [1, -1]], np.int32),
                page_size=16, num_pages=3, num_q_heads=8, num_kv_heads=2)


def _expect(status_name, **over):
    kw = _good()
    kw.update(over)
    seq = {k: kw.pop(k) for k in ("seq_lens", "cu_q", "q_pos", "block_table")}
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan_create(seq["seq_lens"], seq["cu_q"], seq["q_pos"], seq["block_table"], **kw)
    assert e.value.name == status_name, str(e.value)
    assert pa.pa_last_error()


@pytest.mark.parametrize("over,status", [
    (dict(num_q_heads=6, num_kv_heads=4), "PA_ERR_SHAPE"),
    (dict(num_kv_heads=0), "PA_ERR_SHAPE"),
    (dict(page_size=12), "PA_ERR_UNSUPPORTED"),
    (dict(page_size=0), "PA_ERR_PLAN"),
    (dict(max_splits=0), "PA_ERR_INVALID"),
    (dict(max_splits=65), "PA_ERR_INVALID"),
    (dict(window=-1), "PA_ERR_INVALID"),
    (dict(q_pos=np.array([20, 5, 6], np.int32)), "PA_ERR_PLAN"),        # position == length
    (dict(q_pos=np.array([19, -1, 6], np.int32)), "PA_ERR_PLAN"),
    (dict(cu_q=np.array([1, 1, 3], np.int32)), "PA_ERR_PLAN"),
    (dict(cu_q=np.array([0, 2, 1], np.int32), q_pos=np.array([19], np.int32)), "PA_ERR_PLAN"),
    (dict(block_table=np.array([[0, 3], [1, -1]], np.int32)), "PA_ERR_PLAN"),  # page outside pool
    (dict(block_table=np.array([[0, -1], [1, -1]], np.int32)), "PA_ERR_PLAN"),  # used entry missing
    (dict(seq_lens=np.array([33, 7], np.int32)), "PA_ERR_PLAN"),         # longer than the table
    (dict(seq_lens=np.array([-1, 7], np.int32)), "PA_ERR_PLAN"),
    (dict(mla=True), "PA_ERR_SHAPE"),                                    # MLA needs one KV head
    (dict(num_pages=0), "PA_ERR_PLAN"),
])
def test_plan_rejects_malformed_schedules(over, status):
    _expect(status, **over)


def test_forward_rejects_null_plan():
    lib = pa.load_library()
    rc = lib.pa_attention_fwd(None, 0, None, None, None, None, None, 64, 64, 1.0, None, 0, None, None)
    assert rc == -1 and "plan" in pa.pa_last_error()
    rc = lib.pa_mla_fwd(None, 1, None, None, None, None, None, None, 512, 64, 1.0, None, 0, None, None)
    assert rc == -1


def test_plan_create_rejects_null_descriptor():
    lib = pa.load_library()
    h = ctypes.c_void_p()
    assert lib.pa_plan_create(None, None, ctypes.byref(h)) == -1
    assert lib.pa_plan_create(None, None, None) == -1
    assert not h.value


def test_destroy_null_is_ok():
    assert pa.load_library().pa_plan_destroy(None) == 0


def test_info_and_workspace_reject_null():
    lib = pa.load_library()
    n = ctypes.c_size_t()
    assert lib.pa_plan_workspace_bytes(None, 128, ctypes.byref(n)) == -1
    assert lib.pa_plan_get_info(None, None) == -1
