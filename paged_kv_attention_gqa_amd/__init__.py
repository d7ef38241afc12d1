"""MI355X (gfx950) paged-KV attention: a C-ABI HIP library (libpaged_attn.so,
declared in include/paged_attn.h) and its thin ctypes binding.

The library is loaded on first use; importing this package loads nothing."""
from ._binding import (  # noqa: F401
    PaError, Plan, load_library, pa_append_kv, pa_attention_bwd, pa_attention_fwd, pa_attention_fwd_noalloc,
    pa_last_error, pa_mla_bwd, pa_mla_fwd, pa_sparse_attention_fwd, pa_sparse_workspace_bytes,
    pa_plan_bwd_workspace_bytes, pa_plan_create, pa_plan_create_host,
    pa_plan_destroy, pa_plan_get_info, pa_plan_get_work, pa_plan_workspace_bytes, pa_status_string, EXPORTED,
    LIB_PATH, STATUS_NAMES,
)
