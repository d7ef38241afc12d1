// Host-visible launchers of the paged-attention kernels (internal to the
// library; the public boundary is include/paged_attn.h).
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"

namespace pa {

// Optional timing events of a main attention launch: when set, the launch
// records the start and end of the kernel's own execution into them
// (hipExtLaunchKernel).
struct MainEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// dtype: 0 = f32, 1 = bf16, 2 = f16.  d, dv: K and V head sizes.  g: query
// heads per KV head.
bool gqa_supported(int dtype, int d, int dv, int g);
bool prefill_supported(int dtype, int d, int dv, int g);
// Main GQA launch over the a.n_items entries of a.items: decode-only, or one
// mixed launch when the list holds prefill tiles.
hipError_t launch_gqa_main(int dtype, int d, int dv, int g, bool has_prefill, const KernelArgs& a,
                           const MainEvents& ev, hipStream_t stream);
// Log-sum-exp merge of split rows into the output.
hipError_t launch_gqa_merge(int dtype, int d, int dv, int g, const KernelArgs& a, const MergeItem* merges,
                            int n_merges, hipStream_t stream);

// Workgroups of the decode-only (group size g) and MLA kernels that one CU
// holds at once; the planner balances decode work over CUs x this many.
int decode_wgs_per_cu(int g);
// Waves of one decode-only workgroup (group size g): an item may cover up to
// this many KV heads.
int decode_waves(int g);
int mla_wgs_per_cu();

// Absorbed MLA: h query heads, latent rank r, position width p.
bool mla_supported(int dtype, int h, int r, int p);
// has_prefill: the item list holds chunked-prefill items.
hipError_t launch_mla_main(int dtype, bool has_prefill, const KernelArgs& a, const MainEvents& ev,
                           hipStream_t stream);
hipError_t launch_mla_merge(int dtype, const KernelArgs& a, const MergeItem* merges, int n_merges,
                            hipStream_t stream);

// Paged K/V append: rows (i, h) of k_new [Q, heads, k_row_bytes] and v_new
// [Q, heads, v_row_bytes] to pool rows (slot_of[i], h).  Row sizes are
// multiples of 16 bytes; n_cu sizes the grid.
hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* slot_of,
                         int64_t queries, int heads, int k_row_bytes, int v_row_bytes, int n_cu, hipStream_t stream);

// Paged GQA/MHA backward: zero dk / dv (pool shaped, pool_slots rows of each),
// D = dO . O for the `rows` (query, head) rows into delta, then dQ (per-query
// items [0, n_dq), or on MFMA the row tiles [n_dq + n_kv, + n_dqt)) and
// dK / dV over items [n_dq, n_dq + n_kv).  `shared` (a pool page holds two
// key positions): dK / dV are added up in f32 -- in the pools for f32 data,
// else in `acc` (pool_slots x (d + dv) floats) rounded into the pools last.
bool bwd_supported(int dtype, int d, int dv, int g);
hipError_t launch_gqa_bwd(int dtype, int d, int dv, int g, const KernelArgs& a, const void* dout, void* dq, void* dk,
                          void* dvp, float* delta, float* acc, bool shared, const BwdItem* items, int n_dq, int n_kv,
                          int n_dqt, int64_t rows, int64_t pool_slots, int n_cu, hipStream_t stream);


}  // namespace pa
