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

// Launcher of one GQA kernel (decode, mixed or merge) for one data type, head
// size pair and group size.
using LaunchFn = hipError_t (*)(const KernelArgs&, int n_wg, const MergeItem* merges, int n_merges,
                                const MainEvents& ev, hipStream_t stream);
// The kernels of one group size (a launcher is null when no kernel exists
// for that data type and head size pair) and the decode launch shape.
struct GqaFamily {
  LaunchFn decode = nullptr, decode_short = nullptr, mixed = nullptr, merge = nullptr;
  int waves = 1, wgs_per_cu = 1;
};
// Lookups of the two translation units that instantiate the group sizes
// (false when g is not among theirs).
bool gqa_family_pow2(int dtype, int d, int dv, int g, GqaFamily* out);
bool gqa_family_other(int dtype, int d, int dv, int g, GqaFamily* out);

bool gqa_supported(int dtype, int d, int dv, int g);
bool prefill_supported(int dtype, int d, int dv, int g);
// Main GQA launch over the a.n_items entries of a.items: decode-only, or one
// mixed launch when the list holds prefill tiles.
hipError_t launch_gqa_main(int dtype, int d, int dv, int g, bool has_prefill, const KernelArgs& a,
                           const MainEvents& ev, hipStream_t stream);
// Waves per workgroup of the decode launch for short items.
constexpr int kShortItemWaves = 2;
// Decode launch over a list of short items (a few key blocks each): fewer
// waves per workgroup than the main decode launch.
hipError_t launch_gqa_short(int dtype, int d, int dv, int g, const KernelArgs& a, hipStream_t stream);
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

// Absorbed MLA: h query heads, latent rank r, position width p.  The kernels
// take the heads in groups of kMlaGroupHeads (the MFMA columns): a work item
// or dQ item covers one group (the last one may be partial), and split
// partials hold kMlaGroupHeads heads per slot.
constexpr int kMlaGroupHeads = 16;
constexpr int kMlaMaxRank = 1024, kMlaMaxRope = 256;
// Forward: any dtype, 1 <= r <= kMlaMaxRank, 1 <= p <= kMlaMaxRope, h >= 1
// (16-bit data with r = 512, p = 64 on MFMA, the rest on the vector kernel).
bool mla_supported(int dtype, int h, int r, int p);
// Backward: 16-bit data, r = 512, p = 64, h >= 1.
bool mla_bwd_supported(int dtype, int h, int r, int p);
// has_prefill: the item list holds chunked-prefill items.
hipError_t launch_mla_main(int dtype, int r, int p, bool has_prefill, const KernelArgs& a, const MainEvents& ev,
                           hipStream_t stream);
hipError_t launch_mla_merge(int dtype, int r, int p, const KernelArgs& a, const MergeItem* merges, int n_merges,
                            hipStream_t stream);

// The vector-ALU forward for every shape the specialised kernels do not take
// (pa_generic.hip).  Key rows are [k1 | k2] (d1 + d2 wide; GQA: d2 = 0, MLA:
// latent | kpos), query rows [q1 | q2], value rows dv wide (v_is_k: the
// first dv dims of k1, as the MLA latent).  Work unit u of a plan covers
// query heads (u / nsub) g + (u % nsub) unit_heads .. + unit_heads - 1 (at
// most g - (u % nsub) unit_heads of them) of KV head u / nsub; a decode
// item covers hw consecutive units (nsub = 1).  Split partials hold
// unit_heads heads per slot.
constexpr int kGenericUnitHeads = 16;
constexpr int kGenericMaxKeyWidth = kMlaMaxRank + kMlaMaxRope, kGenericMaxValueWidth = 1024;
struct GenericShape {
  int32_t d1, d2, dv, g, nsub, unit_heads, hw, v_is_k;
};
bool generic_shape_ok(const GenericShape& s);
hipError_t launch_generic(int dtype, const GenericShape& s, const KernelArgs& a, const MainEvents& ev,
                          hipStream_t stream);
hipError_t launch_generic_merge(int dtype, const GenericShape& s, const KernelArgs& a, const MergeItem* merges,
                                int n_merges, hipStream_t stream);

// Paged K/V append: rows (i, h) of k_new [Q, heads, k_row_bytes] and v_new
// [Q, heads, v_row_bytes] to pool rows (slot_of[i], h).  Row sizes are
// multiples of 16 bytes; n_cu sizes the grid.
hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* slot_of,
                         int64_t queries, int heads, int k_row_bytes, int v_row_bytes, int n_cu, hipStream_t stream);

// Absorbed-MLA backward (16-bit data, H = 16, R = 512, P = 64): zero the
// latent / rotary gradient pools (or their f32 sums `acc`, pool_slots x (R +
// P) floats, when pages are shared), D = dO . O, dq_abs / dq_rope over items
// [0, n_dq) (one per query), dlatent / dkpos over [n_dq, n_dq + n_kv) (one
// per block of keys), then the sums rounded into the pools.
hipError_t launch_mla_bwd(int dtype, const KernelArgs& a, const void* dout, void* dq_abs, void* dq_rope, void* dlat,
                          void* dkpos, float* delta, float* acc, bool shared, const BwdItem* items, int n_dq, int n_kv,
                          const int32_t* zero_runs, int n_zero_runs, int64_t rows, int64_t pool_slots, int n_cu,
                          hipStream_t stream);

// Block-sparse top-k selection: one workgroup per (query, KV head) row
// scores the row's candidate blocks, keeps `topk` of them (all when topk is
// 0 or covers every candidate) and writes, at [row * width, + width), one
// decode item per kept block (increasing block order, kEmpty padding), the
// identity workgroup map and the row's merge record.
constexpr int kSparseMaxBlocks = 8192;  // candidate blocks of one row (LDS scores)
constexpr int kSparseMaxDim = 1024;     // K head size (LDS proxy query)
struct SparseArgs {
  const void* q;  // [Q, Hq, D]
  const void* k;  // [pages, ps, Hkv, D]
  const int32_t* block_table;
  const int32_t* q_pos;
  const int32_t* seq_lens;
  const int32_t* seq_of;  // sequence of each packed query
  int32_t table_width, page_shift, hq, hkv, d, causal, window;
  int32_t block_size, topk, width;
  int32_t* selection;  // [Q, Hkv, width] kept blocks, -1 padded, or null
  WorkItem* items;     // [Q * Hkv * width]
  int32_t* wg_first;   // [Q * Hkv * width + 1]
  MergeItem* merges;   // [Q * Hkv]
  uint32_t* scores;    // [Q * Hkv, cand_width] order-mapped block scores of the candidates
  int32_t cand_width;  // candidate blocks of the widest row
  int32_t span;        // keys per scoring workgroup: a multiple of block_size, aligned to itself
  int32_t spans;       // scoring workgroups per row (the widest row's span count)
  int32_t items_per_wg;  // kept blocks per attention workgroup
};
// Kept blocks one attention workgroup runs (one after another).
constexpr int kSparseItemsPerWg = 1;
// Keys one scoring workgroup covers for blocks of `block_size` keys.
inline int sparse_span(int block_size) { return block_size * (block_size >= 1024 ? 1 : 1024 / block_size); }
hipError_t launch_sparse_select(int dtype, const SparseArgs& a, int rows, hipStream_t stream);

// Paged GQA/MHA backward: zero the dk / dv rows (pool shaped, pool_slots rows
// of each) that no dK/dV item writes (zero_runs: n_zero_runs pairs (first
// slot, count); with shared pages the whole f32 sums instead),
// D = dO . O for the `rows` (query, head) rows into delta, then dQ (per-query
// items [0, n_dq), or on MFMA the row tiles [n_dq + n_kv, + n_dqt)) and
// dK / dV over items [n_dq, n_dq + n_kv).  `shared` (a pool page holds two
// key positions): dK / dV are added up in f32 -- in the pools for f32 data,
// else in `acc` (pool_slots x (d + dv) floats) rounded into the pools last.
bool bwd_supported(int dtype, int d, int dv, int g);
// The vector-ALU backward of every other shape (GQA or MLA in the forward
// vector kernel's description): the same items (dQ per (query, work unit),
// dK/dV per (key block, KV head)), zeroing, f32 sums for shared pages and
// D pass as the specialised launches.  dq / dq2: gradients of the q1 / q2
// query parts; dk / dvp: pools of rows s.d1 wide and (GQA) s.dv or (MLA)
// s.d2 wide, pool_rows rows each (MLA: dk is the latent pool, receiving
// the key and value terms).  acc: f32 sums of pool_rows x (both widths).
hipError_t launch_generic_bwd(int dtype, const GenericShape& s, const KernelArgs& a, const void* dout, void* dq,
                              void* dq2, void* dk, void* dvp, float* delta, float* acc, bool shared,
                              const BwdItem* items, int n_dq, int n_kv, const int32_t* zero_runs, int n_zero_runs,
                              int64_t rows, int64_t pool_rows, int n_cu, hipStream_t stream);
hipError_t launch_gqa_bwd(int dtype, int d, int dv, int g, const KernelArgs& a, const void* dout, void* dq, void* dk,
                          void* dvp, float* delta, float* acc, bool shared, const BwdItem* items, int n_dq, int n_kv,
                          int n_dqt, const int32_t* zero_runs, int n_zero_runs, int64_t rows, int64_t pool_slots,
                          int n_cu, hipStream_t stream);


}  // namespace pa
