// Host side of the C ABI declared in include/paged_attn.h: schedule
// validation, work-list planning, plan upload, argument checks and kernel
// dispatch.  Nothing here synchronises with the device or reads device memory
// back on the forward path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <tuple>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <new>
#include <string>
#include <mutex>
#include <vector>

#include "paged_attn.h"
#include "pa_host.h"
#include "pa_launch.h"
#include "pa_prefill.h"

using pa::MergeItem;
using pa::WorkItem;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

// Sequences with at most this many queries run as per-query decode items;
// longer runs of queries become prefill tiles of kPrefillRows query rows.
constexpr int kDecodeMaxQueries = 4;
constexpr int kPrefillRows = pa::kPrefillRows;
constexpr int kDefaultSplitTokens = 512;
// In a launch that also runs prefill tiles, a decode item is worked by the
// prefill workgroup's eight waves: give it proportionally more keys (on the
// mixed batch with its 4096-key window, rows cut at 4096 keys -- whole rows --
// ran 2% faster than rows cut at 2048, 3% faster than at 1024).
constexpr int kMixedSplitTokens = 4096;
constexpr int kDefaultMlaSplitTokens = 1024;
constexpr int kSplitAlign = 64;
// Shortest piece of a split decode row in a balanced plan: a piece's partial
// results (G x Dv floats for GQA, 16 x 512 for MLA) should stay small next to
// the keys it reads.
constexpr int kMinPieceKeys = 128;
constexpr int kMlaMinPieceKeys = 256;
// Waves that share one KV head of a balanced decode item.  Fewer waves per
// head (more heads per workgroup) means shorter pieces for the same number
// of workgroups, so more splits per row; four keeps the piece count of a
// one-head workgroup of four waves.
constexpr int kDecodeWavesPerHead = 4;
constexpr int kMaxSplitsLimit = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

int pa::host_fail(int status, const char* msg) { return fail(status, "%s", msg); }

struct pa_plan {
  int device = -1;
  // every device-side use of the plan (upload, forward, append, backward and
  // the final free) is ordered on this stream
  hipStream_t created_on = nullptr;
  hipEvent_t uploaded = nullptr;  // the upload copy (reads the host blob) has finished
  // schedule, host copy
  int32_t S = 0, Q = 0, W = 0, ps = 1, page_shift = 0, num_pages = 0;
  int32_t hq = 0, hkv = 0, causal = 0, window = 0, max_splits = 1, mla = 0, split_tokens = 0;
  std::vector<int32_t> seq_lens, cu_q, q_pos, bt;
  // work lists, host copy
  std::vector<WorkItem> items;    // grouped by workgroup, launch order
  std::vector<int32_t> wg_first;  // workgroup b runs items wg_first[b] .. wg_first[b + 1] - 1
  std::vector<MergeItem> merges;
  int32_t n_decode = 0, n_prefill = 0, n_slots = 0;
  int32_t heads_shift = 0;        // decode items cover 2^heads_shift consecutive units (KV heads, MLA head groups)
  int32_t n_wg = 0;               // workgroups of the main launch
  int32_t n_cu = 0;               // compute units of the plan's device
  // append: pool slot (page * page_size + slot) of every query's position,
  // and the first query whose slot another query also writes (-1: none)
  std::vector<int32_t> slot_of;
  int32_t dup_query = -1;
  std::vector<int32_t> seq_of;    // sequence of each packed query (block-sparse selection)
  // backward (GQA plans): dQ items, then dK/dV items; a page that two key
  // positions share (-1: none) makes the single-writer dK/dV pass impossible
  std::vector<pa::BwdItem> bwd_items;
  int32_t n_bwd_dq = 0, n_bwd_kv = 0, n_bwd_dqt = 0;
  // backward, single-writer mode: runs (first pool slot, count) of the slots
  // no dK/dV item writes, which are zeroed instead
  std::vector<int32_t> zero_runs;
  int32_t shared_page = -1;
  // The backward lists are built on first need (a backward call, its
  // workspace size or pa_plan_get_info), so that forward-only plans do not
  // pay for them; the device copy is uploaded by the first backward call.
  std::mutex bwd_mu;
  bool bwd_built = false;
  std::vector<char> bwd_blob;
  char* bwd_dev = nullptr;
  hipEvent_t bwd_uploaded = nullptr;
  // device copy: one allocation
  std::vector<char> blob;
  char* dev = nullptr;
  const int32_t* d_bt = nullptr;
  const int32_t* d_qpos = nullptr;
  const int32_t* d_lens = nullptr;
  const WorkItem* d_items = nullptr;
  const int32_t* d_wg_first = nullptr;
  const int32_t* d_slot_of = nullptr;
  const int32_t* d_seq_of = nullptr;
  const MergeItem* d_merges = nullptr;
  const pa::BwdItem* d_bwd = nullptr;
  const int32_t* d_zero_runs = nullptr;

  int group() const { return hq / hkv; }
  // Work units of one query row.  GQA with G <= kGenericUnitHeads: its KV
  // heads (a unit: one KV head and its G query heads).  MLA (one shared
  // latent head) and GQA with a larger G: the query heads of each KV head
  // in groups of kGenericUnitHeads (= kMlaGroupHeads), nsub groups per KV
  // head, the last one possibly partial.  unit_heads: query heads per unit
  // (and per split-partial slot).
  bool grouped() const { return mla || hq / hkv > pa::kGenericUnitHeads; }
  int nsub() const { return grouped() ? (group() + pa::kGenericUnitHeads - 1) / pa::kGenericUnitHeads : 1; }
  int units() const { return hkv * nsub(); }
  int unit_heads() const { return grouped() ? pa::kGenericUnitHeads : group(); }
};

namespace {

// Keys visible to a query at position p in a sequence of L keys form one
// contiguous range [lo, hi] (boostr `build_attention_mask` on absolute
// positions); p < L guarantees it holds p itself.
void visible_range(int p, int L, int causal, int window, int* lo, int* hi) {
  *hi = causal ? p : L - 1;
  *lo = window > 0 ? std::max(0, p - window + 1) : 0;
}

int validate_desc(const pa_plan_desc* d) {
  if (!d) return fail(PA_ERR_INVALID, "plan descriptor is NULL");
  if (d->num_seqs < 0) return fail(PA_ERR_PLAN, "num_seqs %d < 0", d->num_seqs);
  if (d->num_seqs > 0 && (!d->seq_lens || !d->cu_q || !d->block_table))
    return fail(PA_ERR_INVALID, "seq_lens, cu_q and block_table are required when num_seqs > 0");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "head counts Hq=%d Hkv=%d: need Hkv > 0 dividing Hq", d->num_q_heads,
                d->num_kv_heads);
  if (d->mla != 0 && d->mla != 1) return fail(PA_ERR_INVALID, "mla must be 0 or 1");
  if (d->mla && d->num_kv_heads != 1) return fail(PA_ERR_SHAPE, "MLA latent cache must have one shared head");
  if (d->causal != 0 && d->causal != 1) return fail(PA_ERR_INVALID, "causal must be 0 or 1");
  if (d->window < 0) return fail(PA_ERR_INVALID, "window %d < 0", d->window);
  if (d->max_splits < 1 || d->max_splits > kMaxSplitsLimit)
    return fail(PA_ERR_INVALID, "max_splits %d outside [1, %d]", d->max_splits, kMaxSplitsLimit);
  if (d->split_tokens < 0) return fail(PA_ERR_INVALID, "split_tokens %d < 0", d->split_tokens);
  if (d->page_size <= 0) return fail(PA_ERR_PLAN, "page_size %d <= 0", d->page_size);
  if ((d->page_size & (d->page_size - 1)) != 0 || d->page_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "page_size %d: kernels need a power of two <= 1024", d->page_size);
  if (d->num_pages <= 0) return fail(PA_ERR_PLAN, "num_pages %d <= 0", d->num_pages);
  if (d->num_seqs > 0 && d->table_width <= 0) return fail(PA_ERR_PLAN, "table_width %d <= 0", d->table_width);
  if ((int64_t)d->num_seqs * std::max(d->table_width, 1) > INT32_MAX)
    return fail(PA_ERR_RANGE, "block table exceeds 32-bit indexing");
  if ((int64_t)d->num_pages * d->page_size > INT32_MAX)
    return fail(PA_ERR_RANGE, "pool slots exceed 32-bit indexing");
  if (d->num_seqs == 0) return PA_OK;
  if (d->cu_q[0] != 0) return fail(PA_ERR_PLAN, "cu_q[0] = %d, expected 0", d->cu_q[0]);
  for (int s = 0; s < d->num_seqs; ++s)
    if (d->cu_q[s + 1] < d->cu_q[s]) return fail(PA_ERR_PLAN, "cu_q decreases at sequence %d", s);
  const int64_t Q = d->cu_q[d->num_seqs];
  if (Q * d->num_q_heads > INT32_MAX) return fail(PA_ERR_RANGE, "queries x heads exceed 32-bit indexing");
  if (Q > 0 && !d->q_pos) return fail(PA_ERR_INVALID, "q_pos is required when there are queries");
  for (int s = 0; s < d->num_seqs; ++s) {
    const int L = d->seq_lens[s];
    if (L < 0) return fail(PA_ERR_PLAN, "seq_lens[%d] = %d < 0", s, L);
    if ((int64_t)L > (int64_t)d->table_width * d->page_size)
      return fail(PA_ERR_PLAN, "seq_lens[%d] = %d exceeds table_width x page_size", s, L);
    for (int i = d->cu_q[s]; i < d->cu_q[s + 1]; ++i)
      if (d->q_pos[i] < 0 || d->q_pos[i] >= L)
        return fail(PA_ERR_PLAN, "q_pos[%d] = %d outside [0, seq_lens[%d] = %d)", i, d->q_pos[i], s, L);
    const int pages = (L + d->page_size - 1) / d->page_size;
    for (int j = 0; j < pages; ++j) {
      const int pg = d->block_table[(int64_t)s * d->table_width + j];
      if (pg < 0 || pg >= d->num_pages)
        return fail(PA_ERR_PLAN, "block_table[%d][%d] = %d outside [0, %d)", s, j, pg, d->num_pages);
    }
  }
  return PA_OK;
}

// Split one decode query row's visible range into page-friendly key ranges,
// one item per (range, group of 2^heads_shift KV heads), KV heads innermost:
// the heads of one key range run side by side and together read whole
// [Hkv, D] slot rows of each page.  Partial slots of a split row are laid out
// [range][KV head]; an item's slot is its first head's.
void plan_decode_row(pa_plan* p, int s, int i, int split_tokens, std::vector<WorkItem>& out) {
  const int hw = 1 << p->heads_shift, U = p->units();
  int lo, hi;
  visible_range(p->q_pos[i], p->seq_lens[s], p->causal, p->window, &lo, &hi);
  const int n = hi - lo + 1;
  int nsplit = std::min(p->max_splits, (n + split_tokens - 1) / split_tokens);
  nsplit = std::max(nsplit, 1);
  int chunk = n;
  if (nsplit > 1) {
    chunk = (n + nsplit - 1) / nsplit;
    chunk = (chunk + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    nsplit = (n + chunk - 1) / chunk;
  }
  if (nsplit == 1) {
    for (int kvh = 0; kvh < U; kvh += hw) out.push_back(WorkItem{pa::kDecode, kvh, s, i, 1, lo, hi + 1, -1});
    return;
  }
  const int base = p->n_slots;
  for (int j = 0; j < nsplit; ++j) {
    const int b = lo + j * chunk, e = std::min(hi + 1, b + chunk);
    for (int kvh = 0; kvh < U; kvh += hw)
      out.push_back(WorkItem{pa::kDecode, kvh, s, i, 1, b, e, base + j * U + kvh});
  }
  for (int kvh = 0; kvh < U; ++kvh) p->merges.push_back(MergeItem{i, kvh, base + kvh, nsplit, U});
  p->n_slots += nsplit * U;
}

// Estimated run time of an item, in units of one decode key: a decode item
// streams its keys once; a prefill tile of kPrefillTileKeys keys times up to
// kPrefillRows query rows costs about kPrefillKeyCost decode keys per key;
// every item pays a fixed start-up cost.
constexpr int64_t kPrefillKeyCost = 2;
constexpr int64_t kItemStartCost = 64;
int64_t item_cost(const WorkItem& w) {
  if (w.kind == pa::kPrefill) {
    constexpr int NT = pa::kPrefillTileKeys;
    const int64_t tiles = (w.tok_end - (w.tok_begin & ~(NT - 1)) + NT - 1) / NT;
    return tiles * NT * kPrefillKeyCost + kItemStartCost;
  }
  return (int64_t)(w.tok_end - w.tok_begin) + kItemStartCost;
}

// Dispatch order of the work list.  Workgroup b of a launch goes to XCD b % 8
// and each XCD starts its workgroups in order as CUs free up, so the list is
// built per XCD and interleaved.  Units of work are dealt, largest first, to
// the XCD with the least estimated work so far; a unit is one decode item or
// all prefill tiles of one (sequence, KV head), which read the same keys and
// so share one L2 (with head groups, as in MLA: all prefill tiles of one
// sequence and KV head, and the decode items of all head groups of one KV
// head and key range).  Each XCD then runs its items longest first; XCDs with
// fewer items are padded with empty items.
constexpr int kXcds = 8;
void order_items(pa_plan* p, const std::vector<WorkItem>& pre, const std::vector<WorkItem>& dec) {
  std::vector<std::vector<WorkItem>> units;
  std::vector<int64_t> unit_cost;
  std::map<std::tuple<int, int, int>, size_t> group_of;
  auto add = [&](std::tuple<int, int, int> key, const WorkItem& w) {
    auto g = group_of.find(key);
    if (g == group_of.end()) {
      g = group_of.emplace(key, units.size()).first;
      units.emplace_back();
      unit_cost.push_back(0);
    }
    units[g->second].push_back(w);
    unit_cost[g->second] += item_cost(w);
  };
  const int nsub = p->nsub();
  for (const WorkItem& w : pre) add({w.seq, w.kvh / nsub, 0}, w);
  for (const WorkItem& w : dec) {
    if (nsub > 1) {
      // the head groups of one KV head and key range read the same K/V rows
      add({-1 - w.q_begin, w.tok_begin, w.kvh / nsub}, w);
    } else {
      units.push_back({w});
      unit_cost.push_back(item_cost(w));
    }
  }
  std::vector<size_t> order(units.size());
  for (size_t u = 0; u < order.size(); ++u) order[u] = u;
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return unit_cost[a] > unit_cost[b]; });
  std::vector<std::vector<WorkItem>> bins(kXcds);
  int64_t load[kXcds] = {};
  for (size_t u : order) {
    const int x = (int)(std::min_element(load, load + kXcds) - load);
    bins[x].insert(bins[x].end(), units[u].begin(), units[u].end());
    load[x] += unit_cost[u];
  }
  size_t rows = 0;
  for (auto& b : bins) {
    std::stable_sort(b.begin(), b.end(), [](const WorkItem& a, const WorkItem& c) { return item_cost(a) > item_cost(c); });
    rows = std::max(rows, b.size());
  }
  p->items.clear();
  p->items.reserve(rows * kXcds);
  for (size_t j = 0; j < rows; ++j)
    for (int x = 0; x < kXcds; ++x)
      p->items.push_back(j < bins[x].size() ? bins[x][j] : WorkItem{pa::kEmpty, 0, 0, 0, 0, 0, 0, -1});
  while (!p->items.empty() && p->items.back().kind == pa::kEmpty) p->items.pop_back();
  p->wg_first.resize(p->items.size() + 1);
  for (size_t i = 0; i < p->wg_first.size(); ++i) p->wg_first[i] = (int32_t)i;
}

// Decode rows balanced over the workgroups resident at once (`slots` = CUs x
// workgroups per CU).  The key range of every query is cut into pieces and
// the pieces are dealt to groups of Hkv / 2^heads_shift workgroups, each
// workgroup taking 2^heads_shift consecutive KV heads, so that every
// workgroup gets about the same number of keys and the workgroups of a group
// (consecutive, so dispatched together) read the same page slots at the same
// time; the launch has no tail of lone workgroups.  Cuts fall on multiples
// of kSplitAlign keys; pieces are at least `min_piece` keys (each split piece
// costs a partial write and a merge read); a row is cut into at most
// max_splits pieces, earlier pieces growing
// when the rest of the row would not fit the remaining pieces at about one
// target each; a row cut into several pieces gets one partial slot per piece
// and a merge.  The target of each group is recomputed from the keys
// still unassigned, and the last group takes whatever remains.
void plan_balanced(pa_plan* p, int slots, int min_piece) {
  struct Row {
    int s, q, lo, hi;  // keys [lo, hi)
  };
  std::vector<Row> rows;
  int64_t left = 0;
  for (int s = 0; s < p->S; ++s)
    for (int i = p->cu_q[s]; i < p->cu_q[s + 1]; ++i) {
      int lo, hi;
      visible_range(p->q_pos[i], p->seq_lens[s], p->causal, p->window, &lo, &hi);
      rows.push_back(Row{s, i, lo, hi + 1});
      left += hi + 1 - lo;
    }
  const int hw = 1 << p->heads_shift, U = p->units();
  const int groups = std::max(1, slots / ((U + hw - 1) / hw));
  auto align_up = [](int64_t x) { return (x + kSplitAlign - 1) / kSplitAlign * kSplitAlign; };
  auto align_down = [](int64_t x) { return x / kSplitAlign * kSplitAlign; };
  struct Piece {
    int row, b, e, part;
  };
  std::vector<std::vector<Piece>> grp(1);
  std::vector<int> nparts(rows.size(), 0);
  int64_t fill = 0, target = (left + groups - 1) / groups;
  auto close_group = [&]() {
    if ((int)grp.size() >= groups) return;
    grp.emplace_back();
    fill = 0;
    const int64_t rest = groups - (int64_t)grp.size() + 1;
    target = (left + rest - 1) / rest;
  };
  for (size_t ri = 0; ri < rows.size(); ++ri) {
    const Row& r = rows[ri];
    int b = r.lo;
    while (b < r.hi) {
      const int64_t rem = r.hi - b, room = target - fill;
      // this piece must be long enough for the rest of the row to fit in the
      // pieces max_splits still allows, at about one target each
      const int64_t pieces_left = p->max_splits - nparts[ri];
      const int64_t min_len = std::max<int64_t>(min_piece, rem - (pieces_left - 1) * target);
      int64_t take = rem;
      if ((int)grp.size() < groups && rem > room && pieces_left > 1) {
        if (fill > 0 && room < min_len) {  // too little room left: start the piece in the next group
          close_group();
          continue;
        }
        take = std::min(align_up(b + std::max<int64_t>(room, min_len)) - b, rem);
        if (rem - take < min_piece) {
          // the tail would be too short: either take it too, or leave a
          // min_piece tail, whichever lands nearer the target
          const int64_t shorter = align_down(r.hi - min_piece) - b;
          take = (shorter >= min_len && room - shorter < rem - room) ? shorter : rem;
        }
      }
      grp.back().push_back(Piece{(int)ri, b, (int)(b + take), nparts[ri]++});
      fill += take;
      left -= take;
      b += (int)take;
      if (fill >= target) close_group();
    }
  }
  while (!grp.empty() && grp.back().empty()) grp.pop_back();
  // partial slots: row r, piece j, unit h -> first[r] + j * U + h
  std::vector<int> first(rows.size(), -1);
  for (size_t ri = 0; ri < rows.size(); ++ri) {
    if (nparts[ri] < 2) continue;
    first[ri] = p->n_slots;
    for (int h = 0; h < U; ++h) p->merges.push_back(MergeItem{rows[ri].q, h, p->n_slots + h, nparts[ri], U});
    p->n_slots += U * nparts[ri];
  }
  p->items.clear();
  p->wg_first.assign(1, 0);
  auto emit = [&](const std::vector<Piece>* g, int h) {
    if (g)
      for (const Piece& pc : *g) {
        const Row& r = rows[pc.row];
        const int slot = first[pc.row] < 0 ? -1 : first[pc.row] + pc.part * U + h;
        p->items.push_back(WorkItem{pa::kDecode, h, r.s, r.q, 1, pc.b, pc.e, slot});
      }
    p->wg_first.push_back((int32_t)p->items.size());
  };
  if (p->nsub() > 1) {
    // the head groups of one group of pieces read the same K/V rows: put
    // their workgroups kXcds apart (one XCD, one L2), the groups of a block
    // of kXcds side by side; missing groups of the last block leave empty
    // workgroups
    for (size_t b0 = 0; b0 < grp.size(); b0 += kXcds)
      for (int h = 0; h < U; h += hw)
        for (size_t j = b0; j < b0 + kXcds; ++j) emit(j < grp.size() ? &grp[j] : nullptr, h);
  } else {
    for (const auto& g : grp)
      for (int h = 0; h < U; h += hw) emit(&g, h);
  }
  p->n_decode = (int32_t)p->items.size();
  p->n_prefill = 0;
}

void build_work(pa_plan* p) {
  std::vector<WorkItem> dec, pre;
  const int G = p->group();
  bool has_prefill = false;
  for (int s = 0; s < p->S; ++s) has_prefill |= (p->cu_q[s + 1] - p->cu_q[s]) > kDecodeMaxQueries;
  // MLA decode-only plans of several head groups: items of two groups, which
  // share each latent tile (the MFMA kernel's head-group pairs)
  if (p->mla && !has_prefill && p->units() > 1) p->heads_shift = 1;
  if (!has_prefill && p->split_tokens == 0 && p->max_splits > 1 && p->n_cu > 0) {
    int per_cu = pa::mla_wgs_per_cu();
    if (!p->mla) {
      per_cu = pa::decode_wgs_per_cu(G);
      // heads per item: the largest power of two dividing Hkv that leaves
      // kDecodeWavesPerHead waves to each head
      while ((p->hkv % (2 << p->heads_shift)) == 0 &&
             (2 << p->heads_shift) * kDecodeWavesPerHead <= pa::decode_waves(G))
        ++p->heads_shift;
    }
    plan_balanced(p, p->n_cu * per_cu, p->mla ? kMlaMinPieceKeys : kMinPieceKeys);
    p->n_wg = (int32_t)p->wg_first.size() - 1;
    return;
  }
  const int split_tokens =
      p->split_tokens > 0 ? std::max(kSplitAlign, (p->split_tokens + kSplitAlign - 1) / kSplitAlign * kSplitAlign)
                          : (p->mla ? kDefaultMlaSplitTokens : (has_prefill ? kMixedSplitTokens : kDefaultSplitTokens));
  for (int s = 0; s < p->S; ++s) {
    const int q0 = p->cu_q[s], q1 = p->cu_q[s + 1];
    const int nq = q1 - q0;
    if (nq == 0) continue;
    if (nq <= kDecodeMaxQueries) {
      for (int i = q0; i < q1; ++i) plan_decode_row(p, s, i, split_tokens, dec);
    } else if (p->mla) {
      // MLA chunks: items of kMlaPrefillQueries consecutive queries and one
      // head group over the union of their visible keys, one query per two waves
      for (int t0 = q0; t0 < q1; t0 += pa::kMlaPrefillQueries) {
        const int t1 = std::min(q1, t0 + pa::kMlaPrefillQueries);
        int lo = INT32_MAX, hi = -1;
        for (int i = t0; i < t1; ++i) {
          int a, b;
          visible_range(p->q_pos[i], p->seq_lens[s], p->causal, p->window, &a, &b);
          lo = std::min(lo, a);
          hi = std::max(hi, b);
        }
        for (int h = 0; h < p->units(); ++h) pre.push_back(WorkItem{pa::kPrefill, h, s, t0, t1 - t0, lo, hi + 1, -1});
      }
    } else {
      const int tile_q = std::max(1, kPrefillRows / G);
      for (int kvh = 0; kvh < p->units(); ++kvh)
        for (int t0 = q0; t0 < q1; t0 += tile_q) {
          const int t1 = std::min(q1, t0 + tile_q);
          int lo = INT32_MAX, hi = -1;
          for (int i = t0; i < t1; ++i) {
            int a, b;
            visible_range(p->q_pos[i], p->seq_lens[s], p->causal, p->window, &a, &b);
            lo = std::min(lo, a);
            hi = std::max(hi, b);
          }
          pre.push_back(WorkItem{pa::kPrefill, kvh, s, t0, t1 - t0, lo, hi + 1, -1});
        }
    }
  }
  p->n_prefill = (int32_t)pre.size();
  p->n_decode = (int32_t)dec.size();
  order_items(p, pre, dec);
  p->n_wg = (int32_t)p->wg_first.size() - 1;
}

// Backward work (ruDNN `attention_backward`: scores recomputed from Q and K,
// a second scan of the history).  dK/dV items stream only the queries from
// the first to the last that see their block.  dQ: one item per (query, KV head) over the
// query's visible keys (vector kernel), and one per tile of kBwdQRows query
// rows and KV head over the union of their visible keys (MFMA kernel; the
// launch picks one list by data type and head size).  dK/dV: one item per (block of kBwdBlockKeys keys,
// KV head) of every sequence with queries, skipping blocks no query sees;
// every pool row then has a single writer when each referenced page holds key
// positions of one sequence only (else the launch adds the rows up in f32 and
// shared_page names the first shared page).  The lists run longest first.
void build_bwd(pa_plan* p) {
  std::vector<int32_t> owner(p->num_pages, -1);
  for (int s = 0; s < p->S && p->shared_page < 0; ++s) {
    const int pages = (p->seq_lens[s] + p->ps - 1) / p->ps;
    for (int j = 0; j < pages; ++j) {
      const int page = p->bt[(size_t)s * p->W + j];
      if (owner[page] >= 0) {
        p->shared_page = page;
        break;
      }
      owner[page] = s;
    }
  }
  std::vector<std::pair<int64_t, pa::BwdItem>> dq, kv, dqt;
  const int tile_q = std::max(1, pa::kBwdQRows / p->group());
  for (int s = 0; s < p->S; ++s) {
    const int q0 = p->cu_q[s], q1 = p->cu_q[s + 1], L = p->seq_lens[s];
    if (q0 == q1) continue;
    for (int i = q0; i < q1; ++i) {
      int lo, hi;
      visible_range(p->q_pos[i], L, p->causal, p->window, &lo, &hi);
      for (int kvh = 0; kvh < p->units(); ++kvh) dq.push_back({hi + 1 - lo, pa::BwdItem{s, kvh, i, i + 1, lo, hi + 1}});
    }
    for (int a0 = q0; a0 < q1 && !p->mla; a0 += tile_q) {  // MLA: per-query dQ items only
      const int a1 = std::min(q1, a0 + tile_q);
      int lo = INT32_MAX, hi = -1;
      for (int i = a0; i < a1; ++i) {
        int x, y;
        visible_range(p->q_pos[i], L, p->causal, p->window, &x, &y);
        lo = std::min(lo, x);
        hi = std::max(hi, y);
      }
      for (int kvh = 0; kvh < p->hkv; ++kvh)
        dqt.push_back({(int64_t)(hi + 1 - lo) * (a1 - a0), pa::BwdItem{s, kvh, a0, a1, lo, hi + 1}});
    }
    for (int t0 = 0; t0 < L; t0 += pa::kBwdBlockKeys) {
      const int t1 = std::min(L, t0 + pa::kBwdBlockKeys);
      int64_t rows = 0;  // queries that see a key of the block, and the first and last of them
      int first = -1, last = -1;
      for (int i = q0; i < q1; ++i) {
        int lo, hi;
        visible_range(p->q_pos[i], L, p->causal, p->window, &lo, &hi);
        if (lo < t1 && hi >= t0) {
          ++rows;
          if (first < 0) first = i;
          last = i;
        }
      }
      if (rows == 0) continue;
      // (MLA: one item per block, which takes every head group of its queries)
      for (int kvh = 0; kvh < p->hkv; ++kvh) kv.push_back({rows, pa::BwdItem{s, kvh, first, last + 1, t0, t1}});
    }
  }
  auto longest_first = [](const std::pair<int64_t, pa::BwdItem>& a, const std::pair<int64_t, pa::BwdItem>& b) {
    return a.first > b.first;
  };
  std::stable_sort(dq.begin(), dq.end(), longest_first);
  std::stable_sort(kv.begin(), kv.end(), longest_first);
  std::stable_sort(dqt.begin(), dqt.end(), longest_first);
  p->bwd_items.clear();
  for (auto& x : dq) p->bwd_items.push_back(x.second);
  for (auto& x : kv) p->bwd_items.push_back(x.second);
  for (auto& x : dqt) p->bwd_items.push_back(x.second);
  p->n_bwd_dq = (int32_t)dq.size();
  p->n_bwd_kv = (int32_t)kv.size();
  p->n_bwd_dqt = (int32_t)dqt.size();
  // Each dK/dV item writes every slot of its block (zero where no query sees
  // the key); the other slots of the pools are zeroed by runs of at most
  // kZeroRunSlots slots.
  constexpr int kZeroRunSlots = 64;
  const int64_t pool_slots = (int64_t)p->num_pages * p->ps;
  std::vector<char> owned((size_t)pool_slots, 0);
  for (const auto& x : kv) {
    const pa::BwdItem& b = x.second;
    if (b.kvh != 0) continue;  // the items of all KV heads cover the same slots
    for (int t = b.tok_begin; t < b.tok_end; ++t)
      owned[(size_t)p->bt[(size_t)b.seq * p->W + t / p->ps] * p->ps + t % p->ps] = 1;
  }
  p->zero_runs.clear();
  for (int64_t i = 0; i < pool_slots;) {
    if (owned[(size_t)i]) {
      ++i;
      continue;
    }
    int64_t j = i;
    while (j < pool_slots && !owned[(size_t)j] && j - i < kZeroRunSlots) ++j;
    p->zero_runs.push_back((int32_t)i);
    p->zero_runs.push_back((int32_t)(j - i));
    i = j;
  }
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The backward lists of a plan, built once on the host (thread-safe: the
// plan's lock).  The plan is logically const; the lists are a cache.
void ensure_bwd_host(const pa_plan* cp) {
  pa_plan* p = const_cast<pa_plan*>(cp);
  std::lock_guard<std::mutex> lock(p->bwd_mu);
  if (p->bwd_built) return;
  build_bwd(p);
  p->bwd_built = true;
}

// ... and their device copy, uploaded on the plan's stream by the first
// backward call (ordered before that call's kernels; freed with the plan).
int ensure_bwd_device(const pa_plan* cp) {
  ensure_bwd_host(cp);
  pa_plan* p = const_cast<pa_plan*>(cp);
  std::lock_guard<std::mutex> lock(p->bwd_mu);
  if (p->bwd_dev) return PA_OK;
  const size_t off_zr = align_up(p->bwd_items.size() * sizeof(pa::BwdItem), kAlign);
  const size_t total = std::max(align_up(off_zr + p->zero_runs.size() * 4, kAlign), kAlign);
  p->bwd_blob.assign(total, 0);
  if (!p->bwd_items.empty()) memcpy(p->bwd_blob.data(), p->bwd_items.data(), p->bwd_items.size() * sizeof(pa::BwdItem));
  if (!p->zero_runs.empty()) memcpy(p->bwd_blob.data() + off_zr, p->zero_runs.data(), p->zero_runs.size() * 4);
  char* dev = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&dev), total, p->created_on);
  if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(backward lists)");
  e = hipMemcpyAsync(dev, p->bwd_blob.data(), total, hipMemcpyHostToDevice, p->created_on);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->bwd_uploaded, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(p->bwd_uploaded, p->created_on);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(p->created_on);
    (void)hipFreeAsync(dev, p->created_on);
    if (p->bwd_uploaded) (void)hipEventDestroy(p->bwd_uploaded);
    p->bwd_uploaded = nullptr;
    return hip_fail(e, "backward list upload");
  }
  p->bwd_dev = dev;
  p->d_bwd = reinterpret_cast<const pa::BwdItem*>(dev);
  p->d_zero_runs = reinterpret_cast<const int32_t*>(dev + off_zr);
  return PA_OK;
}

// Workspace: partial sums [slots, G, Dv] | (max, sum, unrounded sum) [slots, G, 3].
size_t ws_o_bytes(const pa_plan* p, int dv) { return align_up((size_t)p->n_slots * p->unit_heads() * dv * 4, kAlign); }
size_t ws_ml_bytes(const pa_plan* p) { return align_up((size_t)p->n_slots * p->unit_heads() * 3 * 4, kAlign); }

size_t workspace_bytes_for(const pa_plan* p, int dv) {
  if (p->n_slots == 0) return 0;
  return ws_o_bytes(p, dv) + ws_ml_bytes(p);
}

struct Extent {
  const void* p;
  size_t n;
  const char* name;
};

bool overlaps(const Extent& a, const Extent& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
  return x < y + b.n && y < x + a.n;
}

// (initializer lists: argument checks make no heap allocation)
int check_disjoint(std::initializer_list<Extent> outs, std::initializer_list<Extent> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Extent& in : ins)
      if (overlaps(*o, in)) return fail(PA_ERR_OVERLAP, "%s overlaps %s", o->name, in.name);
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlaps(*o, *o2)) return fail(PA_ERR_OVERLAP, "%s overlaps %s", o->name, o2->name);
  }
  return PA_OK;
}

// The kernels move tensor rows in 16-byte pieces.
int check_aligned(std::initializer_list<Extent> ts) {
  for (const Extent& t : ts)
    if (t.p && t.n && reinterpret_cast<uintptr_t>(t.p) % 16)
      return fail(PA_ERR_INVALID, "%s must be 16-byte aligned", t.name);
  return PA_OK;
}

// A plan (and the workspace used with it) lives on the device and the
// stream it was made on (ruDNN: metadata and split workspaces belong to one
// device queue).
int check_device(const pa_plan* p, void* stream) {
  if (!p->dev) return fail(PA_ERR_DEVICE, "plan was built on the host only (pa_plan_create_host)");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  if (dev != p->device) return fail(PA_ERR_DEVICE, "plan was made on device %d; the current device is %d", p->device, dev);
  if (reinterpret_cast<hipStream_t>(stream) != p->created_on)
    return fail(PA_ERR_DEVICE, "plan was made on stream %p and is used on that stream only (call on %p)",
                (void*)p->created_on, stream);
  return PA_OK;
}

pa::MainEvents main_events_of(void* const* ev) {
  if (!ev) return {};
  return {reinterpret_cast<hipEvent_t>(ev[0]), reinterpret_cast<hipEvent_t>(ev[1])};
}

// Common forward path once the kernel family is chosen.
struct FwdCall {
  const pa_plan* plan;
  int dtype, d, dv;  // MLA: d = latent rank, dv = rotary width
  pa::KernelArgs args;
  pa::MainEvents events;
  hipStream_t stream;
  bool generic = false;  // GQA on the vector kernel (pa_generic.hip), with this shape
  pa::GenericShape shape{};
};

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// Host copy of a validated schedule (no device access).
pa_plan* new_plan(const pa_plan_desc* desc) {
  pa_plan* p = new (std::nothrow) pa_plan();
  if (!p) return nullptr;
  p->S = desc->num_seqs;
  p->W = std::max(desc->table_width, 1);
  p->ps = desc->page_size;
  while ((1 << p->page_shift) < p->ps) ++p->page_shift;
  p->num_pages = desc->num_pages;
  p->hq = desc->num_q_heads;
  p->hkv = desc->num_kv_heads;
  p->causal = desc->causal;
  p->window = desc->window;
  p->max_splits = desc->max_splits;
  p->mla = desc->mla;
  p->split_tokens = desc->split_tokens;
  p->cu_q.assign(1, 0);
  if (p->S > 0) {
    p->seq_lens.assign(desc->seq_lens, desc->seq_lens + p->S);
    p->cu_q.assign(desc->cu_q, desc->cu_q + p->S + 1);
    p->bt.assign(desc->block_table, desc->block_table + (size_t)p->S * p->W);
  }
  p->Q = p->cu_q.back();
  if (p->Q > 0) p->q_pos.assign(desc->q_pos, desc->q_pos + p->Q);
  // append slots (positions are validated: every one maps to a pool page)
  p->slot_of.resize(p->Q);
  p->seq_of.resize(p->Q);
  for (int s = 0; s < p->S; ++s)
    for (int i = p->cu_q[s]; i < p->cu_q[s + 1]; ++i) {
      p->seq_of[i] = s;
      const int pos = p->q_pos[i];
      p->slot_of[i] = p->bt[(size_t)s * p->W + pos / p->ps] * p->ps + pos % p->ps;
    }
  std::vector<std::pair<int32_t, int32_t>> order(p->Q);
  for (int i = 0; i < p->Q; ++i) order[i] = {p->slot_of[i], i};
  std::sort(order.begin(), order.end());
  for (int i = 1; i < p->Q; ++i)
    if (order[i].first == order[i - 1].first) {
      p->dup_query = std::max(order[i].second, order[i - 1].second);
      break;
    }
  return p;
}

}  // namespace

extern "C" {

int pa_plan_create(const pa_plan_desc* desc, void* stream, pa_plan** out_plan) {
  if (!out_plan) return fail(PA_ERR_INVALID, "out_plan is NULL");
  int rc = validate_desc(desc);
  if (rc != PA_OK) return rc;

  pa_plan* p = new_plan(desc);
  if (!p) return fail(PA_ERR_HIP, "host allocation failed");
  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&p->n_cu, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "device query");
  }
  build_work(p);

  // one blob: block table | q_pos | seq_lens | items | workgroup ranges | merges | append slots | query sequences
  size_t off_bt = 0;
  size_t off_qpos = align_up(off_bt + p->bt.size() * 4, kAlign);
  size_t off_lens = align_up(off_qpos + p->q_pos.size() * 4, kAlign);
  size_t off_items = align_up(off_lens + p->seq_lens.size() * 4, kAlign);
  size_t off_wg = align_up(off_items + p->items.size() * sizeof(WorkItem), kAlign);
  size_t off_merges = align_up(off_wg + p->wg_first.size() * 4, kAlign);
  size_t off_slots = align_up(off_merges + p->merges.size() * sizeof(MergeItem), kAlign);
  size_t off_seq = align_up(off_slots + p->slot_of.size() * 4, kAlign);
  size_t total = align_up(off_seq + p->seq_of.size() * 4, kAlign);
  total = std::max(total, kAlign);
  p->blob.assign(total, 0);
  if (!p->bt.empty()) memcpy(p->blob.data() + off_bt, p->bt.data(), p->bt.size() * 4);
  if (!p->q_pos.empty()) memcpy(p->blob.data() + off_qpos, p->q_pos.data(), p->q_pos.size() * 4);
  if (!p->seq_lens.empty()) memcpy(p->blob.data() + off_lens, p->seq_lens.data(), p->seq_lens.size() * 4);
  if (!p->items.empty()) memcpy(p->blob.data() + off_items, p->items.data(), p->items.size() * sizeof(WorkItem));
  memcpy(p->blob.data() + off_wg, p->wg_first.data(), p->wg_first.size() * 4);
  if (!p->merges.empty())
    memcpy(p->blob.data() + off_merges, p->merges.data(), p->merges.size() * sizeof(MergeItem));
  if (!p->slot_of.empty()) memcpy(p->blob.data() + off_slots, p->slot_of.data(), p->slot_of.size() * 4);
  if (!p->seq_of.empty()) memcpy(p->blob.data() + off_seq, p->seq_of.data(), p->seq_of.size() * 4);

  // stream-ordered allocation, upload and (in pa_plan_destroy) free: no call
  // of the plan's life waits for the device
  p->created_on = reinterpret_cast<hipStream_t>(stream);
  e = hipMallocAsync(reinterpret_cast<void**>(&p->dev), total, p->created_on);
  if (e != hipSuccess) {
    p->dev = nullptr;
    delete p;
    return hip_fail(e, "hipMallocAsync(plan)");
  }
  e = hipMemcpyAsync(p->dev, p->blob.data(), total, hipMemcpyHostToDevice, p->created_on);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->uploaded, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(p->uploaded, p->created_on);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(p->created_on);
    (void)hipFreeAsync(p->dev, p->created_on);
    if (p->uploaded) (void)hipEventDestroy(p->uploaded);
    delete p;
    return hip_fail(e, "plan upload");
  }
  p->d_bt = reinterpret_cast<const int32_t*>(p->dev + off_bt);
  p->d_qpos = reinterpret_cast<const int32_t*>(p->dev + off_qpos);
  p->d_lens = reinterpret_cast<const int32_t*>(p->dev + off_lens);
  p->d_items = reinterpret_cast<const WorkItem*>(p->dev + off_items);
  p->d_wg_first = reinterpret_cast<const int32_t*>(p->dev + off_wg);
  p->d_merges = reinterpret_cast<const MergeItem*>(p->dev + off_merges);
  p->d_slot_of = reinterpret_cast<const int32_t*>(p->dev + off_slots);
  p->d_seq_of = reinterpret_cast<const int32_t*>(p->dev + off_seq);
  *out_plan = p;
  return ok();
}

int pa_plan_create_host(const pa_plan_desc* desc, int32_t num_cus, pa_plan** out_plan) {
  if (!out_plan) return fail(PA_ERR_INVALID, "out_plan is NULL");
  if (num_cus <= 0 || num_cus > 65536) return fail(PA_ERR_INVALID, "num_cus %d outside [1, 65536]", num_cus);
  int rc = validate_desc(desc);
  if (rc != PA_OK) return rc;
  pa_plan* p = new_plan(desc);
  if (!p) return fail(PA_ERR_HIP, "host allocation failed");
  p->n_cu = num_cus;
  build_work(p);
  *out_plan = p;
  return ok();
}

int pa_plan_get_work(const pa_plan* plan, int32_t* items, int32_t* n_items, int32_t* wg_first, int32_t* n_wg,
                     int32_t* merges, int32_t* n_merges) {
  if (!plan || !n_items || !n_wg || !n_merges) return fail(PA_ERR_INVALID, "plan and the count pointers are required");
  static_assert(sizeof(WorkItem) == 8 * sizeof(int32_t) && sizeof(MergeItem) == 5 * sizeof(int32_t),
                "work records are exported as plain int32 rows");
  *n_items = (int32_t)plan->items.size();
  *n_wg = plan->n_wg;
  *n_merges = (int32_t)plan->merges.size();
  if (items && !plan->items.empty()) memcpy(items, plan->items.data(), plan->items.size() * sizeof(WorkItem));
  if (wg_first) memcpy(wg_first, plan->wg_first.data(), (size_t)(plan->n_wg + 1) * sizeof(int32_t));
  if (merges && !plan->merges.empty()) memcpy(merges, plan->merges.data(), plan->merges.size() * sizeof(MergeItem));
  return ok();
}

int pa_plan_destroy(pa_plan* plan) {
  if (!plan) return ok();
  if (!plan->dev) {  // built on the host only (pa_plan_create_host)
    delete plan;
    return ok();
  }
  // Every kernel that reads the plan was enqueued on its stream, so a free
  // ordered after them on that stream needs no wait for them.  The host
  // blob is the source of the upload copy, enqueued when the plan was made:
  // wait for that copy alone before the blob goes.
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (prev != plan->device) (void)hipSetDevice(plan->device);
  if (plan->uploaded) (void)hipEventSynchronize(plan->uploaded);
  if (plan->bwd_uploaded) (void)hipEventSynchronize(plan->bwd_uploaded);
  hipError_t e = hipFreeAsync(plan->dev, plan->created_on);
  if (plan->bwd_dev) {
    const hipError_t e2 = hipFreeAsync(plan->bwd_dev, plan->created_on);
    if (e == hipSuccess) e = e2;
  }
  if (plan->uploaded) (void)hipEventDestroy(plan->uploaded);
  if (plan->bwd_uploaded) (void)hipEventDestroy(plan->bwd_uploaded);
  if (prev >= 0 && prev != plan->device) (void)hipSetDevice(prev);
  delete plan;
  if (e != hipSuccess) return hip_fail(e, "hipFreeAsync(plan)");
  return ok();
}

int pa_plan_get_info(const pa_plan* plan, pa_plan_info* info) {
  if (!plan || !info) return fail(PA_ERR_INVALID, "plan or info is NULL");
  info->num_queries = plan->Q;
  info->decode_items = plan->n_decode;
  info->prefill_items = plan->n_prefill;
  info->split_rows = (int32_t)plan->merges.size();
  info->split_slots = plan->n_slots;
  info->launches = plan->items.empty() ? 0 : (plan->merges.empty() ? 1 : 2);
  info->workgroups = plan->n_wg;
  info->heads_per_item = 1 << plan->heads_shift;
  ensure_bwd_host(plan);
  info->bwd_dq_items = plan->n_bwd_dq;
  info->bwd_kv_items = plan->n_bwd_kv;
  info->bwd_shared_pages = plan->shared_page >= 0 ? 1 : 0;
  return ok();
}

int pa_plan_workspace_bytes(const pa_plan* plan, int32_t v_head_dim, size_t* bytes) {
  if (!plan || !bytes) return fail(PA_ERR_INVALID, "plan or bytes is NULL");
  if (v_head_dim <= 0 || v_head_dim > 1024) return fail(PA_ERR_SHAPE, "v_head_dim %d outside [1, 1024]", v_head_dim);
  *bytes = workspace_bytes_for(plan, v_head_dim);
  return ok();
}

static int launch_common(FwdCall& c, bool is_mla) {
  const pa_plan* p = c.plan;
  if (p->Q == 0 || p->items.empty()) return ok();
  hipError_t e;
  if (c.generic) {
    e = pa::launch_generic(c.dtype, c.shape, c.args, c.events, c.stream);
  } else if (is_mla) {
    e = pa::launch_mla_main(c.dtype, c.d, c.dv, p->n_prefill > 0, c.args, c.events, c.stream);
  } else {
    e = pa::launch_gqa_main(c.dtype, c.d, c.dv, p->group(), p->n_prefill > 0, c.args, c.events, c.stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (!p->merges.empty()) {
    const int nm = (int)p->merges.size();
    e = c.generic ? pa::launch_generic_merge(c.dtype, c.shape, c.args, p->d_merges, nm, c.stream)
        : is_mla  ? pa::launch_mla_merge(c.dtype, c.d, c.dv, c.args, p->d_merges, nm, c.stream)
                  : pa::launch_gqa_merge(c.dtype, c.d, c.dv, p->group(), c.args, p->d_merges, nm, c.stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return ok();
}

static int check_workspace(const pa_plan* p, int dv, void* workspace, size_t workspace_bytes, float** ws_o,
                           float** ws_ml, size_t* need_out) {
  const size_t need = workspace_bytes_for(p, dv);
  *need_out = need;
  *ws_o = *ws_ml = nullptr;
  if (need == 0) return PA_OK;
  if (!workspace) return fail(PA_ERR_WORKSPACE, "plan splits %d query rows: a %zu-byte workspace is required",
                              (int)p->merges.size(), need);
  if (workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "split workspace has %zu bytes, plan needs %zu", workspace_bytes, need);
  if ((uintptr_t)workspace % kAlign) return fail(PA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  char* base = reinterpret_cast<char*>(workspace);
  *ws_o = reinterpret_cast<float*>(base);
  *ws_ml = reinterpret_cast<float*>(base + ws_o_bytes(p, dv));
  return PA_OK;
}

int pa_attention_fwd(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool, const void* v_pool,
                     void* out, float* lse, int32_t head_dim, int32_t v_head_dim, float scale, void* workspace,
                     size_t workspace_bytes, void* const* main_events, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID, "plan is NULL");
  if (plan->mla) return fail(PA_ERR_INVALID, "plan was made for MLA (use pa_mla_fwd)");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!k_pool || !v_pool) return fail(PA_ERR_INVALID, "k_pool and v_pool are required");
  if (plan->Q > 0 && (!q || !out)) return fail(PA_ERR_INVALID, "q and out are required when there are queries");
  if (head_dim <= 0 || v_head_dim <= 0 || head_dim > 1024 || v_head_dim > 1024)
    return fail(PA_ERR_SHAPE, "head sizes D=%d Dv=%d outside [1, 1024]", head_dim, v_head_dim);
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PA_ERR_SHAPE, "scale %g must be finite and > 0", scale);
  int rc = check_device(plan, stream);
  if (rc != PA_OK) return rc;
  float *ws_o, *ws_ml;
  size_t need;
  rc = check_workspace(plan, v_head_dim, workspace, workspace_bytes, &ws_o, &ws_ml, &need);
  if (rc != PA_OK) return rc;
  // the specialised kernels when they cover the plan's items, else the
  // vector kernel (any group size and head sizes up to 1024)
  const int G = plan->group();
  const bool generic = plan->grouped() || (plan->n_decode > 0 && !pa::gqa_supported(dtype, head_dim, v_head_dim, G)) ||
                       (plan->n_prefill > 0 && !pa::prefill_supported(dtype, head_dim, v_head_dim, G));
  const size_t es = dtype == PA_F32 ? 4 : 2;
  const size_t slots = (size_t)plan->num_pages * plan->ps * plan->hkv;
  const Extent e_out{out, (size_t)plan->Q * plan->hq * v_head_dim * es, "out"};
  const Extent e_lse{lse, lse ? (size_t)plan->Q * plan->hq * 4 : 0, "lse"};
  const Extent e_ws{workspace, need, "workspace"};
  const Extent e_q{q, (size_t)plan->Q * plan->hq * head_dim * es, "q"};
  const Extent e_k{k_pool, slots * head_dim * es, "k_pool"};
  const Extent e_v{v_pool, slots * v_head_dim * es, "v_pool"};
  rc = check_disjoint({e_out, e_lse, e_ws}, {e_q, e_k, e_v});
  if (rc == PA_OK) rc = check_aligned({e_out, e_q, e_k, e_v});
  if (rc != PA_OK) return rc;

  FwdCall c{plan, dtype, head_dim, v_head_dim, {}, main_events_of(main_events), reinterpret_cast<hipStream_t>(stream)};
  c.generic = generic;
  c.shape = pa::GenericShape{head_dim, 0, v_head_dim, G, plan->nsub(), plan->unit_heads(), 1 << plan->heads_shift, 0};
  pa::KernelArgs& a = c.args;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.out = out;
  a.lse = lse;
  a.ws_o = ws_o;
  a.ws_ml = ws_ml;
  a.block_table = plan->d_bt;
  a.q_pos = plan->d_qpos;
  a.seq_lens = plan->d_lens;
  a.items = plan->d_items;
  a.n_items = (int32_t)plan->items.size();
  a.wg_first = plan->d_wg_first;
  a.n_wg = plan->n_wg;
  a.heads_shift = plan->heads_shift;
  a.table_width = plan->W;
  a.page_shift = plan->page_shift;
  a.hq = plan->hq;
  a.hkv = plan->hkv;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.causal = plan->causal;
  a.window = plan->window;
  return launch_common(c, false);
}

int pa_mla_fwd(const pa_plan* plan, int32_t dtype, const void* q_abs, const void* q_rope, const void* latent,
               const void* kpos, void* out, float* lse, int32_t rank, int32_t rope_dim, float scale,
               void* workspace, size_t workspace_bytes, void* const* main_events, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID, "plan is NULL");
  if (!plan->mla) return fail(PA_ERR_INVALID, "plan was made for GQA (use pa_attention_fwd)");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!latent || !kpos) return fail(PA_ERR_INVALID, "latent and kpos are required");
  if (plan->Q > 0 && (!q_abs || !q_rope || !out))
    return fail(PA_ERR_INVALID, "q_abs, q_rope and out are required when there are queries");
  if (rank <= 0 || rank > 1024) return fail(PA_ERR_SHAPE, "latent rank %d outside [1, 1024]", rank);
  if (rope_dim <= 0 || rope_dim > 256)
    return fail(PA_ERR_SHAPE, "rotary width rope_dim %d outside [1, 256]", rope_dim);
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PA_ERR_SHAPE, "scale %g must be finite and > 0", scale);
  int rc = check_device(plan, stream);
  if (rc != PA_OK) return rc;
  float *ws_o, *ws_ml;
  size_t need;
  rc = check_workspace(plan, rank, workspace, workspace_bytes, &ws_o, &ws_ml, &need);
  if (rc != PA_OK) return rc;
  if (!pa::mla_supported(dtype, plan->hq, rank, rope_dim))
    return fail(PA_ERR_UNSUPPORTED, "no MLA kernel for dtype %d, H=%d, rank=%d, rope_dim=%d", dtype, plan->hq, rank,
                rope_dim);
  const size_t es = dtype == PA_F32 ? 4 : 2;
  const size_t slots = (size_t)plan->num_pages * plan->ps;
  const Extent e_out{out, (size_t)plan->Q * plan->hq * rank * es, "out"};
  const Extent e_lse{lse, lse ? (size_t)plan->Q * plan->hq * 4 : 0, "lse"};
  const Extent e_ws{workspace, need, "workspace"};
  const Extent e_qa{q_abs, (size_t)plan->Q * plan->hq * rank * es, "q_abs"};
  const Extent e_qr{q_rope, (size_t)plan->Q * plan->hq * rope_dim * es, "q_rope"};
  const Extent e_lat{latent, slots * rank * es, "latent"};
  const Extent e_kp{kpos, slots * rope_dim * es, "kpos"};
  rc = check_disjoint({e_out, e_lse, e_ws}, {e_qa, e_qr, e_lat, e_kp});
  if (rc == PA_OK) rc = check_aligned({e_out, e_qa, e_qr, e_lat, e_kp});
  if (rc != PA_OK) return rc;

  FwdCall c{plan, dtype, rank, rope_dim, {}, main_events_of(main_events), reinterpret_cast<hipStream_t>(stream)};
  pa::KernelArgs& a = c.args;
  a.q = q_abs;
  a.k = latent;
  a.v = latent;
  a.qr = q_rope;
  a.kr = kpos;
  a.out = out;
  a.lse = lse;
  a.ws_o = ws_o;
  a.ws_ml = ws_ml;
  a.block_table = plan->d_bt;
  a.q_pos = plan->d_qpos;
  a.seq_lens = plan->d_lens;
  a.items = plan->d_items;
  a.n_items = (int32_t)plan->items.size();
  a.wg_first = plan->d_wg_first;
  a.n_wg = plan->n_wg;
  a.heads_shift = plan->heads_shift;
  a.table_width = plan->W;
  a.page_shift = plan->page_shift;
  a.hq = plan->hq;
  a.hkv = 1;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.causal = plan->causal;
  a.window = plan->window;
  return launch_common(c, true);
}

int pa_append_kv(const pa_plan* plan, int32_t dtype, const void* k_new, const void* v_new, void* k_pool,
                 void* v_pool, int32_t head_dim, int32_t v_head_dim, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID, "plan is NULL");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!k_pool || !v_pool) return fail(PA_ERR_INVALID, "k_pool and v_pool are required");
  if (plan->Q > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID, "k_new and v_new are required when there are queries");
  if (head_dim <= 0 || v_head_dim <= 0 || head_dim > 1024 || v_head_dim > 1024)
    return fail(PA_ERR_SHAPE, "row widths %d, %d outside [1, 1024]", head_dim, v_head_dim);
  const size_t es = dtype == PA_F32 ? 4 : 2;
  const int heads = plan->mla ? 1 : plan->hkv;
  if ((head_dim * es) % 16 || (v_head_dim * es) % 16)
    return fail(PA_ERR_UNSUPPORTED, "this build appends rows of whole 16-byte chunks (widths %d, %d)", head_dim,
                v_head_dim);
  if (plan->dup_query >= 0)
    return fail(PA_ERR_PLAN, "query %d writes the pool slot of another query of the plan", plan->dup_query);
  const size_t slots = (size_t)plan->num_pages * plan->ps * heads;
  const Extent e_kp{k_pool, slots * head_dim * es, "k_pool"}, e_vp{v_pool, slots * v_head_dim * es, "v_pool"};
  const Extent e_kn{k_new, (size_t)plan->Q * heads * head_dim * es, "k_new"};
  const Extent e_vn{v_new, (size_t)plan->Q * heads * v_head_dim * es, "v_new"};
  int rc = check_disjoint({e_kp, e_vp}, {e_kn, e_vn});
  if (rc == PA_OK) rc = check_aligned({e_kp, e_vp, e_kn, e_vn});
  if (rc != PA_OK) return rc;
  rc = check_device(plan, stream);
  if (rc != PA_OK) return rc;
  if (plan->Q == 0) return ok();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = pa::launch_append(k_new, v_new, k_pool, v_pool, plan->d_slot_of, plan->Q, heads,
                                   (int)(head_dim * es), (int)(v_head_dim * es), std::max(plan->n_cu, 1), st);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

// f32 D = dO . O per (query, head) row at the start of the backward workspace.
static size_t bwd_delta_bytes(const pa_plan* plan) {
  return plan->Q > 0 ? align_up((size_t)plan->Q * plan->hq * 4, kAlign) : 0;
}

// Some pool row takes dK / dV from two key positions (only matters when
// there are queries).
static bool bwd_shared(const pa_plan* plan) {
  ensure_bwd_host(plan);
  return plan->shared_page >= 0 && plan->Q > 0;
}

int pa_plan_bwd_workspace_bytes(const pa_plan* plan, int32_t dtype, int32_t head_dim, int32_t v_head_dim,
                                size_t* bytes) {
  if (!plan || !bytes) return fail(PA_ERR_INVALID, "plan or bytes is NULL");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (head_dim <= 0 || v_head_dim <= 0 || head_dim > 1024 || v_head_dim > 1024)
    return fail(PA_ERR_SHAPE, "head sizes D=%d Dv=%d outside [1, 1024]", head_dim, v_head_dim);
  *bytes = bwd_delta_bytes(plan);
  if (bwd_shared(plan) && dtype != PA_F32)
    *bytes += align_up((size_t)plan->num_pages * plan->ps * plan->hkv * (head_dim + v_head_dim) * 4, kAlign);
  return ok();
}

int pa_attention_bwd(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool, const void* v_pool,
                     const void* out, const float* lse, const void* dout, void* dq, void* dk_pool, void* dv_pool,
                     int32_t head_dim, int32_t v_head_dim, float scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!plan) return fail(PA_ERR_INVALID, "plan is NULL");
  if (plan->mla) return fail(PA_ERR_INVALID, "plan was made for MLA (use pa_mla_bwd)");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!k_pool || !v_pool || !dk_pool || !dv_pool)
    return fail(PA_ERR_INVALID, "k_pool, v_pool, dk_pool and dv_pool are required");
  if (plan->Q > 0 && (!q || !out || !lse || !dout || !dq))
    return fail(PA_ERR_INVALID, "q, out, lse, dout and dq are required when there are queries");
  if (head_dim <= 0 || v_head_dim <= 0 || head_dim > 1024 || v_head_dim > 1024)
    return fail(PA_ERR_SHAPE, "head sizes D=%d Dv=%d outside [1, 1024]", head_dim, v_head_dim);
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PA_ERR_SHAPE, "scale %g must be finite and > 0", scale);
  // the specialised kernels where they exist, else the vector kernels (any
  // group size and head sizes up to 1024)
  const int G = plan->group();
  const bool generic = plan->grouped() || !pa::bwd_supported(dtype, head_dim, v_head_dim, G);
  size_t need = 0;
  pa_plan_bwd_workspace_bytes(plan, dtype, head_dim, v_head_dim, &need);
  if (need > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "backward needs %zu bytes of workspace", need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "backward workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const size_t es = dtype == PA_F32 ? 4 : 2;
  const size_t slots = (size_t)plan->num_pages * plan->ps * plan->hkv;
  const size_t rows = (size_t)plan->Q * plan->hq;
  const Extent e_dq{dq, rows * head_dim * es, "dq"}, e_dk{dk_pool, slots * head_dim * es, "dk_pool"};
  const Extent e_dv{dv_pool, slots * v_head_dim * es, "dv_pool"}, e_ws{workspace, need, "workspace"};
  const Extent e_q{q, rows * head_dim * es, "q"}, e_k{k_pool, slots * head_dim * es, "k_pool"};
  const Extent e_v{v_pool, slots * v_head_dim * es, "v_pool"}, e_o{out, rows * v_head_dim * es, "out"};
  const Extent e_l{lse, rows * 4, "lse"}, e_do{dout, rows * v_head_dim * es, "dout"};
  int rc = check_disjoint({e_dq, e_dk, e_dv, e_ws}, {e_q, e_k, e_v, e_o, e_l, e_do});
  if (rc == PA_OK) rc = check_aligned({e_dq, e_dk, e_dv, e_q, e_k, e_v, e_o, e_do});
  if (rc != PA_OK) return rc;
  rc = check_device(plan, stream);
  if (rc != PA_OK) return rc;
  rc = ensure_bwd_device(plan);
  if (rc != PA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  pa::KernelArgs a{};
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.out = const_cast<void*>(out);
  a.lse = const_cast<float*>(lse);
  a.block_table = plan->d_bt;
  a.q_pos = plan->d_qpos;
  a.seq_lens = plan->d_lens;
  a.table_width = plan->W;
  a.page_shift = plan->page_shift;
  a.hq = plan->hq;
  a.hkv = plan->hkv;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.causal = plan->causal;
  a.window = plan->window;
  float* delta = reinterpret_cast<float*>(workspace);
  float* acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_delta_bytes(plan));
  const int n_runs = (int)(plan->zero_runs.size() / 2);
  hipError_t e;
  if (generic) {
    const pa::GenericShape shape{head_dim, 0, v_head_dim, G, plan->nsub(), plan->unit_heads(), 1, 0};
    e = pa::launch_generic_bwd(dtype, shape, a, dout, dq, nullptr, dk_pool, dv_pool, delta, acc, bwd_shared(plan),
                               plan->d_bwd, plan->n_bwd_dq, plan->n_bwd_kv, plan->d_zero_runs, n_runs, (int64_t)rows,
                               (int64_t)slots, std::max(plan->n_cu, 1), st);
  } else {
    e = pa::launch_gqa_bwd(dtype, head_dim, v_head_dim, G, a, dout, dq, dk_pool, dv_pool, delta, acc,
                           bwd_shared(plan), plan->d_bwd, plan->n_bwd_dq, plan->n_bwd_kv, plan->n_bwd_dqt,
                           plan->d_zero_runs, n_runs, (int64_t)rows, (int64_t)slots, std::max(plan->n_cu, 1), st);
  }
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

int pa_mla_bwd(const pa_plan* plan, int32_t dtype, const void* q_abs, const void* q_rope, const void* latent,
               const void* kpos, const void* out, const float* lse, const void* dout, void* dq_abs, void* dq_rope,
               void* dlatent, void* dkpos, int32_t rank, int32_t rope_dim, float scale, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID, "plan is NULL");
  if (!plan->mla) return fail(PA_ERR_INVALID, "plan was made for GQA (use pa_attention_bwd)");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!latent || !kpos || !dlatent || !dkpos)
    return fail(PA_ERR_INVALID, "latent, kpos, dlatent and dkpos are required");
  if (plan->Q > 0 && (!q_abs || !q_rope || !out || !lse || !dout || !dq_abs || !dq_rope))
    return fail(PA_ERR_INVALID, "q_abs, q_rope, out, lse, dout, dq_abs and dq_rope are required when there are queries");
  if (rank <= 0 || rank > 1024) return fail(PA_ERR_SHAPE, "latent rank %d outside [1, 1024]", rank);
  if (rope_dim <= 0 || rope_dim > 256) return fail(PA_ERR_SHAPE, "rotary width rope_dim %d outside [1, 256]", rope_dim);
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PA_ERR_SHAPE, "scale %g must be finite and > 0", scale);
  // the MFMA kernels for 16-bit rank 512 / width 64, else the vector kernels
  const bool generic = !pa::mla_bwd_supported(dtype, plan->hq, rank, rope_dim);
  size_t need = 0;
  pa_plan_bwd_workspace_bytes(plan, dtype, rank, rope_dim, &need);
  if (need > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "MLA backward needs %zu bytes of workspace", need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "MLA backward workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
      return fail(PA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  }
  const size_t es = dtype == PA_F32 ? 4 : 2;
  const size_t slots = (size_t)plan->num_pages * plan->ps;
  const size_t rows = (size_t)plan->Q * plan->hq;
  const Extent e_dqa{dq_abs, rows * rank * es, "dq_abs"}, e_dqr{dq_rope, rows * rope_dim * es, "dq_rope"};
  const Extent e_dl{dlatent, slots * rank * es, "dlatent"}, e_dk{dkpos, slots * rope_dim * es, "dkpos"};
  const Extent e_ws{workspace, need, "workspace"};
  const Extent e_qa{q_abs, rows * rank * es, "q_abs"}, e_qr{q_rope, rows * rope_dim * es, "q_rope"};
  const Extent e_l{latent, slots * rank * es, "latent"}, e_k{kpos, slots * rope_dim * es, "kpos"};
  const Extent e_o{out, rows * rank * es, "out"}, e_lse{lse, rows * 4, "lse"}, e_do{dout, rows * rank * es, "dout"};
  int rc = check_disjoint({e_dqa, e_dqr, e_dl, e_dk, e_ws}, {e_qa, e_qr, e_l, e_k, e_o, e_lse, e_do});
  if (rc == PA_OK) rc = check_aligned({e_dqa, e_dqr, e_dl, e_dk, e_qa, e_qr, e_l, e_k, e_o, e_do});
  if (rc != PA_OK) return rc;
  rc = check_device(plan, stream);
  if (rc != PA_OK) return rc;
  rc = ensure_bwd_device(plan);
  if (rc != PA_OK) return rc;
  pa::KernelArgs a{};
  a.q = q_abs;
  a.qr = q_rope;
  a.k = latent;
  a.v = latent;
  a.kr = kpos;
  a.out = const_cast<void*>(out);
  a.lse = const_cast<float*>(lse);
  a.block_table = plan->d_bt;
  a.q_pos = plan->d_qpos;
  a.seq_lens = plan->d_lens;
  a.table_width = plan->W;
  a.page_shift = plan->page_shift;
  a.hq = plan->hq;
  a.hkv = 1;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.causal = plan->causal;
  a.window = plan->window;
  float* delta = reinterpret_cast<float*>(workspace);
  float* acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_delta_bytes(plan));
  const int n_runs = (int)(plan->zero_runs.size() / 2);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (generic) {
    const pa::GenericShape shape{rank, rope_dim, rank, plan->hq, plan->nsub(), plan->unit_heads(), 1, 1};
    e = pa::launch_generic_bwd(dtype, shape, a, dout, dq_abs, dq_rope, dlatent, dkpos, delta, acc, bwd_shared(plan),
                               plan->d_bwd, plan->n_bwd_dq, plan->n_bwd_kv, plan->d_zero_runs, n_runs, (int64_t)rows,
                               (int64_t)slots, std::max(plan->n_cu, 1), st);
  } else {
    e = pa::launch_mla_bwd(dtype, a, dout, dq_abs, dq_rope, dlatent, dkpos, delta, acc, bwd_shared(plan), plan->d_bwd,
                           plan->n_bwd_dq, plan->n_bwd_kv, plan->d_zero_runs, n_runs, (int64_t)rows, (int64_t)slots,
                           std::max(plan->n_cu, 1), st);
  }
  if (e != hipSuccess) return hip_fail(e, "MLA backward launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Block-sparse top-k attention (alice-llm 2.0.0, sparse_attention/
// llama3_bridge.rs, `llama3_sparse_attention`).  Workspace: decode items and
// identity workgroup map [rows * width], merge records [rows], split partials
// of rows * width slots (rows = Q * Hkv, one slot per kept block), then (when
// topk > 0) the candidate block scores [rows, widest row's candidates].
// ---------------------------------------------------------------------------
namespace {

struct SparseLayout {
  int32_t width = 0, cand = 0, span = 0, spans = 0;
  size_t off_items = 0, off_wg = 0, off_merges = 0, off_o = 0, off_ml = 0, off_scores = 0, total = 0;
};

int sparse_layout(const pa_plan* p, int dv, int block_size, int topk, SparseLayout* out) {
  if (p->mla) return fail(PA_ERR_INVALID, "block-sparse attention runs on GQA plans (mla == 0)");
  if (block_size <= 0 || block_size % p->ps != 0)
    return fail(PA_ERR_SHAPE, "block_size %d must be a positive multiple of page_size %d", block_size, p->ps);
  if (topk < 0) return fail(PA_ERR_INVALID, "topk %d < 0", topk);
  if (dv <= 0 || dv > 1024) return fail(PA_ERR_SHAPE, "v_head_dim %d outside [1, 1024]", dv);
  const int span = pa::sparse_span(block_size);
  int32_t most = 0, spans = 0;  // candidate blocks and scoring spans of the widest row
  for (int s = 0; s < p->S; ++s)
    for (int i = p->cu_q[s]; i < p->cu_q[s + 1]; ++i) {
      int lo, hi;
      visible_range(p->q_pos[i], p->seq_lens[s], p->causal, p->window, &lo, &hi);
      most = std::max(most, hi / block_size - lo / block_size + 1);
      spans = std::max(spans, hi / span - lo / span + 1);
    }
  if (most > pa::kSparseMaxBlocks)
    return fail(PA_ERR_UNSUPPORTED, "a row spans %d blocks of %d keys; the selection holds at most %d", most,
                block_size, pa::kSparseMaxBlocks);
  SparseLayout L;
  L.width = topk > 0 ? topk : std::max(most, 1);
  L.cand = std::max(most, 1);
  L.span = span;
  L.spans = std::max(spans, 1);
  const size_t rows = (size_t)p->Q * p->hkv, slots = rows * L.width;
  if (slots > (size_t)INT32_MAX) return fail(PA_ERR_RANGE, "rows x kept blocks exceed 32-bit indexing");
  if (L.spans > 65535) return fail(PA_ERR_UNSUPPORTED, "a row spans %d scoring spans of %d keys", L.spans, span);
  L.off_items = 0;
  L.off_wg = align_up(slots * sizeof(WorkItem), kAlign);
  L.off_merges = align_up(L.off_wg + (slots + 1) * 4, kAlign);
  L.off_o = align_up(L.off_merges + rows * sizeof(MergeItem), kAlign);
  L.off_ml = align_up(L.off_o + slots * p->group() * dv * 4, kAlign);
  // block scores only when some blocks are dropped
  L.off_scores = align_up(L.off_ml + slots * p->group() * 3 * 4, kAlign);
  const size_t score_bytes = topk > 0 ? rows * L.cand * 4 : 0;
  L.total = p->Q > 0 ? align_up(L.off_scores + score_bytes, kAlign) : 0;
  *out = L;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_sparse_workspace_bytes(const pa_plan* plan, int32_t v_head_dim, int32_t block_size, int32_t topk,
                              size_t* bytes, int32_t* width) {
  if (!plan || !bytes || !width) return fail(PA_ERR_INVALID, "plan, bytes and width are required");
  SparseLayout L;
  const int rc = sparse_layout(plan, v_head_dim, block_size, topk, &L);
  if (rc != PA_OK) return rc;
  *bytes = L.total;
  *width = L.width;
  return ok();
}

int pa_sparse_attention_fwd(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool,
                            const void* v_pool, void* out, float* lse, int32_t head_dim, int32_t v_head_dim,
                            float scale, int32_t block_size, int32_t topk, int32_t* selection, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID, "plan is NULL");
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16) return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!k_pool || !v_pool) return fail(PA_ERR_INVALID, "k_pool and v_pool are required");
  if (plan->Q > 0 && (!q || !out)) return fail(PA_ERR_INVALID, "q and out are required when there are queries");
  if (head_dim <= 0 || head_dim > pa::kSparseMaxDim || v_head_dim <= 0 || v_head_dim > 1024)
    return fail(PA_ERR_SHAPE, "head sizes D=%d Dv=%d outside [1, 1024]", head_dim, v_head_dim);
  const size_t es = dtype == PA_F32 ? 4 : 2;
  if ((head_dim * es) % 16) return fail(PA_ERR_UNSUPPORTED, "K rows of %d elements are not whole 16-byte pieces", head_dim);
  if (!std::isfinite(scale) || scale <= 0.f) return fail(PA_ERR_SHAPE, "scale %g must be finite and > 0", scale);
  SparseLayout L;
  int rc = sparse_layout(plan, v_head_dim, block_size, topk, &L);
  if (rc != PA_OK) return rc;
  rc = check_device(plan, stream);
  if (rc != PA_OK) return rc;
  const int G = plan->group();
  if (!pa::gqa_supported(dtype, head_dim, v_head_dim, G))
    return fail(PA_ERR_UNSUPPORTED, "no decode kernel for dtype %d, D=%d, Dv=%d, G=%d", dtype, head_dim, v_head_dim,
                G);
  if (L.total > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "block-sparse attention needs %zu bytes of workspace", L.total);
    if (workspace_bytes < L.total)
      return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, block-sparse attention needs %zu", workspace_bytes,
                  L.total);
    if ((uintptr_t)workspace % kAlign) return fail(PA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  }
  const size_t rows = (size_t)plan->Q * plan->hkv;
  const size_t slots = (size_t)plan->num_pages * plan->ps * plan->hkv;
  const Extent e_out{out, (size_t)plan->Q * plan->hq * v_head_dim * es, "out"};
  const Extent e_lse{lse, lse ? (size_t)plan->Q * plan->hq * 4 : 0, "lse"};
  const Extent e_ws{workspace, L.total, "workspace"};
  const Extent e_sel{selection, selection ? rows * L.width * 4 : 0, "selection"};
  const Extent e_q{q, (size_t)plan->Q * plan->hq * head_dim * es, "q"};
  const Extent e_k{k_pool, slots * head_dim * es, "k_pool"};
  const Extent e_v{v_pool, slots * v_head_dim * es, "v_pool"};
  rc = check_disjoint({e_out, e_lse, e_ws, e_sel}, {e_q, e_k, e_v});
  if (rc == PA_OK) rc = check_aligned({e_out, e_q, e_k, e_v});
  if (rc != PA_OK) return rc;
  if (plan->Q == 0) return ok();

  char* ws = static_cast<char*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  pa::SparseArgs sa{};
  sa.q = q;
  sa.k = k_pool;
  sa.block_table = plan->d_bt;
  sa.q_pos = plan->d_qpos;
  sa.seq_lens = plan->d_lens;
  sa.seq_of = plan->d_seq_of;
  sa.table_width = plan->W;
  sa.page_shift = plan->page_shift;
  sa.hq = plan->hq;
  sa.hkv = plan->hkv;
  sa.d = head_dim;
  sa.causal = plan->causal;
  sa.window = plan->window;
  sa.block_size = block_size;
  sa.topk = topk;
  sa.width = L.width;
  sa.selection = selection;
  sa.items = reinterpret_cast<WorkItem*>(ws + L.off_items);
  sa.wg_first = reinterpret_cast<int32_t*>(ws + L.off_wg);
  sa.merges = reinterpret_cast<MergeItem*>(ws + L.off_merges);
  sa.scores = reinterpret_cast<uint32_t*>(ws + L.off_scores);
  sa.cand_width = L.cand;
  sa.span = L.span;
  sa.spans = L.spans;
  sa.items_per_wg = pa::kSparseItemsPerWg;
  hipError_t e = pa::launch_sparse_select(dtype, sa, (int)rows, st);
  if (e != hipSuccess) return hip_fail(e, "block selection launch");

  pa::KernelArgs a{};
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.out = out;
  a.lse = lse;
  a.ws_o = reinterpret_cast<float*>(ws + L.off_o);
  a.ws_ml = reinterpret_cast<float*>(ws + L.off_ml);
  a.block_table = plan->d_bt;
  a.q_pos = plan->d_qpos;
  a.seq_lens = plan->d_lens;
  a.items = sa.items;
  a.n_items = (int32_t)(rows * L.width);
  a.wg_first = sa.wg_first;
  a.n_wg = (int32_t)((rows * L.width + pa::kSparseItemsPerWg - 1) / pa::kSparseItemsPerWg);
  a.heads_shift = 0;
  a.table_width = plan->W;
  a.page_shift = plan->page_shift;
  a.hq = plan->hq;
  a.hkv = plan->hkv;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.causal = plan->causal;
  a.window = plan->window;
  e = pa::launch_gqa_short(dtype, head_dim, v_head_dim, G, a, st);
  if (e != hipSuccess) return hip_fail(e, "block attention launch");
  e = pa::launch_gqa_merge(dtype, head_dim, v_head_dim, G, a, sa.merges, (int)rows, st);
  if (e != hipSuccess) return hip_fail(e, "block merge launch");
  return ok();
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_INVALID: return "bad argument: null pointer, unknown data type or flag out of range";
    case PA_ERR_SHAPE: return "tensor sizes, head counts or softmax scale do not fit together";
    case PA_ERR_PLAN: return "schedule is inconsistent (offsets, positions or block table)";
    case PA_ERR_UNSUPPORTED: return "valid request that no kernel of this build handles";
    case PA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PA_ERR_OVERLAP: return "an output shares memory with an input or another output";
    case PA_ERR_RANGE: return "a size does not fit 32-bit element indexing";
    case PA_ERR_HIP: return "the HIP runtime reported a failure";
    case PA_ERR_DEVICE: return "plan used away from the device or stream it was made for";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
