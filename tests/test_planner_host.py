"""Host checks of the work planner (no GPU): plans built with
pa_plan_create_host for a device of a given CU count are read back with
pa_plan_get_work and checked against the visibility rule of the header
(key t of a sequence of L keys is visible to a query at position p iff
t < L, t <= p when causal, and t > p - window when windowed):

- every visible (query, KV head, key) is covered by exactly one item, decode
  pieces tile each row's visible range without gaps, prefill tiles contain
  the visible range of each of their queries;
- split rows have one partial slot per piece, every slot is used once, and
  each merge record lists exactly the slots of its row;
- no row is cut into more than max_splits pieces, cuts are 64-aligned and
  the pieces of balanced plans are at least the planner's minimum unless the
  row is shorter;
- workgroup ranges partition the item list, and the balanced decode plans
  give every workgroup about the same number of keys.
"""
import numpy as np
import pytest

import paged_kv_attention_gqa_amd as pa

KIND_DECODE, KIND_PREFILL, KIND_EMPTY = 0, 1, 2


def schedule(seed, q_counts, histories, page_size, *, hq, hkv, causal=True, window=0, max_splits=16,
             split_tokens=0, mla=False):
    """Sequences whose queries sit at the end of their context (decode steps
    and prefill chunks after `histories[s]` cached keys), pages in a shuffled
    pool."""
    rng = np.random.default_rng(seed)
    seq_lens = np.array([h + c for h, c in zip(histories, q_counts)], np.int32)
    pages = [-(-int(L) // page_size) for L in seq_lens]
    width = max(max(pages), 1)
    perm = rng.permutation(sum(pages) + 3).astype(np.int32)
    bt = np.full((len(seq_lens), width), -1, np.int32)
    o = 0
    for s, n in enumerate(pages):
        bt[s, :n] = perm[o:o + n]
        o += n
    cu_q = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    q_pos = np.concatenate([np.arange(L - c, L) for L, c in zip(seq_lens, q_counts)] + [np.zeros(0)]).astype(np.int32)
    return dict(seq_lens=seq_lens, cu_q=cu_q, q_pos=q_pos, block_table=bt, page_size=page_size,
                num_pages=int(perm.size), num_q_heads=hq, num_kv_heads=hkv, causal=causal, window=window,
                max_splits=max_splits, split_tokens=split_tokens, mla=mla)


def visible(s, i):
    """[lo, hi) of query i's visible keys, from the header's rule."""
    seq = int(np.searchsorted(s["cu_q"], i, side="right") - 1)
    L, p = int(s["seq_lens"][seq]), int(s["q_pos"][i])
    hi = p + 1 if s["causal"] else L
    lo = max(0, p - s["window"] + 1) if s["window"] > 0 else 0
    return seq, lo, hi


def plan_of(s, num_cus):
    p = pa.pa_plan_create_host(num_cus=num_cus, **s)
    items, wg, merges = pa.pa_plan_get_work(p)
    info = pa.pa_plan_get_info(p)
    pa.pa_plan_destroy(p)
    return items, wg, merges, info


def check_plan(s, items, wg, merges, info, min_piece):
    # work units of a row: KV heads, or (MLA, and groups of more than 16
    # query heads) each KV head's query heads in groups of 16
    G = s["num_q_heads"] // s["num_kv_heads"]
    hkv = s["num_kv_heads"] * (-(-G // 16) if s["mla"] or G > 16 else 1)
    Q = int(s["cu_q"][-1])
    hpi = info["heads_per_item"]
    # MLA pairs head groups: with an odd number of groups the last item's second is past the end
    assert hpi >= 1 and (hkv % hpi == 0 or s["mla"]) and (hpi & (hpi - 1)) == 0
    # workgroup ranges partition the item list
    assert wg[0] == 0 and wg[-1] == len(items) and np.all(np.diff(wg) >= 0)
    assert info["workgroups"] == len(wg) - 1
    assert info["decode_items"] == int((items[:, 0] == KIND_DECODE).sum())
    assert info["prefill_items"] == int((items[:, 0] == KIND_PREFILL).sum())
    assert set(np.unique(items[:, 0])) <= {KIND_DECODE, KIND_PREFILL, KIND_EMPTY}

    pieces = {}   # (query, head) -> [(b, e, slot)]
    tiles = {}    # (query, head) -> number of prefill tiles holding it
    for kind, kvh, seq, q0, qn, b, e, slot in items.tolist():
        if kind == KIND_EMPTY:
            continue
        if kind == KIND_DECODE:
            assert qn == 1 and 0 <= kvh < hkv and kvh % hpi == 0
            vs, lo, hi = visible(s, q0)
            assert vs == seq and lo <= b < e <= hi, (q0, b, e, lo, hi)
            for h in range(kvh, min(kvh + hpi, hkv)):
                pieces.setdefault((q0, h), []).append((b, e, slot + (h - kvh) if slot >= 0 else -1))
        else:
            assert hpi == 1 and 0 <= kvh < hkv and qn >= 1
            for i in range(q0, q0 + qn):
                vs, lo, hi = visible(s, i)
                assert vs == seq and b <= lo and hi <= e, (i, b, e, lo, hi)
                tiles[(i, kvh)] = tiles.get((i, kvh), 0) + 1
    # every (query, head) exactly once: one prefill tile, or decode pieces
    assert all(v == 1 for v in tiles.values())
    assert not set(tiles) & set(pieces)
    assert set(tiles) | set(pieces) == {(i, h) for i in range(Q) for h in range(hkv)}

    used = []
    merge_of = {(q, h): (slot, n, stride) for q, h, slot, n, stride in merges.tolist()}
    assert len(merge_of) == len(merges)
    for (i, h), ps in pieces.items():
        ps.sort()
        _, lo, hi = visible(s, i)
        assert ps[0][0] == lo and ps[-1][1] == hi
        assert all(a[1] == c[0] for a, c in zip(ps, ps[1:])), f"gap or overlap in row {(i, h)}"
        assert len(ps) <= s["max_splits"]
        if len(ps) == 1:
            assert ps[0][2] == -1 and (i, h) not in merge_of
            continue
        assert all(b % 64 == 0 for b, _, _ in ps[1:]), "cuts fall on multiples of 64 keys"
        assert all(e - b >= min(min_piece, hi - lo) for b, e, _ in ps)
        slots = [sl for _, _, sl in ps]
        first, n, stride = merge_of[(i, h)]
        assert n == len(ps) and sorted(slots) == sorted(first + j * stride for j in range(n))
        used += slots
    assert len(used) == len(set(used)), "a partial slot is used twice"
    assert all(0 <= x < info["split_slots"] for x in used)
    assert info["split_rows"] == len(merges)
    return pieces


DECODE_SCHEDULES = [
    # the decode-batch shape: 32 single-query rows of 512..8192 keys
    dict(seed=1, q_counts=[1] * 32, histories=list(np.random.default_rng(2).integers(511, 8192, 32)),
         page_size=16, hq=32, hkv=8),
    dict(seed=2, q_counts=[1, 2, 1, 3, 4], histories=[0, 5000, 130, 20000, 77], page_size=64, hq=64, hkv=8,
         window=700),
    dict(seed=3, q_counts=[1] * 7, histories=[300, 1, 4000, 9000, 63, 64, 65], page_size=16, hq=12, hkv=6),
    dict(seed=4, q_counts=[1, 1], histories=[2100, 1], page_size=1, hq=16, hkv=1),
    dict(seed=5, q_counts=[1, 1, 1], histories=[20000, 16385, 4095], page_size=16, hq=8, hkv=2, max_splits=1),
    dict(seed=6, q_counts=[1, 1, 1], histories=[20000, 16385, 4095], page_size=32, hq=24, hkv=3, split_tokens=300),
    dict(seed=7, q_counts=[2, 1], histories=[12345, 9999], page_size=16, hq=16, hkv=4, window=7001, causal=False),
]


@pytest.mark.parametrize("num_cus", [256, 80, 1])
@pytest.mark.parametrize("k", range(len(DECODE_SCHEDULES)))
def test_decode_plans_cover_every_visible_key_once(k, num_cus):
    s = schedule(**DECODE_SCHEDULES[k])
    items, wg, merges, info = plan_of(s, num_cus)
    assert info["prefill_items"] == 0
    # balanced plans keep pieces >= 128 keys; fixed split_tokens cuts leave a remainder
    check_plan(s, items, wg, merges, info, min_piece=1 if s["split_tokens"] else 128)


def test_balanced_decode_plan_evens_out_workgroups():
    """The decode-batch shape on 256 CUs: one group of workgroups per piece
    list, each workgroup within 10% of the mean number of (key, head) pairs,
    and no more workgroups than fit on the device at once."""
    s = schedule(**DECODE_SCHEDULES[0])
    items, wg, merges, info = plan_of(s, 256)
    check_plan(s, items, wg, merges, info, min_piece=128)
    hpi = info["heads_per_item"]
    assert hpi == 2  # G = 4: eight waves, four per head
    work = np.array([sum((items[i, 6] - items[i, 5]) * hpi for i in range(wg[b], wg[b + 1]))
                     for b in range(len(wg) - 1)])
    assert len(work) <= 256 * 2
    assert work.max() <= 1.1 * work.mean(), (work.max(), work.mean())
    # the workgroups of one piece list run the same pieces for different heads
    assert len(work) % (s["num_kv_heads"] // hpi) == 0


def test_unsplit_rows_write_the_output_directly():
    s = schedule(**DECODE_SCHEDULES[4])
    items, wg, merges, info = plan_of(s, 256)
    assert len(merges) == 0 and info["split_slots"] == 0 and np.all(items[:, 7] == -1)


@pytest.mark.parametrize("num_cus", [256, 13])
@pytest.mark.parametrize("window,causal", [(0, True), (300, True), (0, False)])
def test_mixed_plans_tile_prefill_rows_and_split_decode_rows(num_cus, window, causal):
    """Chunks of 2048 / 700 / 33 queries next to decode rows: prefill tiles of
    256 query rows per KV head, decode rows cut by split_tokens."""
    s = schedule(11, q_counts=[2048, 1, 700, 1, 33, 2], histories=[0, 30000, 4000, 9000, 100, 50],
                 page_size=16, hq=32, hkv=8, window=window, causal=causal)
    items, wg, merges, info = plan_of(s, num_cus)
    assert info["prefill_items"] > 0 and info["decode_items"] > 0 and info["heads_per_item"] == 1
    check_plan(s, items, wg, merges, info, min_piece=1)
    # one item per workgroup, empty items only as padding
    assert np.array_equal(wg, np.arange(len(items) + 1))
    G = 32 // 8
    pre = items[items[:, 0] == KIND_PREFILL]
    assert np.all(pre[:, 4] <= 256 // G)


@pytest.mark.parametrize("num_cus", [256, 7])
def test_mla_plans(num_cus):
    """MLA: one shared latent head, 16 query heads; balanced pieces of at
    least 256 keys."""
    rng = np.random.default_rng(5)
    s = schedule(5, q_counts=[1] * 64, histories=list(rng.integers(1023, 16384, 64)), page_size=64, hq=16, hkv=1,
                 mla=True)
    items, wg, merges, info = plan_of(s, num_cus)
    assert info["heads_per_item"] == 1
    check_plan(s, items, wg, merges, info, min_piece=256)
    work = np.array([sum(items[i, 6] - items[i, 5] for i in range(wg[b], wg[b + 1])) for b in range(len(wg) - 1)])
    assert len(work) <= num_cus * 2 and work.max() <= 1.1 * work.mean() + 512


def test_host_plans_are_rejected_by_forward_calls():
    """Checked before any HIP call: the (never dereferenced) tensor pointers
    are placeholders."""
    s = schedule(**DECODE_SCHEDULES[2])
    p = pa.pa_plan_create_host(num_cus=256, **s)
    lib = pa.load_library()
    rc = lib.pa_attention_fwd(p.handle, 1, 16, 16, 16, 16, None, 128, 128, 1.0, None, 0, None, None)
    assert rc == -9 and "host only" in pa.pa_last_error()
    pa.pa_plan_destroy(p)


def test_host_plan_rejects_bad_cu_counts():
    s = schedule(**DECODE_SCHEDULES[2])
    for n in (0, -3, 1 << 20):
        with pytest.raises(pa.PaError):
            pa.pa_plan_create_host(num_cus=n, **s)


def test_query_pointers_may_be_null_only_without_queries():
    """q and out are required when the plan has queries (PA_ERR_INVALID, -1);
    without queries NULL passes the argument checks and the host-only plan is
    then refused for the device (PA_ERR_DEVICE, -9)."""
    lib = pa.load_library()
    s = schedule(**DECODE_SCHEDULES[2])
    p = pa.pa_plan_create_host(num_cus=256, **s)
    assert lib.pa_attention_fwd(p.handle, 1, None, 16, 16, None, None, 128, 128, 1.0, None, 0, None, None) == -1
    pa.pa_plan_destroy(p)
    s0 = schedule(9, q_counts=[0, 0], histories=[40, 0], page_size=16, hq=8, hkv=2)
    p0 = pa.pa_plan_create_host(num_cus=256, **s0)
    assert pa.pa_plan_get_info(p0)["launches"] == 0
    assert lib.pa_attention_fwd(p0.handle, 1, None, 16, 16, None, None, 128, 128, 1.0, None, 0, None, None) == -9
    pa.pa_plan_destroy(p0)


def test_append_rejects_two_queries_writing_one_slot():
    """pa_append_kv refuses a plan in which two queries name one pool slot
    (PA_ERR_PLAN, -3) before any device check; a plan without such a pair
    passes the argument checks and the host-only plan is then refused for the
    device (PA_ERR_DEVICE, -9).  Tensor pointers are never dereferenced."""
    lib = pa.load_library()
    s = schedule(8, q_counts=[1, 3], histories=[20, 50], page_size=16, hq=8, hkv=2)
    p = pa.pa_plan_create_host(num_cus=256, **s)
    assert lib.pa_append_kv(p.handle, 1, 1 << 20, 2 << 20, 3 << 20, 1 << 30, 64, 64, None) == -9
    pa.pa_plan_destroy(p)
    s["q_pos"] = s["q_pos"].copy()
    s["q_pos"][2] = s["q_pos"][1]
    p = pa.pa_plan_create_host(num_cus=256, **s)
    assert lib.pa_append_kv(p.handle, 1, 1 << 20, 2 << 20, 3 << 20, 1 << 30, 64, 64, None) == -3
    assert "writes the pool slot" in pa.pa_last_error()
    pa.pa_plan_destroy(p)


def test_backward_workspace_and_shared_page_detection():
    """The backward workspace holds one f32 D = dO . O per (query, head) row
    (256-byte aligned); a table that points two positions at one pool page
    sets bwd_shared_pages and, for 16-bit data, adds f32 sums of the whole dK
    and dV pools; f32 data need none (the sums are the pools).  Bad dtype or
    head sizes are refused."""
    s = schedule(10, q_counts=[3, 2], histories=[40, 30], page_size=16, hq=8, hkv=2)
    p = pa.pa_plan_create_host(num_cus=256, **s)
    assert pa.pa_plan_get_info(p)["bwd_shared_pages"] == 0
    assert pa.pa_plan_bwd_workspace_bytes(p, "bf16", 64, 64) == 256
    assert pa.pa_plan_bwd_workspace_bytes(p, "f32", 64, 64) == 256
    with pytest.raises(ValueError):
        pa.pa_plan_bwd_workspace_bytes(p, "f64", 64, 64)
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan_bwd_workspace_bytes(p, "bf16", 0, 64)
    assert e.value.status == -2
    pa.pa_plan_destroy(p)
    s["block_table"] = s["block_table"].copy()
    s["block_table"][1, 0] = s["block_table"][0, 0]  # prefix sharing of the first page
    p = pa.pa_plan_create_host(num_cus=256, **s)
    assert pa.pa_plan_get_info(p)["bwd_shared_pages"] == 1
    slots = s["num_pages"] * 16 * 2
    assert pa.pa_plan_bwd_workspace_bytes(p, "bf16", 64, 32) == 256 + -(-slots * 96 * 4 // 256) * 256
    assert pa.pa_plan_bwd_workspace_bytes(p, "f32", 64, 32) == 256
    pa.pa_plan_destroy(p)
    s0 = schedule(11, q_counts=[0, 0], histories=[40, 30], page_size=16, hq=8, hkv=2)
    s0["block_table"][1, 0] = s0["block_table"][0, 0]
    p = pa.pa_plan_create_host(num_cus=256, **s0)
    assert pa.pa_plan_bwd_workspace_bytes(p, "bf16", 64, 64) == 0  # no queries: nothing to add up
    pa.pa_plan_destroy(p)


def test_backward_lists_on_first_use_match_the_visibility_rule():
    """The backward work lists are built when first asked for (here by
    pa_plan_get_info): one dQ item per (query, KV head), one dK/dV item per
    (128-key block of a sequence that some query sees, KV head); asking twice
    gives the same counts, and a plan with prefill chunks and decode rows
    counts both."""
    s = schedule(12, q_counts=[1, 37, 0, 2], histories=[300, 129, 50, 0], page_size=16, hq=12, hkv=3,
                 window=90)
    p = pa.pa_plan_create_host(num_cus=64, **s)
    first = pa.pa_plan_get_info(p)
    again = pa.pa_plan_get_info(p)
    pa.pa_plan_destroy(p)
    nq = int(s["cu_q"][-1])
    assert first["bwd_dq_items"] == again["bwd_dq_items"] == nq * s["num_kv_heads"]
    blocks = set()
    for i in range(nq):
        seq, lo, hi = visible(s, i)
        for blk in range(lo // 128, (hi - 1) // 128 + 1):
            blocks.add((seq, blk))
    assert first["bwd_kv_items"] == again["bwd_kv_items"] == len(blocks) * s["num_kv_heads"]


def sparse_candidates(s, block):
    """Candidate blocks per query (those holding a key it sees)."""
    out = []
    for i in range(int(s["cu_q"][-1])):
        _, lo, hi = visible(s, i)
        out.append((hi - 1) // block - lo // block + 1)
    return out


@pytest.mark.parametrize("block", [16, 48, 2048])
def test_sparse_workspace_and_width(block):
    """pa_sparse_workspace_bytes: the selection width is topk, or the largest
    candidate count of any row for topk = 0; the workspace is 256-byte
    aligned, grows with topk, and with topk > 0 holds the candidate block
    scores of every (query, KV head) row as well."""
    s = schedule(13, q_counts=[1, 20, 3], histories=[5000, 700, 33], page_size=16, hq=8, hkv=2, window=0)
    p = pa.pa_plan_create_host(num_cus=256, **s)
    most = max(sparse_candidates(s, block))
    n0, w0 = pa.pa_sparse_workspace_bytes(p, 64, block, 0)
    n1, w1 = pa.pa_sparse_workspace_bytes(p, 64, block, 1)
    n3, w3 = pa.pa_sparse_workspace_bytes(p, 64, block, 3)
    pa.pa_plan_destroy(p)
    assert (w0, w1, w3) == (most, 1, 3)
    assert all(n % 256 == 0 and n > 0 for n in (n0, n1, n3))
    rows = int(s["cu_q"][-1]) * s["num_kv_heads"]
    assert n3 > n1
    assert n1 >= rows * most * 4  # the score buffer alone


def test_sparse_layout_errors():
    """Block sizes that are not positive multiples of the page size, a
    negative topk, rows of more than 8192 blocks and MLA plans are refused
    before any device work."""
    s = schedule(14, q_counts=[1, 2], histories=[9000, 100], page_size=1, hq=4, hkv=1)
    p = pa.pa_plan_create_host(num_cus=256, **s)
    for block, topk, status in [(0, 1, -2), (3, -1, -1)]:
        with pytest.raises(pa.PaError) as e:
            pa.pa_sparse_workspace_bytes(p, 64, block, topk)
        assert e.value.status == status
    with pytest.raises(pa.PaError) as e:
        pa.pa_sparse_workspace_bytes(p, 64, 1, 4)  # 9001 one-key blocks in a row
    assert e.value.status == -4
    assert pa.pa_sparse_workspace_bytes(p, 64, 2, 4)[1] == 4  # 4501 blocks: accepted
    pa.pa_plan_destroy(p)
    s = schedule(15, q_counts=[1], histories=[100], page_size=16, hq=16, hkv=1, mla=True)
    p = pa.pa_plan_create_host(num_cus=256, **s)
    with pytest.raises(pa.PaError) as e:
        pa.pa_sparse_workspace_bytes(p, 512, 64, 4)
    assert e.value.status == -1
    pa.pa_plan_destroy(p)


@pytest.mark.parametrize("hq", [128, 48, 20, 8])
@pytest.mark.parametrize("num_cus", [256, 7])
def test_mla_head_groups(hq, num_cus):
    """MLA with other head counts: one unit per group of 16 query heads (the
    last one partial), covering every (query, group) once; in balanced plans
    the groups of one key range sit kXcds = 8 workgroups apart (one XCD), and
    in mixed plans every item of a sequence lands on one XCD."""
    rng = np.random.default_rng(6)
    units = -(-hq // 16)
    s = schedule(6, q_counts=[1] * 40, histories=list(rng.integers(1023, 16384, 40)), page_size=64, hq=hq, hkv=1,
                 mla=True)
    items, wg, merges, info = plan_of(s, num_cus)
    check_plan(s, items, wg, merges, info, min_piece=256)
    # decode-only plans pair the head groups (two per item)
    assert info["heads_per_item"] == (2 if units > 1 else 1)
    assert set(items[:, 1].tolist()) == set(range(0, units, info["heads_per_item"]))
    xcd_of = {}
    for b in range(len(wg) - 1):
        for i in range(wg[b], wg[b + 1]):
            key = (int(items[i, 3]), int(items[i, 5]), int(items[i, 6]))
            xcd_of.setdefault(key, set()).add(b % 8)
    if units > 1:
        assert all(len(x) == 1 for x in xcd_of.values())
    assert all(m[1] < units and m[4] == units for m in merges.tolist())

    s = schedule(7, q_counts=[40, 1, 9, 1], histories=[100, 5000, 700, 20], page_size=16, hq=hq, hkv=1, mla=True)
    items, wg, merges, info = plan_of(s, num_cus)
    check_plan(s, items, wg, merges, info, min_piece=1)
    assert info["prefill_items"] == units * (20 + 5)
    assert np.array_equal(wg, np.arange(len(items) + 1))
    seq_xcd = {}
    for i, it in enumerate(items.tolist()):
        if it[0] == KIND_PREFILL:
            seq_xcd.setdefault(it[2], set()).add(i % 8)
    assert all(len(x) == 1 for x in seq_xcd.values())


@pytest.mark.parametrize("hq,hkv", [(32, 1), (72, 8), (71, 1)])
@pytest.mark.parametrize("num_cus", [256, 7])
def test_large_group_sizes_use_head_groups(hq, hkv, num_cus):
    """G > 16: one work unit per group of 16 query heads of each KV head (the
    last one partial), in balanced decode plans (the groups of one KV head
    and piece on one XCD) and in mixed plans."""
    G = hq // hkv
    units = hkv * -(-G // 16)
    rng = np.random.default_rng(8)
    s = schedule(8, q_counts=[1] * 30, histories=list(rng.integers(100, 9000, 30)), page_size=16, hq=hq, hkv=hkv)
    items, wg, merges, info = plan_of(s, num_cus)
    check_plan(s, items, wg, merges, info, min_piece=128)
    assert set(items[items[:, 0] == KIND_DECODE][:, 1].tolist()) == set(range(units))
    nsub = units // hkv
    xcd_of = {}
    for b in range(len(wg) - 1):
        for i in range(wg[b], wg[b + 1]):
            xcd_of.setdefault((int(items[i, 3]), int(items[i, 5]), int(items[i, 1]) // nsub), set()).add(b % 8)
    assert all(len(x) == 1 for x in xcd_of.values())

    s = schedule(9, q_counts=[40, 1, 9, 1], histories=[100, 5000, 700, 20], page_size=16, hq=hq, hkv=hkv)
    items, wg, merges, info = plan_of(s, num_cus)
    check_plan(s, items, wg, merges, info, min_piece=1)
    assert info["prefill_items"] > 0 and set(items[items[:, 0] == KIND_PREFILL][:, 1].tolist()) == set(range(units))
