"""Seeded synthetic paged-KV workloads.

Every array is plain numpy.  bf16 and f16 (IEEE binary16) tensors are carried
as their raw 16-bit patterns (uint16), produced from float32 draws by
round-to-nearest-even; the same rounded bits feed both the HIP path and the
oracle.

Layouts follow ruDNN 0.1.107 paged_attention/mod.rs (`DevicePlan::attention`,
`DevicePlan::mla`): packed Q [queries, Hq, D]; K pool [pages, page_size, Hkv,
D]; V pool [pages, page_size, Hkv, Dv]; MLA latent [pages, page_size, 1, R] and
rotated position cache [pages, page_size, 1, P].  Queries are packed per
sequence (offsets cu_q), each with an explicit absolute position q_pos; the
block table maps logical page j of sequence s to a physical pool page.

Recipe per named workload (draw order: lengths, page permutation, Q, K, V):
integers "uniform in [a, b]" include both ends; the pool holds exactly the
pages the sequences need (unless stated), assigned by a seeded permutation in
logical order; values are N(0, 1) float32 rounded to the storage type.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Callable, Dict, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
F16_NAN = np.uint16(0x7E00)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even; NaN -> quiet NaN.
    (For every non-NaN input the 32-bit sum below cannot overflow.)"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (numpy's conversion: round to
    nearest even, overflow to infinity, NaN -> NaN)."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(rng: np.random.Generator, n: int, fill, chunk: int = _CHUNK):
    """Run fill(child_generator, start, end) over fixed chunks of `chunk`
    (4M) elements.  Each chunk draws from its own child stream spawned from
    one seed taken from `rng`, so the values do not depend on the thread
    count."""
    seed = int(rng.integers(0, 2 ** 63 - 1))
    starts = list(range(0, n, chunk))
    children = np.random.SeedSequence(seed).spawn(len(starts))

    def work(k):
        fill(np.random.default_rng(children[k]), starts[k], min(n, starts[k] + chunk))

    if len(starts) <= 1:
        for k in range(len(starts)):
            work(k)
    else:
        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws rounded to the storage type."""
    n = int(np.prod(shape))
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown storage type {dtype!r}")
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(g, s, e):
        x = g.standard_normal(e - s, dtype=np.float32)
        out[s:e] = x if dtype == "f32" else (f32_to_bf16_bits(x) if dtype == "bf16" else f32_to_f16_bits(x))

    _chunked(rng, n, fill)
    return out.reshape(shape)


def _nan_value(dtype: str):
    return {"f32": np.float32(np.nan), "bf16": BF16_NAN, "f16": F16_NAN}[dtype]


@dataclasses.dataclass
class PagedBatch:
    """One packed batch over a paged K/V pool (GQA/MHA)."""
    name: str
    dtype: str                      # "f32" | "bf16" | "f16"
    seq_lens: np.ndarray            # int32 [S]
    cu_q: np.ndarray                # int32 [S+1]
    q_pos: np.ndarray               # int32 [Q]
    block_table: np.ndarray         # int32 [S, W]; entries past a sequence's pages are -1
    page_size: int
    num_pages: int
    hq: int
    hkv: int
    d: int
    dv: int
    scale: float
    causal: bool
    window: int                     # 0 = unlimited
    q: np.ndarray                   # [Q, hq, d]
    k: np.ndarray                   # [pages, ps, hkv, d]
    v: np.ndarray                   # [pages, ps, hkv, dv]
    seed: int = 0
    max_splits: int = 16

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_queries(self) -> int:
        return int(self.cu_q[-1])

    @property
    def table_width(self) -> int:
        return int(self.block_table.shape[1])


@dataclasses.dataclass
class MlaBatch:
    """One packed batch over a paged absorbed-MLA latent cache."""
    name: str
    dtype: str
    seq_lens: np.ndarray
    cu_q: np.ndarray
    q_pos: np.ndarray
    block_table: np.ndarray
    page_size: int
    num_pages: int
    heads: int
    r: int
    p: int
    scale: float
    causal: bool
    window: int
    q_abs: np.ndarray               # [Q, H, R]
    q_rope: np.ndarray              # [Q, H, P]
    latent: np.ndarray              # [pages, ps, 1, R]
    kpos: np.ndarray                # [pages, ps, 1, P]
    seed: int = 0
    max_splits: int = 16

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_queries(self) -> int:
        return int(self.cu_q[-1])

    @property
    def table_width(self) -> int:
        return int(self.block_table.shape[1])


def _tables(rng: np.random.Generator, seq_lens, page_size: int, pool_pages: Optional[int] = None,
            table_width: Optional[int] = None):
    """Seeded permutation of the pool assigned to the sequences' pages in
    logical order.  Returns (block_table, num_pages, used page ids)."""
    pages = [max(0, -(-int(L) // page_size)) for L in seq_lens]
    total = sum(pages)
    pool = total if pool_pages is None else pool_pages
    assert pool >= total
    perm = rng.permutation(pool).astype(np.int32)
    width = max(1, max(pages) if pages else 1) if table_width is None else table_width
    bt = np.full((len(pages), width), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(pages):
        bt[s, :n] = perm[off:off + n]
        off += n
    return bt, pool, perm[:total]


def _packed(q_counts):
    cu = np.zeros(len(q_counts) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_counts)
    return cu


def _poison_unused(pool: np.ndarray, used_pages: np.ndarray, seq_lens, block_table, page_size, dtype,
                   tails: bool):
    """NaN-fill pages no sequence references and (optionally) the slots past
    each sequence's length in its last page."""
    nan = _nan_value(dtype)
    mask = np.ones(pool.shape[0], dtype=bool)
    mask[used_pages] = False
    pool[mask] = nan
    if tails:
        for s, L in enumerate(seq_lens):
            L = int(L)
            if L % page_size:
                last = block_table[s, L // page_size]
                pool[last, L % page_size:] = nan


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def config_tiny_f32_decode(seed: int = 1) -> PagedBatch:
    """Tiny f32 paged GQA decode: 1 sequence of 256 tokens in 16 pages placed
    in seeded-shuffled slots of a 32-page pool (other pages NaN), one query
    at position 255, Hq=4, Hkv=1, D=64, page 16, causal, scale 1/8."""
    rng = np.random.default_rng(seed)
    ps, L, hq, hkv, d = 16, 256, 4, 1, 64
    seq_lens = np.array([L], dtype=np.int32)
    used = rng.permutation(32)[:16].astype(np.int32)
    bt = used.reshape(1, 16).copy()
    q = _normal(rng, (1, hq, d), "f32")
    k = _normal(rng, (32, ps, hkv, d), "f32")
    v = _normal(rng, (32, ps, hkv, d), "f32")
    _poison_unused(k, used, seq_lens, bt, ps, "f32", tails=False)
    _poison_unused(v, used, seq_lens, bt, ps, "f32", tails=False)
    return PagedBatch("tiny_f32_decode", "f32", seq_lens, _packed([1]), np.array([L - 1], np.int32), bt,
                      ps, 32, hq, hkv, d, d, 1.0 / 8.0, True, 0, q, k, v, seed, 16)


def config_bf16_decode_batch(seed: int = 2) -> PagedBatch:
    """bf16 paged GQA decode batch: 32 sequences, one query each at L-1,
    contexts uniform in [512, 8192], Hq=32, Hkv=8, D=128, page 16, pool sized
    to the total and permuted, scale 1/sqrt(128), up to 16 splits."""
    rng = np.random.default_rng(seed)
    S, ps, hq, hkv, d = 32, 16, 32, 8, 128
    seq_lens = rng.integers(512, 8192 + 1, size=S).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q = _normal(rng, (S, hq, d), "bf16")
    k = _normal(rng, (pool, ps, hkv, d), "bf16")
    v = _normal(rng, (pool, ps, hkv, d), "bf16")
    return PagedBatch("bf16_decode_batch", "bf16", seq_lens, _packed([1] * S), seq_lens - 1, bt, ps, pool,
                      hq, hkv, d, d, 1.0 / math.sqrt(128.0), True, 0, q, k, v, seed, 16)


def config_bf16_chunked_prefill(seed: int = 3) -> PagedBatch:
    """bf16 chunked prefill: 8 sequences, history uniform in [0, 4096] plus a
    512-query chunk at the following positions; causal, Hq=32, Hkv=8, D=128,
    page 16, scale 1/sqrt(128)."""
    rng = np.random.default_rng(seed)
    S, C, ps, hq, hkv, d = 8, 512, 16, 32, 8, 128
    hist = rng.integers(0, 4096 + 1, size=S).astype(np.int32)
    seq_lens = (hist + C).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_pos = np.concatenate([np.arange(h, h + C, dtype=np.int32) for h in hist])
    q = _normal(rng, (S * C, hq, d), "bf16")
    k = _normal(rng, (pool, ps, hkv, d), "bf16")
    v = _normal(rng, (pool, ps, hkv, d), "bf16")
    return PagedBatch("bf16_chunked_prefill", "bf16", seq_lens, _packed([C] * S), q_pos, bt, ps, pool,
                      hq, hkv, d, d, 1.0 / math.sqrt(128.0), True, 0, q, k, v, seed, 16)


def config_bf16_mixed_batch(seed: int = 4) -> PagedBatch:
    """bf16 mixed packed batch: 64 decode queries with contexts uniform in
    [1024, 32768] followed by 4 prefill chunks of 1024 queries with histories
    uniform in [0, 8192]; Hq=64, Hkv=8, D=128, page 64, causal, sliding window
    4096, scale 1/sqrt(128) (the workload names no scale; 1/sqrt(D) is the
    standard one)."""
    rng = np.random.default_rng(seed)
    nd, npf, C, ps, hq, hkv, d = 64, 4, 1024, 64, 64, 8, 128
    dec_lens = rng.integers(1024, 32768 + 1, size=nd).astype(np.int32)
    hist = rng.integers(0, 8192 + 1, size=npf).astype(np.int32)
    seq_lens = np.concatenate([dec_lens, hist + C]).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_pos = np.concatenate([dec_lens - 1] + [np.arange(h, h + C, dtype=np.int32) for h in hist])
    Q = nd + npf * C
    q = _normal(rng, (Q, hq, d), "bf16")
    k = _normal(rng, (pool, ps, hkv, d), "bf16")
    v = _normal(rng, (pool, ps, hkv, d), "bf16")
    return PagedBatch("bf16_mixed_batch", "bf16", seq_lens, _packed([1] * nd + [C] * npf), q_pos.astype(np.int32),
                      bt, ps, pool, hq, hkv, d, d, 1.0 / math.sqrt(128.0), True, 4096, q, k, v, seed, 16)


def _unit_rms(rng: np.random.Generator, shape, dtype: str = "bf16") -> np.ndarray:
    """N(0,1) rows rescaled in float32 to unit RMS (no epsilon, no weight),
    then rounded to the storage type (kept as is for f32)."""
    to_bits = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits, "f32": lambda x: x}[dtype]
    width = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = np.empty(rows * width, dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(g, s, e):
        x = g.standard_normal(e - s, dtype=np.float32).reshape(-1, width)
        rms = np.sqrt(np.mean(x * x, axis=1, dtype=np.float32), dtype=np.float32)
        out[s:e] = to_bits(x / rms[:, None]).reshape(-1)

    # whole rows per chunk (the chunk size stays 4M elements for widths dividing it)
    _chunked(rng, rows * width, fill, _CHUNK if _CHUNK % width == 0 else _CHUNK // width * width)
    return out.reshape(shape)


def config_bf16_mla_decode(seed: int = 5) -> MlaBatch:
    """bf16 absorbed-MLA decode: 64 sequences, one query each at L-1, H=16,
    R=512, P=64, contexts uniform in [1024, 16384], page 64, unit-RMS latent
    rows, scale 1/sqrt(576), causal."""
    rng = np.random.default_rng(seed)
    S, H, R, P, ps = 64, 16, 512, 64, 64
    seq_lens = rng.integers(1024, 16384 + 1, size=S).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_abs = _normal(rng, (S, H, R), "bf16")
    q_rope = _normal(rng, (S, H, P), "bf16")
    latent = _unit_rms(rng, (pool, ps, 1, R))
    kpos = _normal(rng, (pool, ps, 1, P), "bf16")
    return MlaBatch("bf16_mla_decode", "bf16", seq_lens, _packed([1] * S), seq_lens - 1, bt, ps, pool,
                    H, R, P, 1.0 / math.sqrt(576.0), True, 0, q_abs, q_rope, latent, kpos, seed, 16)


def config_bf16_mla_decode_h128(seed: int = 5) -> MlaBatch:
    """The MLA decode shape with all 128 query heads of a DeepSeek-V3-sized
    model on one GPU (a workload of this library): 64 sequences, one query
    each at L-1, H=128, R=512, P=64, contexts uniform in [1024, 16384], page
    64, unit-RMS latent rows, scale 1/sqrt(576), causal."""
    rng = np.random.default_rng(seed)
    S, H, R, P, ps = 64, 128, 512, 64, 64
    seq_lens = rng.integers(1024, 16384 + 1, size=S).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_abs = _normal(rng, (S, H, R), "bf16")
    q_rope = _normal(rng, (S, H, P), "bf16")
    latent = _unit_rms(rng, (pool, ps, 1, R))
    kpos = _normal(rng, (pool, ps, 1, P), "bf16")
    return MlaBatch("bf16_mla_decode_h128", "bf16", seq_lens, _packed([1] * S), seq_lens - 1, bt, ps, pool,
                    H, R, P, 1.0 / math.sqrt(576.0), True, 0, q_abs, q_rope, latent, kpos, seed, 16)


def config_bf16_chunked_prefill_d192(seed: int = 7) -> PagedBatch:
    """The chunked-prefill shape with K rows of 192 and V rows of 128 (a
    workload of this library): 8 sequences, history uniform in [0, 4096] plus a
    512-query chunk, causal, Hq=32, Hkv=8, page 16, scale 1/sqrt(192)."""
    rng = np.random.default_rng(seed)
    S, C, ps, hq, hkv, d, dv = 8, 512, 16, 32, 8, 192, 128
    hist = rng.integers(0, 4096 + 1, size=S).astype(np.int32)
    seq_lens = (hist + C).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_pos = np.concatenate([np.arange(h, h + C, dtype=np.int32) for h in hist])
    q = _normal(rng, (S * C, hq, d), "bf16")
    k = _normal(rng, (pool, ps, hkv, d), "bf16")
    v = _normal(rng, (pool, ps, hkv, dv), "bf16")
    return PagedBatch("bf16_chunked_prefill_d192", "bf16", seq_lens, _packed([C] * S), q_pos, bt, ps, pool,
                      hq, hkv, d, dv, 1.0 / math.sqrt(192.0), True, 0, q, k, v, seed, 16)


def config_bf16_chunked_prefill_d256(seed: int = 8) -> PagedBatch:
    """The chunked-prefill shape with K and V rows of 256 (a workload of this
    library): 8 sequences, history uniform in [0, 4096] plus a 512-query
    chunk, causal, Hq=32, Hkv=8, page 16, scale 1/sqrt(256)."""
    rng = np.random.default_rng(seed)
    S, C, ps, hq, hkv, d = 8, 512, 16, 32, 8, 256
    hist = rng.integers(0, 4096 + 1, size=S).astype(np.int32)
    seq_lens = (hist + C).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_pos = np.concatenate([np.arange(h, h + C, dtype=np.int32) for h in hist])
    q = _normal(rng, (S * C, hq, d), "bf16")
    k = _normal(rng, (pool, ps, hkv, d), "bf16")
    v = _normal(rng, (pool, ps, hkv, d), "bf16")
    return PagedBatch("bf16_chunked_prefill_d256", "bf16", seq_lens, _packed([C] * S), q_pos, bt, ps, pool,
                      hq, hkv, d, d, 1.0 / math.sqrt(256.0), True, 0, q, k, v, seed, 16)


def config_bf16_mla_chunked_prefill(seed: int = 6) -> MlaBatch:
    """bf16 absorbed-MLA chunked prefill (a workload of this library, beside
    the MLA decode one): 8 sequences, each a 256-query chunk after a history
    uniform in [0, 4096], H=16, R=512, P=64, page 64, unit-RMS latent rows,
    scale 1/sqrt(576), causal."""
    rng = np.random.default_rng(seed)
    S, H, R, P, ps, C = 8, 16, 512, 64, 64, 256
    hist = rng.integers(0, 4096 + 1, size=S)
    seq_lens = (hist + C).astype(np.int32)
    bt, pool, _ = _tables(rng, seq_lens, ps)
    q_pos = np.concatenate([np.arange(h, h + C, dtype=np.int32) for h in hist])
    q_abs = _normal(rng, (S * C, H, R), "bf16")
    q_rope = _normal(rng, (S * C, H, P), "bf16")
    latent = _unit_rms(rng, (pool, ps, 1, R))
    kpos = _normal(rng, (pool, ps, 1, P), "bf16")
    return MlaBatch("bf16_mla_chunked_prefill", "bf16", seq_lens, _packed([C] * S), q_pos, bt, ps, pool,
                    H, R, P, 1.0 / math.sqrt(576.0), True, 0, q_abs, q_rope, latent, kpos, seed, 16)


CONFIGS: Dict[str, Callable] = {
    "tiny_f32_decode": config_tiny_f32_decode,
    "bf16_decode_batch": config_bf16_decode_batch,
    "bf16_chunked_prefill": config_bf16_chunked_prefill,
    "bf16_mixed_batch": config_bf16_mixed_batch,
    "bf16_mla_decode": config_bf16_mla_decode,
    "bf16_mla_decode_h128": config_bf16_mla_decode_h128,
    "bf16_mla_chunked_prefill": config_bf16_mla_chunked_prefill,
    "bf16_chunked_prefill_d192": config_bf16_chunked_prefill_d192,
    "bf16_chunked_prefill_d256": config_bf16_chunked_prefill_d256,
}


# ---------------------------------------------------------------------------
# Small randomized batches for parity and property tests
# ---------------------------------------------------------------------------

def random_batch(seed: int, *, dtype: str = "bf16", hq: int = 8, hkv: int = 2, d: int = 64,
                 page_size: int = 16, q_counts=(1, 1, 5, 1), histories=None, max_len: int = 300,
                 causal: bool = True, window: int = 0, extra_pages: int = 3, poison: bool = True,
                 scale: Optional[float] = None, max_splits: int = 16, dv: Optional[int] = None) -> PagedBatch:
    """A small ragged batch: sequence s has q_counts[s] queries that sit at the
    end of its context (the last q_counts[s] positions), like a decode step or
    a prefill chunk after `histories[s]` cached tokens.  Extra pool pages and
    (with `poison`) tail slots of each last page are NaN."""
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    S = len(q_counts)
    if histories is None:
        histories = rng.integers(0, max_len + 1, size=S)
    seq_lens = np.array([int(h) + int(c) for h, c in zip(histories, q_counts)], dtype=np.int32)
    need = sum(-(-int(L) // page_size) for L in seq_lens)
    bt, pool, used = _tables(rng, seq_lens, page_size, pool_pages=need + extra_pages)
    q_pos = np.concatenate([np.arange(L - c, L, dtype=np.int32) for L, c in zip(seq_lens, q_counts)]
                           + [np.zeros(0, np.int32)])
    Q = int(sum(q_counts))
    q = _normal(rng, (Q, hq, d), dtype)
    k = _normal(rng, (pool, page_size, hkv, d), dtype)
    v = _normal(rng, (pool, page_size, hkv, dv), dtype)
    if poison:
        _poison_unused(k, used, seq_lens, bt, page_size, dtype, tails=True)
        _poison_unused(v, used, seq_lens, bt, page_size, dtype, tails=True)
    sc = (1.0 / math.sqrt(d)) if scale is None else scale
    return PagedBatch(f"random_{seed}", dtype, seq_lens, _packed(list(q_counts)), q_pos.astype(np.int32), bt,
                      page_size, pool, hq, hkv, d, dv, sc, causal, window, q, k, v, seed, max_splits)


def with_shared_pages(b: PagedBatch, links) -> PagedBatch:
    """A copy of `b` whose block table points page slot j_dst of sequence
    s_dst at the pool page of slot j_src of sequence s_src, for each
    (s_dst, j_dst, s_src, j_src) in `links` (prefix sharing between sequences,
    or one page at two positions of a sequence).  The pools are unchanged; the
    rows the new reader sees must be rows the source sequence holds (so no
    poisoned tail slot becomes visible)."""
    bt = b.block_table.copy()
    ps = b.page_size
    for s_dst, j_dst, s_src, j_src in links:
        need = min(ps, int(b.seq_lens[s_dst]) - j_dst * ps)
        have = min(ps, int(b.seq_lens[s_src]) - j_src * ps)
        assert 0 < need <= have, (s_dst, j_dst, s_src, j_src)
        bt[s_dst, j_dst] = b.block_table[s_src, j_src]
    return dataclasses.replace(b, name=b.name + "+shared", block_table=bt)


def random_mla_batch(seed: int, *, heads: int = 16, r: int = 512, p: int = 64, page_size: int = 64,
                     q_counts=(1, 1, 1), histories=None, max_len: int = 700, causal: bool = True,
                     window: int = 0, extra_pages: int = 2, poison: bool = True,
                     max_splits: int = 16, dtype: str = "bf16") -> MlaBatch:
    """A small ragged absorbed-MLA batch (f32, bf16 or f16), laid out like the
    MLA workload above, with NaN in unreferenced pages and tail slots."""
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown storage type {dtype!r}")
    rng = np.random.default_rng(seed)
    S = len(q_counts)
    if histories is None:
        histories = rng.integers(0, max_len + 1, size=S)
    seq_lens = np.array([int(h) + int(c) for h, c in zip(histories, q_counts)], dtype=np.int32)
    need = sum(-(-int(L) // page_size) for L in seq_lens)
    bt, pool, used = _tables(rng, seq_lens, page_size, pool_pages=need + extra_pages)
    q_pos = np.concatenate([np.arange(L - c, L, dtype=np.int32) for L, c in zip(seq_lens, q_counts)]
                           + [np.zeros(0, np.int32)])
    Q = int(sum(q_counts))
    q_abs = _normal(rng, (Q, heads, r), dtype)
    q_rope = _normal(rng, (Q, heads, p), dtype)
    latent = _unit_rms(rng, (pool, page_size, 1, r), dtype)
    kpos = _normal(rng, (pool, page_size, 1, p), dtype)
    if poison:
        for t in (latent, kpos):
            _poison_unused(t, used, seq_lens, bt, page_size, dtype, tails=True)
    return MlaBatch(f"random_mla_{seed}", dtype, seq_lens, _packed(list(q_counts)), q_pos.astype(np.int32), bt,
                    page_size, pool, heads, r, p, 1.0 / math.sqrt(r + p), causal, window, q_abs, q_rope, latent,
                    kpos, seed, max_splits)
