// Chunked-prefill body (bf16 MFMA): up to 256 query rows -- 256/G consecutive
// queries of one sequence times the G query heads of one KV head -- against
// the keys the plan assigns to the tile, gathered page by page through the
// block table.
//
// Definition followed: boostr 0.2.0-beta.2 `standard_attention_fwd` (scores
// Q K^T * scale, additive causal / sliding-window mask of
// `build_attention_mask`, softmax, weights times V, logsumexp) with queries at
// absolute positions as ruDNN 0.1.107 `DevicePlan::attention` specifies for
// prefill chunks.  Both products are dense contractions and run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; softmax statistics are
// fp32 and kept per query row in registers (online softmax across key tiles).
//
// Data flow per 64-key tile (three LDS stages, two tiles in flight, one
// barrier per tile):
//   HBM --global_load_lds_dwordx4 (page-gathered, no registers)--> LDS
//     K, V row-major [64 keys][D], the 16-byte pieces of key row t stored at
//     piece ^ swz(t) so that column reads hit distinct bank groups
//   each wave (32 rows):  S^T[64 x 32] = K . Q^T      (Q^T held in registers)
//                         O^T[D x 32] += V^T . P^T    (V^T read with
//                         ds_read_b64_tr_b16, P^T straight from S^T)
// In the S^T / O^T accumulator layout every lane owns one query row, so the
// row max, the rescale and the row sum need at most one cross-lane step.
#pragma once

#include "pa_decode.h"
#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefillTileKeys = 64;
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillRows = kPrefillWaves * kPrefillRowsPerWave;
constexpr int kPrefillStages = 4;  // K/V tiles in the LDS ring

template <int D>
struct PrefillSmem {
  static constexpr int kTile = kPrefillTileKeys * D * 2;  // bytes of one K or V tile
  static constexpr int kStage = 2 * kTile;
  static constexpr int kBytes = kPrefillStages * kStage;
};

__device__ __forceinline__ floatx16_t mfma_32x32x16(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// 16 bytes from global memory to LDS at (wave-uniform base) + 16 * lane
// (global_load_lds_dwordx4; M0 holds the LDS base).
//
// Written as inline assembly on purpose: the compiler's wait-count insertion
// treats every transposed LDS read (ds_read_b64_tr_b16) as possibly aliasing
// any LDS DMA still in flight and drains the vector-memory counter before it,
// which would wait for the tiles being prefetched.  Hidden from that pass,
// the DMA is ordered by the callers' own s_waitcnt vmcnt + barrier pairs.  The
// instruction writes no VGPR, so there is no in-flight register to track.
__device__ __forceinline__ void load_to_lds(const void* src, char* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void_t*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0");
}

// Transposed read: in each 16-lane group, lane 4r + j supplies the address of
// 4 halfwords of row r; lane i receives halfword i % 4 of lane 4r + i / 4's
// chunk for r = 0..3.
__device__ __forceinline__ short4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

// Where piece `piece` of key row `key` is stored: piece ^ swz(key), a
// bit-rotated copy of the low key bits.  Sixteen consecutive keys reading the
// same piece (16-byte operand reads) and four consecutive keys reading four
// neighbouring pieces (transpose reads) then hit distinct 16-byte bank groups.
template <int PIECES>
__device__ __forceinline__ int swz(int key) {
  if constexpr (PIECES >= 16)
    return ((key & 3) << 2) | ((key >> 2) & 3);
  else
    return ((key & 3) << 1) | ((key >> 2) & 1);
}

// Byte offset of 16-byte piece `piece` of key row `key` inside a tile.
template <int D>
__device__ __forceinline__ int tile_off(int key, int piece) {
  return key * (D * 2) + ((piece ^ swz<D / 8>(key)) << 4);
}

// UNIFORM: pages hold >= 16 keys, so a tile's page numbers are scalar loads
// and the loop body issues no other vector-memory loads (a single per-lane
// lookup would make the compiler drain the vector-memory counter before
// every tile issue).
template <int D, int G, bool UNIFORM>
__device__ __forceinline__ void prefill_item_impl(const KernelArgs& a, const WorkItem& it, char* smem) {
  constexpr int NT = kPrefillTileKeys;
  constexpr int KS = D / 16;                         // MFMA k-steps of S^T (over head dims)
  constexpr int DB = D / 32;                         // 32-dim blocks of O^T
  constexpr int PIECES = D / 8;                      // 16-byte pieces per key row
  constexpr int TILE = PrefillSmem<D>::kTile;
  constexpr int STAGE = PrefillSmem<D>::kStage;
  constexpr int NS = kPrefillStages;
  constexpr int KEYS_PER_LOAD = kWave / PIECES;      // key rows one wave-wide load covers
  constexpr int LOADS_PER_TILE = NT / KEYS_PER_LOAD; // per K (or V) tile
  constexpr int LOADS_PER_WAVE = 2 * LOADS_PER_TILE / kPrefillWaves;
  static_assert(PIECES >= 8 && kWave % PIECES == 0, "head size must be a multiple of 64");
  static_assert((2 * LOADS_PER_TILE) % kPrefillWaves == 0, "tile loads must split over the waves");
  static_assert(KEYS_PER_LOAD <= 16, "one load must stay inside a page of 16 keys");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int row = wave * kPrefillRowsPerWave + n;
  const int qloc = row / G, g = row % G;
  const bool row_valid = qloc < it.q_count;
  const int qi = it.q_begin + min(qloc, it.q_count - 1);
  const int head = it.kvh * G + g;
  const int pos = a.q_pos[qi];
  const int tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint32_t row_stride = (uint32_t)a.hkv * D;
  const float c2 = a.scale_log2;

  // Q^T operand: lane (n, h) holds dims 16 ks + 8 h .. +7 of row n
  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((uint64_t)qi * a.hq + head) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * k + 8 * h);
  }

  // positions spanned by this wave's valid rows, for skipping masked tiles
  int pmin = row_valid ? pos : INT32_MAX, pmax = row_valid ? pos : -1;
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
    pmin = min(pmin, __shfl_xor(pmin, s));
    pmax = max(pmax, __shfl_xor(pmax, s));
  }

  floatx16_t o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[b][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  // This wave issues loads wave * LOADS_PER_WAVE .. +LOADS_PER_WAVE of each
  // tile; load i covers K (i < LOADS_PER_TILE) or V rows KEYS_PER_LOAD *
  // (i % LOADS_PER_TILE) + lane / PIECES at stored piece lane % PIECES.  The
  // KEYS_PER_LOAD keys of one load share a page; a load starting past the
  // last key is pulled back to the last group and keys past tok_end read the
  // last key (so every row in LDS is finite sequence data).
  const int my_key_in_load = lane / PIECES;
  const int my_stored_piece = lane % PIECES;
  constexpr int MAXP = NT / 16;
  const int last_page = (te - 1) >> a.page_shift;
  const int last_grp = (te - 1) & ~(KEYS_PER_LOAD - 1);
  // wave-uniform page numbers of the (at most MAXP) pages tile t0 spans
  auto fetch_pages = [&](int t0, int (&tp)[MAXP]) {
    if constexpr (UNIFORM) {
      const int p0 = t0 >> a.page_shift;
#pragma unroll
      for (int q = 0; q < MAXP; ++q) tp[q] = load_uniform(bt, min(p0 + q, last_page));
    }
  };
  auto issue_tile = [&](int t0, char* stage, const int (&tp)[MAXP]) {
    const int p0 = t0 >> a.page_shift;
#pragma unroll
    for (int j = 0; j < LOADS_PER_WAVE; ++j) {
      const int i = wave * LOADS_PER_WAVE + j;
      const int kl = KEYS_PER_LOAD * (i % LOADS_PER_TILE);  // first key of the load within the tile
      const int grp = min(t0 + kl, last_grp);              // wave-uniform
      const int t = min(grp + my_key_in_load, te - 1);
      int page;
      if constexpr (UNIFORM) {
        const int q = (grp >> a.page_shift) - p0;  // 0 .. MAXP-1
        page = tp[0];
#pragma unroll
        for (int k = 1; k < MAXP; ++k) page = q == k ? tp[k] : page;
      } else {
        page = bt[t >> a.page_shift];
      }
      const int piece = my_stored_piece ^ swz<PIECES>(kl + my_key_in_load);
      const uint16_t* pool = reinterpret_cast<const uint16_t*>(i < LOADS_PER_TILE ? a.k : a.v) +
                             (uint64_t)page * ps * row_stride + (uint64_t)it.kvh * D;
      const uint32_t off = (uint32_t)(t & (ps - 1)) * row_stride + piece * 8;
      load_to_lds(pool + off, stage + (i < LOADS_PER_TILE ? 0 : TILE) + (i % LOADS_PER_TILE) * 1024);
    }
  };
  // wait until at most `ahead` tiles of this wave's loads are still in flight
  auto wait_tiles = [&](int ahead) {
    if (!UNIFORM || ahead <= 0)
      wait_vmcnt<0>();
    else if (ahead == 1)
      wait_vmcnt<LOADS_PER_WAVE>();
    else
      wait_vmcnt<2 * LOADS_PER_WAVE>();
  };

  // tile entirely hidden from every row of this wave?
  auto hidden = [&](int t0) {
    return pmax < 0 || (a.causal && t0 > pmax) || (a.window > 0 && t0 + NT - 1 <= pmin - a.window);
  };
  // S^T = K . Q^T : two 32-key blocks; lane (n, h) reads dims 16 k + 8 h of key row n
  auto scores = [&](const char* ks, floatx16_t (&s)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks + tile_off<D>(mb * 32 + n, 2 * k + h));
        s[mb] = mfma_32x32x16(kf, qf[k], s[mb]);
      }
  };
  // mask, new running max and rescale of the accumulators; returns the
  // subtrahend of the exponent (max in log2 units)
  auto row_max = [&](int t0, floatx16_t (&s)[2]) {
    const bool full = t0 >= tb && t0 + NT <= te && (!a.causal || t0 + NT - 1 <= pmin) &&
                      (a.window == 0 || t0 > pmax - a.window);
    // accumulator element e of block mb holds key t0 + 32 mb + 8 (e/4) + 4 h + e%4
    if (!full) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = t0 + 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
          const bool vis = row_valid && t >= tb && t < te && (!a.causal || t <= pos) &&
                           (a.window == 0 || t > pos - a.window);
          s[mb][e] = vis ? s[mb][e] : -INFINITY;
        }
    }
    float mx = m;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
    mx = pair32_max(mx);  // both lane halves hold the same row
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    const float alpha = fast_exp2((m - mu) * c2);
    m = mx;
    l *= alpha;
    if (__any(alpha != 1.f)) {  // no row of the wave raised its max: nothing to rescale
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[b][e] *= alpha;
    }
    return mu * c2;
  };
  // P^T = 2^(S^T c - max) rounded to bf16 and O^T += V^T . P^T.  k-step kk
  // covers keys 16 kk .. +15; lane (n, h) feeds keys 16 kk + 8 (e/4) + 4 h +
  // e%4 (e = 0..7): elements 8 (kk % 2) + e of S^T block kk / 2, and the V^T
  // rows of the same keys by two transposed reads (4 keys each) of dims 32 b
  // + 16 (lane/16 % 2) + lane % 16.
  const int grp16 = lane >> 4, gi = lane & 15;
  const int hh = grp16 >> 1, d16 = grp16 & 1;
  const int rr = gi >> 2, jj = gi & 3;
  auto weights_pv = [&](const char* vs, const floatx16_t (&s)[2], float sub) {
#pragma unroll
    for (int kk = 0; kk < NT / 16; ++kk) {
      const int mb = kk >> 1, e0 = 8 * (kk & 1);
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(__builtin_fmaf(s[mb][e0 + 2 * j], c2, -sub));
        const float p1 = fast_exp2(__builtin_fmaf(s[mb][e0 + 2 * j + 1], c2, -sub));
        pw[j] = pack_bf16(p0, p1);
        l += p0 + p1;
      }
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      const int key0 = 16 * kk + 4 * hh + rr;  // rows r of the first read; +8 for the second
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const int dim = 32 * b + 16 * d16 + 4 * jj;
        const int piece = dim >> 3, half = (dim & 7) * 2;
        const short4_t v0 = lds_read_tr16(vs + tile_off<D>(key0, piece) + half);
        const short4_t v1 = lds_read_tr16(vs + tile_off<D>(key0 + 8, piece) + half);
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))));
        o[b] = mfma_32x32x16(vf, pf, o[b]);
      }
    }
  };

  // Software pipeline over the key tiles: iteration j computes the scores of
  // tile j + 1 on MFMA while the vector units turn the scores of tile j into
  // weights, then accumulates tile j.  The ring holds tile j (V being read),
  // j + 1 (K being read), j + 2 (in flight) and j + 3 (issued at the top of
  // iteration j into the stage tile j - 1 used).  Page numbers run one tile
  // ahead of the loads that use them.
  const int t_first = tb & ~(NT - 1);
  const int ntiles = (te - t_first + NT - 1) / NT;
  int tp_next[MAXP];
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) {
    if (j < ntiles) {
      fetch_pages(t_first + j * NT, tp_next);
      issue_tile(t_first + j * NT, smem + j * STAGE, tp_next);
    }
  }
  fetch_pages(t_first + (NS - 1) * NT, tp_next);

  floatx16_t s_cur[2];
  wait_tiles(min(ntiles - 1, NS - 2));
  __syncthreads();  // tile 0 has landed everywhere
  if (!hidden(t_first)) scores(smem, s_cur);

  for (int j = 0; j < ntiles; ++j) {
    const int t0 = t_first + j * NT;
    const bool has_next = j + 1 < ntiles;
    if (has_next) {
      wait_tiles(min(ntiles - 2 - j, 1));  // tile j + 1 has landed, j + 2 may be in flight
      __syncthreads();  // ... for every wave; every wave is done with tile j - 1
      if (j + NS - 1 < ntiles) {
        issue_tile(t_first + (j + NS - 1) * NT, smem + ((j + NS - 1) % NS) * STAGE, tp_next);
        fetch_pages(t_first + (j + NS) * NT, tp_next);
      }
    }
    const char* vs = smem + (j % NS) * STAGE + TILE;
    const char* ks_next = smem + ((j + 1) % NS) * STAGE;
    const bool cur = !hidden(t0);
    const bool nxt = has_next && !hidden(t0 + NT);
    floatx16_t s_next[2];
    if (cur) {
      const float sub = row_max(t0, s_cur);
      if (nxt) {
        scores(ks_next, s_next);
        weights_pv(vs, s_cur, sub);
      } else {
        weights_pv(vs, s_cur, sub);
      }
    } else if (nxt) {
      scores(ks_next, s_next);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) s_cur[mb] = s_next[mb];
  }

  l = pair32_sum(l);
  if (!row_valid) return;
  const float inv = 1.f / l;
  uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((uint64_t)qi * a.hq + head) * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // dims 32 b + 8 k + 4 h + 0..3
      uint2 w;
      w.x = pack_bf16(o[b][4 * k + 0] * inv, o[b][4 * k + 1] * inv);
      w.y = pack_bf16(o[b][4 * k + 2] * inv, o[b][4 * k + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * b + 8 * k + 4 * h) = w;
    }
  if (a.lse && h == 0) a.lse[(uint64_t)qi * a.hq + head] = m * a.scale + logf(l);
}

template <int D, int G>
__device__ __forceinline__ void prefill_item(const KernelArgs& a, const WorkItem& it, char* smem) {
  if (a.page_shift >= 4)
    prefill_item_impl<D, G, true>(a, it, smem);
  else
    prefill_item_impl<D, G, false>(a, it, smem);
}

// A prefill tile handled one query at a time by the decode body (f32 data and
// head sizes without an MFMA tile): each query's keys [lo, hi] are its own
// visible range.
template <typename T, int D, int G, int NW, int U>
__device__ __forceinline__ void prefill_item_by_queries(const KernelArgs& a, const WorkItem& it, float* smem) {
  const int L = a.seq_lens[it.seq];
  for (int j = 0; j < it.q_count; ++j) {
    const int qi = it.q_begin + j;
    const int p = a.q_pos[qi];
    WorkItem d = it;
    d.kind = kDecode;
    d.q_begin = qi;
    d.q_count = 1;
    d.tok_end = (a.causal ? p : L - 1) + 1;
    d.tok_begin = a.window > 0 ? max(0, p - a.window + 1) : 0;
    d.slot = -1;
    decode_item<T, D, G, NW, U>(a, d, smem);
    __syncthreads();
  }
}

}  // namespace pa
