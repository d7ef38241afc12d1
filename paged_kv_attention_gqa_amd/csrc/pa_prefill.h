// Chunked-prefill body (16-bit MFMA, bf16 or f16): up to 256 query rows -- 256/G consecutive
// queries of one sequence times the G query heads of one KV head -- against
// the keys the plan assigns to the tile, gathered page by page through the
// block table.
//
// Definition followed: boostr 0.2.0-beta.2 `standard_attention_fwd` (scores
// Q K^T * scale, additive causal / sliding-window mask of
// `build_attention_mask`, softmax, weights times V, logsumexp) with queries at
// absolute positions as ruDNN 0.1.107 `DevicePlan::attention` specifies for
// prefill chunks.  Both products are dense contractions and run on
// v_mfma_f32_32x32x16_bf16 (_f16 for f16 data) with fp32 accumulation; softmax statistics are
// fp32 and kept per query row in registers (online softmax across key tiles).
//
// Data flow per 64-key tile (three LDS stages, two tiles in flight, one
// barrier per tile):
//   HBM --global_load_lds_dwordx4 (page-gathered, no registers)--> LDS
//     K [64 keys][D], V [64 keys][Dv] row-major, the 16-byte pieces of key row t stored at
//     piece ^ swz(t) so that column reads hit distinct bank groups
//   each wave (32 rows):  S^T[64 x 32] = K . Q^T      (Q^T held in registers)
//                         O^T[Dv x 32] += V^T . P^T   (V^T read with
//                         ds_read_b64_tr_b16, P^T straight from S^T)
// In the S^T / O^T accumulator layout every lane owns one query row, so the
// row max, the rescale and the row sum need at most one cross-lane step.
#pragma once

#include "pa_decode.h"
#include "pa_device.h"

namespace pa {

// Eight 16-bit elements of an MFMA operand.  The register type is the same
// for bf16 and f16 data; mfma_* reinterpret it as the storage type T.
typedef __bf16 frag_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefillTileKeys = 64;
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillRows = kPrefillWaves * kPrefillRowsPerWave;
constexpr int kLdsBytes = 160 * 1024;
constexpr bool kPrefillPingPong = true;  // two wave groups in opposite phase (see prefill_item_impl)
constexpr float kLazyRescaleLog2 = 8.f;  // weights may reach 2^8 before the reference max moves

template <int D, int DV = D>
struct PrefillSmem {
  static constexpr int kTileK = kPrefillTileKeys * D * 2;   // bytes of one K tile
  static constexpr int kTileV = kPrefillTileKeys * DV * 2;  // bytes of one V tile
  static constexpr int kStage = kTileK + kTileV;
  // K/V tiles in the LDS ring: four (two in flight), or three (one in
  // flight) where four stages do not fit the 160 KB of LDS
  static constexpr int kStages = 4 * kStage <= kLdsBytes ? 4 : 3;
  static constexpr int kBytes = kStages * kStage;
};

template <typename T>
__device__ __forceinline__ floatx16_t mfma_32x32x16(const frag_t& a, const frag_t& b, const floatx16_t& c) {
  if constexpr (__is_same(T, _Float16))
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// LDS address of a generic pointer into LDS: its low 32 bits (the LDS
// aperture of the flat address space starts on a 4 GB boundary).  Taken by
// truncation rather than an address-space cast, whose null check hipcc for
// gfx950 can emit as a compare that fails instruction verification.
__device__ __forceinline__ uint32_t lds_address(const void* p) { return (uint32_t)(size_t)p; }

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
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_address(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0");
}
// The same with the non-temporal hint, for data read once (MLA latent and
// rotary rows); prefill tiles are shared by the query tiles of a sequence
// through L2 and keep the default policy (nt measured 1-6% slower there).
__device__ __forceinline__ void load_to_lds_stream(const void* src, char* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_address(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "s"(lds) : "m0");
}
// The same load from (wave-uniform base) + 32-bit per-lane byte offset
// (global_load_lds_dwordx4 with a scalar base address).
__device__ __forceinline__ void load_to_lds_sv(const char* base, uint32_t off, char* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_address(lds_base));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(lds) : "m0");
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
// Rows of a multiple of 16 pieces use four key bits, other rows (8 or 24
// pieces) three, so that the XOR stays inside the row.
template <int PIECES>
__device__ __forceinline__ int swz(int key) {
  if constexpr (PIECES % 16 == 0)
    return ((key & 3) << 2) | ((key >> 2) & 3);
  else
    return ((key & 3) << 1) | ((key >> 2) & 1);
}

// Load piece idx (16 bytes) of a block of key rows W 16-bit elements wide,
// stored with the tile swizzle: it is stored piece idx % (W / 8) of row
// idx / (W / 8) and carries that row's logical piece (stored ^ swz(row)).
// Returns the row and the source byte offset within it.
template <int W>
__device__ __forceinline__ uint32_t piece_src(int idx, int* row) {
  constexpr int P = W / 8;
  const int r = idx / P, p = idx - r * P;
  *row = r;
  return (uint32_t)((p ^ swz<P>(r)) << 4);
}
template <int W>
struct RowWidth {
  static constexpr int value = W;
};

// Byte offset of 16-byte piece `piece` of key row `key` inside a tile.
template <int D>
__device__ __forceinline__ int tile_off(int key, int piece) {
  return key * (D * 2) + ((piece ^ swz<D / 8>(key)) << 4);
}

// UNIFORM: pages hold >= 16 keys, so each wave's tile rows share one page,
// whose number comes from a per-lane window of 64 tiles loaded once per 64
// tiles; the loop body issues no other vector-memory loads (a per-tile
// per-lane lookup would make the compiler drain the vector-memory counter
// before every tile issue).
//
// DVM: the width of the V and output rows in memory; a tile computes output
// dims dv0 .. dv0 + DV - 1 of them (DV < DVM: one pass of several, each
// recomputing the scores).
template <typename T, int D, int DV, int G, bool UNIFORM, int DVM = DV>
__device__ __forceinline__ void prefill_item_impl(const KernelArgs& a, const WorkItem& it, char* smem, int dv0 = 0) {
  constexpr int NT = kPrefillTileKeys;
  constexpr int KS = D / 16;                         // MFMA k-steps of S^T (over head dims)
  constexpr int DB = DV / 32;                        // 32-dim blocks of O^T
  constexpr int TILE_K = PrefillSmem<D, DV>::kTileK;
  constexpr int STAGE = PrefillSmem<D, DV>::kStage;
  constexpr int NS = PrefillSmem<D, DV>::kStages;
  static_assert(NS >= 3, "the ring holds the V tile read, the K tile scored and one in flight");
  constexpr int MB = NT / 32;                        // 32-key MFMA blocks per tile
  constexpr int HALF = kPrefillWaves / 2;            // waves loading K (the others load V)
  constexpr int KEYS_PER_WAVE = NT / HALF;           // consecutive key rows one wave loads per tile
  constexpr int LOADS_K = KEYS_PER_WAVE * D * 2 / 1024, LOADS_V = KEYS_PER_WAVE * DV * 2 / 1024;
  static_assert(KEYS_PER_WAVE == 16 && NT % 32 == 0 && D % 32 == 0 && DV % 32 == 0,
                "each wave loads 16 consecutive key rows of K (first half of the waves) or V in whole 1 KB loads");

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
  const float c2 = a.scale_log2;

  // Q^T operand: lane (n, h) holds dims 16 ks + 8 h .. +7 of row n
  frag_t qf[KS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((uint64_t)qi * a.hq + head) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = *reinterpret_cast<const frag_t*>(qrow + 16 * k + 8 * h);
  }
  // The tile loads are inline assembly that the compiler's wait-count pass
  // does not see; it would count only these query loads as outstanding and,
  // at every use of a query register in the tile loop, wait until that few
  // loads remain, i.e. for the tile loads still in flight.  Finishing the
  // query loads here leaves it nothing to wait for in the loop.
  wait_vmcnt<0>();

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
  // m: reference max of the row (raised lazily, see row_max); l: sum of the
  // (unrounded) weights relative to it
  float m = -INFINITY, l = 0.f;

  // Tile loads.  Wave w fills key rows 16 (w % 4) .. +15 of the K tile (w < 4)
  // or the V tile (w >= 4) with LOADS_K (LOADS_V) loads of 1 KB; lane l of
  // load j carries 16-byte piece 64 j + l of the 16 rows' stored layout (see
  // piece_src; the swizzle takes the low key bits, which 16 (w % 4) leaves
  // alone).  Sixteen aligned keys never straddle a page of >= 16 keys, so one
  // page number per wave and tile is enough (see page_of).  Keys past tok_end
  // read the last key instead (every row in LDS is finite sequence data; such
  // keys are masked); keys before tok_begin are sequence keys and are masked
  // as well.
  const int wq = wave % HALF;
  const bool loads_v = wave >= HALF;
  const uint32_t rs_k = (uint32_t)a.hkv * D * 2, rs_v = (uint32_t)a.hkv * DVM * 2;  // bytes between key rows
  const char* pool_k = reinterpret_cast<const char*>(a.k) + (uint64_t)it.kvh * D * 2;
  const char* pool_v = reinterpret_cast<const char*>(a.v) + ((uint64_t)it.kvh * DVM + dv0) * 2;
  // Page numbers of this wave's key group in 64 consecutive tiles are one
  // vector load (lane k holding tile win + k's, handed out with v_readlane),
  // reloaded every 64 tiles: a scalar load per tile would make the first
  // LDS-read wait after it (lgkmcnt(0)) also wait for that load's trip to
  // memory.
  const int t_base = tb & ~(NT - 1);
  int win = 0, win_pages = 0;
  auto load_window = [&](int w) {
    return bt[min(t_base + (w + lane) * NT + KEYS_PER_WAVE * wq, te - 1) >> a.page_shift];
  };
  if constexpr (UNIFORM) {
    win_pages = load_window(0);
    wait_vmcnt<0>();
  }
  auto page_of = [&](int t0) {
    if constexpr (UNIFORM) {
      const int jt = (t0 - t_base) / NT;
      if (jt - win >= kWave) {
        win += kWave;
        win_pages = load_window(win);
        // wait here, once per 64 tiles: left pending, the load would make the
        // compiler wait for all memory operations where the paths merge
        wait_vmcnt<0>();
      }
      return __builtin_amdgcn_readlane(win_pages, jt - win);
    } else {
      return 0;
    }
  };
  // Equal K and V widths of 8 or 16 pieces: a load covers whole rows
  // (KPL of them), lane l carries stored piece l % PIECES of row l / PIECES;
  // swz permutes the low key bits, so for row KPL j + my_key the stored
  // piece's offset is lane_piece0 ^ (swz(KPL j) << 4) (rows are >= 128 bytes
  // apart, the XOR stays in the piece bits), computed from one per-lane value.
  constexpr int PIECES = D / 8;
  constexpr bool WHOLE_ROWS = D == DV && kWave % PIECES == 0;
  constexpr int KPL = WHOLE_ROWS ? kWave / PIECES : 1;
  const int my_key = lane / PIECES;
  const uint32_t lane_piece0 = (uint32_t)(((lane % PIECES) ^ swz<PIECES>(my_key)) << 4);
  const uint32_t lane_off0 = (uint32_t)my_key * rs_k + lane_piece0;
  // row and stored-piece offset of load j for this lane (rows W elements wide)
  auto load_piece = [&](auto width, int j, int* r) {
    constexpr int W = decltype(width)::value;
    if constexpr (WHOLE_ROWS) {
      *r = KPL * j + my_key;
      return lane_piece0 ^ (uint32_t)(swz<PIECES>(KPL * j) << 4);
    } else {
      return piece_src<W>(kWave * j + lane, r);
    }
  };
  // this wave's 16 rows of one tile (rows W elements wide, rs bytes apart in the pool)
  auto issue_rows = [&](auto width, const char* pool, uint32_t rs, char* dst, int k0, int page) {
    constexpr int W = decltype(width)::value;
    constexpr int LOADS = KEYS_PER_WAVE * W * 2 / 1024;
    if (UNIFORM && k0 + KEYS_PER_WAVE <= te) {
      // whole group in range: one scalar base, fixed lane offsets
      const char* base = pool + ((uint64_t)page * ps + (k0 & (ps - 1))) * rs;
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        if constexpr (WHOLE_ROWS) {
          const uint32_t off = (lane_off0 ^ (uint32_t)(swz<PIECES>(KPL * j) << 4)) + (uint32_t)(KPL * j) * rs;
          load_to_lds_sv(base, off, dst + j * 1024);
        } else {
          int r;
          const uint32_t piece = load_piece(width, j, &r);
          load_to_lds_sv(base, (uint32_t)r * rs + piece, dst + j * 1024);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        int r;
        const uint32_t piece = load_piece(width, j, &r);
        const int t = min(k0 + r, te - 1);
        const uint32_t off = (uint32_t)(t & (ps - 1)) * rs + piece;
        if constexpr (UNIFORM) {
          load_to_lds_sv(pool + (uint64_t)page * ps * rs, off, dst + j * 1024);
        } else {
          const char* src = pool + (uint64_t)bt[t >> a.page_shift] * ps * rs + off;  // per-lane page
          load_to_lds(src, dst + j * 1024);
        }
      }
    }
  };
  auto issue_tile = [&](int t0, char* stage, int page) {
    const int k0 = t0 + KEYS_PER_WAVE * wq;  // first key of this wave's rows
    if constexpr (D == DV && DV == DVM) {  // one code path for both halves of the waves
      issue_rows(RowWidth<D>{}, loads_v ? pool_v : pool_k, rs_k,
                 stage + (loads_v ? TILE_K : 0) + KEYS_PER_WAVE * wq * (D * 2), k0, page);
    } else if (loads_v) {
      issue_rows(RowWidth<DV>{}, pool_v, rs_v, stage + TILE_K + KEYS_PER_WAVE * wq * (DV * 2), k0, page);
    } else {
      issue_rows(RowWidth<D>{}, pool_k, rs_k, stage + KEYS_PER_WAVE * wq * (D * 2), k0, page);
    }
  };
  // wait until at most `ahead` tiles of this wave's loads are still in flight
  auto wait_tiles = [&](int ahead) {
    if (!UNIFORM || ahead <= 0)
      wait_vmcnt<0>();
    else if (ahead == 1)
      loads_v ? wait_vmcnt<LOADS_V>() : wait_vmcnt<LOADS_K>();
    else
      loads_v ? wait_vmcnt<2 * LOADS_V>() : wait_vmcnt<2 * LOADS_K>();
  };

  // tile entirely hidden from every row of this wave?
  auto hidden = [&](int t0) {
    return pmax < 0 || (a.causal && t0 > pmax) || (a.window > 0 && t0 + NT - 1 <= pmin - a.window);
  };
  // LDS byte offsets of this lane's operand reads within a tile, computed once:
  // K fragment k (key row n, piece 2k + h; +32 rows for the second block) and
  // V^T half-fragments (b, r) of k-step 0 (later k-steps add 16 rows).
  uint32_t koff[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) koff[k] = (uint32_t)tile_off<D>(n, 2 * k + h);
  uint32_t voff[DB][2];
  {
    const int grp16 = lane >> 4, gi = lane & 15;
    const int key0 = 4 * (grp16 >> 1) + (gi >> 2);
    const int dim0 = 16 * (grp16 & 1) + 4 * (gi & 3);
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int dim = 32 * b + dim0;
        voff[b][r] = (uint32_t)(tile_off<DV>(key0 + 8 * r, dim >> 3) + (dim & 7) * 2);
      }
  }
  // S^T = K . Q^T : two 32-key blocks; lane (n, h) reads dims 16 k + 8 h of key row n
  auto scores = [&](const char* ks, floatx16_t (&s)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
    // K fragments run kAhead MFMAs ahead of their use (a small register ring)
    constexpr int kSteps = MB * KS, kAhead = 4;
    auto frag = [&](int i) {
      return *reinterpret_cast<const frag_t*>(ks + koff[i / MB] + (i % MB) * 32 * (D * 2));
    };
    frag_t ring[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = frag(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const frag_t kf = ring[i % kAhead];
      if (i + kAhead < kSteps) ring[i % kAhead] = frag(i + kAhead);
      s[i % MB] = mfma_32x32x16<T>(kf, qf[i / MB], s[i % MB]);
      __builtin_amdgcn_sched_barrier(0);  // keep the read distance (the scheduler would shorten it)
    }
  };
  // Mask the tile and update the reference max; returns the exponent offset
  // (reference max in log2 units).  The reference is raised only when a row's
  // tile max exceeds it by more than 2^kLazyRescaleLog2 in weight, so weights
  // stay <= 2^kLazyRescaleLog2 and the accumulators are rescaled only on the
  // few tiles that raise some row's max that far.  Numerator and denominator
  // share the reference, so the result does not depend on when it moves.
  auto row_max = [&](int t0, floatx16_t (&s)[MB]) {
    const bool full = t0 >= tb && t0 + NT <= te && (!a.causal || t0 + NT - 1 <= pmin) &&
                      (a.window == 0 || t0 > pmax - a.window);
    // accumulator element e of block mb holds key t0 + 32 mb + 8 (e/4) + 4 h + e%4
    if (!full) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = t0 + 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
          const bool vis = row_valid && t >= tb && t < te && (!a.causal || t <= pos) &&
                           (a.window == 0 || t > pos - a.window);
          s[mb][e] = vis ? s[mb][e] : -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
    mx = pair32_max(mx);  // both lane halves hold the same row
    if (__any(mx * c2 > m * c2 + kLazyRescaleLog2)) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2((m - (mn == -INFINITY ? 0.f : mn)) * c2);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[b][e] *= alpha;
    }
    return (m == -INFINITY ? 0.f : m) * c2;
  };
  // P^T = 2^(S^T c - ref) rounded to the storage type (vector work only).  k-step kk
  // covers keys 16 kk .. +15; lane (n, h) feeds keys 16 kk + 8 (e/4) + 4 h +
  // e%4 (e = 0..7): elements 8 (kk % 2) + e of S^T block kk / 2.
  auto weights = [&](const floatx16_t (&s)[MB], float sub, frag_t (&pf)[NT / 16]) {
#pragma unroll
    for (int kk = 0; kk < NT / 16; ++kk) {
      const int mb = kk >> 1, e0 = 8 * (kk & 1);
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(__builtin_fmaf(s[mb][e0 + 2 * j], c2, -sub));
        const float p1 = fast_exp2(__builtin_fmaf(s[mb][e0 + 2 * j + 1], c2, -sub));
        pw[j] = Pair16<T>::pack(p0, p1);
        l += p0 + p1;
      }
      pf[kk] = __builtin_bit_cast(frag_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    }
  };
  // O^T += V^T . P^T (matrix work only): the V^T rows of k-step kk's keys by
  // two transposed reads (4 keys each) of dims 32 b + 16 (lane/16 % 2) +
  // lane % 16 (offsets voff, plus 16 rows per k-step).
  auto pv = [&](const char* vs, const frag_t (&pf)[NT / 16]) {
#pragma unroll
    for (int kk = 0; kk < NT / 16; ++kk) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const short4_t v0 = lds_read_tr16(vs + voff[b][0] + kk * 16 * (DV * 2));
        const short4_t v1 = lds_read_tr16(vs + voff[b][1] + kk * 16 * (DV * 2));
        const frag_t vf = __builtin_bit_cast(
            frag_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))));
        o[b] = mfma_32x32x16<T>(vf, pf[kk], o[b]);
      }
    }
  };

  // Two wave groups in opposite phase, each alternating a matrix phase M(j)
  // (P.V of tile j - 1, then the scores of tile j) with a vector phase V(j)
  // (mask, reference max and weights of tile j).  Between the barriers that
  // publish tiles j and j + 1 the leading waves (0-3) run M(j) then V(j) and
  // the trailing waves (4-7) V(j - 1) then M(j).  Each SIMD holds one wave of
  // each group, so while one runs its matrix phase the other runs its vector
  // phase: the two never wait on each other for the MFMA pipe, and a wave's
  // in-order issue never holds its vector work behind its own MFMAs.  Tiles
  // land two barriers after their loads are issued; the ring holds tile
  // j - 1 (V, read in M(j)), j (being read), j + 1 (in flight) and j + 2
  // (issued after the barrier of tile j into the stage of tile j - 2, whose
  // last reader was M(j - 1)).
  const int t_first = tb & ~(NT - 1);
  const int ntiles = (te - t_first + NT - 1) / NT;
  const bool lead = !kPrefillPingPong || wave < kPrefillWaves / 2;
  int page_next = 0;
#pragma unroll
  for (int j = 0; j < NS - 2; ++j) {
    if (j < ntiles) {
      page_next = page_of(t_first + j * NT);
      issue_tile(t_first + j * NT, smem + j * STAGE, page_next);
    }
  }
  page_next = page_of(t_first + (NS - 2) * NT);

  floatx16_t s[MB];
  frag_t pf[NT / 16];
  auto sync = [&](int j) {
    wait_tiles(min(ntiles - 1 - j, NS - 3));  // tile j has landed, j + 1 may be in flight (four stages)
    barrier_keep_loads();                // ... for every wave; tile j - 2 is no longer read
    if (j + NS - 2 < ntiles) {
      issue_tile(t_first + (j + NS - 2) * NT, smem + ((j + NS - 2) % NS) * STAGE, page_next);
      page_next = page_of(t_first + (j + NS - 1) * NT);
    }
  };
  auto vector_phase = [&](int jj) {  // tile jj's scores -> weights
    if (jj >= 0 && jj < ntiles && !hidden(t_first + jj * NT)) weights(s, row_max(t_first + jj * NT, s), pf);
  };
  // The matrix phase runs at wave priority 1, so that where both waves of a
  // SIMD have an instruction ready the MFMA chain and its operand reads
  // issue first (chunked prefill +2%, mixed batch +1.6%; the vector phase
  // raised instead: -1.5%).
  auto matrix_phase = [&](int jj) {  // P.V of tile jj - 1, scores of tile jj
    __builtin_amdgcn_s_setprio(1);
    if (jj > 0 && !hidden(t_first + (jj - 1) * NT)) pv(smem + ((jj - 1) % NS) * STAGE + TILE_K, pf);
    if (jj < ntiles && !hidden(t_first + jj * NT)) scores(smem + (jj % NS) * STAGE, s);
    __builtin_amdgcn_s_setprio(0);
  };
  // One loop body for both groups, V(j - 1) then M(j); only the barrier
  // (and the loads issued after it) sits before V(j - 1) in the trailing
  // waves and after it in the leading ones.
  for (int j = 0; j <= ntiles; ++j) {
    const bool more = j < ntiles;
    if (!lead && more) sync(j);
    vector_phase(j - 1);
    if (lead && more) sync(j);
    matrix_phase(j);
  }

  l = pair32_sum(l);
  if (!row_valid) return;
  const float inv = 1.f / l;
  uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((uint64_t)qi * a.hq + head) * DVM + dv0;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // dims 32 b + 8 k + 4 h + 0..3
      uint2 w;
      w.x = Pair16<T>::pack(o[b][4 * k + 0] * inv, o[b][4 * k + 1] * inv);
      w.y = Pair16<T>::pack(o[b][4 * k + 2] * inv, o[b][4 * k + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * b + 8 * k + 4 * h) = w;
    }
  if (a.lse && h == 0 && dv0 == 0) a.lse[(uint64_t)qi * a.hq + head] = m * a.scale + logf(l);
}

// D = Dv = 256 runs in two passes of 128 output dims (the output sums of 256
// dims and the 256-dim query operand would not fit one wave's registers).
template <int D, int DV>
struct PrefillPass {
  static constexpr int kDims = (D == 256 && DV == 256) ? 128 : DV;
};

template <typename T, int D, int DV, int G>
__device__ __forceinline__ void prefill_item(const KernelArgs& a, const WorkItem& it, char* smem) {
  static_assert(sizeof(T) == 2, "the MFMA tile runs on 16-bit data");
  constexpr int DP = PrefillPass<D, DV>::kDims;
#pragma unroll 1
  for (int dv0 = 0; dv0 < DV; dv0 += DP) {
    if (dv0 > 0) __syncthreads();  // every wave is done with the previous pass's ring
    if (a.page_shift >= 4)
      prefill_item_impl<T, D, DP, G, true, DV>(a, it, smem, dv0);
    else
      prefill_item_impl<T, D, DP, G, false, DV>(a, it, smem, dv0);
  }
}

// A prefill tile handled one query at a time by the decode body (f32 data,
// which has no MFMA tile): each query's keys [lo, hi] are its own visible
// range.
template <typename T, int D, int DV, int G, int NW, int U>
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
    decode_item<T, D, DV, G, NW, U>(a, d, smem);
    __syncthreads();
  }
}

}  // namespace pa
