// Absorbed-MLA decode body (16-bit MFMA, bf16 or f16): one query, one group of H = 16 of
// its heads (heads 16 g .. 16 g + 15 of item kvh = g; the last group of a head count
// that is no multiple of 16 is partial), one contiguous range of its visible keys.
//
// Definition followed: ruDNN 0.1.107 paged_attention/mod.rs `DevicePlan::mla`
// -- one shared latent head [pages, page_size, 1, R] serves as key and value,
// a rotated position cache [pages, page_size, 1, P] adds q_rope . kpos to
// every score, scale from the model's original query/key size -- with the
// softmax and masking of boostr 0.2.0-beta.2 `standard_attention_fwd` /
// `build_attention_mask`.
//
// Per key the method reads R + P = 576 16-bit elements (1152 bytes) and does 16 x (576 +
// 512) multiply-adds: ~30 flops per byte, above what the fp32 vector units
// sustain at HBM speed, so both products run on MFMA with the 16 heads as the
// N dimension:
//   S^T[16 keys x 16 heads] = latent . q_abs^T + kpos . q_rope^T   (16x16x32)
//   O^T[R x 16 heads]      += latent^T . P^T                      (16x16x16)
// The four waves of a workgroup share a four-stage LDS ring of 16-key tiles
// (three in flight while one is used, one barrier per tile), loaded with
// global_load_lds_dwordx4 (16-byte pieces of key row t stored at piece ^
// swz(t)); page numbers come from a per-lane window of 64 tiles loaded
// once per 64 tiles, so the vector-memory counter counts tile loads only.  Each
// wave computes the score tile over a quarter of the 576 dims; the four
// partial tiles meet in LDS and every wave sums them in one fixed order, so
// all waves hold the same scores and softmax statistics.  Each wave owns
// R / 4 = 128 output dims; latent^T fragments come from ds_read_b64_tr_b16.
// Every lane owns one head's column, so softmax needs two cross-lane steps
// per tile.
#pragma once

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_prefill.h"

namespace pa {

typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kMlaHeads = 16;
constexpr int kMlaRank = 512;
constexpr int kMlaRope = 64;
constexpr int kMlaTileKeys = 16;
constexpr int kMlaWaves = 4;
constexpr int kMlaStages = 4;  // tiles in the ring: three in flight while one is used

// NG: head groups per decode item (their partial score tiles share the
// exchange area).
template <int NG = 1>
struct MlaSmem {
  static constexpr int kLatTile = kMlaTileKeys * kMlaRank * 2;   // 16 KB
  static constexpr int kPosTile = kMlaTileKeys * kMlaRope * 2;   // 2 KB
  static constexpr int kStage = kLatTile + kPosTile;
  static constexpr int kXchgOff = kMlaStages * kStage;           // 72 KB
  static constexpr int kBytes = kXchgOff + NG * kMlaWaves * 64 * 16;  // + partial scores of the four waves
};

// Wait until at most `ahead` (<= MAXA) tiles of PER loads each are still in
// flight for this wave.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if constexpr (MAXA == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAXA)
      wait_vmcnt<PER * MAXA>();
    else
      wait_tiles_ahead<PER, MAXA - 1>(ahead);
  }
}

template <typename T>
__device__ __forceinline__ floatx4_t mfma_16x16x32(const frag_t& a, const frag_t& b, const floatx4_t& c) {
  if constexpr (__is_same(T, _Float16))
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <typename T>
__device__ __forceinline__ floatx4_t mfma_16x16x16(const short4_t& a, const short4_t& b, const floatx4_t& c) {
  if constexpr (__is_same(T, _Float16))
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c,
                                                 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Byte offset of 16-byte piece `piece` of key row `key` in a tile of WIDTH
// 16-bit elements per row.
template <int WIDTH>
__device__ __forceinline__ int mla_off(int key, int piece) {
  return key * (WIDTH * 2) + ((piece ^ swz<WIDTH / 8>(key)) << 4);
}

// tid: the thread index, as for decode_item.
//
// PREFILL: the item holds up to kMlaPrefillQueries consecutive queries of
// one sequence (chunked prefill); waves 2 i and 2 i + 1 take query q_begin +
// i, its 16 heads as the MFMA columns, each owning half of the R output dims
// (both compute the query's scores), and mask the keys of the shared tiles
// by that query's position.  The tiles are loaded once for the item's
// queries.
//
// SPLIT (decode items): the score tile is split over the waves as above.
// The prefill instantiation runs its decode items with SPLIT = false, every
// wave computing the whole score tile: hipcc for gfx950 fails to generate
// code ("operand has incorrect register class") for the split tile next to
// the prefill body in one kernel.
//
// NG (split decode items only): the item covers head groups kvh .. kvh +
// NG - 1, which share each tile's LDS reads (latent and rotary fragments,
// transposed latent reads), the barriers and the exchange; each group has
// its own query operands, scores, softmax state and output sums.  A group
// past the last head (an odd number of groups) computes copies and stores
// nothing; group g's split partials go to slot + g.
constexpr int kMlaWavesPerQuery = kMlaWaves / kMlaPrefillQueries;
static_assert(kMlaWavesPerQuery == 2, "two waves per prefill query");
template <typename T, bool PREFILL = false, bool SPLIT = true, int NG = 1>
__device__ __forceinline__ void mla_item(const KernelArgs& a, const WorkItem& it, char* smem, int tid = threadIdx.x) {
  constexpr int H = kMlaHeads, R = kMlaRank, P = kMlaRope, NT = kMlaTileKeys;
  constexpr int KS_LAT = R / 32, KS_POS = P / 32;  // 16x16x32 k-steps
  constexpr int DW = PREFILL ? R / kMlaWavesPerQuery : R / kMlaWaves;  // output dims per wave
  constexpr int DB = DW / 16;                       // 16-dim blocks of O^T per wave
  constexpr int ROWS_PER_WAVE = NT / kMlaWaves;     // latent rows each wave loads per tile
  constexpr int LOADS_PER_TILE = ROWS_PER_WAVE + 1; // + a quarter of the rotary tile
  static_assert(NT % kMlaWaves == 0 && DW % 16 == 0, "tile must split over the waves");
  const int lane = tid & 63;
  // wave-uniform (readfirstlane): keeps the tile schedule and its block-table
  // lookups in scalar registers and scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, c = lane >> 4;           // MFMA column (head / key row) and k-group
  const int wq = wave / kMlaWavesPerQuery;          // PREFILL: this wave's query of the item
  const bool q_ok = !PREFILL || wq < it.q_count;
  const int qi = it.q_begin + (PREFILL ? min(wq, it.q_count - 1) : 0);
  const int qpos = PREFILL ? a.q_pos[qi] : 0;
  // row of this lane's query head (its MFMA column) in group g; columns past
  // the last head compute a copy of it and store nothing
  auto head_row = [&](int g) { return (uint64_t)qi * a.hq + min(H * (it.kvh + g) + n, a.hq - 1); };
  const int dim0 = DW * (PREFILL ? wave % kMlaWavesPerQuery : wave);  // first output dim of this wave
  const int tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint16_t* lat = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* kpos = reinterpret_cast<const uint16_t*>(a.kr);

  // q^T operands: lane (n, c) holds dims 32 ks + 8 c .. +7 of head n.
  // Decode: each wave computes the scores over its own quarter of the
  // latent k-steps (4 wave .. 4 wave + 3, 16x16x32) and of the rotary dims
  // (16 wave .. 16 wave + 15, one 16x16x16 step: lane (n, c) holds dims
  // 16 wave + 4 c .. +3); the four partial tiles are summed through LDS.
  constexpr bool SPLIT_S = !PREFILL && SPLIT;
  static_assert(NG == 1 || SPLIT_S, "several head groups per item only on split decode items");
  // Prefill: the two waves of a query split its score tile the same way,
  // wave 2 i + h taking latent k-steps 8 h .. 8 h + 7 and rotary k-step h
  // (16x16x32), their partial tiles summed through LDS.
  constexpr bool SPLIT_P = PREFILL;
  static_assert(!SPLIT_P || (KS_LAT % kMlaWavesPerQuery == 0 && KS_POS == kMlaWavesPerQuery),
                "prefill score tile split over a query's two waves");
  constexpr int QA = SPLIT_S ? KS_LAT / kMlaWaves : (SPLIT_P ? KS_LAT / kMlaWavesPerQuery : KS_LAT);
  constexpr int QP = SPLIT_S ? 0 : (SPLIT_P ? 1 : KS_POS);
  static_assert(P == 16 * kMlaWaves, "one 16-dim rotary step per wave");
  const int half = wave % kMlaWavesPerQuery;  // prefill: this wave's half of the score k-steps
  const int ks0 = SPLIT_S ? QA * wave : (SPLIT_P ? QA * half : 0);
  frag_t qa[NG][QA], qp[QP > 0 ? QP : 1];
  short4_t qp16[NG] = {};
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint64_t hrow = head_row(g);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + hrow * R;
    const uint16_t* prow = reinterpret_cast<const uint16_t*>(a.qr) + hrow * P;
#pragma unroll
    for (int k = 0; k < QA; ++k) qa[g][k] = *reinterpret_cast<const frag_t*>(qrow + 32 * (ks0 + k) + 8 * c);
#pragma unroll
    for (int k = 0; k < QP; ++k) qp[k] = *reinterpret_cast<const frag_t*>(prow + 32 * ((SPLIT_P ? half : 0) + k) + 8 * c);
    if constexpr (SPLIT_S) qp16[g] = *reinterpret_cast<const short4_t*>(prow + 16 * wave + 4 * c);
  }
  // The tile loads below are inline assembly that the compiler's wait-count
  // pass does not see; it would count only these query loads as outstanding
  // and, at every use of a query register in the tile loop, wait until that
  // few loads remain, i.e. for the tile loads still in flight.  Finishing the
  // query loads here leaves it nothing to wait for in the loop.

  floatx4_t o[NG][DB];
  float m[NG], l[NG], lx[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int b = 0; b < DB; ++b) o[g][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m[g] = -INFINITY;
    l[g] = 0.f;
    lx[g] = 0.f;
  }

  auto clamp_key = [&](int t) { return min(max(t, tb), te - 1); };
  // This wave's share of a tile: latent rows ROWS_PER_WAVE * wave + r (one
  // 1 KB load each) and rotary rows 4 wave .. 4 wave + 3 (half a load: lanes
  // 0..31, 8 lanes of 16 bytes per 128-byte row).  With pages of >= 16 keys
  // the 16 keys of a tile (clamped ones included) share one page, and the
  // page numbers of 64 consecutive tiles are one vector load (lane k holding
  // tile win + k's, handed out with v_readlane), reloaded every 64 tiles: a
  // scalar load per tile would make the first LDS-read wait after it
  // (lgkmcnt(0)) also wait for that load's trip to memory.  Smaller pages
  // look each row up.
  const bool uniform = ps >= NT;
  const int first = tb & ~(NT - 1);
  int win = 0, win_pages = 0;
  auto load_window = [&](int w) {
    return bt[clamp_key(first + (w + lane) * NT) >> a.page_shift];
  };
  if (uniform) win_pages = load_window(0);
  wait_vmcnt<0>();  // query loads and the first window (see above)
  auto tile_page = [&](int t0) {
    if (!uniform) return 0;
    const int jt = (t0 - first) / NT;
    if (jt - win >= kWave) {
      win += kWave;
      win_pages = load_window(win);
      // wait here, once per 64 tiles: left pending, the load would make the
      // compiler wait for all memory operations where the paths merge, on
      // every tile
      wait_vmcnt<0>();
    }
    return __builtin_amdgcn_readlane(win_pages, jt - win);
  };
  auto issue_tile = [&](int t0, char* stage, int tpage) {
    int pg[ROWS_PER_WAVE];
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; ++r)
      pg[r] = uniform ? tpage : load_uniform(bt, clamp_key(t0 + ROWS_PER_WAVE * wave + r) >> a.page_shift);
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; ++r) {
      const int row = ROWS_PER_WAVE * wave + r;
      const int t = clamp_key(t0 + row);
      const uint16_t* src = lat + ((uint64_t)pg[r] * ps + (t & (ps - 1))) * R + ((lane ^ swz<R / 8>(row)) * 8);
      load_to_lds_stream(src, stage + row * (R * 2));
    }
    if (lane < 32) {
      const int rl = lane >> 3;  // 0..3
      int page = pg[0];
#pragma unroll
      for (int q = 1; q < ROWS_PER_WAVE; ++q) page = rl == q ? pg[q] : page;
      const int row = ROWS_PER_WAVE * wave + rl;
      const int t = clamp_key(t0 + row);
      const uint16_t* src = kpos + ((uint64_t)page * ps + (t & (ps - 1))) * P + (((lane & 7) ^ swz<P / 8>(row)) * 8);
      load_to_lds_stream(src, stage + MlaSmem<NG>::kLatTile + wave * 512);
    }
  };

  // tiles start on multiples of 16 keys; keys outside [tb, te) are masked
  const int ntiles = (te - first + NT - 1) / NT;
  int page_next = 0;
#pragma unroll
  for (int j = 0; j < kMlaStages - 1; ++j)
    if (j < ntiles) {
      page_next = tile_page(first + j * NT);
      issue_tile(first + j * NT, smem + j * MlaSmem<NG>::kStage, page_next);
    }
  page_next = tile_page(first + (kMlaStages - 1) * NT);
  for (int j = 0; j < ntiles; ++j) {
    // tiles j+1 .. j+2 may stay in flight; this wave's share of tile j has landed
    wait_tiles_ahead<LOADS_PER_TILE, kMlaStages - 2>(min(ntiles - 1 - j, kMlaStages - 2));
    barrier_keep_loads();  // ... every wave's share has; tile j-1's stage is free for reuse
    if (j + kMlaStages - 1 < ntiles) {
      issue_tile(first + (j + kMlaStages - 1) * NT, smem + ((j + kMlaStages - 1) % kMlaStages) * MlaSmem<NG>::kStage,
                 page_next);
      page_next = tile_page(first + (j + kMlaStages) * NT);
    }
    const int t0 = first + j * NT;
    const char* ls = smem + (j % kMlaStages) * MlaSmem<NG>::kStage;
    const char* kps = ls + MlaSmem<NG>::kLatTile;

    // S^T: lane (n, c) holds keys 4 c + r (r = 0..3) of head n; two
    // accumulator chains halve the dependent MFMA latency
    floatx4_t s[NG];
    if constexpr (PREFILL) {
      // this wave's half of the k-steps, fragments read as they are used (the
      // output sums hold 128 registers); the pair's two partial tiles meet in
      // LDS and both waves add them in one order, so they hold the same scores
      floatx4_t sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < QA; ++k)
        sc[k & 1] = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(ls + mla_off<R>(n, 4 * (ks0 + k) + c)),
                                     qa[0][k], sc[k & 1]);
      sc[0] = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(kps + mla_off<P>(n, 4 * half + c)), qp[0], sc[0]);
      typedef __attribute__((address_space(3))) floatx4_t lds_f4_t;
      lds_f4_t* xs = (lds_f4_t*)(size_t)__builtin_amdgcn_readfirstlane(lds_address(smem + MlaSmem<NG>::kXchgOff));
      xs[wave * 64 + lane] = sc[0] + sc[1];
      barrier_keep_loads();  // the exchange is written (the tiles in flight stay in flight)
      const int w0 = wave - half;
      s[0] = xs[w0 * 64 + lane] + xs[(w0 + 1) * 64 + lane];
    } else if constexpr (!SPLIT_S) {
      frag_t kf[KS_LAT + KS_POS];
#pragma unroll
      for (int k = 0; k < KS_LAT; ++k) kf[k] = *reinterpret_cast<const frag_t*>(ls + mla_off<R>(n, 4 * k + c));
#pragma unroll
      for (int k = 0; k < KS_POS; ++k)
        kf[KS_LAT + k] = *reinterpret_cast<const frag_t*>(kps + mla_off<P>(n, 4 * k + c));
      floatx4_t sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < KS_LAT; ++k) sc[k & 1] = mfma_16x16x32<T>(kf[k], qa[0][k], sc[k & 1]);
#pragma unroll
      for (int k = 0; k < KS_POS; ++k) sc[k & 1] = mfma_16x16x32<T>(kf[KS_LAT + k], qp[k], sc[k & 1]);
      s[0] = sc[0] + sc[1];
    } else {
      frag_t kf[QA];
      // pieces 16 wave + 4 k + c: the swizzle (< 16) leaves the 16-piece block in place
      const char* lsw = ls + 256 * wave;
#pragma unroll
      for (int k = 0; k < QA; ++k) kf[k] = *reinterpret_cast<const frag_t*>(lsw + mla_off<R>(n, 4 * k + c));
      const short4_t kp16 = *reinterpret_cast<const short4_t*>(kps + mla_off<P>(n, 2 * wave + (c >> 1)) + (c & 1) * 8);
      // the partial tiles of the four waves, summed in one fixed order so
      // that every wave holds the same scores (the previous tile's reads
      // were done before this tile's barrier)
      typedef __attribute__((address_space(3))) floatx4_t lds_f4_t;
      lds_f4_t* xs = (lds_f4_t*)(size_t)__builtin_amdgcn_readfirstlane(lds_address(smem + MlaSmem<NG>::kXchgOff));
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        floatx4_t sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int k = 0; k < QA; ++k) sc[k & 1] = mfma_16x16x32<T>(kf[k], qa[g][k], sc[k & 1]);
        sc[0] = mfma_16x16x16<T>(kp16, qp16[g], sc[0]);
        xs[(g * kMlaWaves + wave) * 64 + lane] = sc[0] + sc[1];
      }
      barrier_keep_loads();  // the exchange is written (the tiles in flight stay in flight)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const lds_f4_t* xg = xs + g * kMlaWaves * 64;
        s[g] = ((xg[lane] + xg[64 + lane]) + xg[128 + lane]) + xg[192 + lane];
      }
    }
    short4_t pf[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * c + r;
        if constexpr (PREFILL)
          s[g][r] = (t >= tb && t < te && (!a.causal || t <= qpos) && (a.window == 0 || t > qpos - a.window))
                        ? s[g][r]
                        : -INFINITY;
        else
          s[g][r] = (t >= tb && t < te) ? s[g][r] : -INFINITY;
      }

      // Online softmax against a lazily raised reference max (weights stay
      // <= 2^kLazyRescaleLog2; the accumulators are rescaled only when a tile
      // raises some head's max past that).
      float mx = fmaxf(fmaxf(s[g][0], s[g][1]), fmaxf(s[g][2], s[g][3]));
      mx = pair32_max(pair16_max(mx));  // over the four k-groups of lanes
      if (__any(mx * a.scale_log2 > m[g] * a.scale_log2 + kLazyRescaleLog2)) {
        const float mn = fmaxf(m[g], mx);
        const float alpha = fast_exp2((m[g] - (mn == -INFINITY ? 0.f : mn)) * a.scale_log2);
        m[g] = mn;
        l[g] *= alpha;
        lx[g] *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b) o[g][b] *= alpha;
      }
      const float sub = (m[g] == -INFINITY ? 0.f : m[g]) * a.scale_log2;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(__builtin_fmaf(s[g][r], a.scale_log2, -sub));
      const uint32_t w0 = Pair16<T>::pack(p[0], p[1]), w1 = Pair16<T>::pack(p[2], p[3]);
      l[g] += Pair16<T>::lo(w0) + Pair16<T>::hi(w0) + Pair16<T>::lo(w1) + Pair16<T>::hi(w1);
      lx[g] += (p[0] + p[1]) + (p[2] + p[3]);
      pf[g] = __builtin_bit_cast(short4_t, make_uint2(w0, w1));
    }

    // O^T block b (dims dim0 + 16 b ..): lane (i = lane % 16, c) needs
    // latent[4 c + r][dim0 + 16 b + i]: one transposed read, lane 4 r + j
    // giving the address of dims dim0 + 16 b + 4 j of key row 4 c + r.
    const int key = 4 * c + (n >> 2);
    if constexpr (PREFILL) {
      constexpr int VB = 8;  // fragments read per group (the output sums hold 128 registers)
#pragma unroll
      for (int b0 = 0; b0 < DB; b0 += VB) {
        short4_t vf[VB];
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          const int dim = dim0 + 16 * (b0 + b) + 4 * (n & 3);
          vf[b] = lds_read_tr16(ls + mla_off<R>(key, dim >> 3) + (dim & 7) * 2);
        }
#pragma unroll
        for (int b = 0; b < VB; ++b) o[0][b0 + b] = mfma_16x16x16<T>(vf[b], pf[0], o[0][b0 + b]);
      }
    } else {
      short4_t vf[DB];
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const int dim = DW * wave + 16 * b + 4 * (n & 3);
        vf[b] = lds_read_tr16(ls + mla_off<R>(key, dim >> 3) + (dim & 7) * 2);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int b = 0; b < DB; ++b) o[g][b] = mfma_16x16x16<T>(vf[b], pf[g], o[g][b]);
    }
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (H * (it.kvh + g) >= a.hq) break;  // a group past the last head (wave-uniform)
    // full row sums: the four k-groups of lanes hold different keys
    const float lg = pair32_sum(pair16_sum(l[g]));
    const float lxg = pair32_sum(pair16_sum(lx[g]));
    const bool head_ok = H * (it.kvh + g) + n < a.hq;

    // O^T lane (n, c) element r is dim dim0 + 16 b + 4 c + r of head n
    if (PREFILL || it.slot < 0) {
      if ((PREFILL && !q_ok) || !head_ok) continue;
      const uint64_t hrow = head_row(g);
      const float inv = 1.f / lg;
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + hrow * R + (PREFILL ? dim0 : DW * wave);
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        uint2 w;
        w.x = Pair16<T>::pack(o[g][b][0] * inv, o[g][b][1] * inv);
        w.y = Pair16<T>::pack(o[g][b][2] * inv, o[g][b][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * b + 4 * c) = w;
      }
      if (a.lse && (PREFILL ? wave % kMlaWavesPerQuery : wave) == 0 && c == 0)
        a.lse[hrow] = m[g] * a.scale + logf(lxg);
    } else {
      const uint64_t srow = (uint64_t)(it.slot + g) * H + n;
      float* dst = a.ws_o + srow * R + DW * wave;
#pragma unroll
      for (int b = 0; b < DB; ++b) *reinterpret_cast<floatx4_t*>(dst + 16 * b + 4 * c) = o[g][b];
      if (wave == 0 && c == 0) {
        a.ws_ml[srow * 3 + 0] = m[g] * a.scale_log2;
        a.ws_ml[srow * 3 + 1] = lg;
        a.ws_ml[srow * 3 + 2] = lxg;
      }
    }
  }
}

}  // namespace pa
