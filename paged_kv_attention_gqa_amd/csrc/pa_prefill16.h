// Chunked-prefill body on 16x16x32 MFMA for head sizes the prefill_item tile
// does not take (D = Dv = 256, and pairs of multiples of 64 other than
// 192 / 128, in bf16 / f16): the
// rows and keys of a prefill tile as in
// prefill_item (up to 256 query rows -- 256 / G consecutive queries of one
// sequence times the G heads of one KV head -- against the keys the plan
// assigns to the tile), computed with the operand scheme of the backward's
// MFMA kernels.
//
// Definition followed: boostr 0.2.0-beta.2 `standard_attention_fwd` with the
// mask of `build_attention_mask` on absolute positions (ruDNN 0.1.107
// `DevicePlan::attention`, V rows of their own width Dv).
//
// Eight waves of 32 rows (two 16-row blocks); Q^T of a wave's rows stays in
// registers while K and V stream through LDS 32 keys at a time (one tile
// ahead in registers).  Per tile and block:
//   S^T = K Q^T                       (keys x rows: lane (n, g) holds row n,
//                                      keys 4 g .. 4 g + 3 of each 16-key half)
//   P^T = 2^(S^T c - m) with an online max per row (lanes of one column)
//   O  += P V                         (rows x dims: P straight from the S^T
//                                      accumulators, the two halves'
//                                      keys interleaved in the k order; V
//                                      columns by transposed LDS reads in
//                                      that order)
// O's accumulator holds rows 4 g + e in lane (dim, g): its per-row rescale
// and normalisation take the row's value from lane 4 g + e.  Value rows wider
// than 128 run in passes of 128 output dims over the whole key range (the
// scores are recomputed per pass), so that the output sums fit the registers.
#pragma once

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_mla.h"
#include "pa_prefill.h"

namespace pa {

constexpr int kPrefill16Keys = 32;  // keys per LDS tile

// Byte offset of 16-byte piece `piece` of row `row` in a tile of WIDTH
// elements per row: the low three piece bits are XORed with three low row
// bits, so the offset stays inside the row for any number of pieces.
template <int WIDTH>
__device__ __forceinline__ int tile16_off(int row, int piece) {
  return row * (WIDTH * 2) + ((piece ^ (((row & 3) << 1) | ((row >> 2) & 1))) << 4);
}

template <int D, int DV>
struct Prefill16Smem {
  static constexpr int kPasses = DV > 128 ? DV / 128 : 1;
  static constexpr int kPassDims = DV / kPasses;  // output dims per pass
  static constexpr int kK = kPrefill16Keys * D * 2;
  static constexpr int kV = kPrefill16Keys * kPassDims * 2;
  static constexpr int kBytes = kK + kV;
};

template <typename T, int D, int DV, int G>
__device__ __forceinline__ void prefill16_item(const KernelArgs& a, const WorkItem& it, char* smem) {
  constexpr int NT = kPrefill16Keys;
  constexpr int PASSES = Prefill16Smem<D, DV>::kPasses, DVP = Prefill16Smem<D, DV>::kPassDims;
  constexpr int KS = D / 32, VB = DVP / 16;     // k-steps of S^T; 16-dim blocks of O per pass
  constexpr int PK = D / 8, PV = DVP / 8;       // 16-byte pieces per K / V tile row
  constexpr int CHUNKS = NT * (PK + PV);        // 16-byte pieces per tile
  constexpr int THREADS = kPrefillWaves * kWave;
  constexpr int PER_THREAD = (CHUNKS + THREADS - 1) / THREADS;
  static_assert(D % 32 == 0 && DVP * PASSES == DV && PK % 8 == 0 && PV % 8 == 0, "unsupported head sizes");
  static_assert(kPrefillWaves * 32 == kPrefillRows, "eight waves of 32 rows");
  char* ks = smem;
  char* vs = smem + Prefill16Smem<D, DV>::kK;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g4 = lane >> 4;
  const int kvh = it.kvh;
  const int tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D, vrow = (uint64_t)a.hkv * DV;
  const int nrows = it.q_count * G;
  const float c2 = a.scale_log2;

  // this lane's two rows (MFMA column n of blocks 0 and 1): Q^T operands,
  // position and softmax state
  frag_t qb[2][KS];
  int pos[2];
  bool row_ok[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int rho = wave * 32 + blk * 16 + n;
    row_ok[blk] = rho < nrows;
    const int rg = row_ok[blk] ? rho : 0;
    const uint64_t row = (uint64_t)(it.q_begin + rg / G) * a.hq + (uint64_t)kvh * G + rg % G;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qb[blk][k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(a.q) + row * D + 32 * k + 8 * g4);
    pos[blk] = a.q_pos[it.q_begin + rg / G];
  }

  for (int pass = 0; pass < PASSES; ++pass) {
  const int vd0 = pass * DVP;  // first output dim of this pass
  float m[2], l[2];
  floatx4_t o[2][VB];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    m[blk] = -INFINITY;
    l[blk] = 0.f;
#pragma unroll
    for (int b = 0; b < VB; ++b) o[blk][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // tile loads: piece c < NT PK of K (key c / PK, piece c % PK), then of V
  u32x4_t pre[PER_THREAD];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_k = c < NT * PK;
        const int cc = is_k ? c : c - NT * PK;
        const int key = is_k ? cc / PK : cc / PV, piece = is_k ? cc % PK : cc % PV;
        const int t = min(t0 + key, te - 1);
        const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
        const uint16_t* src = is_k ? reinterpret_cast<const uint16_t*>(a.k) + slot * krow + (uint64_t)kvh * D
                                   : reinterpret_cast<const uint16_t*>(a.v) + slot * vrow + (uint64_t)kvh * DV + vd0;
        pre[j] = *reinterpret_cast<const u32x4_t*>(src + piece * 8);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_k = c < NT * PK;
        const int cc = is_k ? c : c - NT * PK;
        char* dst = is_k ? ks + tile16_off<D>(cc / PK, cc % PK) : vs + tile16_off<DVP>(cc / PV, cc % PV);
        *reinterpret_cast<u32x4_t*>(dst) = pre[j];
      }
    }
  };
  // transposed reads of V: 16-lane group g4, lane 4 r + j -> key 4 g4 + r
  // (+16 for the second read), dims 16 b + 4 j
  uint32_t troff[VB][2];
#pragma unroll
  for (int b = 0; b < VB; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = 4 * g4 + (n >> 2) + 16 * h, dim = 16 * b + 4 * (n & 3);
      troff[b][h] = (uint32_t)(tile16_off<DVP>(key, dim >> 3) + (dim & 7) * 2);
    }

  const int t_first = tb & ~(NT - 1);
  fetch(t_first);
  for (int t0 = t_first; t0 < te; t0 += NT) {
    __syncthreads();  // every wave is done with the previous tile
    store();
    __syncthreads();
    if (t0 + NT < te) fetch(t0 + NT);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      floatx4_t s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k)
          s[h] = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(ks + tile16_off<D>(16 * h + n, 4 * k + g4)),
                                  qb[blk][k], s[h]);
      }
      // mask: lane (n, g4) element e of half h is key t0 + 16 h + 4 g4 + e of row n
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = t0 + 16 * h + 4 * g4 + e;
          const bool vis = row_ok[blk] && t >= tb && t < te && (!a.causal || t <= pos[blk]) &&
                           (a.window == 0 || t > pos[blk] - a.window);
          s[h][e] = vis ? s[h][e] : -INFINITY;
          mx = fmaxf(mx, s[h][e]);
        }
      mx = pair32_max(pair16_max(mx));  // the row's max over the tile (four k-groups of lanes)
      if (__any(mx * c2 > m[blk] * c2 + kLazyRescaleLog2)) {
        const float mn = fmaxf(m[blk], mx);
        const float alpha = fast_exp2((m[blk] - (mn == -INFINITY ? 0.f : mn)) * c2);
        m[blk] = mn;
        l[blk] *= alpha;
        float al[4];  // alpha of O's rows 4 g4 + e
#pragma unroll
        for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g4 + e);
#pragma unroll
        for (int b = 0; b < VB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[blk][b][e] *= al[e];
      }
      const float sub = (m[blk] == -INFINITY ? 0.f : m[blk]) * c2;
      uint32_t pw[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = fast_exp2(__builtin_fmaf(s[h][e], c2, -sub));
          l[blk] += p[e];
        }
        pw[2 * h] = Pair16<T>::pack(p[0], p[1]);
        pw[2 * h + 1] = Pair16<T>::pack(p[2], p[3]);
      }
      const frag_t pf = __builtin_bit_cast(frag_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const short4_t v0 = lds_read_tr16(vs + troff[b][0]);
        const short4_t v1 = lds_read_tr16(vs + troff[b][1]);
        const frag_t vf = __builtin_bit_cast(
            frag_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))));
        o[blk][b] = mfma_16x16x32<T>(pf, vf, o[blk][b]);
      }
    }
  }

  // row sums over the four k-groups; O rows 4 g4 + e take theirs from lane 4 g4 + e
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float lt = pair32_sum(pair16_sum(l[blk]));
    const int rho_n = wave * 32 + blk * 16 + n;
    if (a.lse && pass == 0 && g4 == 0 && rho_n < nrows) {
      const uint64_t row = (uint64_t)(it.q_begin + rho_n / G) * a.hq + (uint64_t)kvh * G + rho_n % G;
      a.lse[row] = m[blk] * a.scale + logf(lt);
    }
    const float inv = 1.f / lt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ie = __shfl(inv, 4 * g4 + e);
      const int rho = wave * 32 + blk * 16 + 4 * g4 + e;
      if (rho >= nrows) continue;
      const uint64_t row = (uint64_t)(it.q_begin + rho / G) * a.hq + (uint64_t)kvh * G + rho % G;
#pragma unroll
      for (int b = 0; b < VB; ++b) store_out<T>(a.out, row * DV + vd0 + 16 * b + n, o[blk][b][e] * ie);
    }
  }
  }
}

}  // namespace pa
