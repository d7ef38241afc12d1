// Chunked-prefill body (bf16 MFMA): up to 128 query rows -- 128/G consecutive
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
// Data flow per 64-key tile:
//   HBM --(16-byte loads, page-gathered)--> registers --> LDS:
//     K  row-major   [64 keys][D]     (rows padded by 16 bytes)
//     V^T            [D][64 keys]     (keys permuted to the MFMA k order,
//                                      16-byte groups XOR-swizzled by dim)
//   each wave (32 rows):  S^T[64 x 32] = K . Q^T      (Q^T held in registers)
//                         O^T[D x 32] += V^T . P^T    (P^T straight from S^T)
// In the S^T / O^T accumulator layout every lane owns one query row, so the
// row max, the rescale and the row sum need at most one cross-lane step.
#pragma once

#include "pa_decode.h"
#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefillTileKeys = 64;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowsPerWave = 32;

template <int D>
struct PrefillSmem {
  static constexpr int kRow = D * 2 + 16;                   // bytes per K row
  static constexpr int kVRow = kPrefillTileKeys * 2 + 16;  // bytes per V^T row
  static constexpr int kBytes = kPrefillTileKeys * kRow + D * kVRow;
};

__device__ __forceinline__ floatx16_t mfma_32x32x16(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key t inside the V^T tile: swap bits 2 and 3 so that the eight
// keys one lane feeds to a P.V k-step are contiguous.
__device__ __forceinline__ int vt_col(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// Byte offset of 16-byte group `grp` (8 keys) of V^T row `d`.
__device__ __forceinline__ int vt_off(int d, int grp, int vrow) { return d * vrow + ((grp ^ ((d >> 3) & 7)) << 4); }

template <int D, int G>
__device__ __forceinline__ void prefill_item(const KernelArgs& a, const WorkItem& it, char* smem) {
  constexpr int NT = kPrefillTileKeys;
  constexpr int KS = D / 16;      // MFMA k-steps of S^T (over head dims)
  constexpr int DB = D / 32;      // 32-dim blocks of O^T
  constexpr int PIECES = D / 8;   // 16-byte pieces per key row
  constexpr int KROW = PrefillSmem<D>::kRow;
  constexpr int VROW = PrefillSmem<D>::kVRow;
  constexpr int NTHR = kPrefillWaves * kWave;
  constexpr int KCH = NT * PIECES / NTHR;        // K pieces per thread per tile
  constexpr int VCH = (NT / 2) * PIECES / NTHR;  // V key-pair pieces per thread per tile
  static_assert(KCH >= 1 && VCH >= 1 && (NT * PIECES) % NTHR == 0, "tile does not divide over the workgroup");
  static_assert(kPrefillWaves * kPrefillRowsPerWave % G == 0 || G > 128, "rows per tile must hold whole queries");

  char* ks = smem;
  char* vs = smem + NT * KROW;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const uint64_t row_stride = (uint64_t)a.hkv * D;
  const uint64_t head_off = (uint64_t)it.kvh * D;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(a.v);

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
  float m = -INFINITY, l = 0.f, lx = 0.f;  // lx: unrounded weights, for the logsumexp

  // global -> register staging of one tile
  uint4 kreg[KCH], vreg[VCH][2];
  auto slot_offset = [&](int t) -> uint64_t {
    const int tc = min(max(t, tb), te - 1);  // out-of-range keys read an in-range key, masked below
    const int page = bt[tc >> a.page_shift];
    return ((uint64_t)page * ps + (tc & (ps - 1))) * row_stride + head_off;
  };
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = i * NTHR + tid;
      const int key = c / PIECES, piece = c % PIECES;
      kreg[i] = *reinterpret_cast<const uint4*>(kpool + slot_offset(t0 + key) + piece * 8);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = i * NTHR + tid;
      const int pair = c / PIECES, piece = c % PIECES;
      vreg[i][0] = *reinterpret_cast<const uint4*>(vpool + slot_offset(t0 + 2 * pair) + piece * 8);
      vreg[i][1] = *reinterpret_cast<const uint4*>(vpool + slot_offset(t0 + 2 * pair + 1) + piece * 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = i * NTHR + tid;
      const int key = c / PIECES, piece = c % PIECES;
      *reinterpret_cast<uint4*>(ks + key * KROW + piece * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = i * NTHR + tid;
      const int pair = c / PIECES, piece = c % PIECES;
      const int col = vt_col(2 * pair);  // even; its odd partner lands next to it
      const uint32_t w0[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
      const uint32_t w1[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = piece * 8 + 2 * j;
        *reinterpret_cast<uint32_t*>(vs + vt_off(d0, col >> 3, VROW) + (col & 7) * 2) = interleave_lo(w0[j], w1[j]);
        *reinterpret_cast<uint32_t*>(vs + vt_off(d0 + 1, col >> 3, VROW) + (col & 7) * 2) =
            interleave_hi(w0[j], w1[j]);
      }
    }
  };

  const int t_first = tb & ~(NT - 1);
  if (t_first < te) load_tile(t_first);
  for (int t0 = t_first; t0 < te; t0 += NT) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t0 + NT < te) load_tile(t0 + NT);  // in flight while this tile is computed

    // tile entirely hidden from every row of this wave?
    const bool hidden = pmax < 0 || (a.causal && t0 > pmax) || (a.window > 0 && t0 + NT - 1 <= pmin - a.window);
    if (hidden) continue;
    const bool full = t0 >= tb && t0 + NT <= te && (!a.causal || t0 + NT - 1 <= pmin) &&
                      (a.window == 0 || t0 > pmax - a.window) && pmax >= 0;

    // S^T = K . Q^T : two 32-key blocks
    floatx16_t s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks + (mb * 32 + n) * KROW + 32 * k + 16 * h);
        s[mb] = mfma_32x32x16(kf, qf[k], s[mb]);
      }
    }

    // mask: accumulator element e of block mb holds key t0 + 32 mb + 8 (e/4) + 4 h + e%4
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

    // online softmax for this lane's row (both lane halves hold the same row)
    float mx = m;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    const float alpha = fast_exp2((m - mu) * a.scale_log2);
    m = mx;
    l *= alpha;
    lx *= alpha;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][e] *= alpha;

    // P^T operand for k-step kk: elements 8 (kk % 2) .. +7 of block kk / 2
#pragma unroll
    for (int kk = 0; kk < NT / 16; ++kk) {
      const int mb = kk >> 1, e0 = 8 * (kk & 1);
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2((s[mb][e0 + 2 * j] - mu) * a.scale_log2);
        const float p1 = fast_exp2((s[mb][e0 + 2 * j + 1] - mu) * a.scale_log2);
        pw[j] = pack_bf16(p0, p1);
        l += bf16_lo(pw[j]) + bf16_hi(pw[j]);
        lx += p0 + p1;
      }
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const int d = 32 * b + n;
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(vs + vt_off(d, 2 * kk + h, VROW));
        o[b] = mfma_32x32x16(vf, pf, o[b]);
      }
    }
  }

  l += __shfl_xor(l, 32);
  lx += __shfl_xor(lx, 32);
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
  if (a.lse && h == 0) a.lse[(uint64_t)qi * a.hq + head] = m * a.scale + logf(lx);
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
