// Absorbed-MLA decode body (bf16 MFMA): one query, all H = 16 heads, one
// contiguous range of its visible keys.
//
// Definition followed: ruDNN 0.1.107 paged_attention/mod.rs `DevicePlan::mla`
// -- one shared latent head [pages, page_size, 1, R] serves as key and value,
// a rotated position cache [pages, page_size, 1, P] adds q_rope . kpos to
// every score, scale from the model's original query/key size -- with the
// softmax and masking of boostr 0.2.0-beta.2 `standard_attention_fwd` /
// `build_attention_mask`.
//
// Per key the method reads R + P = 576 bf16 (1152 bytes) and does 16 x (576 +
// 512) multiply-adds: ~30 flops per byte, above what the fp32 vector units
// sustain at HBM speed, so both products run on MFMA with the 16 heads as the
// N dimension:
//   S^T[16 keys x 16 heads] = latent . q_abs^T + kpos . q_rope^T   (16x16x32)
//   O^T[R x 16 heads]      += latent^T . P^T                      (16x16x16)
// Each wave streams its own 16-key tiles (wave w takes tiles w, w+4, ...)
// into a private two-stage LDS ring with global_load_lds_dwordx4 (16-byte
// pieces of key row t stored at piece ^ (t & 7)); latent^T fragments come from
// ds_read_b64_tr_b16.  Every lane owns one head's column, so softmax needs two
// cross-lane steps per tile.  The four waves merge through LDS at the end.
#pragma once

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_prefill.h"

namespace pa {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kMlaHeads = 16;
constexpr int kMlaRank = 512;
constexpr int kMlaRope = 64;
constexpr int kMlaTileKeys = 16;
constexpr int kMlaWaves = 4;

struct MlaSmem {
  static constexpr int kLatTile = kMlaTileKeys * kMlaRank * 2;   // 16 KB
  static constexpr int kPosTile = kMlaTileKeys * kMlaRope * 2;   // 2 KB
  static constexpr int kStage = kLatTile + kPosTile;
  static constexpr int kWaveRing = 2 * kStage;
  static constexpr int kRing = kMlaWaves * kWaveRing;           // 144 KB
  // end-of-item combine: O [wave][head][R] f32 + (m, l, lx) [wave][head]
  static constexpr int kCombine = kMlaWaves * kMlaHeads * (kMlaRank + 3) * 4;
  static constexpr int kBytes = kRing > kCombine ? kRing : kCombine;
};

__device__ __forceinline__ floatx4_t mfma_16x16x32(const bf16x8_t& a, const bf16x8_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma_16x16x16(const short4_t& a, const short4_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Byte offset of 16-byte piece `piece` of key row `key` in a tile of `width`
// bf16 per row.
template <int WIDTH>
__device__ __forceinline__ int mla_off(int key, int piece) {
  return key * (WIDTH * 2) + ((piece ^ (key & 7)) << 4);
}

template <typename T>
__device__ __forceinline__ void mla_item(const KernelArgs& a, const WorkItem& it, char* smem) {
  constexpr int H = kMlaHeads, R = kMlaRank, P = kMlaRope, NT = kMlaTileKeys;
  constexpr int KS_LAT = R / 32, KS_POS = P / 32;  // 16x16x32 k-steps
  constexpr int DB = R / 16;                        // 16-dim blocks of O^T
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, c = lane >> 4;           // MFMA column (head / key row) and k-group
  const int qi = it.q_begin;
  const int tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint16_t* lat = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* kpos = reinterpret_cast<const uint16_t*>(a.kr);

  // q^T operands: lane (n, c) holds dims 32 ks + 8 c .. +7 of head n
  bf16x8_t qa[KS_LAT], qp[KS_POS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((uint64_t)qi * H + n) * R;
    const uint16_t* prow = reinterpret_cast<const uint16_t*>(a.qr) + ((uint64_t)qi * H + n) * P;
#pragma unroll
    for (int k = 0; k < KS_LAT; ++k) qa[k] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * k + 8 * c);
#pragma unroll
    for (int k = 0; k < KS_POS; ++k) qp[k] = *reinterpret_cast<const bf16x8_t*>(prow + 32 * k + 8 * c);
  }

  floatx4_t o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f, lx = 0.f;

  char* ring = smem + wave * MlaSmem::kWaveRing;
  auto clamp_key = [&](int t) { return min(max(t, tb), te - 1); };
  // One tile: 16 latent rows (one 1 KB load each; the row's page number is
  // wave-uniform) and 16 rotary rows (two loads of 8 rows x 128 bytes).
  auto issue_tile = [&](int t0, char* stage) {
#pragma unroll
    for (int r = 0; r < NT; ++r) {  // latent row r: lane loads piece lane ^ (r & 7)
      const int t = clamp_key(t0 + r);
      const int page = bt[t >> a.page_shift];
      const uint16_t* src = lat + ((uint64_t)page * ps + (t & (ps - 1))) * R + ((lane ^ (r & 7)) * 8);
      load_to_lds(src, stage + r * (R * 2));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // rotary rows 8 i .. 8 i + 7: lane covers row 8 i + lane / 8
      const int r = 8 * i + (lane >> 3);
      const int t = clamp_key(t0 + r);
      const int page = bt[t >> a.page_shift];
      const uint16_t* src = kpos + ((uint64_t)page * ps + (t & (ps - 1))) * P + (((lane & 7) ^ (r & 7)) * 8);
      load_to_lds(src, stage + MlaSmem::kLatTile + i * 1024);
    }
  };

  const int first = tb + wave * NT;
  int stage = 0;
  if (first < te) issue_tile(first, ring);
  for (int t0 = first; t0 < te; t0 += kMlaWaves * NT, stage ^= 1) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's tile has landed (the ring is private to the wave)
    if (t0 + kMlaWaves * NT < te) issue_tile(t0 + kMlaWaves * NT, ring + (stage ^ 1) * MlaSmem::kStage);
    const char* ls = ring + stage * MlaSmem::kStage;
    const char* kps = ls + MlaSmem::kLatTile;

    // S^T: lane (n, c) holds keys 4 c + r (r = 0..3) of head n
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS_LAT; ++k) {
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ls + mla_off<R>(n, 4 * k + c));
      s = mfma_16x16x32(kf, qa[k], s);
    }
#pragma unroll
    for (int k = 0; k < KS_POS; ++k) {
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kps + mla_off<P>(n, 4 * k + c));
      s = mfma_16x16x32(kf, qp[k], s);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * c + r;
      s[r] = (t >= tb && t < te) ? s[r] : -INFINITY;
    }

    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx = fmaxf(mx, m);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    const float alpha = fast_exp2((m - mu) * a.scale_log2);
    m = mx;
    l *= alpha;
    lx *= alpha;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2((s[r] - mu) * a.scale_log2);
    const uint32_t w0 = pack_bf16(p[0], p[1]), w1 = pack_bf16(p[2], p[3]);
    l += bf16_lo(w0) + bf16_hi(w0) + bf16_lo(w1) + bf16_hi(w1);
    lx += (p[0] + p[1]) + (p[2] + p[3]);
    const short4_t pf = __builtin_bit_cast(short4_t, make_uint2(w0, w1));

    // O^T block b: lane (i = lane % 16, c) needs latent[4 c + r][16 b + i]:
    // one transposed read, lane 4 r + j giving the address of dims 16 b + 4 j
    // of key row 4 c + r.
    const int rr = n >> 2, jj = n & 3;
    const int key = 4 * c + rr;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int dim = 16 * b + 4 * jj;
      const short4_t vf = lds_read_tr16(ls + mla_off<R>(key, dim >> 3) + (dim & 7) * 2);
      o[b] = mfma_16x16x16(vf, pf, o[b]);
    }
  }

  // full row sums of this wave: the four k-groups hold different keys
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  lx += __shfl_xor(lx, 16);
  lx += __shfl_xor(lx, 32);

  // combine the waves: O^T lane (n, c) element r is dim 16 b + 4 c + r of head n
  __syncthreads();  // every wave is done with its ring; reuse it for the combine
  float* so = reinterpret_cast<float*>(smem);                   // [wave][head][R]
  float* sml = so + kMlaWaves * H * R;                          // [wave][head][3]
#pragma unroll
  for (int b = 0; b < DB; ++b)
    *reinterpret_cast<floatx4_t*>(so + ((size_t)wave * H + n) * R + 16 * b + 4 * c) = o[b];
  if (c == 0) {
    sml[(wave * H + n) * 3 + 0] = m;
    sml[(wave * H + n) * 3 + 1] = l;
    sml[(wave * H + n) * 3 + 2] = lx;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < H * R; idx += kMlaWaves * kWave) {
    const int hd = idx / R, d = idx % R;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) M = fmaxf(M, sml[(w * H + hd) * 3]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, LX = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) {
      const float f = fast_exp2((sml[(w * H + hd) * 3] - mu) * a.scale_log2);
      L += sml[(w * H + hd) * 3 + 1] * f;
      LX += sml[(w * H + hd) * 3 + 2] * f;
      O += so[((size_t)w * H + hd) * R + d] * f;
    }
    if (it.slot < 0) {
      store_out<T>(a.out, ((uint64_t)qi * H + hd) * R + d, O / L);
      if (a.lse && d == 0) a.lse[(uint64_t)qi * H + hd] = M * a.scale + logf(LX);
    } else {
      a.ws_o[((uint64_t)it.slot * H + hd) * R + d] = O;
      if (d == 0) {
        a.ws_ml[((uint64_t)it.slot * H + hd) * 3 + 0] = M * a.scale_log2;
        a.ws_ml[((uint64_t)it.slot * H + hd) * 3 + 1] = L;
        a.ws_ml[((uint64_t)it.slot * H + hd) * 3 + 2] = LX;
      }
    }
  }
}

}  // namespace pa
