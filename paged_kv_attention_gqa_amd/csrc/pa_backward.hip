// Paged GQA/MHA backward (VALU): gradients of the forward pass with respect
// to the queries and to the K/V pools.
//
// Definition followed: ruDNN 0.1.107 paged_attention/mod.rs
// `attention_backward` (first-order gradients, scores recomputed from Q and K
// in a second scan of the history) with the formulas of boostr 0.2.0-beta.2
// attention/flash_standard.rs `standard_attention_bwd`: with P the softmax
// weights of a row (recomputed from the forward's logsumexp) and dO its
// output gradient,
//   D = dO . O,   dP_t = dO . V_t,   dS_t = P_t (dP_t - D),
//   dQ = scale sum_t dS_t K_t,   dK_t = scale sum_rows dS_t Q,   dV_t = sum_rows P_t dO,
// the GQA map summing the rows of the G query heads that share a KV head.
//
// Four launches: zero the K/V gradient pools, D per row, dQ (one workgroup
// per (query, KV head), keys strided over lanes as in the decode body), and
// dK/dV (one workgroup per 128-key block and KV head, looping over the
// sequence's query rows): on 16-bit MFMA for bf16 / f16, on the vector units
// for f32.  Each pool row has a single writer, so the result
// does not depend on scheduling (ruDNN's ordered, atomic-free variant).
#include <algorithm>

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_launch.h"
#include "pa_mla.h"

namespace pa {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBwdDqWaves = 4;
constexpr int kBwdKvWaves = 8;

struct BwdArgs {
  KernelArgs a;        // q, k, v, out, lse, block table, positions, lengths, geometry, scale
  const void* dout;    // [Q, Hq, Dv]
  void* dq;            // [Q, Hq, D]
  void* dk;            // pool shaped [pages, ps, Hkv, D]
  void* dv;            // pool shaped [pages, ps, Hkv, Dv]
  float* delta;        // [Q, Hq]: D = dO . O
  const BwdItem* items;
  float* acc_k;        // null: dK rows are stored (one writer each); else f32 sums shaped like dk
  float* acc_v;        // likewise for dV
};

// One dK or dV element of a pool row: stored when every pool row has a
// single writer, added to the f32 sums when pages are shared (several
// sequences, or several positions of one, contribute to the row).
template <typename T>
__device__ __forceinline__ void put_grad(void* pool, float* acc, uint64_t idx, float v) {
  if (acc)
    unsafeAtomicAdd(acc + idx, v);
  else
    store_out<T>(pool, idx, v);
}

// Element e of a lane's chunk as float.
template <typename T, int N>
__device__ __forceinline__ float chunk_elem(const Words<N>& w, int e) {
  if constexpr (sizeof(T) == 2)
    return (e & 1) ? Pair16<T>::hi(w.w[e >> 1]) : Pair16<T>::lo(w.w[e >> 1]);
  else
    return __uint_as_float(w.w[e]);
}

template <typename T>
__device__ __forceinline__ float load_elem(const void* base, uint64_t idx) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t b = reinterpret_cast<const uint16_t*>(base)[idx];
    return Pair16<T>::lo(b);
  } else {
    return reinterpret_cast<const float*>(base)[idx];
  }
}

// Zero n 16-byte chunks (grid-stride).
__global__ __launch_bounds__(256) void bwd_zero_kernel(u32x4_t* p, int64_t n) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// The f32 sums of shared-page gradients rounded into the 16-bit pool, four
// elements per thread (grid-stride).
template <typename T>
__global__ __launch_bounds__(256) void bwd_cast_kernel(const float4* src, uint2* dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 x = src[i];
    dst[i] = uint2{Pair16<T>::pack(x.x, x.y), Pair16<T>::pack(x.z, x.w)};
  }
}

// D = dO . O per (query, head) row: one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs b, int64_t rows, int dv) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int c = lane; c < dv; c += kWave)
    acc = fmaf(load_elem<T>(b.dout, row * dv + c), load_elem<T>(b.a.out, row * dv + c), acc);
  acc = group_sum<kWave>(acc);
  if (lane == 0) b.delta[row] = acc;
}

// dQ of one (query, KV head) item for its G query heads.
template <typename T, int D, int DV, int G>
__global__ __launch_bounds__(kBwdDqWaves* kWave) void bwd_dq_kernel(BwdArgs b) {
  using Lay = DecodeLayout<T, D, DV>;
  constexpr int LPT = Lay::kLanes, KW = Lay::kKWords, VW = Lay::kVWords, EK = Lay::kKElems, EV = Lay::kVElems;
  constexpr int TPW = kWave / LPT, NW = kBwdDqWaves, SZ = (int)sizeof(T);
  __shared__ float smem[NW * G * D];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[blockIdx.x];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane / LPT, c = lane % LPT;
  const int qi = it.q_begin, kvh = it.kvh;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D, vrow = (uint64_t)a.hkv * DV;

  Words<KW> qv[G];
  Words<VW> gv[G];
  float l2[G], dl[G], acc[G][EK];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t row = (uint64_t)qi * a.hq + (uint64_t)kvh * G + g;
    qv[g] = load_words<KW, false>(reinterpret_cast<const char*>(a.q) + (row * D + c * EK) * SZ);
    gv[g] = load_words<VW, false>(reinterpret_cast<const char*>(b.dout) + (row * DV + c * EV) * SZ);
    l2[g] = a.lse[row] * kLog2e;
    dl[g] = b.delta[row];
#pragma unroll
    for (int e = 0; e < EK; ++e) acc[g][e] = 0.f;
  }

  for (int t0 = it.tok_begin + wave * TPW; t0 < it.tok_end; t0 += NW * TPW) {
    const int t = t0 + r;
    const bool valid = t < it.tok_end;
    const int tc = valid ? t : it.tok_end - 1;
    const uint64_t slot = (uint64_t)bt[tc >> a.page_shift] * ps + (tc & (ps - 1));
    const Words<KW> kw =
        load_words<KW, false>(reinterpret_cast<const char*>(a.k) + ((slot * krow) + (uint64_t)kvh * D + c * EK) * SZ);
    const Words<VW> vw =
        load_words<VW, false>(reinterpret_cast<const char*>(a.v) + ((slot * vrow) + (uint64_t)kvh * DV + c * EV) * SZ);
    float s[G], dp[G];
    chunk_scores<T, G, KW>(qv, kw, s);
    chunk_scores<T, G, VW>(gv, vw, dp);
    group_sum_all<LPT, G>(s);
    group_sum_all<LPT, G>(dp);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = fast_exp2(__builtin_fmaf(s[g], a.scale_log2, -l2[g]));
      const float ds = valid ? p * (dp[g] - dl[g]) : 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) acc[g][e] = fmaf(ds, chunk_elem<T, KW>(kw, e), acc[g][e]);
    }
  }

  // rows of the wave (lanes c, c + LPT, ...), then the waves through LDS
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EK; ++e) acc[g][e] = column_sum<LPT>(acc[g][e]);
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EK; ++e) smem[(wave * G + g) * D + c * EK + e] = acc[g][e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int g = idx / D, d = idx % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += smem[(w * G + g) * D + d];
    store_out<T>(b.dq, ((uint64_t)qi * a.hq + (uint64_t)kvh * G + g) * D + d, sum * a.scale);
  }
}

// dK and dV of one block of up to kBwdBlockKeys keys and one KV head, in
// sub-blocks of 64 keys.  Lane (r, c) of wave w holds chunk c of keys
// sub + (u NW + w) TPW + r, u < U, and their gradient sums; the sequence's
// query rows stream past.
constexpr int kBwdSubKeys = 64;
template <typename T, int D, int DV, int G>
__global__ __launch_bounds__(kBwdKvWaves* kWave) void bwd_dkv_kernel(BwdArgs b, int first_item) {
  using Lay = DecodeLayout<T, D, DV>;
  constexpr int LPT = Lay::kLanes, KW = Lay::kKWords, VW = Lay::kVWords, EK = Lay::kKElems, EV = Lay::kVElems;
  constexpr int TPW = kWave / LPT, NW = kBwdKvWaves, SZ = (int)sizeof(T);
  constexpr int U = kBwdSubKeys / (NW * TPW);
  static_assert(U >= 1 && U * NW * TPW == kBwdSubKeys && kBwdBlockKeys % kBwdSubKeys == 0,
                "a sub-block must split evenly over the lanes");
  const KernelArgs& a = b.a;
  const BwdItem item = b.items[first_item + blockIdx.x];
  for (int sub = item.tok_begin; sub < item.tok_end; sub += kBwdSubKeys) {
  BwdItem it = item;
  it.tok_begin = sub;
  it.tok_end = min(item.tok_end, sub + kBwdSubKeys);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane / LPT, c = lane % LPT;
  const int kvh = it.kvh;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D, vrow = (uint64_t)a.hkv * DV;
  const int L = a.seq_lens[it.seq];

  int key[U];
  bool valid[U];
  uint64_t slot[U];
  Words<KW> kw[U];
  Words<VW> vw[U];
  float dk[U][EK], dv[U][EV];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    key[u] = it.tok_begin + (u * NW + wave) * TPW + r;
    valid[u] = key[u] < it.tok_end;
    const int tc = valid[u] ? key[u] : it.tok_end - 1;
    slot[u] = (uint64_t)bt[tc >> a.page_shift] * ps + (tc & (ps - 1));
    kw[u] = load_words<KW, false>(reinterpret_cast<const char*>(a.k) + ((slot[u] * krow) + (uint64_t)kvh * D + c * EK) * SZ);
    vw[u] = load_words<VW, false>(reinterpret_cast<const char*>(a.v) + ((slot[u] * vrow) + (uint64_t)kvh * DV + c * EV) * SZ);
#pragma unroll
    for (int e = 0; e < EK; ++e) dk[u][e] = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) dv[u][e] = 0.f;
  }

  for (int i = it.q_begin; i < it.q_end; ++i) {
    const int pos = a.q_pos[i];
    const int hi = a.causal ? pos : L - 1;
    const int lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;
    if (hi < it.tok_begin || lo >= it.tok_end) continue;  // the row sees no key of the block
    for (int g = 0; g < G; ++g) {
      const uint64_t row = (uint64_t)i * a.hq + (uint64_t)kvh * G + g;
      Words<KW> qw[1];
      Words<VW> gw[1];
      qw[0] = load_words<KW, false>(reinterpret_cast<const char*>(a.q) + (row * D + c * EK) * SZ);
      gw[0] = load_words<VW, false>(reinterpret_cast<const char*>(b.dout) + (row * DV + c * EV) * SZ);
      const float l2 = a.lse[row] * kLog2e, dl = b.delta[row];
      float s[U], dp[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float t1[1], t2[1];
        chunk_scores<T, 1, KW>(qw, kw[u], t1);
        chunk_scores<T, 1, VW>(gw, vw[u], t2);
        s[u] = t1[0];
        dp[u] = t2[0];
      }
      group_sum_all<LPT, U>(s);
      group_sum_all<LPT, U>(dp);
      float qf[EK], gf[EV];
#pragma unroll
      for (int e = 0; e < EK; ++e) qf[e] = chunk_elem<T, KW>(qw[0], e);
#pragma unroll
      for (int e = 0; e < EV; ++e) gf[e] = chunk_elem<T, VW>(gw[0], e);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool vis = valid[u] && key[u] >= lo && key[u] <= hi;
        const float p = vis ? fast_exp2(__builtin_fmaf(s[u], a.scale_log2, -l2)) : 0.f;
        const float ds = p * (dp[u] - dl) * a.scale;
#pragma unroll
        for (int e = 0; e < EV; ++e) dv[u][e] = fmaf(p, gf[e], dv[u][e]);
#pragma unroll
        for (int e = 0; e < EK; ++e) dk[u][e] = fmaf(ds, qf[e], dk[u][e]);
      }
    }
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!valid[u]) continue;
#pragma unroll
    for (int e = 0; e < EK; ++e) put_grad<T>(b.dk, b.acc_k, slot[u] * krow + (uint64_t)kvh * D + c * EK + e, dk[u][e]);
#pragma unroll
    for (int e = 0; e < EV; ++e) put_grad<T>(b.dv, b.acc_v, slot[u] * vrow + (uint64_t)kvh * DV + c * EV + e, dv[u][e]);
  }
  }
}

// dK and dV of one block of kBwdBlockKeys keys and one KV head on 16-bit
// MFMA (v_mfma_f32_16x16x32): eight waves of 16 keys; the sequence's query
// rows (query, head of the group) stream through LDS in tiles of 32 rows.
// Per tile and wave, with the 16x16 accumulator layout (lane (n, g) holds
// column n, rows 4 g .. 4 g + 3):
//   S  = Q K^T,  dP = dO V^T          (rows x keys; K^T and V^T of the wave's
//                                      keys stay in registers)
//   P  = 2^(S c - lse2) masked,  dS = P (dP - D) scale
//   dV += P^T dO,  dK += dS^T Q       (keys x dims; P^T / dS^T straight from
//                                      the S / dP accumulators, with the
//                                      row order of the two 16-row halves
//                                      interleaved; dO and Q columns by
//                                      transposed LDS reads in that order)
constexpr int kBwdMfmaWaves = 8;
constexpr int kBwdRowTile = 32;

// Tile layout of the backward's LDS tiles: rows of WIDTH elements in 16-byte
// pieces, stored at piece ^ (three low row bits), which stays inside the row
// for any multiple of 8 pieces (D = 192 has 24).
template <int WIDTH>
__device__ __forceinline__ int bwd_off(int row, int piece) {
  return row * (WIDTH * 2) + ((piece ^ (((row & 3) << 1) | ((row >> 2) & 1))) << 4);
}

// Eight 16-bit elements of column dims 16 blk + (lane % 16) from the rows
// 4 g + 0..3 and 16 + 4 g + 0..3 of a tile (g = lane / 16): two transposed
// reads, the order in which the 16x16 accumulators hold their rows.
template <int WIDTH>
__device__ __forceinline__ uint32_t bwd_troff(int blk, int h, int n, int g4) {
  const int row = 4 * g4 + (n >> 2) + 16 * h, dim = 16 * blk + 4 * (n & 3);
  return (uint32_t)(bwd_off<WIDTH>(row, dim >> 3) + (dim & 7) * 2);
}
__device__ __forceinline__ frag_t bwd_tfrag(const char* t, uint32_t off0, uint32_t off1) {
  const short4_t v0 = lds_read_tr16(t + off0);
  const short4_t v1 = lds_read_tr16(t + off1);
  return __builtin_bit_cast(frag_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))));
}

template <typename T, int D, int DV>
__global__ __launch_bounds__(kBwdMfmaWaves* kWave) void bwd_dkv_mfma_kernel(BwdArgs b, int first_item, int G) {
  constexpr int KSK = D / 32, KSV = DV / 32;  // 16x16x32 k-steps over the K / V dims
  constexpr int DBK = D / 16, DBV = DV / 16;  // 16-dim blocks of dK / dV
  constexpr int PK = D / 8, PV = DV / 8;      // 16-byte pieces per Q / dO row
  constexpr int CHUNKS = kBwdRowTile * (PK + PV);
  constexpr int THREADS = kBwdMfmaWaves * kWave;
  constexpr int PER_THREAD = (CHUNKS + THREADS - 1) / THREADS;
  static_assert(kBwdMfmaWaves * 16 == kBwdBlockKeys, "eight waves of 16 keys");
  static_assert(D % 64 == 0 && DV % 64 == 0, "rows of whole 8-piece groups");
  __shared__ __attribute__((aligned(16))) char qs[kBwdRowTile * D * 2];
  __shared__ __attribute__((aligned(16))) char gs[kBwdRowTile * DV * 2];
  __shared__ float lse2s[kBwdRowTile], dls[kBwdRowTile];
  __shared__ int poss[kBwdRowTile];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g4 = lane >> 4;  // MFMA column and k-group
  const int kvh = it.kvh;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D, vrow = (uint64_t)a.hkv * DV;
  const int nrows = (it.q_end - it.q_begin) * G;
  const float c2 = a.scale_log2;

  // K^T and V^T operands of this wave's 16 keys (key column n, dims 32 k + 8 g4 ..)
  const int my_key = it.tok_begin + wave * 16 + n;
  const bool key_ok = my_key < it.tok_end;
  frag_t kb[KSK], vb[KSV];
  {
    const int tc = key_ok ? my_key : it.tok_end - 1;
    const uint64_t slot = (uint64_t)bt[tc >> a.page_shift] * ps + (tc & (ps - 1));
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(a.k) + slot * krow + (uint64_t)kvh * D;
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(a.v) + slot * vrow + (uint64_t)kvh * DV;
#pragma unroll
    for (int k = 0; k < KSK; ++k) kb[k] = *reinterpret_cast<const frag_t*>(kr + 32 * k + 8 * g4);
#pragma unroll
    for (int k = 0; k < KSV; ++k) vb[k] = *reinterpret_cast<const frag_t*>(vr + 32 * k + 8 * g4);
  }
  floatx4_t dk[DBK], dv[DBV];
#pragma unroll
  for (int i = 0; i < DBK; ++i) dk[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < DBV; ++i) dv[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // keys of this lane's dK / dV accumulator rows: 4 g4 + e, e < 4
  const int key_lo = it.tok_begin + wave * 16;

  // Tile loads: piece c < 32 PK of Q (row c / PK), then of dO (rows past the
  // item's last are row 0 again, masked through lse2 = +inf); threads below
  // 32 the row statistics.
  auto row_addr = [&](int rho) -> uint64_t {  // (query, head) row of tile row rho
    const int rg = rho < nrows ? rho : 0;
    return ((uint64_t)(it.q_begin + rg / G) * a.hq + (uint64_t)kvh * G + rg % G);
  };
  u32x4_t pre[PER_THREAD];
  float pl = 0.f, pd = 0.f;
  int pp = 0;
  auto fetch = [&](int r0) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_q = c < kBwdRowTile * PK;
        const int cc = is_q ? c : c - kBwdRowTile * PK;
        const int r = is_q ? cc / PK : cc / PV, piece = is_q ? cc % PK : cc % PV;
        const uint64_t row = row_addr(r0 + r);
        pre[j] = is_q ? *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.q) + row * D + piece * 8)
                      : *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(b.dout) + row * DV +
                                                          piece * 8);
      }
    }
    if (tid < kBwdRowTile) {
      const int rho = r0 + tid;
      const uint64_t row = row_addr(rho);
      const bool ok = rho < nrows;
      pl = ok ? a.lse[row] * kLog2e : INFINITY;
      pd = ok ? b.delta[row] : 0.f;
      pp = a.q_pos[it.q_begin + (ok ? rho : 0) / G];
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_q = c < kBwdRowTile * PK;
        const int cc = is_q ? c : c - kBwdRowTile * PK;
        char* dst = is_q ? qs + bwd_off<D>(cc / PK, cc % PK) : gs + bwd_off<DV>(cc / PV, cc % PV);
        *reinterpret_cast<u32x4_t*>(dst) = pre[j];
      }
    }
    if (tid < kBwdRowTile) {
      lse2s[tid] = pl;
      dls[tid] = pd;
      poss[tid] = pp;
    }
  };

  if (nrows > 0) fetch(0);
  for (int r0 = 0; r0 < nrows; r0 += kBwdRowTile) {
    __syncthreads();  // every wave is done with the previous tile
    store();
    __syncthreads();
    if (r0 + kBwdRowTile < nrows) fetch(r0 + kBwdRowTile);

    // S and dP of the two 16-row halves
    floatx4_t s[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      dp[h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSK; ++k)
        s[h] = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(qs + bwd_off<D>(16 * h + n, 4 * k + g4)), kb[k], s[h]);
#pragma unroll
      for (int k = 0; k < KSV; ++k)
        dp[h] = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(gs + bwd_off<DV>(16 * h + n, 4 * k + g4)), vb[k],
                                 dp[h]);
    }
    // P and dS; lane (n, g4) element e of half h is row 16 h + 4 g4 + e, key n
    uint32_t pw[4], dw[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const floatx4_t l4 = *reinterpret_cast<const floatx4_t*>(lse2s + 16 * h + 4 * g4);
      const floatx4_t d4 = *reinterpret_cast<const floatx4_t*>(dls + 16 * h + 4 * g4);
      float p[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = poss[16 * h + 4 * g4 + e];
        const bool vis = key_ok && (!a.causal || my_key <= pos) && (a.window == 0 || my_key > pos - a.window);
        p[e] = vis ? fast_exp2(__builtin_fmaf(s[h][e], c2, -l4[e])) : 0.f;
        ds[e] = p[e] * (dp[h][e] - d4[e]) * a.scale;
      }
      pw[2 * h] = Pair16<T>::pack(p[0], p[1]);
      pw[2 * h + 1] = Pair16<T>::pack(p[2], p[3]);
      dw[2 * h] = Pair16<T>::pack(ds[0], ds[1]);
      dw[2 * h + 1] = Pair16<T>::pack(ds[2], ds[3]);
    }
    const frag_t pf = __builtin_bit_cast(frag_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    const frag_t df = __builtin_bit_cast(frag_t, make_uint4(dw[0], dw[1], dw[2], dw[3]));
    // dV += P^T dO, dK += dS^T Q over the tile's 32 rows
#pragma unroll
    for (int blk = 0; blk < DBV; ++blk)
      dv[blk] = mfma_16x16x32<T>(pf, bwd_tfrag(gs, bwd_troff<DV>(blk, 0, n, g4), bwd_troff<DV>(blk, 1, n, g4)),
                                 dv[blk]);
#pragma unroll
    for (int blk = 0; blk < DBK; ++blk)
      dk[blk] = mfma_16x16x32<T>(df, bwd_tfrag(qs, bwd_troff<D>(blk, 0, n, g4), bwd_troff<D>(blk, 1, n, g4)),
                                 dk[blk]);
  }

  // lane (n, g4) of block blk holds dims 16 blk + n of keys key_lo + 4 g4 + e
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = key_lo + 4 * g4 + e;
    if (t >= it.tok_end) continue;
    const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
#pragma unroll
    for (int blk = 0; blk < DBK; ++blk)
      put_grad<T>(b.dk, b.acc_k, slot * krow + (uint64_t)kvh * D + 16 * blk + n, dk[blk][e]);
#pragma unroll
    for (int blk = 0; blk < DBV; ++blk)
      put_grad<T>(b.dv, b.acc_v, slot * vrow + (uint64_t)kvh * DV + 16 * blk + n, dv[blk][e]);
  }
}

// dQ of one tile of up to kBwdQRows query rows (queries q_begin .. q_end of
// one sequence times the G heads of one KV head) on 16-bit MFMA: eight waves
// of 16 rows; the keys the tile sees stream through LDS 32 at a time.  The
// mirror image of bwd_dkv_mfma_kernel: Q^T and dO^T of the wave's rows stay
// in registers,
//   S^T = K Q^T, dP^T = V dO^T          (keys x rows, per 16-key half)
//   P^T, dS^T as there (row statistics are per lane: lane column = row)
//   dQ += dS K                          (rows x dims; dS straight from the
//                                        dS^T accumulators, K columns by
//                                        transposed LDS reads)
constexpr int kBwdKeyTile = 32;
template <typename T, int D, int DV>
__global__ __launch_bounds__(kBwdMfmaWaves* kWave) void bwd_dq_mfma_kernel(BwdArgs b, int first_item, int G) {
  constexpr int KSK = D / 32, KSV = DV / 32, DBK = D / 16;
  constexpr int PK = D / 8, PV = DV / 8;
  constexpr int CHUNKS = kBwdKeyTile * (PK + PV);
  constexpr int THREADS = kBwdMfmaWaves * kWave;
  constexpr int PER_THREAD = (CHUNKS + THREADS - 1) / THREADS;
  static_assert(kBwdMfmaWaves * 16 == kBwdQRows, "eight waves of 16 rows");
  static_assert(D % 64 == 0 && DV % 64 == 0, "rows of whole 8-piece groups");
  __shared__ __attribute__((aligned(16))) char ks[kBwdKeyTile * D * 2];
  __shared__ __attribute__((aligned(16))) char vs[kBwdKeyTile * DV * 2];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g4 = lane >> 4;
  const int kvh = it.kvh;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D, vrow = (uint64_t)a.hkv * DV;
  const int nrows = (it.q_end - it.q_begin) * G;
  const float c2 = a.scale_log2;

  // this lane's row (MFMA column n): Q^T and dO^T operands, statistics, position
  const int my_row = wave * 16 + n;
  const bool row_ok = my_row < nrows;
  const int rg = row_ok ? my_row : 0;
  const uint64_t row = (uint64_t)(it.q_begin + rg / G) * a.hq + (uint64_t)kvh * G + rg % G;
  frag_t qb[KSK], gb[KSV];
#pragma unroll
  for (int k = 0; k < KSK; ++k)
    qb[k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(a.q) + row * D + 32 * k + 8 * g4);
#pragma unroll
  for (int k = 0; k < KSV; ++k)
    gb[k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(b.dout) + row * DV + 32 * k + 8 * g4);
  const float l2 = row_ok ? a.lse[row] * kLog2e : INFINITY;
  const float dl = row_ok ? b.delta[row] : 0.f;
  const int pos = a.q_pos[it.q_begin + rg / G];
  floatx4_t dq[DBK];
#pragma unroll
  for (int i = 0; i < DBK; ++i) dq[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // tile loads: piece c < 32 PK of K (key c / PK), then of V
  u32x4_t pre[PER_THREAD];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_k = c < kBwdKeyTile * PK;
        const int cc = is_k ? c : c - kBwdKeyTile * PK;
        const int key = is_k ? cc / PK : cc / PV, piece = is_k ? cc % PK : cc % PV;
        const int t = min(t0 + key, it.tok_end - 1);
        const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
        pre[j] = is_k ? *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.k) + slot * krow +
                                                          (uint64_t)kvh * D + piece * 8)
                      : *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.v) + slot * vrow +
                                                          (uint64_t)kvh * DV + piece * 8);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_k = c < kBwdKeyTile * PK;
        const int cc = is_k ? c : c - kBwdKeyTile * PK;
        char* dst = is_k ? ks + bwd_off<D>(cc / PK, cc % PK) : vs + bwd_off<DV>(cc / PV, cc % PV);
        *reinterpret_cast<u32x4_t*>(dst) = pre[j];
      }
    }
  };

  fetch(it.tok_begin);
  for (int t0 = it.tok_begin; t0 < it.tok_end; t0 += kBwdKeyTile) {
    __syncthreads();  // every wave is done with the previous tile
    store();
    __syncthreads();
    if (t0 + kBwdKeyTile < it.tok_end) fetch(t0 + kBwdKeyTile);

    uint32_t dw[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      floatx4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSK; ++k)
        s = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(ks + bwd_off<D>(16 * h + n, 4 * k + g4)), qb[k], s);
#pragma unroll
      for (int k = 0; k < KSV; ++k)
        dp = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(vs + bwd_off<DV>(16 * h + n, 4 * k + g4)), gb[k], dp);
      // lane (n, g4) element e: key t0 + 16 h + 4 g4 + e, row my_row
      float ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * h + 4 * g4 + e;
        const bool vis = row_ok && t < it.tok_end && (!a.causal || t <= pos) && (a.window == 0 || t > pos - a.window);
        const float p = vis ? fast_exp2(__builtin_fmaf(s[e], c2, -l2)) : 0.f;
        ds[e] = p * (dp[e] - dl) * a.scale;
      }
      dw[2 * h] = Pair16<T>::pack(ds[0], ds[1]);
      dw[2 * h + 1] = Pair16<T>::pack(ds[2], ds[3]);
    }
    const frag_t df = __builtin_bit_cast(frag_t, make_uint4(dw[0], dw[1], dw[2], dw[3]));
#pragma unroll
    for (int blk = 0; blk < DBK; ++blk)
      dq[blk] = mfma_16x16x32<T>(df, bwd_tfrag(ks, bwd_troff<D>(blk, 0, n, g4), bwd_troff<D>(blk, 1, n, g4)), dq[blk]);
  }

  // lane (n, g4) of block blk holds dims 16 blk + n of rows wave 16 + 4 g4 + e
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = wave * 16 + 4 * g4 + e;
    if (r >= nrows) continue;
    const uint64_t orow = (uint64_t)(it.q_begin + r / G) * a.hq + (uint64_t)kvh * G + r % G;
#pragma unroll
    for (int blk = 0; blk < DBK; ++blk) store_out<T>(b.dq, orow * D + 16 * blk + n, dq[blk][e]);
  }
}

namespace {

using BwdFn = hipError_t (*)(const BwdArgs&, int, int, int, hipStream_t);

// items: [0, n_dq) dQ per (query, KV head), [n_dq, n_dq + n_kv) dK/dV per
// key block, then n_dqt dQ row tiles
template <typename T, int D, int DV, int G>
hipError_t launch_bwd_t(const BwdArgs& b, int n_dq, int n_kv, int n_dqt, hipStream_t stream) {
  constexpr bool kMfma = sizeof(T) == 2 && D % 64 == 0 && DV % 64 == 0;
  if (kMfma && n_dqt > 0) {
    if constexpr (kMfma)
      hipLaunchKernelGGL((bwd_dq_mfma_kernel<T, D, DV>), dim3(n_dqt), dim3(kBwdMfmaWaves * kWave), 0, stream, b,
                         n_dq + n_kv, G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (n_dq > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, DV, G>), dim3(n_dq), dim3(kBwdDqWaves * kWave), 0, stream, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_kv > 0) {
    if constexpr (kMfma)
      hipLaunchKernelGGL((bwd_dkv_mfma_kernel<T, D, DV>), dim3(n_kv), dim3(kBwdMfmaWaves * kWave), 0, stream, b, n_dq,
                         G);
    else
      hipLaunchKernelGGL((bwd_dkv_kernel<T, D, DV, G>), dim3(n_kv), dim3(kBwdKvWaves * kWave), 0, stream, b, n_dq);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int D, int DV>
BwdFn pick_bwd_g(int g) {
  switch (g) {
    case 1: return launch_bwd_t<T, D, DV, 1>;
    case 2: return launch_bwd_t<T, D, DV, 2>;
    case 4: return launch_bwd_t<T, D, DV, 4>;
    case 8: return launch_bwd_t<T, D, DV, 8>;
    case 16: return launch_bwd_t<T, D, DV, 16>;
    default: return nullptr;
  }
}

template <typename T>
BwdFn pick_bwd_d(int d, int dv, int g) {
  if (d == 64 && dv == 64) return pick_bwd_g<T, 64, 64>(g);
  if (d == 128 && dv == 128) return pick_bwd_g<T, 128, 128>(g);
  if (d == 256 && dv == 256) return pick_bwd_g<T, 256, 256>(g);
  if (d == 192 && dv == 128) return pick_bwd_g<T, 192, 128>(g);
  return nullptr;
}

BwdFn pick_bwd(int dtype, int d, int dv, int g) {
  if (dtype == 0) return pick_bwd_d<float>(d, dv, g);
  if (dtype == 1) return pick_bwd_d<uint16_t>(d, dv, g);
  if (dtype == 2) return pick_bwd_d<_Float16>(d, dv, g);
  return nullptr;
}

}  // namespace

bool bwd_supported(int dtype, int d, int dv, int g) { return pick_bwd(dtype, d, dv, g) != nullptr; }

hipError_t launch_gqa_bwd(int dtype, int d, int dv, int g, const KernelArgs& a, const void* dout, void* dq, void* dk,
                          void* dvp, float* delta, float* acc, bool shared, const BwdItem* items, int n_dq, int n_kv,
                          int n_dqt, int64_t rows, int64_t pool_slots, int n_cu, hipStream_t stream) {
  BwdFn f = pick_bwd(dtype, d, dv, g);
  if (!f) return hipErrorInvalidValue;
  const int es = dtype == 0 ? 4 : 2;
  // Shared pages: f32 gradients are added into the pools themselves, 16-bit
  // ones into f32 sums in the workspace that are rounded into the pools last.
  float* acc_k = nullptr;
  float* acc_v = nullptr;
  if (shared) {
    acc_k = dtype == 0 ? static_cast<float*>(dk) : acc;
    acc_v = dtype == 0 ? static_cast<float*>(dvp) : acc + pool_slots * d;
  }
  // the gradient sums start at zero: rows no query sees keep it
  for (int pass = 0; pass < 2; ++pass) {
    void* base = pass == 0 ? (acc_k ? static_cast<void*>(acc_k) : dk) : (acc_v ? static_cast<void*>(acc_v) : dvp);
    const int64_t chunks = pool_slots * (pass == 0 ? d : dv) * (acc_k ? 4 : es) / 16;
    if (chunks == 0) continue;
    const int64_t grid = std::min<int64_t>((chunks + 255) / 256, (int64_t)std::max(n_cu, 1) * 16);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream, reinterpret_cast<u32x4_t*>(base),
                       chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs b{a, dout, dq, dk, dvp, delta, items, acc_k, acc_v};
  if (rows > 0) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
    if (dtype == 0)
      hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3(grid), dim3(256), 0, stream, b, rows, dv);
    else if (dtype == 1)
      hipLaunchKernelGGL(bwd_delta_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, b, rows, dv);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<_Float16>, dim3(grid), dim3(256), 0, stream, b, rows, dv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = f(b, n_dq, n_kv, n_dqt, stream);
  if (e != hipSuccess || !shared || dtype == 0) return e;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t n4 = pool_slots * (pass == 0 ? d : dv) / 4;
    if (n4 == 0) continue;
    const int64_t grid = std::min<int64_t>((n4 + 255) / 256, (int64_t)std::max(n_cu, 1) * 16);
    const float4* src = reinterpret_cast<const float4*>(pass == 0 ? acc_k : acc_v);
    uint2* dst = reinterpret_cast<uint2*>(pass == 0 ? dk : dvp);
    if (dtype == 1)
      hipLaunchKernelGGL(bwd_cast_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, n4);
    else
      hipLaunchKernelGGL(bwd_cast_kernel<_Float16>, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, n4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
