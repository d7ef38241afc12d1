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
  void* dq2;           // MLA: dq_rope [Q, H, P] (dq is dq_abs, dk the latent pool, dv the rotary pool)
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

// Zero the pool rows of the slot runs (first, count) no dK/dV item writes:
// one workgroup per run, rows of k_row / v_row bytes (multiples of 16) in
// the two gradient pools.
__global__ __launch_bounds__(256) void bwd_zero_runs_kernel(char* dk, char* dv, const int32_t* runs, int k_row,
                                                            int v_row) {
  const int64_t first = runs[2 * blockIdx.x], count = runs[2 * blockIdx.x + 1];
  const u32x4_t z = {0u, 0u, 0u, 0u};
  const int64_t nk = count * k_row / 16, nv = count * v_row / 16;
  u32x4_t* pk = reinterpret_cast<u32x4_t*>(dk + first * k_row);
  u32x4_t* pv = reinterpret_cast<u32x4_t*>(dv + first * v_row);
  for (int64_t i = threadIdx.x; i < nk; i += blockDim.x) pk[i] = z;
  for (int64_t i = threadIdx.x; i < nv; i += blockDim.x) pv[i] = z;
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
  // two LDS buffers: tile i in buffer i % 2
  __shared__ __attribute__((aligned(16))) char qs2[2][kBwdRowTile * D * 2];
  __shared__ __attribute__((aligned(16))) char gs2[2][kBwdRowTile * DV * 2];
  __shared__ float lse2s2[2][kBwdRowTile], dls2[2][kBwdRowTile];
  __shared__ int poss2[2][kBwdRowTile];
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
  // Tiles of query rows: registers two tiles ahead (fetched while the two
  // tiles before them are computed), then one LDS buffer per tile parity.
  struct Staged {
    u32x4_t v[PER_THREAD];
    float pl, pd;
    int pp;
  };
  auto fetch = [&](Staged& st, int r0) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_q = c < kBwdRowTile * PK;
        const int cc = is_q ? c : c - kBwdRowTile * PK;
        const int r = is_q ? cc / PK : cc / PV, piece = is_q ? cc % PK : cc % PV;
        const uint64_t row = row_addr(r0 + r);
        st.v[j] = is_q ? *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.q) + row * D + piece * 8)
                       : *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(b.dout) + row * DV +
                                                           piece * 8);
      }
    }
    if (tid < kBwdRowTile) {
      const int rho = r0 + tid;
      const uint64_t row = row_addr(rho);
      const bool ok = rho < nrows;
      st.pl = ok ? a.lse[row] * kLog2e : INFINITY;
      st.pd = ok ? b.delta[row] : 0.f;
      st.pp = a.q_pos[it.q_begin + (ok ? rho : 0) / G];
    }
  };
  auto store = [&](const Staged& st, int buf) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_q = c < kBwdRowTile * PK;
        const int cc = is_q ? c : c - kBwdRowTile * PK;
        char* dst = is_q ? qs2[buf] + bwd_off<D>(cc / PK, cc % PK) : gs2[buf] + bwd_off<DV>(cc / PV, cc % PV);
        *reinterpret_cast<u32x4_t*>(dst) = st.v[j];
      }
    }
    if (tid < kBwdRowTile) {
      lse2s2[buf][tid] = st.pl;
      dls2[buf][tid] = st.pd;
      poss2[buf][tid] = st.pp;
    }
  };
  auto compute = [&](int buf) {
    const char* qs = qs2[buf];
    const char* gs = gs2[buf];
    const float* lse2s = lse2s2[buf];
    const float* dls = dls2[buf];
    const int* poss = poss2[buf];
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
  };

  // tile i: stored into buffer i % 2 after the barrier that follows the
  // compute of tile i - 2 (its last readers), made visible by the next
  // barrier, which also lets the fetch of tile i + 2 reuse its registers;
  // the barriers leave the row fetches in flight
  const int ntile = (nrows + kBwdRowTile - 1) / kBwdRowTile;
  if constexpr (D + DV <= 256) {
    Staged sa{}, sb{};
    if (ntile > 0) fetch(sa, 0);
    if (ntile > 1) fetch(sb, kBwdRowTile);
    for (int i = 0; i < ntile; i += 2) {
      store(sa, 0);
      barrier_keep_loads();
      if (i + 2 < ntile) fetch(sa, (i + 2) * kBwdRowTile);
      compute(0);
      if (i + 1 >= ntile) break;
      store(sb, 1);
      barrier_keep_loads();
      if (i + 3 < ntile) fetch(sb, (i + 3) * kBwdRowTile);
      compute(1);
    }
  } else {
    // wider rows: one tile ahead in registers (two would spill)
    Staged sa{};
    if (ntile > 0) fetch(sa, 0);
    for (int i = 0; i < ntile; ++i) {
      store(sa, i & 1);
      barrier_keep_loads();
      if (i + 1 < ntile) fetch(sa, (i + 1) * kBwdRowTile);
      compute(i & 1);
    }
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

// dQ per 128-row tile on the 32x32x16 MFMA (K = V head sizes 64 and 128):
// four waves of 32 rows, so that each K and V fragment read from LDS feeds a
// 32-row product (twice the rows of the 16x16x32 kernel above, half the LDS
// bytes per flop).  The tile of 32 keys is held as in the forward's prefill
// tile (pieces of key row t at piece ^ swz(t)):
//   S^T[32 keys x 32 rows]  = K . Q^T       dP^T = V . dO^T
//   dQ^T[D x 32 rows]      += K^T . dS^T    (K^T by transposed reads, dS^T
//                                             straight from the accumulators)
// Every lane owns one row (its accumulator column); dS is rounded to the
// storage type for the product, as in the kernel above.
constexpr int kBwdDq32Waves = 4;
template <typename T, int D, int DV>
__global__ __launch_bounds__(kBwdDq32Waves* kWave) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_mfma32_kernel(BwdArgs b, int first_item, int G) {
  constexpr int NT = kBwdKeyTile;
  constexpr int KSK = D / 16, KSV = DV / 16, DB = D / 32;
  constexpr int PK = D / 8, PV = DV / 8;
  constexpr int CHUNKS = NT * (PK + PV);
  constexpr int THREADS = kBwdDq32Waves * kWave;
  constexpr int PER_THREAD = (CHUNKS + THREADS - 1) / THREADS;
  static_assert(kBwdDq32Waves * 32 == kBwdQRows, "four waves of 32 rows");
  static_assert(NT == 32 && D % 32 == 0 && DV % 16 == 0, "one 32-key block per tile");
  __shared__ __attribute__((aligned(16))) char ks[NT * D * 2];
  __shared__ __attribute__((aligned(16))) char vs[NT * DV * 2];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 31, h = lane >> 5;
  const int kvh = it.kvh;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D, vrow = (uint64_t)a.hkv * DV;
  const int nrows = (it.q_end - it.q_begin) * G;
  const float c2 = a.scale_log2;

  // this lane's row (accumulator column n): Q^T and dO^T operands (dims
  // 16 k + 8 h .. +7), statistics, position
  const int my_row = wave * 32 + n;
  const bool row_ok = my_row < nrows;
  const int rg = row_ok ? my_row : 0;
  const uint64_t row = (uint64_t)(it.q_begin + rg / G) * a.hq + (uint64_t)kvh * G + rg % G;
  frag_t qb[KSK], gb[KSV];
#pragma unroll
  for (int k = 0; k < KSK; ++k)
    qb[k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(a.q) + row * D + 16 * k + 8 * h);
#pragma unroll
  for (int k = 0; k < KSV; ++k)
    gb[k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(b.dout) + row * DV + 16 * k + 8 * h);
  const float l2 = row_ok ? a.lse[row] * kLog2e : INFINITY;
  const float dl = row_ok ? b.delta[row] : 0.f;
  const int pos = a.q_pos[it.q_begin + rg / G];
  floatx16_t dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.f;

  // K^T fragments of dim block blk and k-step kk: two transposed reads (4
  // keys each) at toff[blk][r] + kk * 16 rows, the forward's V^T pattern
  uint32_t toff[DB][2];
  {
    const int grp16 = lane >> 4, gi = lane & 15;
    const int key0 = 4 * (grp16 >> 1) + (gi >> 2);
    const int d0 = 16 * (grp16 & 1) + 4 * (gi & 3);
#pragma unroll
    for (int blk = 0; blk < DB; ++blk)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int dim = 32 * blk + d0;
        toff[blk][r] = (uint32_t)(tile_off<D>(key0 + 8 * r, dim >> 3) + (dim & 7) * 2);
      }
  }

  // tile loads: piece c < NT PK of K (key c / PK), then of V
  u32x4_t pre[PER_THREAD];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * THREADS;
      if (c < CHUNKS) {
        const bool is_k = c < NT * PK;
        const int cc = is_k ? c : c - NT * PK;
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
        const bool is_k = c < NT * PK;
        const int cc = is_k ? c : c - NT * PK;
        char* dst = is_k ? ks + tile_off<D>(cc / PK, cc % PK) : vs + tile_off<DV>(cc / PV, cc % PV);
        *reinterpret_cast<u32x4_t*>(dst) = pre[j];
      }
    }
  };

  fetch(it.tok_begin);
  for (int t0 = it.tok_begin; t0 < it.tok_end; t0 += NT) {
    __syncthreads();  // every wave is done with the previous tile
    store();
    __syncthreads();
    if (t0 + NT < it.tok_end) fetch(t0 + NT);

    floatx16_t s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
    for (int k = 0; k < KSK; ++k)
      s = mfma_32x32x16<T>(*reinterpret_cast<const frag_t*>(ks + tile_off<D>(n, 2 * k + h)), qb[k], s);
#pragma unroll
    for (int k = 0; k < KSV; ++k)
      dp = mfma_32x32x16<T>(*reinterpret_cast<const frag_t*>(vs + tile_off<DV>(n, 2 * k + h)), gb[k], dp);
    // element e: key t0 + 8 (e / 4) + 4 h + e % 4 of row my_row; k-step kk
    // of dQ^T takes elements 8 kk .. 8 kk + 7 (keys 16 kk .. 16 kk + 15)
    frag_t df[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float ds[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int e = 8 * kk + 2 * j + i;
          const int t = t0 + 8 * (e >> 2) + 4 * h + (e & 3);
          const bool vis =
              row_ok && t < it.tok_end && (!a.causal || t <= pos) && (a.window == 0 || t > pos - a.window);
          const float p = vis ? fast_exp2(__builtin_fmaf(s[e], c2, -l2)) : 0.f;
          ds[i] = p * (dp[e] - dl) * a.scale;
        }
        w[j] = Pair16<T>::pack(ds[0], ds[1]);
      }
      df[kk] = __builtin_bit_cast(frag_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int blk = 0; blk < DB; ++blk) {
        const short4_t v0 = lds_read_tr16(ks + toff[blk][0] + kk * 16 * (D * 2));
        const short4_t v1 = lds_read_tr16(ks + toff[blk][1] + kk * 16 * (D * 2));
        const frag_t kf = __builtin_bit_cast(
            frag_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))));
        dq[blk] = mfma_32x32x16<T>(kf, df[kk], dq[blk]);
      }
  }

  // dQ^T block blk: lane (n, h) element 4 k + i is dim 32 blk + 8 k + 4 h + i of row my_row
  if (!row_ok) return;
  uint16_t* orow = reinterpret_cast<uint16_t*>(b.dq) + row * D;
#pragma unroll
  for (int blk = 0; blk < DB; ++blk)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint2 w;
      w.x = Pair16<T>::pack(dq[blk][4 * k + 0], dq[blk][4 * k + 1]);
      w.y = Pair16<T>::pack(dq[blk][4 * k + 2], dq[blk][4 * k + 3]);
      *reinterpret_cast<uint2*>(orow + 32 * blk + 8 * k + 4 * h) = w;
    }
}

// ---------------------------------------------------------------------------
// Absorbed-MLA backward (ruDNN 0.1.107 paged_attention `mla_backward` /
// `mla_backward_into`), on 16-bit MFMA.  The latent is both key and value,
// so its gradient receives the key term and the value term; the rotated
// position cache and the position query receive the terms of their own dot
// product.  With s = scale (q_abs . lat_t + q_rope . kpos_t), P = exp(s -
// lse), dP_t = dO . lat_t, D = dO . O and dS = P (dP - D):
//   dq_abs = scale sum_t dS_t lat_t     dq_rope = scale sum_t dS_t kpos_t
//   dlat_t = sum_rows (scale dS_t q_abs + P_t dO)   dkpos_t = sum_rows scale dS_t q_rope
// Four waves per workgroup split the 512 latent dims (128 each) and the 64
// rotary dims (16 each) of every product; the partial score and dP tiles
// of the waves meet in LDS and are summed in one fixed order, as in the
// forward's split score tile.  LDS rows are padded by 16 bytes so that the
// 16 rows one operand read touches fall in distinct banks.
// ---------------------------------------------------------------------------
constexpr int kMlaBwdWaves = 4;
constexpr int kMlaLatRow = kMlaRank * 2 + 16;  // padded LDS bytes of a 512-wide row
constexpr int kMlaPosRow = kMlaRope * 2 + 16;  // padded LDS bytes of a 64-wide row

// Copy rows [0, ROWS) of a [ROWS, WIDTH] 16-bit tile into LDS (padded rows
// of ROW bytes); row r comes from src(r).
template <int WIDTH, int ROW, int ROWS = 16, typename Src>
__device__ __forceinline__ void mla_tile_to_lds(char* dst, Src src) {
  constexpr int PIECES = WIDTH / 8;  // 16-byte pieces per row
  for (int idx = threadIdx.x; idx < ROWS * PIECES; idx += kMlaBwdWaves * kWave) {
    const int r = idx / PIECES, piece = idx % PIECES;
    *reinterpret_cast<u32x4_t*>(dst + r * ROW + piece * 16) =
        *reinterpret_cast<const u32x4_t*>(src(r) + piece * 8);
  }
}

// dq_abs and dq_rope of one query and group of 16 heads (item kvh = g: heads
// 16 g .. 16 g + 15, the last group possibly partial) over its visible keys
// [tok_begin, tok_end), 16 keys per tile:
//   S^T, dP^T [16 keys x 16 heads]    (partial over each wave's dims, summed)
//   dq_abs^T [dims x heads] += lat^T . dS^T,  dq_rope^T += kpos^T . dS^T
template <typename T>
__global__ __launch_bounds__(kMlaBwdWaves* kWave) void mla_bwd_dq_kernel(BwdArgs b, int first_item) {
  constexpr int H = kMlaHeads, R = kMlaRank, P = kMlaRope, NT = 16;
  __shared__ __attribute__((aligned(16))) char lat_s[NT * kMlaLatRow];
  __shared__ __attribute__((aligned(16))) char kp_s[NT * kMlaPosRow];
  __shared__ floatx4_t xs[2][kMlaBwdWaves][kWave];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, c = lane >> 4;
  const int qi = it.q_begin, tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint16_t* lat = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* kpos = reinterpret_cast<const uint16_t*>(a.kr);

  // this wave's operands: q_abs^T and dO^T over latent dims 128 wave .. +127
  // (lane (n, c): head 16 g + n, dims 32 k + 8 c), q_rope^T over rotary dims
  // 16 wave ..; columns past the last head repeat it and are not stored
  const int head = H * it.kvh + n;
  const bool head_ok = head < a.hq;
  const uint64_t row = (uint64_t)qi * a.hq + min(head, a.hq - 1);
  frag_t qa[4], go[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d0 = 32 * (4 * wave + k) + 8 * c;
    qa[k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(a.q) + row * R + d0);
    go[k] = *reinterpret_cast<const frag_t*>(reinterpret_cast<const uint16_t*>(b.dout) + row * R + d0);
  }
  const short4_t qr = *reinterpret_cast<const short4_t*>(reinterpret_cast<const uint16_t*>(a.qr) + row * P +
                                                         16 * wave + 4 * c);
  const float l2 = a.lse[row] * kLog2e, dl = b.delta[row];
  const float c2 = a.scale_log2;

  floatx4_t dqa[8], dqr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) dqa[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = tb & ~(NT - 1); t0 < te; t0 += NT) {
    auto slot_of = [&](int r) {
      const int t = min(max(t0 + r, tb), te - 1);  // clamped keys are masked below
      return (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
    };
    mla_tile_to_lds<R, kMlaLatRow>(lat_s, [&](int r) { return lat + slot_of(r) * R; });
    mla_tile_to_lds<P, kMlaPosRow>(kp_s, [&](int r) { return kpos + slot_of(r) * P; });
    __syncthreads();
    floatx4_t sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const frag_t lf = *reinterpret_cast<const frag_t*>(lat_s + n * kMlaLatRow + (32 * (4 * wave + k) + 8 * c) * 2);
      sc = mfma_16x16x32<T>(lf, qa[k], sc);
      dp = mfma_16x16x32<T>(lf, go[k], dp);
    }
    sc = mfma_16x16x16<T>(*reinterpret_cast<const short4_t*>(kp_s + n * kMlaPosRow + (16 * wave + 4 * c) * 2), qr,
                          sc);
    xs[0][wave][lane] = sc;
    xs[1][wave][lane] = dp;
    __syncthreads();
    sc = ((xs[0][0][lane] + xs[0][1][lane]) + xs[0][2][lane]) + xs[0][3][lane];
    dp = ((xs[1][0][lane] + xs[1][1][lane]) + xs[1][2][lane]) + xs[1][3][lane];
    // lane (n, c): keys t0 + 4 c + r of head n
    float ds[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * c + r;
      const float p = (t >= tb && t < te) ? fast_exp2(__builtin_fmaf(sc[r], c2, -l2)) : 0.f;
      ds[r] = p * (dp[r] - dl);
    }
    const short4_t dsf =
        __builtin_bit_cast(short4_t, make_uint2(Pair16<T>::pack(ds[0], ds[1]), Pair16<T>::pack(ds[2], ds[3])));
    // A = lat^T [16 dims x 16 keys] by transposed reads: lane 4 r + j of a
    // 16-lane group gives dims .. + 4 j of key row 4 c + r
    const int key = 4 * c + (n >> 2);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int dim = 128 * wave + 16 * blk + 4 * (n & 3);
      dqa[blk] = mfma_16x16x16<T>(lds_read_tr16(lat_s + key * kMlaLatRow + dim * 2), dsf, dqa[blk]);
    }
    dqr = mfma_16x16x16<T>(lds_read_tr16(kp_s + key * kMlaPosRow + (16 * wave + 4 * (n & 3)) * 2), dsf, dqr);
    __syncthreads();  // the tiles and the exchange are rewritten next
  }

  // lane (n, c) element e: dim (block base) + 4 c + e of head 16 g + n
  if (!head_ok) return;
  uint16_t* oa = reinterpret_cast<uint16_t*>(b.dq) + row * R + 128 * wave + 4 * c;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    uint2 w;
    w.x = Pair16<T>::pack(dqa[blk][0] * a.scale, dqa[blk][1] * a.scale);
    w.y = Pair16<T>::pack(dqa[blk][2] * a.scale, dqa[blk][3] * a.scale);
    *reinterpret_cast<uint2*>(oa + 16 * blk) = w;
  }
  uint2 w;
  w.x = Pair16<T>::pack(dqr[0] * a.scale, dqr[1] * a.scale);
  w.y = Pair16<T>::pack(dqr[2] * a.scale, dqr[3] * a.scale);
  *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(b.dq2) + row * P + 16 * wave + 4 * c) = w;
}

// dlatent and dkpos of one block of up to kBwdBlockKeys keys, 64 keys (four
// 16-key tiles) at a time, against the queries [q_begin, q_end) that see
// them, each query one 16-row tile per group of 16 heads (a partial last
// group repeats its last head in the missing rows, weighted zero); a
// (query, head group)'s operand tiles are loaded once for the 64 keys:
//   S, dP [16 heads x 16 keys] per key tile (partial over each wave's dims,
//   summed)
//   dlat^T [dims x keys] += dO^T . P + scale q_abs^T . dS
//   dkpos^T [dims x keys] += scale q_rope^T . dS
template <typename T>
__global__ __launch_bounds__(kMlaBwdWaves* kWave) void mla_bwd_dkv_kernel(BwdArgs b, int first_item) {
  constexpr int H = kMlaHeads, R = kMlaRank, P = kMlaRope, NT = 16, KT = 4;
  __shared__ __attribute__((aligned(16))) char lat_s[KT * NT * kMlaLatRow];
  __shared__ __attribute__((aligned(16))) char kp_s[KT * NT * kMlaPosRow];
  __shared__ __attribute__((aligned(16))) char qa_s[H * kMlaLatRow];
  __shared__ __attribute__((aligned(16))) char go_s[H * kMlaLatRow];
  __shared__ __attribute__((aligned(16))) char qr_s[H * kMlaPosRow];
  __shared__ floatx4_t xs[2][KT][kMlaBwdWaves][kWave];
  __shared__ float l2s[H], dls[H];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, c = lane >> 4;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const int L = a.seq_lens[it.seq];
  const uint16_t* lat = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* kpos = reinterpret_cast<const uint16_t*>(a.kr);
  const float c2 = a.scale_log2;

  for (int sub = it.tok_begin; sub < it.tok_end; sub += KT * NT) {
    const int te = min(it.tok_end, sub + KT * NT);
    auto slot_of = [&](int r) {
      const int t = min(sub + r, te - 1);
      return (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
    };
    mla_tile_to_lds<R, kMlaLatRow, KT * NT>(lat_s, [&](int r) { return lat + slot_of(r) * R; });
    mla_tile_to_lds<P, kMlaPosRow, KT * NT>(kp_s, [&](int r) { return kpos + slot_of(r) * P; });
    __syncthreads();
    // B operands of S = q_abs lat^T (+ q_rope kpos^T) and dP = dO lat^T:
    // lane (n, c) holds key 16 kt + n's dims 32 k + 8 c (this wave's k-steps)
    frag_t lb[KT][4];
    short4_t kb[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        lb[kt][k] = *reinterpret_cast<const frag_t*>(lat_s + (NT * kt + n) * kMlaLatRow + (32 * (4 * wave + k) + 8 * c) * 2);
      kb[kt] = *reinterpret_cast<const short4_t*>(kp_s + (NT * kt + n) * kMlaPosRow + (16 * wave + 4 * c) * 2);
    }
    floatx4_t dla[KT][8], dkp[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      dkp[kt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 8; ++i) dla[kt][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }

    for (int qi = it.q_begin; qi < it.q_end; ++qi) {
      const int pos = a.q_pos[qi];
      const int hi = a.causal ? pos : L - 1;
      const int lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;
      if (hi < sub || lo >= te) continue;  // this query sees none of the keys
      for (int g0 = 0; g0 < a.hq; g0 += H) {
        const int nh = min(H, a.hq - g0);  // heads of this group
        const uint64_t row0 = (uint64_t)qi * a.hq + g0;
        auto hrow = [&](int r) { return row0 + min(r, nh - 1); };
        __syncthreads();  // the previous (query, head group)'s tiles and partials are no longer read
        mla_tile_to_lds<R, kMlaLatRow>(qa_s, [&](int r) { return reinterpret_cast<const uint16_t*>(a.q) + hrow(r) * R; });
        mla_tile_to_lds<R, kMlaLatRow>(go_s,
                                       [&](int r) { return reinterpret_cast<const uint16_t*>(b.dout) + hrow(r) * R; });
        mla_tile_to_lds<P, kMlaPosRow>(qr_s, [&](int r) { return reinterpret_cast<const uint16_t*>(a.qr) + hrow(r) * P; });
        if (tid < H) {
          l2s[tid] = a.lse[hrow(tid)] * kLog2e;
          dls[tid] = b.delta[hrow(tid)];
        }
        __syncthreads();
        // this wave's partial S and dP of every key tile
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          floatx4_t sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int off = n * kMlaLatRow + (32 * (4 * wave + k) + 8 * c) * 2;
            sc = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(qa_s + off), lb[kt][k], sc);
            dp = mfma_16x16x32<T>(*reinterpret_cast<const frag_t*>(go_s + off), lb[kt][k], dp);
          }
          sc = mfma_16x16x16<T>(*reinterpret_cast<const short4_t*>(qr_s + n * kMlaPosRow + (16 * wave + 4 * c) * 2),
                                kb[kt], sc);
          xs[0][kt][wave][lane] = sc;
          xs[1][kt][wave][lane] = dp;
        }
        __syncthreads();
        // A = dO^T / q_abs^T [16 dims x 16 heads] by transposed reads: lane
        // 4 r + j of a 16-lane group gives dims .. + 4 j of head row 4 c + r
        const int head = 4 * c + (n >> 2);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const floatx4_t sc = ((xs[0][kt][0][lane] + xs[0][kt][1][lane]) + xs[0][kt][2][lane]) + xs[0][kt][3][lane];
          const floatx4_t dp = ((xs[1][kt][0][lane] + xs[1][kt][1][lane]) + xs[1][kt][2][lane]) + xs[1][kt][3][lane];
          // lane (n, c): heads 4 c + r of key t
          const int t = sub + NT * kt + n;
          const bool vis = t < te && t >= lo && t <= hi;
          float pv[4], ds[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = 4 * c + r;
            pv[r] = vis && h < nh ? fast_exp2(__builtin_fmaf(sc[r], c2, -l2s[h])) : 0.f;
            ds[r] = pv[r] * (dp[r] - dls[h]) * a.scale;
          }
          const short4_t pf =
              __builtin_bit_cast(short4_t, make_uint2(Pair16<T>::pack(pv[0], pv[1]), Pair16<T>::pack(pv[2], pv[3])));
          const short4_t dsf =
              __builtin_bit_cast(short4_t, make_uint2(Pair16<T>::pack(ds[0], ds[1]), Pair16<T>::pack(ds[2], ds[3])));
#pragma unroll
          for (int blk = 0; blk < 8; ++blk) {
            const int off = head * kMlaLatRow + (128 * wave + 16 * blk + 4 * (n & 3)) * 2;
            dla[kt][blk] = mfma_16x16x16<T>(lds_read_tr16(go_s + off), pf, dla[kt][blk]);
            dla[kt][blk] = mfma_16x16x16<T>(lds_read_tr16(qa_s + off), dsf, dla[kt][blk]);
          }
          dkp[kt] = mfma_16x16x16<T>(lds_read_tr16(qr_s + head * kMlaPosRow + (16 * wave + 4 * (n & 3)) * 2), dsf,
                                     dkp[kt]);
        }
      }
    }
    // lane (n, c) element e: dim (block base) + 4 c + e of key sub + 16 kt + n
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int t = sub + NT * kt + n;
      if (t < te) {
        const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
#pragma unroll
        for (int blk = 0; blk < 8; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            put_grad<T>(b.dk, b.acc_k, slot * R + 128 * wave + 16 * blk + 4 * c + e, dla[kt][blk][e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) put_grad<T>(b.dv, b.acc_v, slot * P + 16 * wave + 4 * c + e, dkp[kt][e]);
      }
    }
    __syncthreads();  // the key tiles are rewritten by the next 64 keys
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU backward for every shape the kernels above do not take (any
// group size, head sizes up to 1024, MLA with f32 data or other widths), in
// the forward vector kernel's description (GenericShape: key rows [k1 | k2],
// value rows V or, for MLA, k1 itself), fp32 throughout:
//   dQ: one workgroup per dQ item (one query, one work unit of up to 16
//       heads, its visible keys); the unit's heads in passes of 8, keys in
//       tiles of 8: S and dP of the 64 (key, head) pairs (four threads per
//       pair over a quarter of the dims each), dS = P (dP - D), then
//       dq += dS k (d1 + d2 dims);
//   dK/dV: one workgroup per dK/dV item (a block of keys of one KV head),
//       8 keys at a time, their sums in registers while every (query, head)
//       pair that sees them streams past 8 heads at a time:
//       dk += scale dS q, dv += P dO; MLA adds dv to the latent's dk part.
// Same items, zeroing, f32 sums for shared pages and D = dO . O pass as the
// specialised kernels.
// ---------------------------------------------------------------------------
constexpr int kGbThreads = 256;
constexpr int kGbHeads = 8;                                  // query heads per pass
constexpr int kGbKeys = 8;                                   // keys per tile
constexpr int kGbMaxW = kGenericMaxKeyWidth;                 // key row (d1 + d2) <= 1280
constexpr int kGbMaxV = kGenericMaxValueWidth;               // value row <= 1024
constexpr int kGbPhases = kGbThreads / kGbKeys;              // 32 threads per key / head of a pass
constexpr int kGbW = kGbMaxW / kGbPhases, kGbV = kGbMaxV / kGbPhases;  // dims per thread: 40, 32
static_assert(kGbThreads == 4 * kGbKeys * kGbHeads && kGbKeys == kGbHeads, "four threads per (key, head) pair");

// First query head and head count of work unit u (as the forward kernel).
__device__ __forceinline__ void gb_unit_heads(const GenericShape& s, int u, int* h0, int* nh) {
  const int kv = u / s.nsub, sub = u - kv * s.nsub;
  *h0 = kv * s.g + sub * s.unit_heads;
  *nh = min(s.unit_heads, s.g - sub * s.unit_heads);
}

// The query rows (q1 | q2 -> qs, W wide) and output-gradient rows (-> gs,
// DV wide) of heads h0 .. h0 + 7 of query qi (rows past n repeat the last),
// their lse in log2 units and D = dO . O, as f32 in LDS.
template <typename T>
__device__ __forceinline__ void gb_load_rows(const BwdArgs& b, const GenericShape& s, int qi, int h0, int n, float* qs,
                                             float* gs, float* st) {
  const KernelArgs& a = b.a;
  const int W = s.d1 + s.d2, DV = s.dv;
  for (int idx = threadIdx.x; idx < kGbHeads * W; idx += kGbThreads) {
    const int h = idx / W, d = idx - h * W;
    const uint64_t row = (uint64_t)qi * a.hq + h0 + min(h, n - 1);
    qs[idx] = d < s.d1 ? load_elem<T>(a.q, row * s.d1 + d) : load_elem<T>(a.qr, row * s.d2 + (d - s.d1));
  }
  for (int idx = threadIdx.x; idx < kGbHeads * DV; idx += kGbThreads) {
    const int h = idx / DV, d = idx - h * DV;
    gs[idx] = load_elem<T>(b.dout, ((uint64_t)qi * a.hq + h0 + min(h, n - 1)) * DV + d);
  }
  if (threadIdx.x < kGbHeads) {
    const uint64_t row = (uint64_t)qi * a.hq + h0 + min((int)threadIdx.x, n - 1);
    st[threadIdx.x] = a.lse[row] * kLog2e;
    st[kGbHeads + threadIdx.x] = b.delta[row];
  }
}

// Key rows (k1 | k2 -> ks, W wide) and value rows (-> vs, DV wide, unless V
// is k1) of keys t0 .. t0 + 7 of KV head kv (keys from `last` on repeat it).
template <typename T>
__device__ __forceinline__ void gb_load_keys(const KernelArgs& a, const GenericShape& s, const int32_t* bt, int kv,
                                             int t0, int last, float* ks, float* vs) {
  const int W = s.d1 + s.d2, DV = s.dv, ps = 1 << a.page_shift;
  for (int idx = threadIdx.x; idx < kGbKeys * W; idx += kGbThreads) {
    const int k = idx / W, d = idx - k * W;
    const int t = min(t0 + k, last);
    const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
    ks[idx] = d < s.d1 ? load_elem<T>(a.k, (slot * a.hkv + kv) * s.d1 + d)
                       : load_elem<T>(a.kr, slot * s.d2 + (d - s.d1));
  }
  if (!s.v_is_k) {
    for (int idx = threadIdx.x; idx < kGbKeys * DV; idx += kGbThreads) {
      const int k = idx / DV, d = idx - k * DV;
      const int t = min(t0 + k, last);
      const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
      vs[idx] = load_elem<T>(a.v, (slot * a.hkv + kv) * DV + d);
    }
  }
}

// S (log2 units) and dP of this thread's (key, head) pair: four threads per
// pair, each over a quarter of the dims, summed by lane exchange.
__device__ __forceinline__ void gb_pair_dots(const GenericShape& s, const float* qs, const float* gs, const float* ks,
                                             const float* vt, int vstride, float scale_log2, int* sk, int* sh,
                                             float* sc, float* dp) {
  const int W = s.d1 + s.d2, DV = s.dv;
  const int pair = threadIdx.x >> 2, part = threadIdx.x & 3;
  *sk = pair / kGbHeads;
  *sh = pair % kGbHeads;
  const float* q = qs + *sh * W;
  const float* k = ks + *sk * W;
  const float* g = gs + *sh * DV;
  const float* v = vt + *sk * vstride;
  float a0 = 0.f, a1 = 0.f;
  for (int d = part; d < W; d += 4) a0 = __builtin_fmaf(q[d], k[d], a0);
  for (int d = part; d < DV; d += 4) a1 = __builtin_fmaf(g[d], v[d], a1);
  a0 += __shfl_xor(a0, 1);
  a1 += __shfl_xor(a1, 1);
  a0 += __shfl_xor(a0, 2);
  a1 += __shfl_xor(a1, 2);
  *sc = a0 * scale_log2;
  *dp = a1;
}

// Pool rows of any width: zero the runs of slots no dK/dV item writes, zero
// f32 sums, round f32 sums into a 16-bit pool -- element by element (2-byte
// units for the runs), since rows need not be whole 16-byte pieces here.
__global__ __launch_bounds__(256) void gbwd_zero_runs_kernel(char* dk, char* dv, const int32_t* runs, int k_row,
                                                             int v_row) {
  const int64_t first = runs[2 * blockIdx.x], count = runs[2 * blockIdx.x + 1];
  uint16_t* pk = reinterpret_cast<uint16_t*>(dk + first * k_row);
  uint16_t* pv = reinterpret_cast<uint16_t*>(dv + first * v_row);
  for (int64_t i = threadIdx.x; i < count * k_row / 2; i += blockDim.x) pk[i] = 0;
  for (int64_t i = threadIdx.x; i < count * v_row / 2; i += blockDim.x) pv[i] = 0;
}
__global__ __launch_bounds__(256) void gbwd_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0.f;
}
template <typename T>
__global__ __launch_bounds__(256) void gbwd_cast_kernel(const float* src, void* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    store_out<T>(dst, i, src[i]);
}

template <typename T>
__global__ __launch_bounds__(kGbThreads) void gbwd_dq_kernel(BwdArgs b, GenericShape s) {
  __shared__ float q_s[kGbHeads * kGbMaxW];
  __shared__ float g_s[kGbHeads * kGbMaxV];
  __shared__ float k_s[kGbKeys * kGbMaxW];
  __shared__ float v_s[kGbKeys * kGbMaxV];
  __shared__ float st_s[2 * kGbHeads];
  __shared__ float ds_s[kGbKeys * kGbHeads];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[blockIdx.x];
  const int W = s.d1 + s.d2;
  const float* vt = s.v_is_k ? k_s : v_s;
  const int vstride = s.v_is_k ? W : s.dv;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const int qi = it.q_begin, pos = a.q_pos[qi];
  const int kv = it.kvh / s.nsub;
  int h0, nh;
  gb_unit_heads(s, it.kvh, &h0, &nh);
  const int oh = threadIdx.x / kGbPhases, od = threadIdx.x % kGbPhases;  // output head of the pass, dim phase
  for (int p0 = 0; p0 < nh; p0 += kGbHeads) {
    const int np = min(kGbHeads, nh - p0);
    __syncthreads();  // the previous pass's rows are no longer read
    gb_load_rows<T>(b, s, qi, h0 + p0, np, q_s, g_s, st_s);
    float acc[kGbW];
#pragma unroll
    for (int j = 0; j < kGbW; ++j) acc[j] = 0.f;
    for (int t0 = it.tok_begin; t0 < it.tok_end; t0 += kGbKeys) {
      __syncthreads();  // the previous tile is consumed (and the rows are written)
      gb_load_keys<T>(a, s, bt, kv, t0, it.tok_end - 1, k_s, v_s);
      __syncthreads();
      int sk, sh;
      float sc, dp;
      gb_pair_dots(s, q_s, g_s, k_s, vt, vstride, a.scale_log2, &sk, &sh, &sc, &dp);
      if ((threadIdx.x & 3) == 0) {
        const int t = t0 + sk;
        const bool vis = t < it.tok_end && (!a.causal || t <= pos) && (a.window == 0 || t > pos - a.window);
        const float p = vis ? fast_exp2(sc - st_s[sh]) : 0.f;
        ds_s[sk * kGbHeads + sh] = p * (dp - st_s[kGbHeads + sh]);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kGbW; ++j) {
        const int d = od + kGbPhases * j;
        if (d < W) {
          float x = acc[j];
#pragma unroll
          for (int k = 0; k < kGbKeys; ++k) x = __builtin_fmaf(ds_s[k * kGbHeads + oh], k_s[k * W + d], x);
          acc[j] = x;
        }
      }
    }
    if (oh < np) {
      const uint64_t row = (uint64_t)qi * a.hq + h0 + p0 + oh;
#pragma unroll
      for (int j = 0; j < kGbW; ++j) {
        const int d = od + kGbPhases * j;
        if (d < s.d1)
          store_out<T>(b.dq, row * s.d1 + d, acc[j] * a.scale);
        else if (d < W)
          store_out<T>(b.dq2, row * s.d2 + (d - s.d1), acc[j] * a.scale);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kGbThreads) void gbwd_dkv_kernel(BwdArgs b, GenericShape s, int first_item) {
  __shared__ float q_s[kGbHeads * kGbMaxW];
  __shared__ float g_s[kGbHeads * kGbMaxV];
  __shared__ float k_s[kGbKeys * kGbMaxW];
  __shared__ float v_s[kGbKeys * kGbMaxV];
  __shared__ float st_s[2 * kGbHeads];
  __shared__ float p_s[kGbKeys * kGbHeads], ds_s[kGbKeys * kGbHeads];
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
  const int W = s.d1 + s.d2, DV = s.dv;
  const float* vt = s.v_is_k ? k_s : v_s;
  const int vstride = s.v_is_k ? W : DV;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const int L = a.seq_lens[it.seq], ps = 1 << a.page_shift;
  const int kv = it.kvh;
  const int ok = threadIdx.x / kGbPhases, od = threadIdx.x % kGbPhases;  // key of the tile, dim phase
  for (int sub = it.tok_begin; sub < it.tok_end; sub += kGbKeys) {
    const int te = min(it.tok_end, sub + kGbKeys);
    __syncthreads();  // the previous keys are no longer read
    gb_load_keys<T>(a, s, bt, kv, sub, te - 1, k_s, v_s);
    float dk[kGbW], dv[kGbV];
#pragma unroll
    for (int j = 0; j < kGbW; ++j) dk[j] = 0.f;
#pragma unroll
    for (int j = 0; j < kGbV; ++j) dv[j] = 0.f;
    for (int qi = it.q_begin; qi < it.q_end; ++qi) {
      const int pos = a.q_pos[qi];
      const int hi = a.causal ? pos : L - 1;
      const int lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;
      if (hi < sub || lo >= te) continue;  // this query sees none of the keys
      for (int p0 = 0; p0 < s.g; p0 += kGbHeads) {
        const int np = min(kGbHeads, s.g - p0);
        __syncthreads();  // the previous rows and weights are no longer read (and the keys are written)
        gb_load_rows<T>(b, s, qi, kv * s.g + p0, np, q_s, g_s, st_s);
        __syncthreads();
        int sk, sh;
        float sc, dp;
        gb_pair_dots(s, q_s, g_s, k_s, vt, vstride, a.scale_log2, &sk, &sh, &sc, &dp);
        if ((threadIdx.x & 3) == 0) {
          const int t = sub + sk;
          const bool vis = sh < np && t < te && t >= lo && t <= hi;
          const float p = vis ? fast_exp2(sc - st_s[sh]) : 0.f;
          p_s[sk * kGbHeads + sh] = p;
          ds_s[sk * kGbHeads + sh] = p * (dp - st_s[kGbHeads + sh]) * a.scale;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kGbW; ++j) {
          const int d = od + kGbPhases * j;
          if (d < W) {
            float x = dk[j];
#pragma unroll
            for (int h = 0; h < kGbHeads; ++h) x = __builtin_fmaf(ds_s[ok * kGbHeads + h], q_s[h * W + d], x);
            dk[j] = x;
          }
        }
#pragma unroll
        for (int j = 0; j < kGbV; ++j) {
          const int d = od + kGbPhases * j;
          if (d < DV) {
            float x = dv[j];
#pragma unroll
            for (int h = 0; h < kGbHeads; ++h) x = __builtin_fmaf(p_s[ok * kGbHeads + h], g_s[h * DV + d], x);
            dv[j] = x;
          }
        }
      }
    }
    // key sub + ok: GQA writes dk (d1 wide) and dv (DV wide) rows of KV head
    // kv; MLA the latent row (dk's first d1 dims plus dv) and the rotary row
    const int t = sub + ok;
    if (t < te) {
      const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
      const uint64_t ra = (slot * a.hkv + kv) * s.d1;
      if (s.v_is_k) {
#pragma unroll
        for (int j = 0; j < kGbW; ++j) {
          const int d = od + kGbPhases * j;
          if (d < s.d1)
            put_grad<T>(b.dk, b.acc_k, ra + d, dk[j] + (j < kGbV ? dv[j] : 0.f));
          else if (d < W)
            put_grad<T>(b.dv, b.acc_v, slot * s.d2 + (d - s.d1), dk[j]);
        }
      } else {
        const uint64_t rb = (slot * a.hkv + kv) * DV;
#pragma unroll
        for (int j = 0; j < kGbW; ++j) {
          const int d = od + kGbPhases * j;
          if (d < s.d1) put_grad<T>(b.dk, b.acc_k, ra + d, dk[j]);
        }
#pragma unroll
        for (int j = 0; j < kGbV; ++j) {
          const int d = od + kGbPhases * j;
          if (d < DV) put_grad<T>(b.dv, b.acc_v, rb + d, dv[j]);
        }
      }
    }
  }
}

namespace {

using BwdFn = hipError_t (*)(const BwdArgs&, int, int, int, hipStream_t);

// items: [0, n_dq) dQ per (query, KV head), [n_dq, n_dq + n_kv) dK/dV per
// key block, then n_dqt dQ row tiles
template <typename T, int D, int DV, int G>
hipError_t launch_bwd_t(const BwdArgs& b, int n_dq, int n_kv, int n_dqt, hipStream_t stream) {
  constexpr bool kMfma = sizeof(T) == 2 && D % 64 == 0 && DV % 64 == 0;
  constexpr bool kMfma32 = kMfma && D == DV && D <= 128;  // the 32x32x16 dQ kernel's registers
  if (kMfma && n_dqt > 0) {
    if constexpr (kMfma32)
      hipLaunchKernelGGL((bwd_dq_mfma32_kernel<T, D, DV>), dim3(n_dqt), dim3(kBwdDq32Waves * kWave), 0, stream, b,
                         n_dq + n_kv, G);
    else if constexpr (kMfma)
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
                          int n_dqt, const int32_t* zero_runs, int n_zero_runs, int64_t rows, int64_t pool_slots,
                          int n_cu, hipStream_t stream) {
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
  if (shared) {
    // the sums start at zero everywhere: several items add into a row
    for (int pass = 0; pass < 2; ++pass) {
      void* base = pass == 0 ? static_cast<void*>(acc_k) : static_cast<void*>(acc_v);
      const int64_t chunks = pool_slots * (pass == 0 ? d : dv) * 4 / 16;
      if (chunks == 0) continue;
      const int64_t grid = std::min<int64_t>((chunks + 255) / 256, (int64_t)std::max(n_cu, 1) * 16);
      hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                         reinterpret_cast<u32x4_t*>(base), chunks);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else if (n_zero_runs > 0) {
    // single writer per row: only the rows no item writes are zeroed
    const int hkv = a.hkv;
    hipLaunchKernelGGL(bwd_zero_runs_kernel, dim3(n_zero_runs), dim3(256), 0, stream, static_cast<char*>(dk),
                       static_cast<char*>(dvp), zero_runs, hkv * d * es, hkv * dv * es);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs b{a, dout, dq, dk, dvp, delta, items, acc_k, acc_v, nullptr};
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


hipError_t launch_mla_bwd(int dtype, const KernelArgs& a, const void* dout, void* dq_abs, void* dq_rope, void* dlat,
                          void* dkpos, float* delta, float* acc, bool shared, const BwdItem* items, int n_dq, int n_kv,
                          const int32_t* zero_runs, int n_zero_runs, int64_t rows, int64_t pool_slots, int n_cu,
                          hipStream_t stream) {
  if (dtype != 1 && dtype != 2) return hipErrorInvalidValue;
  constexpr int R = kMlaRank, P = kMlaRope;
  float* acc_k = shared ? acc : nullptr;
  float* acc_v = shared ? acc + pool_slots * R : nullptr;
  if (shared) {
    // the f32 sums start at zero everywhere: several items add into a row
    for (int pass = 0; pass < 2; ++pass) {
      void* base = pass == 0 ? static_cast<void*>(acc_k) : static_cast<void*>(acc_v);
      const int64_t chunks = pool_slots * (pass == 0 ? R : P) * 4 / 16;
      if (chunks == 0) continue;
      const int64_t grid = std::min<int64_t>((chunks + 255) / 256, (int64_t)std::max(n_cu, 1) * 16);
      hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                         reinterpret_cast<u32x4_t*>(base), chunks);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else if (n_zero_runs > 0) {
    // single writer per row: only the rows no item writes are zeroed
    hipLaunchKernelGGL(bwd_zero_runs_kernel, dim3(n_zero_runs), dim3(256), 0, stream, static_cast<char*>(dlat),
                       static_cast<char*>(dkpos), zero_runs, R * 2, P * 2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs b{a, dout, dq_abs, dlat, dkpos, delta, items, acc_k, acc_v, dq_rope};
  if (rows > 0) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
    if (dtype == 1)
      hipLaunchKernelGGL(bwd_delta_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, b, rows, R);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<_Float16>, dim3(grid), dim3(256), 0, stream, b, rows, R);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_dq > 0) {
    if (dtype == 1)
      hipLaunchKernelGGL(mla_bwd_dq_kernel<uint16_t>, dim3(n_dq), dim3(kMlaBwdWaves * kWave), 0, stream, b, 0);
    else
      hipLaunchKernelGGL(mla_bwd_dq_kernel<_Float16>, dim3(n_dq), dim3(kMlaBwdWaves * kWave), 0, stream, b, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_kv > 0) {
    if (dtype == 1)
      hipLaunchKernelGGL(mla_bwd_dkv_kernel<uint16_t>, dim3(n_kv), dim3(kMlaBwdWaves * kWave), 0, stream, b, n_dq);
    else
      hipLaunchKernelGGL(mla_bwd_dkv_kernel<_Float16>, dim3(n_kv), dim3(kMlaBwdWaves * kWave), 0, stream, b, n_dq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!shared) return hipSuccess;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t n4 = pool_slots * (pass == 0 ? R : P) / 4;
    const int64_t grid = std::min<int64_t>((n4 + 255) / 256, (int64_t)std::max(n_cu, 1) * 16);
    const float4* src = reinterpret_cast<const float4*>(pass == 0 ? acc_k : acc_v);
    uint2* dst = reinterpret_cast<uint2*>(pass == 0 ? dlat : dkpos);
    if (dtype == 1)
      hipLaunchKernelGGL(bwd_cast_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, n4);
    else
      hipLaunchKernelGGL(bwd_cast_kernel<_Float16>, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


hipError_t launch_generic_bwd(int dtype, const GenericShape& s, const KernelArgs& a, const void* dout, void* dq,
                              void* dq2, void* dk, void* dvp, float* delta, float* acc, bool shared,
                              const BwdItem* items, int n_dq, int n_kv, const int32_t* zero_runs, int n_zero_runs,
                              int64_t rows, int64_t pool_rows, int n_cu, hipStream_t stream) {
  if (!generic_shape_ok(s) || dtype < 0 || dtype > 2) return hipErrorInvalidValue;
  const int es = dtype == 0 ? 4 : 2;
  const int wa = s.d1, wb = s.v_is_k ? s.d2 : s.dv;  // widths of the two gradient pools' rows
  const int64_t grid_cap = (int64_t)std::max(n_cu, 1) * 16;
  float* acc_k = nullptr;
  float* acc_v = nullptr;
  if (shared) {
    // f32 gradients are added into the pools themselves, 16-bit ones into f32
    // sums in the workspace; either way they start at zero everywhere
    acc_k = dtype == 0 ? static_cast<float*>(dk) : acc;
    acc_v = dtype == 0 ? static_cast<float*>(dvp) : acc + pool_rows * wa;
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t n = pool_rows * (pass == 0 ? wa : wb);
      if (n == 0) continue;
      hipLaunchKernelGGL(gbwd_zero_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, grid_cap)), dim3(256), 0,
                         stream, pass == 0 ? acc_k : acc_v, n);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else if (n_zero_runs > 0) {
    hipLaunchKernelGGL(gbwd_zero_runs_kernel, dim3(n_zero_runs), dim3(256), 0, stream, static_cast<char*>(dk),
                       static_cast<char*>(dvp), zero_runs, a.hkv * wa * es, a.hkv * wb * es);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs b{a, dout, dq, dk, dvp, delta, items, acc_k, acc_v, dq2};
  auto run = [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    if (rows > 0) {
      hipLaunchKernelGGL(bwd_delta_kernel<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, b, rows, s.dv);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (n_dq > 0) {
      hipLaunchKernelGGL(gbwd_dq_kernel<T>, dim3(n_dq), dim3(kGbThreads), 0, stream, b, s);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (n_kv > 0) {
      hipLaunchKernelGGL(gbwd_dkv_kernel<T>, dim3(n_kv), dim3(kGbThreads), 0, stream, b, s, n_dq);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (shared && dtype != 0) {
      for (int pass = 0; pass < 2; ++pass) {
        const int64_t n = pool_rows * (pass == 0 ? wa : wb);
        if (n == 0) continue;
        hipLaunchKernelGGL(gbwd_cast_kernel<T>, dim3((unsigned)std::min<int64_t>((n + 255) / 256, grid_cap)),
                           dim3(256), 0, stream, pass == 0 ? acc_k : acc_v, pass == 0 ? dk : dvp, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  };
  if (dtype == 0) return run(float{});
  if (dtype == 1) return run(uint16_t{});
  return run(_Float16{});
}

}  // namespace pa
