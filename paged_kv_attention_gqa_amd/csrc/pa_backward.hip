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
// dK/dV (one workgroup per 64-key block and KV head, looping over the
// sequence's query rows).  Each pool row has a single writer, so the result
// does not depend on scheduling (ruDNN's ordered, atomic-free variant).
#include <algorithm>

#include "pa_decode.h"
#include "pa_device.h"
#include "pa_launch.h"

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
};

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

// dK and dV of one block of up to kBwdBlockKeys keys and one KV head.  Lane
// (r, c) of wave w holds chunk c of keys tok_begin + (u NW + w) TPW + r,
// u < U, and their gradient sums; the sequence's query rows stream past.
template <typename T, int D, int DV, int G>
__global__ __launch_bounds__(kBwdKvWaves* kWave) void bwd_dkv_kernel(BwdArgs b, int first_item) {
  using Lay = DecodeLayout<T, D, DV>;
  constexpr int LPT = Lay::kLanes, KW = Lay::kKWords, VW = Lay::kVWords, EK = Lay::kKElems, EV = Lay::kVElems;
  constexpr int TPW = kWave / LPT, NW = kBwdKvWaves, SZ = (int)sizeof(T);
  constexpr int U = kBwdBlockKeys / (NW * TPW);
  static_assert(U >= 1 && U * NW * TPW == kBwdBlockKeys, "a block must split evenly over the lanes");
  const KernelArgs& a = b.a;
  const BwdItem it = b.items[first_item + blockIdx.x];
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
    for (int e = 0; e < EK; ++e) store_out<T>(b.dk, slot[u] * krow + (uint64_t)kvh * D + c * EK + e, dk[u][e]);
#pragma unroll
    for (int e = 0; e < EV; ++e) store_out<T>(b.dv, slot[u] * vrow + (uint64_t)kvh * DV + c * EV + e, dv[u][e]);
  }
}

namespace {

using BwdFn = hipError_t (*)(const BwdArgs&, int, int, hipStream_t);

template <typename T, int D, int DV, int G>
hipError_t launch_bwd_t(const BwdArgs& b, int n_dq, int n_kv, hipStream_t stream) {
  if (n_dq > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, DV, G>), dim3(n_dq), dim3(kBwdDqWaves * kWave), 0, stream, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_kv > 0) {
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
                          void* dvp, float* delta, const BwdItem* items, int n_dq, int n_kv, int64_t rows,
                          int64_t pool_slots, int n_cu, hipStream_t stream) {
  BwdFn f = pick_bwd(dtype, d, dv, g);
  if (!f) return hipErrorInvalidValue;
  const int es = dtype == 0 ? 4 : 2;
  // gradient pools start at zero: rows no query sees keep it
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t chunks = pool_slots * (pass == 0 ? d : dv) * es / 16;
    if (chunks == 0) continue;
    const int64_t grid = std::min<int64_t>((chunks + 255) / 256, (int64_t)std::max(n_cu, 1) * 16);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<u32x4_t*>(pass == 0 ? dk : dvp), chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs b{a, dout, dq, dk, dvp, delta, items};
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
  return f(b, n_dq, n_kv, stream);
}

}  // namespace pa
