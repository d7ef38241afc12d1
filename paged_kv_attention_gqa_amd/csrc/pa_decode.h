// Split-KV decode body (VALU): one query, one KV head and all G = Hq/Hkv
// query heads of that KV head, over one contiguous range of visible keys.
//
// Definition followed: boostr 0.2.0-beta.2 `standard_attention_fwd`
// (softmax(scale * q k^T + mask) v) with the GQA head mapping of `expand_kv`,
// evaluated over keys gathered through the block table as ruDNN 0.1.107
// `DevicePlan::attention` lays them out ([pages, page_size, Hkv, D]).  The
// split path follows ruDNN `attention_into_split`: each range keeps fp32
// statistics (running max, sum, unnormalised output) that a second pass
// merges by log-sum-exp weights.
//
// Layout in a wave: a key row of D elements is LPT lanes x 16 bytes, so one
// 16-byte load per lane brings TPW = 64 / LPT keys.  Lane (r, c) handles
// dimension chunk c of the keys assigned to row r.  Rows take consecutive key
// pairs so that a lane holds the same dimensions of two neighbouring keys,
// which lets the bf16 P.V step use packed bf16 dot products.  Each K row is
// read once for all G heads of its group.
#pragma once

#include "pa_device.h"

namespace pa {

// Lane layout of a decode wave for K rows of D elements and V rows of DV
// elements: a key row is spread over kLanes lanes (the smallest power of two
// that keeps a lane's K share within one 16-byte load), each holding kKWords
// 32-bit words of K and kVWords of V.  D = DV = 128 in bf16: 16 lanes x 16
// bytes of K and of V; D = 192, DV = 128 in bf16: 32 lanes x 12 bytes of K and
// 8 bytes of V.
constexpr int decode_lanes(int row_bytes) {
  int p = 1;
  while (row_bytes > 16 * p) p *= 2;
  return p;
}
template <typename T, int D, int DV>
struct DecodeLayout {
  static constexpr int kLanes = decode_lanes(D * (int)sizeof(T));
  static constexpr int kKWords = D * (int)sizeof(T) / kLanes / 4;
  static constexpr int kVWords = DV * (int)sizeof(T) / kLanes / 4;
  static constexpr int kKElems = D / kLanes;
  static constexpr int kVElems = DV / kLanes;
  static_assert(kLanes <= kWave && D % kLanes == 0 && DV % kLanes == 0, "unsupported head sizes");
  static_assert(kKWords * kLanes * 4 == D * (int)sizeof(T) && kVWords * kLanes * 4 == DV * (int)sizeof(T),
                "a lane's share of a row must be whole 32-bit words");
  static_assert(kKWords >= 1 && kVWords >= 1 && kVWords <= 8, "unsupported head sizes");
};

template <int N>
struct Words {
  uint32_t w[N];
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// N words at p (4-byte aligned; 16-byte aligned when N is a multiple of 4,
// 8-byte aligned when N == 2).  NT: non-temporal ("nt") loads.
template <int N, bool NT>
__device__ __forceinline__ Words<N> load_words(const char* p) {
  Words<N> r;
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p) + i;
      const u32x4_t v = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.w[4 * i + j] = v[j];
    }
  } else if constexpr (N == 2) {
    const u32x2_t* q = reinterpret_cast<const u32x2_t*>(p);
    const u32x2_t v = NT ? __builtin_nontemporal_load(q) : *q;
    r.w[0] = v[0];
    r.w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p) + i;
      r.w[i] = NT ? __builtin_nontemporal_load(q) : *q;
    }
  }
  return r;
}

// K/V rows a decode item reads once: non-temporal ("nt") loads.  Measured on
// MI355X: streaming reads reach ~7.0 TB/s with nt against ~6.2 TB/s without,
// and the decode kernel gained 11%.
constexpr float kDecodeLazyLog2 = 8.f;  // weights may reach 2^8 before the reference max moves
constexpr int kStreamLoad = 2;  // cache-policy operand of buffer loads: nt

// N words from a buffer resource at (voffset + soffset) bytes, nt.
template <int N>
__device__ __forceinline__ Words<N> buffer_words(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  Words<N> r;
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 16 * i, soff,
                                                                                           kStreamLoad));
#pragma unroll
      for (int j = 0; j < 4; ++j) r.w[4 * i + j] = v[j];
    }
  } else if constexpr (N == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(rsrc, voff, soff, kStreamLoad);
#pragma unroll
    for (int j = 0; j < 3; ++j) r.w[j] = (uint32_t)v[j];
  } else if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, kStreamLoad);
    r.w[0] = (uint32_t)v[0];
    r.w[1] = (uint32_t)v[1];
  } else {
    static_assert(N == 1, "unsupported chunk");
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, soff, kStreamLoad);
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, uint64_t idx, float v) {
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)(Pair16<T>::pack(v, 0.f) & 0xFFFFu);
  } else {
    reinterpret_cast<float*>(out)[idx] = v;
  }
}

// Raw buffer resource over `base` for 16-byte loads at byte offsets below
// 2^31 (stride 0, 32-bit data format; offsets past the range read zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, 0x7fffffff, 0x00020000);
}

// Scores of G heads against one key chunk held by this lane.
template <typename T, int G, int KW>
__device__ __forceinline__ void chunk_scores(const Words<KW> (&qv)[G], const Words<KW>& kv, float (&s)[G]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) acc = Pair16<T>::dot2(qv[g].w[j], kv.w[j], acc);
      s[g] = acc;
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = __uint_as_float(qv[g].w[0]) * __uint_as_float(kv.w[0]);
#pragma unroll
      for (int j = 1; j < KW; ++j) acc = fmaf(__uint_as_float(qv[g].w[j]), __uint_as_float(kv.w[j]), acc);
      s[g] = acc;
    }
  }
}

// Decode body.  NW waves share one item of HW = 2^hw_shift KV heads (HW
// divides NW): wave w works head it.kvh + w % HW and takes that head's key
// blocks w / HW, w / HW + NW / HW, ...; the statistics of the waves of one
// head are combined through LDS at the end.  With HW = NW every wave walks the
// item's whole key range for its own head, and the waves together read whole
// [Hkv, D] slot rows of each page at the same time.
// K rows hold D elements, V rows DV (DecodeLayout gives the lane shares).
// smem must hold NW * G * (DV + 3) floats.
// tid: the thread index (threadIdx.x); callers that run several items in a
// loop pass a copy the compiler cannot see through, so that per-lane values
// are recomputed per item instead of being kept live across the loop.
template <typename T, int D, int DV, int G, int NW, int U>
__device__ __forceinline__ void decode_item(const KernelArgs& a, const WorkItem& it, float* smem,
                                            int tid = threadIdx.x, int hw_shift = 0) {
  using Lay = DecodeLayout<T, D, DV>;
  constexpr int LPT = Lay::kLanes;       // lanes per key row
  constexpr int KW = Lay::kKWords;       // 32-bit words of K per lane and key
  constexpr int VW = Lay::kVWords;       // 32-bit words of V per lane and key
  constexpr int EK = Lay::kKElems;       // K elements per lane and key
  constexpr int EV = Lay::kVElems;       // V elements (output dims) per lane
  constexpr int TPW = kWave / LPT;       // keys per wave-wide load
  constexpr int BLK = U * TPW;           // keys per wave per block
  constexpr int SZ = (int)sizeof(T);
  static_assert(U % 2 == 0, "keys are processed in pairs");
  static_assert(NW > 1, "waves combine through LDS");

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hsub = wave & ((1 << hw_shift) - 1);  // this wave's head within the item
  const int kpart = wave >> hw_shift;              // this wave's share of the head's blocks
  const int nparts = NW >> hw_shift;               // waves per head
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int qi = it.q_begin;
  const int kvh = it.kvh + hsub;
  const int tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t krow = (uint64_t)a.hkv * D;   // K elements between consecutive slots
  const uint64_t vrow = (uint64_t)a.hkv * DV;  // V elements between consecutive slots

  // This lane's chunk of the G query rows of the group.
  Words<KW> qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qv[g] = load_words<KW, false>(reinterpret_cast<const char*>(a.q) +
                                  (((uint64_t)qi * a.hq + (uint64_t)kvh * G + g) * D + c * EK) * SZ);

  // l sums the weights as the P.V products used them (rounded to the storage
  // type for 16-bit data) and normalises the output; lx sums the unrounded weights for the
  // logsumexp.
  float m[G], l[G], lx[G], o[G][EV];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    lx[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) o[g][e] = 0.f;
  }

  // Key slot u of a block starting at B: rows take consecutive key pairs.
  auto key_of = [&](int B, int u) { return B + 2 * ((u >> 1) * TPW + r) + (u & 1); };
  // byte addresses of this lane's K and V chunks of key tc in pool page `page`
  auto k_addr = [&](int page, int tc) {
    return reinterpret_cast<const char*>(a.k) +
           (((uint64_t)page * ps + (tc & (ps - 1))) * krow + (uint64_t)kvh * D + c * EK) * SZ;
  };
  auto v_addr = [&](int page, int tc) {
    return reinterpret_cast<const char*>(a.v) +
           (((uint64_t)page * ps + (tc & (ps - 1))) * vrow + (uint64_t)kvh * DV + c * EV) * SZ;
  };

  // Scores, online softmax and P.V of one block held in kr / vr.  Keys
  // outside [tb, te) were loaded from a clamped in-range key (every load stays
  // inside the sequence's referenced pages, no branches) and are masked here.
  auto compute_block = [&](int B, const Words<KW> (&kr)[U], const Words<VW> (&vr)[U]) {
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = key_of(B, u);
      valid[u] = (t >= tb) && (t < te);
    }
    // scores, reduced over the LPT lanes of each row (step-major so that
    // independent DPP operations fill each other's hazard slots)
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) chunk_scores<T, G, KW>(qv, kr[u], s[u]);
    group_sum_all<LPT, U * G>(&s[0][0]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) s[u][g] = valid[u] ? s[u][g] : -INFINITY;

    // Online softmax per row and head against a lazily raised reference max:
    // the reference moves (and the sums are rescaled) only when a block's max
    // exceeds it by more than 2^kDecodeLazyLog2 in weight, which after the
    // first blocks is rare; weights stay <= 2^kDecodeLazyLog2.  Numerator and
    // denominators share the reference, so the result does not depend on it.
    float mx[G];
    bool raise = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mx[g] = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx[g] = fmaxf(mx[g], s[u][g]);
      raise |= mx[g] * a.scale_log2 > m[g] * a.scale_log2 + kDecodeLazyLog2;
    }
    if (__any(raise)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], mx[g]);
        const float alpha = fast_exp2((m[g] - (mn == -INFINITY ? 0.f : mn)) * a.scale_log2);
        m[g] = mn;
        l[g] *= alpha;
        lx[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EV; ++e) o[g][e] *= alpha;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sub = (m[g] == -INFINITY ? 0.f : m[g]) * a.scale_log2;
#pragma unroll
      for (int u = 0; u < U; ++u) s[u][g] = fast_exp2(__builtin_fmaf(s[u][g], a.scale_log2, -sub));
    }

    // P.V
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        uint32_t vp[EV];  // (key u, key u + 1) pairs of each output dim
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          vp[2 * j] = interleave_lo(vr[u].w[j], vr[u + 1].w[j]);
          vp[2 * j + 1] = interleave_hi(vr[u].w[j], vr[u + 1].w[j]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t pp = Pair16<T>::pack(s[u][g], s[u + 1][g]);
          l[g] += Pair16<T>::lo(pp) + Pair16<T>::hi(pp);
          lx[g] += s[u][g] + s[u + 1][g];
#pragma unroll
          for (int e = 0; e < EV; ++e) o[g][e] = Pair16<T>::dot2(vp[e], pp, o[g][e]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          l[g] += s[u][g];
          lx[g] += s[u][g];
#pragma unroll
          for (int e = 0; e < EV; ++e) o[g][e] = fmaf(s[u][g], __uint_as_float(vr[u].w[e]), o[g][e]);
        }
      }
    }
  };

  // Blocks start on multiples of BLK; wave w takes blocks B0 + k * step,
  // B0 = tstart + w * BLK.  When a page holds whole blocks:
  //  - the page numbers of 64 consecutive blocks of the wave are one vector
  //    load, lane k holding block k's (v_readlane hands them out);
  //  - a full block (every key < te) loads from one scalar base per block
  //    plus fixed per-lane offsets, and the next full block is always loaded
  //    before the current one is computed (the last one reloads itself), so
  //    every compute follows the same number of newer loads and the
  //    compiler's wait counts keep one block in flight;
  //  - the wave's last block, if it reaches past te, loads clamped keys
  //    (every load inside the sequence's referenced pages) on its own path.
  // Smaller pages look pages up per lane.
  const int tstart = tb & ~(BLK - 1);
  const int step = nparts * BLK;
  if (ps >= BLK) {
    const int B0 = tstart + kpart * BLK;
    const int nb = B0 < te ? (te - 1 - B0) / step + 1 : 0;           // blocks with B < te
    const int nfull = B0 + BLK <= te ? (te - BLK - B0) / step + 1 : 0;  // blocks with B + BLK <= te
    const uint32_t ks2 = (uint32_t)(krow * SZ), vs2 = (uint32_t)(vrow * SZ);  // bytes between consecutive slots
    const char* kbase = reinterpret_cast<const char*>(a.k) + (uint64_t)kvh * D * SZ;
    const char* vbase = reinterpret_cast<const char*>(a.v) + (uint64_t)kvh * DV * SZ;
    // byte offsets of this lane's chunks of key u, from the block's first slot
    uint32_t klane[U], vlane[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      klane[u] = (uint32_t)(key_of(0, u) * ks2 + c * KW * 4);
      vlane[u] = (uint32_t)(key_of(0, u) * vs2 + c * VW * 4);
    }
    const int last_page = (te - 1) >> a.page_shift;
    for (int w0 = 0; w0 < nb; w0 += kWave) {
      const int pv = bt[min((B0 + (w0 + lane) * step) >> a.page_shift, last_page)];
      // buffer loads: the page base in a scalar resource, the slot row as a
      // scalar offset, this lane's chunk as a fixed vector offset (no per-load
      // address arithmetic, no address registers next to in-flight loads)
      auto load_full = [&](int k, Words<KW> (&kr)[U], Words<VW> (&vr)[U]) {
        const int B = B0 + k * step;
        const uint64_t pg = (uint64_t)__builtin_amdgcn_readlane(pv, k - w0) * ps;
        const uint32_t slot = (uint32_t)(B & (ps - 1));
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + pg * ks2), rv = make_rsrc(vbase + pg * vs2);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          kr[u] = buffer_words<KW>(rk, klane[u], slot * ks2);
          vr[u] = buffer_words<VW>(rv, vlane[u], slot * vs2);
        }
      };
      const int kend = min(nfull, w0 + kWave);  // full blocks of this window: w0 .. kend - 1
      if (w0 < kend) {
        Words<KW> ka[U], kb[U];
        Words<VW> va[U], vb[U];
        load_full(w0, ka, va);
        int k = w0;
        while (true) {
          load_full(min(k + 1, kend - 1), kb, vb);
          __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the block they overlap
          compute_block(B0 + k * step, ka, va);
          if (++k >= kend) break;
          load_full(min(k + 1, kend - 1), ka, va);
          __builtin_amdgcn_sched_barrier(0);
          compute_block(B0 + k * step, kb, vb);
          if (++k >= kend) break;
        }
      }
      if (nfull < nb && nfull < w0 + kWave) {  // the wave's partial last block (k = nfull) is in this window
        const int B = B0 + nfull * step;
        const int page = __builtin_amdgcn_readlane(pv, nfull - w0);  // B and te - 1 share this page
        Words<KW> kr[U];
        Words<VW> vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int tc = min(key_of(B, u), te - 1);
          kr[u] = load_words<KW, true>(k_addr(page, tc));
          vr[u] = load_words<VW, true>(v_addr(page, tc));
        }
        compute_block(B, kr, vr);
      }
    }
  } else {
    for (int B = tstart + kpart * BLK; B < te; B += step) {
      int pg[U];
#pragma unroll
      for (int u = 0; u < U; ++u) pg[u] = bt[min(max(key_of(B, u), tb), te - 1) >> a.page_shift];
      Words<KW> kr[U];
      Words<VW> vr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tc = min(max(key_of(B, u), tb), te - 1);
        kr[u] = load_words<KW, true>(k_addr(pg[u], tc));
        vr[u] = load_words<VW, true>(v_addr(pg[u], tc));
      }
      compute_block(B, kr, vr);
    }
  }

  // combine the TPW rows of this wave (lanes c, c+LPT, c+2LPT, ...)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = column_max<LPT>(m[g]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    const float f = fast_exp2((m[g] - mu) * a.scale_log2);
    m[g] = M;
    l[g] = column_sum<LPT>(l[g] * f);
    lx[g] = column_sum<LPT>(lx[g] * f);
#pragma unroll
    for (int e = 0; e < EV; ++e) o[g][e] = column_sum<LPT>(o[g][e] * f);
  }

  // combine the NW waves through LDS: [wave][g][DV] sums, then [wave][g] (m, l, lx)
  float* so = smem;
  float* sml = smem + NW * G * DV;
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EV; ++e) so[(wave * G + g) * DV + c * EV + e] = o[g][e];
      if (c == 0) {
        sml[(wave * G + g) * 3 + 0] = m[g];
        sml[(wave * G + g) * 3 + 1] = l[g];
        sml[(wave * G + g) * 3 + 2] = lx[g];
      }
    }
  }
  __syncthreads();

  // thread x finalises outputs (head, g, d) = x, x + blockDim, ... of the
  // item's HW heads, combining the waves w = head + j * HW
  for (int idx = tid; idx < (G * DV << hw_shift); idx += NW * kWave) {
    const int hs = idx / (G * DV), g = idx / DV % G, d = idx % DV;
    float M = -INFINITY;
    for (int w = hs; w < NW; w += 1 << hw_shift) M = fmaxf(M, sml[(w * G + g) * 3]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, LX = 0.f, O = 0.f;
    for (int w = hs; w < NW; w += 1 << hw_shift) {
      const float f = fast_exp2((sml[(w * G + g) * 3] - mu) * a.scale_log2);
      L += sml[(w * G + g) * 3 + 1] * f;
      LX += sml[(w * G + g) * 3 + 2] * f;
      O += so[(w * G + g) * DV + d] * f;
    }
    const int h = (it.kvh + hs) * G + g;
    if (it.slot < 0) {
      store_out<T>(a.out, ((uint64_t)qi * a.hq + h) * DV + d, O / L);
      if (a.lse && d == 0) a.lse[(uint64_t)qi * a.hq + h] = M * a.scale + logf(LX);
    } else {
      const uint64_t sl = (uint64_t)(it.slot + hs) * G + g;
      a.ws_o[sl * DV + d] = O;
      if (d == 0) {
        a.ws_ml[sl * 3 + 0] = M * a.scale_log2;
        a.ws_ml[sl * 3 + 1] = L;
        a.ws_ml[sl * 3 + 2] = LX;
      }
    }
  }
}

// Log-sum-exp merge of split partials (ruDNN `attention_into_split`: merge the
// fp32 statistics; the weights are alice-llm `lse_combine`'s): for each head
// of the group, M = max_j m_j, w_j = 2^(m_j - M), out = sum_j w_j o_j / sum_j
// w_j l_j, lse = ln 2 * (M + log2 sum_j w_j l_j).  All loads of a row are
// issued before any arithmetic (up to kMergeUnroll splits at a time).
constexpr int kMergeUnroll = 16;

// The (g, d) outputs of a row are spread over `chunks` workgroups; this one
// takes outputs chunk, chunk + chunks, ... in units of blockDim.
// PARTIAL: the row's last group of G heads may reach past head hq - 1 (MLA
// head groups), whose dims are skipped.
template <typename T, int DV, int G, bool PARTIAL = false>
__device__ __forceinline__ void merge_row(const KernelArgs& a, const MergeItem& mi, int chunk, int chunks) {
  // four consecutive output dims per thread (16-byte partial loads)
  static_assert(DV % 4 == 0, "merge reads four dims at a time");
  for (int idx = chunk * blockDim.x + threadIdx.x; idx < G * DV / 4; idx += chunks * blockDim.x) {
    const int g = (4 * idx) / DV, d = (4 * idx) % DV;
    if (PARTIAL && mi.kvh * G + g >= a.hq) break;  // past the last head
    float M = -INFINITY, L = 0.f, LX = 0.f;
    floatx4_t O = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < mi.nsplit; j0 += kMergeUnroll) {
      float mj[kMergeUnroll], lj[kMergeUnroll], lxj[kMergeUnroll];
      floatx4_t oj[kMergeUnroll];
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int j = j0 + u;
        const uint64_t sl = (uint64_t)(mi.slot + min(j, mi.nsplit - 1) * mi.stride) * G + g;
        mj[u] = a.ws_ml[sl * 3];
        lj[u] = a.ws_ml[sl * 3 + 1];
        lxj[u] = a.ws_ml[sl * 3 + 2];
        oj[u] = *reinterpret_cast<const floatx4_t*>(a.ws_o + sl * DV + d);
        if (j >= mi.nsplit) mj[u] = -INFINITY;
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) Mn = fmaxf(Mn, mj[u]);
      const float f = fast_exp2(M - Mn);  // M = -inf on the first pass: f = 0 and L = O = 0
      L *= f;
      LX *= f;
      O *= f;
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const float w = fast_exp2(mj[u] - Mn);
        L += lj[u] * w;
        LX += lxj[u] * w;
        O += oj[u] * w;
      }
      M = Mn;
    }
    const int h = mi.kvh * G + g;
    const uint64_t o0 = ((uint64_t)mi.q * a.hq + h) * DV + d;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<T>(a.out, o0 + e, O[e] / L);
    if (a.lse && d == 0) a.lse[(uint64_t)mi.q * a.hq + h] = (M + log2f(LX)) * 0.69314718055994530942f;
  }
}

}  // namespace pa
