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

template <typename T>
struct Vec16;  // one 16-byte load
template <>
struct Vec16<float> {
  static constexpr int kElems = 4;
};
template <>
struct Vec16<uint16_t> {
  static constexpr int kElems = 8;
};

__device__ __forceinline__ uint4 load16(const void* base, uint64_t elem_off, int esize) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + elem_off * esize);
}

// Scores of G heads against one key chunk held by this lane.
template <typename T, int G>
__device__ __forceinline__ void chunk_scores(const uint4 (&qv)[G], const uint4& kv, float (&s)[G]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
      acc = dot2_bf16(qv[g].x, kv.x, acc);
      acc = dot2_bf16(qv[g].y, kv.y, acc);
      acc = dot2_bf16(qv[g].z, kv.z, acc);
      acc = dot2_bf16(qv[g].w, kv.w, acc);
      s[g] = acc;
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = __uint_as_float(qv[g].x) * __uint_as_float(kv.x);
      acc = fmaf(__uint_as_float(qv[g].y), __uint_as_float(kv.y), acc);
      acc = fmaf(__uint_as_float(qv[g].z), __uint_as_float(kv.z), acc);
      acc = fmaf(__uint_as_float(qv[g].w), __uint_as_float(kv.w), acc);
      s[g] = acc;
    }
  }
}

// Decode body.  NW waves share one item: wave w takes key blocks w, w+NW, ...
// and the waves' statistics are combined through LDS at the end.
// smem must hold NW * G * (EPV * LPT + 2) floats.
template <typename T, int D, int G, int NW, int U>
__device__ __forceinline__ void decode_item(const KernelArgs& a, const WorkItem& it, float* smem) {
  constexpr int EPV = Vec16<T>::kElems;  // elements per 16-byte chunk
  constexpr int LPT = D / EPV;           // lanes per key row
  constexpr int TPW = kWave / LPT;       // keys per wave-wide load
  constexpr int BLK = U * TPW;           // keys per wave per block
  static_assert(D % EPV == 0 && LPT <= kWave && kWave % LPT == 0, "unsupported head size");
  static_assert(U % 2 == 0, "keys are processed in pairs");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int qi = it.q_begin;
  const int kvh = it.kvh;
  const int tb = it.tok_begin, te = it.tok_end;
  const int ps = 1 << a.page_shift;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
  const uint64_t row_stride = (uint64_t)a.hkv * D;  // elements between consecutive slots

  // This lane's chunk of the G query rows of the group.
  uint4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qv[g] = load16(a.q, ((uint64_t)qi * a.hq + (uint64_t)kvh * G + g) * D + c * EPV, sizeof(T));

  float m[G], l[G], o[G][EPV];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[g][e] = 0.f;
  }

  const int t0 = tb & ~1;  // pairs start on even positions
  for (int B = t0 + wave * BLK; B < te; B += NW * BLK) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = B + 2 * ((u >> 1) * TPW + r) + (u & 1);
      valid[u] = (t >= tb) && (t < te);
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (valid[u]) {
        const int page = bt[t >> a.page_shift];
        const uint64_t off = ((uint64_t)page * ps + (t & (ps - 1))) * row_stride + (uint64_t)kvh * D + c * EPV;
        kr[u] = load16(a.k, off, sizeof(T));
        vr[u] = load16(a.v, off, sizeof(T));
      }
    }

    // scores, reduced over the LPT lanes of each row
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      chunk_scores<T, G>(qv, kr[u], s[u]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s[u][g] = group_sum<LPT>(s[u][g]);
        s[u][g] = valid[u] ? s[u][g] : -INFINITY;
      }
    }

    // online softmax per row and head, one rescale per block
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][g]);
      const float mu = (mx == -INFINITY) ? 0.f : mx;
      const float alpha = exp2f((m[g] - mu) * a.scale_log2);
      m[g] = mx;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPV; ++e) o[g][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) s[u][g] = exp2f((s[u][g] - mu) * a.scale_log2);
    }

    // P.V
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const uint32_t v0[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
        const uint32_t v1[4] = {vr[u + 1].x, vr[u + 1].y, vr[u + 1].z, vr[u + 1].w};
        uint32_t vp[EPV];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vp[2 * j] = interleave_lo(v0[j], v1[j]);
          vp[2 * j + 1] = interleave_hi(v0[j], v1[j]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t pp = pack_bf16(s[u][g], s[u + 1][g]);
          l[g] += bf16_lo(pp) + bf16_hi(pp);
#pragma unroll
          for (int e = 0; e < EPV; ++e) o[g][e] = dot2_bf16(vp[e], pp, o[g][e]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float vf[4] = {__uint_as_float(vr[u].x), __uint_as_float(vr[u].y), __uint_as_float(vr[u].z),
                             __uint_as_float(vr[u].w)};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          l[g] += s[u][g];
#pragma unroll
          for (int e = 0; e < EPV; ++e) o[g][e] = fmaf(s[u][g], vf[e], o[g][e]);
        }
      }
    }
  }

  // combine the TPW rows of this wave (lanes c, c+LPT, c+2LPT, ...)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = column_max<LPT>(m[g]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    const float f = exp2f((m[g] - mu) * a.scale_log2);
    m[g] = M;
    l[g] = column_sum<LPT>(l[g] * f);
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[g][e] = column_sum<LPT>(o[g][e] * f);
  }

  // combine the NW waves through LDS: [wave][g][D] sums, then [wave][g] (m, l)
  float* so = smem;
  float* sml = smem + NW * G * D;
  if (NW > 1) {
    if (r == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) so[(wave * G + g) * D + c * EPV + e] = o[g][e];
        if (c == 0) {
          sml[(wave * G + g) * 2 + 0] = m[g];
          sml[(wave * G + g) * 2 + 1] = l[g];
        }
      }
    }
    __syncthreads();
  }

  // final: thread x handles (g, d) outputs x, x + blockDim, ...
  const int nthreads = NW * kWave;
  for (int idx = threadIdx.x; idx < G * D; idx += nthreads) {
    const int g = idx / D, d = idx % D;
    float M, L, O;
    if (NW > 1) {
      M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sml[(w * G + g) * 2]);
      const float mu = (M == -INFINITY) ? 0.f : M;
      L = 0.f;
      O = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f((sml[(w * G + g) * 2] - mu) * a.scale_log2);
        L += sml[(w * G + g) * 2 + 1] * f;
        O += so[(w * G + g) * D + d] * f;
      }
    } else {
      // single wave: lane (0, c) holds dims c*EPV .. c*EPV+EPV-1 of every head
      M = 0.f; L = 0.f; O = 0.f;  // filled below
    }
    if (NW > 1) {
      const int h = kvh * G + g;
      if (it.slot < 0) {
        const float val = O / L;
        if constexpr (sizeof(T) == 2) {
          reinterpret_cast<uint16_t*>(a.out)[((uint64_t)qi * a.hq + h) * D + d] =
              (uint16_t)(pack_bf16(val, 0.f) & 0xFFFFu);
        } else {
          reinterpret_cast<float*>(a.out)[((uint64_t)qi * a.hq + h) * D + d] = val;
        }
        if (a.lse && d == 0) a.lse[(uint64_t)qi * a.hq + h] = M * a.scale + logf(L);
      } else {
        a.ws_o[((uint64_t)it.slot * G + g) * D + d] = O;
        if (d == 0) {
          a.ws_ml[((uint64_t)it.slot * G + g) * 2 + 0] = M * a.scale_log2;
          a.ws_ml[((uint64_t)it.slot * G + g) * 2 + 1] = L;
        }
      }
    }
  }
  if (NW == 1 && r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int h = kvh * G + g;
      if (it.slot < 0) {
        const float inv = 1.f / l[g];
        if constexpr (sizeof(T) == 2) {
          uint4 w;
          w.x = pack_bf16(o[g][0] * inv, o[g][1] * inv);
          w.y = pack_bf16(o[g][2] * inv, o[g][3] * inv);
          w.z = pack_bf16(o[g][4] * inv, o[g][5] * inv);
          w.w = pack_bf16(o[g][6] * inv, o[g][7] * inv);
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + ((uint64_t)qi * a.hq + h) * D + c * EPV) = w;
        } else {
          float4 w = make_float4(o[g][0] * inv, o[g][1] * inv, o[g][2] * inv, o[g][3] * inv);
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + ((uint64_t)qi * a.hq + h) * D + c * EPV) = w;
        }
        if (a.lse && c == 0) a.lse[(uint64_t)qi * a.hq + h] = m[g] * a.scale + logf(l[g]);
      } else {
        float* dst = a.ws_o + ((uint64_t)it.slot * G + g) * D + c * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) dst[e] = o[g][e];
        if (c == 0) {
          a.ws_ml[((uint64_t)it.slot * G + g) * 2 + 0] = m[g] * a.scale_log2;
          a.ws_ml[((uint64_t)it.slot * G + g) * 2 + 1] = l[g];
        }
      }
    }
  }
}

// Log-sum-exp merge of split partials (ruDNN `attention_into_split`: merge the
// fp32 statistics; the weights are alice-llm `lse_combine`'s): for each head
// of the group, M = max_j m_j, w_j = 2^(m_j - M), out = sum_j w_j o_j / sum_j
// w_j l_j, lse = ln 2 * (M + log2 sum_j w_j l_j).
template <typename T, int D, int G>
__device__ __forceinline__ void merge_row(const KernelArgs& a, const MergeItem& mi) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int j = 0; j < mi.nsplit; ++j) M = fmaxf(M, a.ws_ml[((uint64_t)(mi.slot + j) * G + g) * 2]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
    for (int j = 0; j < mi.nsplit; ++j) {
      const uint64_t sl = (uint64_t)(mi.slot + j) * G + g;
      const float w = exp2f(a.ws_ml[sl * 2] - mu);
      L += a.ws_ml[sl * 2 + 1] * w;
      O += a.ws_o[sl * D + d] * w;
    }
    const int h = mi.kvh * G + g;
    const float val = O / L;
    if constexpr (sizeof(T) == 2) {
      reinterpret_cast<uint16_t*>(a.out)[((uint64_t)mi.q * a.hq + h) * D + d] = (uint16_t)(pack_bf16(val, 0.f) & 0xFFFFu);
    } else {
      reinterpret_cast<float*>(a.out)[((uint64_t)mi.q * a.hq + h) * D + d] = val;
    }
    if (a.lse && d == 0) a.lse[(uint64_t)mi.q * a.hq + h] = (M + log2f(L)) * 0.69314718055994530942f;
  }
}

}  // namespace pa
