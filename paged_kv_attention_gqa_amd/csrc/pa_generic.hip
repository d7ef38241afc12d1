// Paged attention forward for the shapes the specialised kernels do not
// take, GQA and absorbed MLA alike:
//   GQA: any group size G = Hq / Hkv (the decode and MFMA kernels are built
//        for 1-8, 12 and 16), any head sizes D, Dv <= 1024 (they are built for
//        64, 128, 256 and 192 / 128);
//   MLA: f32 data, any latent rank R <= 1024 and rotary width P <= 256 (the
//        MFMA kernel takes 16-bit R = 512, P = 64).
//
// Definitions followed: ruDNN 0.1.107 paged_attention/mod.rs
// `execute_attention_into` (GQA head map: query head h reads KV head
// h / G) and `DevicePlan::mla` (one shared latent head is key and value, a
// rotated position cache adds q_rope . kpos to every score), with the
// masking and softmax of boostr 0.2.0-beta.2 `standard_attention_fwd` /
// `build_attention_mask`.  One description covers both: the key row is
// [k1 | k2] (GQA: the K row and nothing; MLA: latent | kpos), the query row
// [q1 | q2], and the value row is the V row (MLA: k1 itself).
//
// The plans and work lists are the specialised kernels': an item is one
// work unit (a KV head with its G <= 16 query heads, or a group of up to 16
// of them when G > 16 or for MLA) of one query or a chunk of queries over
// one key range; decode items may cover hw consecutive units.  Split rows
// leave the same partials (unit_heads heads per slot, max in log2 units,
// sums) for the merge below.
//
// Vector ALU in fp32, one 256-thread workgroup per item at a time.  The
// unit's query rows are converted to f32 in LDS; keys come in tiles of 8 key
// and value rows (f32 in LDS).  Two threads score one (key, head) pair, each
// over half of the key dims, and add through a lane exchange; then the 16
// threads of a head each own the output dims d = their index mod 16 and
// update them with the tile's 8 weights against a running max (online
// softmax in log2 units).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kGenThreads = 256;
constexpr int kGenHeads = kGenericUnitHeads;                         // 16 head slots per workgroup
constexpr int kGenKeys = 8;                                          // keys per tile
constexpr int kGenThreadsPerHead = kGenThreads / kGenHeads;          // 16
constexpr int kGenMaxKey = kGenericMaxKeyWidth;                      // 1280 (MLA 1024 + 256)
constexpr int kGenMaxV = kGenericMaxValueWidth;                      // 1024
constexpr int kGenDimsPerThread = kGenMaxV / kGenThreadsPerHead;     // 64
static_assert(kGenThreads == 2 * kGenKeys * kGenHeads, "two threads per (key, head) score");

template <typename T>
__device__ __forceinline__ float load_f(const void* p, uint64_t i) {
  if constexpr (__is_same(T, float))
    return reinterpret_cast<const float*>(p)[i];
  else if constexpr (__is_same(T, _Float16))
    return (float)reinterpret_cast<const _Float16*>(p)[i];
  else
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}

template <typename T>
__device__ __forceinline__ void store_f(void* p, uint64_t i, float v) {
  if constexpr (__is_same(T, float))
    reinterpret_cast<float*>(p)[i] = v;
  else
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(Pair16<T>::pack(v, 0.f) & 0xFFFFu);
}

// First query head and head count of work unit u.
__device__ __forceinline__ void unit_heads_of(const GenericShape& s, int u, int* h0, int* nh) {
  const int kv = u / s.nsub, sub = u - kv * s.nsub;
  *h0 = kv * s.g + sub * s.unit_heads;
  *nh = min(s.unit_heads, s.g - sub * s.unit_heads);
}

template <typename T>
__global__ __launch_bounds__(kGenThreads) void generic_kernel(KernelArgs a, GenericShape s) {
  __shared__ float q_s[kGenHeads * kGenMaxKey];  // the unit's query rows [q1 | q2], f32
  __shared__ float k_s[kGenKeys * kGenMaxKey];   // one tile of key rows [k1 | k2], f32
  __shared__ float v_s[kGenKeys * kGenMaxV];     // its value rows (unused when V is k1)
  __shared__ float s_s[kGenKeys * kGenHeads];    // the tile's scores in log2 units (-inf: masked)
  const int W = s.d1 + s.d2, DV = s.dv;
  const float* vt = s.v_is_k ? k_s : v_s;
  const int vstride = s.v_is_k ? W : DV;
  const int tid = threadIdx.x;
  const int ps = 1 << a.page_shift;
  const int oh = tid / kGenThreadsPerHead, od = tid % kGenThreadsPerHead;  // output head slot, dim phase
  const int first = a.wg_first[blockIdx.x], last = a.wg_first[blockIdx.x + 1];
  for (int i = first; i < last; ++i) {
    const WorkItem it = a.items[i];
    if (it.kind == kEmpty) continue;
    const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
    for (int j = 0; j < s.hw; ++j) {  // units of a decode item (hw = 1 otherwise)
      const int u = it.kvh + j;
      if (u >= a.hkv * s.nsub) break;  // a unit past the last (an odd number of MLA head groups)
      const int kv = u / s.nsub;
      int h0, nh;
      unit_heads_of(s, u, &h0, &nh);
      for (int qi = it.q_begin; qi < it.q_begin + it.q_count; ++qi) {
        const int qpos = a.q_pos[qi];
        __syncthreads();  // the previous query's reads of q_s, k_s and v_s are done
        // head slots past the unit's heads repeat its last one; their outputs are not stored
        for (int idx = tid; idx < kGenHeads * W; idx += kGenThreads) {
          const int h = idx / W, d = idx - h * W;
          const uint64_t row = (uint64_t)qi * a.hq + h0 + min(h, nh - 1);
          q_s[idx] = d < s.d1 ? load_f<T>(a.q, row * s.d1 + d) : load_f<T>(a.qr, row * s.d2 + (d - s.d1));
        }
        float o[kGenDimsPerThread];
#pragma unroll
        for (int k = 0; k < kGenDimsPerThread; ++k) o[k] = 0.f;
        float m = -INFINITY, l = 0.f;
        for (int t0 = it.tok_begin; t0 < it.tok_end; t0 += kGenKeys) {
          __syncthreads();  // the previous tile is consumed (and the query rows are written)
          for (int idx = tid; idx < kGenKeys * W; idx += kGenThreads) {
            const int k = idx / W, d = idx - k * W;
            const int t = min(t0 + k, it.tok_end - 1);  // keys past the range are masked below
            const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
            k_s[idx] = d < s.d1 ? load_f<T>(a.k, (slot * a.hkv + kv) * s.d1 + d)
                                : load_f<T>(a.kr, slot * s.d2 + (d - s.d1));
          }
          if (!s.v_is_k) {
            for (int idx = tid; idx < kGenKeys * DV; idx += kGenThreads) {
              const int k = idx / DV, d = idx - k * DV;
              const int t = min(t0 + k, it.tok_end - 1);
              const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
              v_s[idx] = load_f<T>(a.v, (slot * a.hkv + kv) * DV + d);
            }
          }
          __syncthreads();
          {
            const int pair = tid >> 1, half = tid & 1;
            const int sk = pair / kGenHeads, sh = pair % kGenHeads;
            const float* qrow = q_s + sh * W;
            const float* krow = k_s + sk * W;
            float acc = 0.f;
            for (int d = half; d < W; d += 2) acc = __builtin_fmaf(qrow[d], krow[d], acc);
            acc += __shfl_xor(acc, 1);
            const int t = t0 + sk;
            const bool vis = t < it.tok_end && (!a.causal || t <= qpos) && (a.window == 0 || t > qpos - a.window);
            if (half == 0) s_s[sk * kGenHeads + sh] = vis ? acc * a.scale_log2 : -INFINITY;
          }
          __syncthreads();
          float mx = -INFINITY;
#pragma unroll
          for (int k = 0; k < kGenKeys; ++k) mx = fmaxf(mx, s_s[k * kGenHeads + oh]);
          if (mx > m) {
            const float alpha = fast_exp2(m - mx);  // 0 while m is -inf
            l *= alpha;
#pragma unroll
            for (int k = 0; k < kGenDimsPerThread; ++k) o[k] *= alpha;
            m = mx;
          }
          float p[kGenKeys];
#pragma unroll
          for (int k = 0; k < kGenKeys; ++k) {
            p[k] = m == -INFINITY ? 0.f : fast_exp2(s_s[k * kGenHeads + oh] - m);
            l += p[k];
          }
#pragma unroll
          for (int k = 0; k < kGenDimsPerThread; ++k) {
            const int d = od + kGenThreadsPerHead * k;
            if (d < DV) {
              float acc = o[k];
#pragma unroll
              for (int e = 0; e < kGenKeys; ++e) acc = __builtin_fmaf(p[e], vt[e * vstride + d], acc);
              o[k] = acc;
            }
          }
        }
        if (oh >= nh) continue;
        if (it.slot < 0) {
          const uint64_t row = (uint64_t)qi * a.hq + h0 + oh;
          const float inv = 1.f / l;
#pragma unroll
          for (int k = 0; k < kGenDimsPerThread; ++k) {
            const int d = od + kGenThreadsPerHead * k;
            if (d < DV) store_f<T>(a.out, row * DV + d, o[k] * inv);
          }
          if (a.lse && od == 0) a.lse[row] = (m + log2f(l)) * 0.69314718055994530942f;
        } else {
          const uint64_t srow = (uint64_t)(it.slot + j) * s.unit_heads + oh;
#pragma unroll
          for (int k = 0; k < kGenDimsPerThread; ++k) {
            const int d = od + kGenThreadsPerHead * k;
            if (d < DV) a.ws_o[srow * DV + d] = o[k];
          }
          if (od == 0) {
            a.ws_ml[srow * 3 + 0] = m;
            a.ws_ml[srow * 3 + 1] = l;
            a.ws_ml[srow * 3 + 2] = l;
          }
        }
      }
    }
  }
}

// Log-sum-exp merge of the split rows (one merge record per (query, work
// unit)); the unit's output dims spread over the grid's y range.
template <typename T>
__global__ __launch_bounds__(kGenThreads) void generic_merge_kernel(KernelArgs a, const MergeItem* merges,
                                                                   GenericShape s) {
  const MergeItem mi = merges[blockIdx.x];
  int h0, nh;
  unit_heads_of(s, mi.kvh, &h0, &nh);
  for (int idx = blockIdx.y * kGenThreads + threadIdx.x; idx < nh * s.dv; idx += gridDim.y * kGenThreads) {
    const int g = idx / s.dv, d = idx - g * s.dv;
    float M = -INFINITY;
    for (int j = 0; j < mi.nsplit; ++j)
      M = fmaxf(M, a.ws_ml[((uint64_t)(mi.slot + j * mi.stride) * s.unit_heads + g) * 3]);
    float L = 0.f, LX = 0.f, O = 0.f;
    for (int j = 0; j < mi.nsplit; ++j) {
      const uint64_t sl = (uint64_t)(mi.slot + j * mi.stride) * s.unit_heads + g;
      const float w = fast_exp2(a.ws_ml[sl * 3] - M);
      L += a.ws_ml[sl * 3 + 1] * w;
      LX += a.ws_ml[sl * 3 + 2] * w;
      O += a.ws_o[sl * s.dv + d] * w;
    }
    const uint64_t row = (uint64_t)mi.q * a.hq + h0 + g;
    store_f<T>(a.out, row * s.dv + d, O / L);
    if (a.lse && d == 0) a.lse[row] = (M + log2f(LX)) * 0.69314718055994530942f;
  }
}

template <typename T>
hipError_t launch_t(const KernelArgs& a, const GenericShape& s, const MainEvents& ev, hipStream_t stream) {
  if (a.n_wg <= 0) return hipSuccess;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(generic_kernel<T>, dim3(a.n_wg), dim3(kGenThreads), 0, stream, ev.start, ev.stop, 0, a, s);
  else
    hipLaunchKernelGGL(generic_kernel<T>, dim3(a.n_wg), dim3(kGenThreads), 0, stream, a, s);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_merge_t(const KernelArgs& a, const GenericShape& s, const MergeItem* merges, int n_merges,
                          hipStream_t stream) {
  if (n_merges <= 0) return hipSuccess;
  const int chunks = (s.unit_heads * s.dv + kGenThreads - 1) / kGenThreads;
  hipLaunchKernelGGL(generic_merge_kernel<T>, dim3(n_merges, chunks), dim3(kGenThreads), 0, stream, a, merges, s);
  return hipGetLastError();
}

}  // namespace

bool generic_shape_ok(const GenericShape& s) {
  return s.d1 >= 1 && s.d2 >= 0 && s.d1 + s.d2 <= kGenMaxKey && s.dv >= 1 && s.dv <= kGenMaxV &&
         (!s.v_is_k || s.dv <= s.d1) && s.g >= 1 && s.nsub >= 1 && s.unit_heads >= 1 &&
         s.unit_heads <= kGenHeads && s.unit_heads * s.nsub >= s.g && s.hw >= 1;
}

hipError_t launch_generic(int dtype, const GenericShape& s, const KernelArgs& a, const MainEvents& ev,
                          hipStream_t stream) {
  if (!generic_shape_ok(s)) return hipErrorInvalidValue;
  if (dtype == 0) return launch_t<float>(a, s, ev, stream);
  if (dtype == 1) return launch_t<uint16_t>(a, s, ev, stream);
  if (dtype == 2) return launch_t<_Float16>(a, s, ev, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_generic_merge(int dtype, const GenericShape& s, const KernelArgs& a, const MergeItem* merges,
                                int n_merges, hipStream_t stream) {
  if (!generic_shape_ok(s)) return hipErrorInvalidValue;
  if (dtype == 0) return launch_merge_t<float>(a, s, merges, n_merges, stream);
  if (dtype == 1) return launch_merge_t<uint16_t>(a, s, merges, n_merges, stream);
  if (dtype == 2) return launch_merge_t<_Float16>(a, s, merges, n_merges, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
