// Absorbed-MLA forward for the shapes the MFMA kernel does not take: f32
// data, latent ranks other than 512 and rotary widths other than 64 (rank
// up to 1024, rotary width up to 256), with any head count.
//
// Definition followed: ruDNN 0.1.107 paged_attention/mod.rs `DevicePlan::mla`
// (one shared latent head [pages, page_size, 1, R] is key and value, a
// rotated position cache [pages, page_size, 1, P] adds q_rope . kpos to every
// score, scale from the model's original query/key size), with the masking
// and softmax of boostr 0.2.0-beta.2 `standard_attention_fwd` /
// `build_attention_mask`.  The work list is the MFMA kernel's: an item is one
// group of 16 heads of one query (decode) or of up to two queries (chunked
// prefill) over one key range, and split rows leave the same partials
// (16 heads per slot, max in log2 units, sums) for the merge below.
//
// Vector ALU in fp32, one 256-thread workgroup per item at a time.  The
// group's 16 query rows [q_abs | q_rope] are converted to f32 in LDS; keys
// come in tiles of 8 latent + rotary rows (f32 in LDS).  Two threads score
// one (key, head) pair, each over half of the R + P dims, and sum through a
// lane exchange; then the 16 threads of a head each own the output dims
// j = their index mod 16 and update them with the tile's 8 weights against
// a running max (online softmax in log2 units).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kGenThreads = 256;
constexpr int kGenHeads = kMlaGroupHeads;
constexpr int kGenKeys = 8;
constexpr int kGenThreadsPerHead = kGenThreads / kGenHeads;            // 16
constexpr int kGenMaxWidth = kMlaMaxRank + kMlaMaxRope;                // 1280
constexpr int kGenDimsPerThread = kMlaMaxRank / kGenThreadsPerHead;    // 64
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

template <typename T>
__global__ __launch_bounds__(kGenThreads) void mla_generic_kernel(KernelArgs a, int R, int P) {
  __shared__ float q_s[kGenHeads * kGenMaxWidth];  // the group's query rows, f32
  __shared__ float k_s[kGenKeys * kGenMaxWidth];   // one tile of latent | rotary rows, f32
  __shared__ float s_s[kGenKeys * kGenHeads];      // the tile's scores in log2 units (-inf: masked)
  const int W = R + P;
  const int tid = threadIdx.x;
  const int ps = 1 << a.page_shift;
  const int oh = tid / kGenThreadsPerHead, od = tid % kGenThreadsPerHead;  // output head and dim phase
  const int first = a.wg_first[blockIdx.x], last = a.wg_first[blockIdx.x + 1];
  for (int i = first; i < last; ++i) {
    const WorkItem it = a.items[i];
    if (it.kind == kEmpty) continue;
    const int32_t* bt = a.block_table + (size_t)it.seq * a.table_width;
    const int g0 = kGenHeads * it.kvh;         // first head of the group
    const int nh = min(kGenHeads, a.hq - g0);  // its heads (the last group may be partial)
    for (int qi = it.q_begin; qi < it.q_begin + it.q_count; ++qi) {
      const int qpos = a.q_pos[qi];
      __syncthreads();  // the previous query's reads of q_s and k_s are done
      // rows past the last head repeat it; their outputs are not stored
      for (int idx = tid; idx < kGenHeads * W; idx += kGenThreads) {
        const int h = idx / W, d = idx - h * W;
        const uint64_t row = (uint64_t)qi * a.hq + g0 + min(h, nh - 1);
        q_s[idx] = d < R ? load_f<T>(a.q, row * R + d) : load_f<T>(a.qr, row * P + (d - R));
      }
      float o[kGenDimsPerThread];
#pragma unroll
      for (int j = 0; j < kGenDimsPerThread; ++j) o[j] = 0.f;
      float m = -INFINITY, l = 0.f;
      for (int t0 = it.tok_begin; t0 < it.tok_end; t0 += kGenKeys) {
        __syncthreads();  // the previous tile is consumed (and the query rows are written)
        for (int idx = tid; idx < kGenKeys * W; idx += kGenThreads) {
          const int k = idx / W, d = idx - k * W;
          const int t = min(t0 + k, it.tok_end - 1);  // keys past the range are masked below
          const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
          k_s[idx] = d < R ? load_f<T>(a.k, slot * R + d) : load_f<T>(a.kr, slot * P + (d - R));
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
          for (int j = 0; j < kGenDimsPerThread; ++j) o[j] *= alpha;
          m = mx;
        }
        float p[kGenKeys];
#pragma unroll
        for (int k = 0; k < kGenKeys; ++k) {
          p[k] = m == -INFINITY ? 0.f : fast_exp2(s_s[k * kGenHeads + oh] - m);
          l += p[k];
        }
#pragma unroll
        for (int j = 0; j < kGenDimsPerThread; ++j) {
          const int d = od + kGenThreadsPerHead * j;
          if (d < R) {
            float acc = o[j];
#pragma unroll
            for (int k = 0; k < kGenKeys; ++k) acc = __builtin_fmaf(p[k], k_s[k * W + d], acc);
            o[j] = acc;
          }
        }
      }
      if (it.slot < 0) {
        if (oh < nh) {
          const uint64_t row = (uint64_t)qi * a.hq + g0 + oh;
          const float inv = 1.f / l;
#pragma unroll
          for (int j = 0; j < kGenDimsPerThread; ++j) {
            const int d = od + kGenThreadsPerHead * j;
            if (d < R) store_f<T>(a.out, row * R + d, o[j] * inv);
          }
          if (a.lse && od == 0) a.lse[row] = (m + log2f(l)) * 0.69314718055994530942f;
        }
      } else {
        const uint64_t srow = (uint64_t)it.slot * kGenHeads + oh;
#pragma unroll
        for (int j = 0; j < kGenDimsPerThread; ++j) {
          const int d = od + kGenThreadsPerHead * j;
          if (d < R) a.ws_o[srow * R + d] = o[j];
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

// Log-sum-exp merge of the split rows (one merge record per (query, head
// group)); output dims of the group's heads spread over the grid's y range.
template <typename T>
__global__ __launch_bounds__(kGenThreads) void mla_generic_merge_kernel(KernelArgs a, const MergeItem* merges, int R) {
  const MergeItem mi = merges[blockIdx.x];
  for (int idx = blockIdx.y * kGenThreads + threadIdx.x; idx < kGenHeads * R; idx += gridDim.y * kGenThreads) {
    const int g = idx / R, d = idx - g * R;
    const int h = mi.kvh * kGenHeads + g;
    if (h >= a.hq) break;  // past the last head of a partial group
    float M = -INFINITY;
    for (int j = 0; j < mi.nsplit; ++j) M = fmaxf(M, a.ws_ml[((uint64_t)(mi.slot + j * mi.stride) * kGenHeads + g) * 3]);
    float L = 0.f, LX = 0.f, O = 0.f;
    for (int j = 0; j < mi.nsplit; ++j) {
      const uint64_t sl = (uint64_t)(mi.slot + j * mi.stride) * kGenHeads + g;
      const float w = fast_exp2(a.ws_ml[sl * 3] - M);
      L += a.ws_ml[sl * 3 + 1] * w;
      LX += a.ws_ml[sl * 3 + 2] * w;
      O += a.ws_o[sl * R + d] * w;
    }
    const uint64_t row = (uint64_t)mi.q * a.hq + h;
    store_f<T>(a.out, row * R + d, O / L);
    if (a.lse && d == 0) a.lse[row] = (M + log2f(LX)) * 0.69314718055994530942f;
  }
}

template <typename T>
hipError_t launch_generic_t(const KernelArgs& a, int R, int P, const MainEvents& ev, hipStream_t stream) {
  if (a.n_wg <= 0) return hipSuccess;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(mla_generic_kernel<T>, dim3(a.n_wg), dim3(kGenThreads), 0, stream, ev.start, ev.stop, 0,
                          a, R, P);
  else
    hipLaunchKernelGGL(mla_generic_kernel<T>, dim3(a.n_wg), dim3(kGenThreads), 0, stream, a, R, P);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_generic_merge_t(const KernelArgs& a, const MergeItem* merges, int n_merges, int R,
                                  hipStream_t stream) {
  if (n_merges <= 0) return hipSuccess;
  const int chunks = (kGenHeads * R + kGenThreads - 1) / kGenThreads;
  hipLaunchKernelGGL(mla_generic_merge_kernel<T>, dim3(n_merges, chunks), dim3(kGenThreads), 0, stream, a, merges,
                     R);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_generic(int dtype, int r, int p, const KernelArgs& a, const MainEvents& ev,
                              hipStream_t stream) {
  if (r < 1 || r > kMlaMaxRank || p < 1 || p > kMlaMaxRope) return hipErrorInvalidValue;
  if (dtype == 0) return launch_generic_t<float>(a, r, p, ev, stream);
  if (dtype == 1) return launch_generic_t<uint16_t>(a, r, p, ev, stream);
  if (dtype == 2) return launch_generic_t<_Float16>(a, r, p, ev, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mla_generic_merge(int dtype, int r, const KernelArgs& a, const MergeItem* merges, int n_merges,
                                    hipStream_t stream) {
  if (r < 1 || r > kMlaMaxRank) return hipErrorInvalidValue;
  if (dtype == 0) return launch_generic_merge_t<float>(a, merges, n_merges, r, stream);
  if (dtype == 1) return launch_generic_merge_t<uint16_t>(a, merges, n_merges, r, stream);
  if (dtype == 2) return launch_generic_merge_t<_Float16>(a, merges, n_merges, r, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
