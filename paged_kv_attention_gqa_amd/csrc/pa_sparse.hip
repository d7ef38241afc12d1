// Block-sparse top-k selection on the GPU (alice-llm 2.0.0,
// sparse_attention/llama3_bridge.rs, `llama3_sparse_attention`): for every
// (query, KV head) row, score each block of block_size consecutive key
// positions by the largest dot product between the group's first query head
// and the block's visible keys (`compute_proxy_block_max_scores`), keep the
// topk best blocks (`sparse_topk_select_batch`), and write one decode work
// item per kept block plus one merge record per row, so that the split-KV
// decode kernel computes a partial per block and the log-sum-exp merge
// combines them (`kvouter_forward` + `lse_combine`).
//
// The proxy score of a key is the f32 product sum in increasing dimension
// order, one fused multiply-add per dimension (for 16-bit data the products
// are exact in f32), so that the choice is reproducible bit for bit; a tie
// goes to the lower block index.  The selection runs once per row and reads
// only K; it is not on the dense path.
#include <hip/hip_runtime.h>

#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kSelThreads = 256;

// Order-preserving map of a float onto an unsigned key (larger float,
// larger key; -inf maps above 0, which marks a block already taken).
__device__ __forceinline__ uint32_t ordered(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ float widen(const T* p, int i) {
  if constexpr (sizeof(T) == 4) {
    return reinterpret_cast<const float*>(p)[i];
  } else {
    const uint16_t u = reinterpret_cast<const uint16_t*>(p)[i];
    return Pair16<T>::lo((uint32_t)u);
  }
}

// Largest 64-bit key of the workgroup (every thread receives it).
__device__ __forceinline__ uint64_t wg_max(uint64_t v, uint64_t* red) {
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, s), hi = __shfl_xor((uint32_t)(v >> 32), s);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  const int wave = threadIdx.x / kWave;
  __syncthreads();  // the previous round's readers are done with red
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
  __syncthreads();
  uint64_t m = red[0];
  for (int w = 1; w < kSelThreads / kWave; ++w) m = red[w] > m ? red[w] : m;
  return m;
}

template <typename T>
__global__ __launch_bounds__(kSelThreads) void sparse_select_kernel(SparseArgs a) {
  __shared__ uint32_t score[kSparseMaxBlocks];
  __shared__ float qp[kSparseMaxDim];
  __shared__ uint64_t red[kSelThreads / kWave];
  __shared__ int32_t wave_count[kSelThreads / kWave];

  const int row = blockIdx.x;  // query * hkv + KV head
  const int i = row / a.hkv, h = row % a.hkv;
  const int s = a.seq_of[i];
  const int L = a.seq_lens[s], p = a.q_pos[i];
  const int hi = a.causal ? p : L - 1;
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int B = a.block_size;
  const int r0 = lo / B, ncand = hi / B - r0 + 1;
  const bool all = a.topk == 0 || a.topk >= ncand;
  const int keep = all ? ncand : a.topk;
  const int tid = threadIdx.x;

  if (!all) {
    // proxy query: the first query head of the group, widened to f32
    const T* q = reinterpret_cast<const T*>(a.q) + ((uint64_t)i * a.hq + (uint64_t)h * (a.hq / a.hkv)) * a.d;
    for (int c = tid; c < a.d; c += kSelThreads) qp[c] = widen(q, c);
    for (int r = tid; r < ncand; r += kSelThreads) score[r] = ordered(-INFINITY);
    __syncthreads();
    // one thread per visible key: the sequential f32 product sum, then the
    // block maximum by an order-preserving atomic max
    const int32_t* bt = a.block_table + (size_t)s * a.table_width;
    const int ps = 1 << a.page_shift;
    for (int t = lo + tid; t <= hi; t += kSelThreads) {
      const uint64_t slot = (uint64_t)bt[t >> a.page_shift] * ps + (t & (ps - 1));
      const T* krow = reinterpret_cast<const T*>(a.k) + (slot * a.hkv + h) * a.d;
      float acc = 0.f;
      for (int c0 = 0; c0 < a.d; c0 += 16 / (int)sizeof(T)) {
        const uint4 w = *reinterpret_cast<const uint4*>(krow + c0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        if constexpr (sizeof(T) == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qp[c0 + e], __uint_as_float(ws[e]), acc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(qp[c0 + 2 * e], Pair16<T>::lo(ws[e]), acc);
            acc = __builtin_fmaf(qp[c0 + 2 * e + 1], Pair16<T>::hi(ws[e]), acc);
          }
        }
      }
      atomicMax(&score[t / B - r0], ordered(acc));
    }
    __syncthreads();
    // keep rounds: the best untaken block (a tie to the lower index) is
    // marked taken (0)
    for (int k = 0; k < keep; ++k) {
      uint64_t best = 0;
      for (int r = tid; r < ncand; r += kSelThreads) {
        const uint64_t key = ((uint64_t)score[r] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)r);
        best = key > best ? key : best;
      }
      best = wg_max(best, red);
      if (tid == 0 && (best >> 32) != 0) score[0xFFFFFFFFu - (uint32_t)best] = 0u;
      __syncthreads();
    }
  }

  // kept blocks in increasing order: a prefix count over the candidates
  const int width = a.width;
  const uint64_t base = (uint64_t)row * width;
  int written = 0;
  for (int c0 = 0; c0 < ncand; c0 += kSelThreads) {
    const int r = c0 + tid;
    const bool kept = r < ncand && (all || score[r] == 0u);
    const uint64_t mask = __ballot(kept);
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int before = __popcll(mask & ((1ull << lane) - 1));
    if (lane == 0) wave_count[wave] = __popcll(mask);
    __syncthreads();
    int off = written;
    for (int w = 0; w < wave; ++w) off += wave_count[w];
    int total = 0;
    for (int w = 0; w < kSelThreads / kWave; ++w) total += wave_count[w];
    if (kept) {
      const int j = off + before;
      const int blk = r0 + r;
      if (a.selection) a.selection[base + j] = blk;
      a.items[base + j] = WorkItem{kDecode, h, s, i, 1, max(blk * B, lo), min((blk + 1) * B, hi + 1),
                                   (int32_t)(base + j)};
    }
    written += total;
    __syncthreads();  // wave_count is rewritten by the next chunk
  }
  for (int j = keep + tid; j < width; j += kSelThreads) {
    if (a.selection) a.selection[base + j] = -1;
    a.items[base + j] = WorkItem{kEmpty, 0, 0, 0, 0, 0, 0, -1};
  }
  for (int j = tid; j < width; j += kSelThreads) a.wg_first[base + j] = (int32_t)(base + j);
  if (row == 0 && tid == 0) a.wg_first[(uint64_t)gridDim.x * width] = (int32_t)((uint64_t)gridDim.x * width);
  if (tid == 0) a.merges[row] = MergeItem{i, h, (int32_t)base, keep, 1};
}

}  // namespace

hipError_t launch_sparse_select(int dtype, const SparseArgs& a, int rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL(sparse_select_kernel<float>, dim3(rows), dim3(kSelThreads), 0, stream, a);
  else if (dtype == 1)
    hipLaunchKernelGGL(sparse_select_kernel<uint16_t>, dim3(rows), dim3(kSelThreads), 0, stream, a);
  else if (dtype == 2)
    hipLaunchKernelGGL(sparse_select_kernel<_Float16>, dim3(rows), dim3(kSelThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
