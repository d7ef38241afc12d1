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
// goes to the lower block index.
//
// Two kernels.  sparse_scores_kernel streams K: one workgroup per row and
// span of keys (a whole number of blocks), each wave 64 keys at a time.  The
// wave reads the keys' rows in 16-byte pieces with consecutive lanes on
// consecutive pieces of a row (coalesced), parks them in LDS with one spare
// piece per key row, and then each lane runs its own key's product sum over
// its row in LDS (the spare piece puts 16 consecutive keys' pieces in 16
// different bank groups).  Block maxima go through LDS to the row's score
// buffer.  sparse_topk_kernel then picks the kept blocks of each row and
// writes the work list.
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

// Largest 64-bit key of the wave (every lane receives it).
__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, s), hi = __shfl_xor((uint32_t)(v >> 32), s);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

constexpr int kPieces = 8;  // 16-byte pieces of a key row per pass (a longer row takes several passes)

template <typename T>
__global__ __launch_bounds__(kSelThreads) void sparse_scores_kernel(SparseArgs a) {
  __shared__ uint4 stage[kSelThreads / kWave][kWave * (kPieces + 1)];
  __shared__ float qp[kSparseMaxDim];
  __shared__ uint32_t bmax[1024];

  const int row = blockIdx.x;  // query * hkv + KV head
  const int i = row / a.hkv, h = row % a.hkv;
  const int s = a.seq_of[i];
  const int L = a.seq_lens[s], p = a.q_pos[i];
  const int hi = a.causal ? p : L - 1;
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int B = a.block_size;
  const int r0 = lo / B, ncand = hi / B - r0 + 1;
  if (a.topk == 0 || a.topk >= ncand) return;  // every block kept: nothing to score
  const int SPAN = a.span;
  const int ks0 = (lo / SPAN + (int)blockIdx.y) * SPAN;  // this workgroup's keys [ks0, ks0 + SPAN)
  if (ks0 > hi) return;
  const int ks_lo = max(ks0, lo), ks_hi = min(ks0 + SPAN - 1, hi);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nb = SPAN / B;

  const T* q = reinterpret_cast<const T*>(a.q) + ((uint64_t)i * a.hq + (uint64_t)h * (a.hq / a.hkv)) * a.d;
  for (int c = tid; c < a.d; c += kSelThreads) qp[c] = widen(q, c);
  for (int j = tid; j < nb; j += kSelThreads) bmax[j] = 0u;
  __syncthreads();

  constexpr int EPP = 16 / (int)sizeof(T);  // elements per piece
  const int P = a.d / EPP;                  // pieces per key row
  const uint64_t row_bytes = (uint64_t)a.d * sizeof(T);
  const char* kbase = reinterpret_cast<const char*>(a.k) + (uint64_t)h * row_bytes;
  const int32_t* bt = a.block_table + (size_t)s * a.table_width;
  const int ps = 1 << a.page_shift;
  uint4* st = stage[wave];
  for (int base = ks0 + kWave * wave; base <= ks_hi; base += kSelThreads) {
    if (base + kWave - 1 < ks_lo) continue;
    const int t = base + lane;
    const bool valid = t >= ks_lo && t <= ks_hi;
    const int tc = min(max(t, ks_lo), ks_hi);  // out-of-range lanes read an in-range key
    const uint64_t slot = (uint64_t)bt[tc >> a.page_shift] * ps + (tc & (ps - 1));
    const uint64_t my_off = slot * a.hkv * row_bytes;  // this lane's key row (KV head offset in kbase)
    float acc = 0.f;
    // one pass: np pieces of the 64 key rows from piece c0 on; the loads are
    // coalesced (piece j * 64 + lane of the 64 x np block is piece (.. % np)
    // of key (.. / np)), parked in LDS, then each lane runs its own key's
    // pieces in dimension order
    // LDS index and source of piece j * 64 + lane of a pass
    auto piece_dst = [&](int j, int np) {
      const int qi = j * kWave + lane, key = qi / np;
      return key * (kPieces + 1) + (qi - key * np);
    };
    auto piece_src = [&](int j, int np, int c0) {
      const int qi = j * kWave + lane, key = qi / np;
      const uint32_t lo32 = __shfl((uint32_t)my_off, key), hi32 = __shfl((uint32_t)(my_off >> 32), key);
      return *reinterpret_cast<const uint4*>(kbase + (((uint64_t)hi32 << 32) | lo32) +
                                             (uint64_t)(c0 + qi - key * np) * 16);
    };
    auto dot = [&](int np, int c0) {
      // other lanes' pieces: keep the reads after the writes (a wave's LDS
      // accesses complete in order) and the next pass's writes after them
      asm volatile("" ::: "memory");
      for (int pc = 0; pc < np; ++pc) {
        const uint4 w = st[lane * (kPieces + 1) + pc];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        const float* qq = qp + (c0 + pc) * EPP;
        if constexpr (sizeof(T) == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qq[e], __uint_as_float(ws[e]), acc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(qq[2 * e], Pair16<T>::lo(ws[e]), acc);
            acc = __builtin_fmaf(qq[2 * e + 1], Pair16<T>::hi(ws[e]), acc);
          }
        }
      }
      asm volatile("" ::: "memory");
    };
    int c0 = 0;
    for (; c0 + kPieces <= P; c0 += kPieces) {  // full passes: all loads in flight together
      uint4 v[kPieces];
#pragma unroll
      for (int j = 0; j < kPieces; ++j) v[j] = piece_src(j, kPieces, c0);
#pragma unroll
      for (int j = 0; j < kPieces; ++j) st[piece_dst(j, kPieces)] = v[j];
      dot(kPieces, c0);
    }
    if (c0 < P) {  // the row's last pieces
      const int np = P - c0;
      for (int j = 0; j < np; ++j) {
        const uint4 v = piece_src(j, np, c0);
        st[piece_dst(j, np)] = v;
      }
      dot(np, c0);
    }
    const uint32_t key = valid ? ordered(acc) : 0u;
    if (B % kWave == 0) {
      // the 64 keys (aligned to 64) lie in one block: one wave maximum
      uint32_t m = key;
#pragma unroll
      for (int sh = 1; sh < kWave; sh <<= 1) m = max(m, (uint32_t)__shfl_xor(m, sh));
      if (lane == 0) atomicMax(&bmax[(base - ks0) / B], m);
    } else if (valid) {
      atomicMax(&bmax[(t - ks0) / B], key);
    }
  }
  __syncthreads();
  // the span's candidate blocks (each has a visible key, so a score above 0)
  uint32_t* out = a.scores + (size_t)row * a.cand_width;
  for (int j = tid; j < nb; j += kSelThreads) {
    const int gb = ks0 / B + j;
    if (gb >= r0 && gb < r0 + ncand) out[gb - r0] = bmax[j];
  }
}

template <typename T>
__global__ __launch_bounds__(kSelThreads) void sparse_topk_kernel(SparseArgs a) {
  __shared__ uint32_t score[kSparseMaxBlocks];
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
    const uint32_t* sc = a.scores + (size_t)row * a.cand_width;
    for (int r = tid; r < ncand; r += kSelThreads) score[r] = sc[r];
    __syncthreads();
    // keep rounds, in the first wave alone (no workgroup barrier per round):
    // the best untaken block (a tie to the lower index) is marked taken (0)
    if (tid < kWave) {
      for (int k = 0; k < keep; ++k) {
        uint64_t best = 0;
        for (int r = tid; r < ncand; r += kWave) {
          const uint64_t key = ((uint64_t)score[r] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)r);
          best = key > best ? key : best;
        }
        best = wave_max(best);
        if (tid == 0 && (best >> 32) != 0) score[0xFFFFFFFFu - (uint32_t)best] = 0u;
        // the mark is read by every lane next round (a wave's LDS accesses
        // complete in order)
        asm volatile("" ::: "memory");
      }
    }
    __syncthreads();
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
  // workgroup w runs items [w * ipw, (w + 1) * ipw) of the row-major list;
  // this row writes the starts that fall in its items
  const int ipw = a.items_per_wg;
  const uint64_t total = (uint64_t)gridDim.x * width;
  for (uint64_t w = (base + ipw - 1) / ipw + tid; w * ipw < base + width; w += kSelThreads)
    a.wg_first[w] = (int32_t)(w * ipw);
  if (row == 0 && tid == 0) a.wg_first[(total + ipw - 1) / ipw] = (int32_t)total;
  if (tid == 0) a.merges[row] = MergeItem{i, h, (int32_t)base, keep, 1};
}

}  // namespace

template <typename T>
hipError_t launch_select_t(const SparseArgs& a, int rows, hipStream_t stream) {
  if (a.topk > 0) {
    hipLaunchKernelGGL(sparse_scores_kernel<T>, dim3(rows, a.spans), dim3(kSelThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sparse_topk_kernel<T>, dim3(rows), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sparse_select(int dtype, const SparseArgs& a, int rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (a.span > 1024 * a.block_size || a.span / a.block_size > 1024) return hipErrorInvalidValue;
  if (dtype == 0) return launch_select_t<float>(a, rows, stream);
  if (dtype == 1) return launch_select_t<uint16_t>(a, rows, stream);
  if (dtype == 2) return launch_select_t<_Float16>(a, rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
