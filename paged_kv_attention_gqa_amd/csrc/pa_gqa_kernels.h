// GQA kernels (split-KV decode, mixed decode + prefill, split merge) as
// templates over the data type, the K and V head sizes and the group size G,
// with their launchers.  Each translation unit that includes this header
// instantiates one set of group sizes (pa_kernels.hip: 1, 2, 4, 8, 16;
// pa_kernels_g.hip: 3, 5, 6, 7, 12) and exports it through a GqaFamily
// lookup; host code reaches the kernels only through pa_launch.h.
#pragma once

#include <hip/hip_ext.h>

#include "pa_decode.h"
#include "pa_launch.h"
#include "pa_prefill.h"

namespace pa {


// U key loads per lane per block.  Small groups (G <= 4) take U = 2 so that
// a wave fits in 128 VGPRs and four waves share a SIMD (measured 2% faster
// than U = 4 at three waves); large groups, whose per-key state grows with G,
// take U = 4 (G = 8) and 2 (G = 16).
template <int G>
struct DecodeUnroll {
  static constexpr int kValue = G <= 4 ? 2 : (G <= 8 ? 4 : 2);
};

// Occupancy targets (waves per SIMD) the register allocator must meet.
// Decode streams HBM and wants several workgroups per CU in flight; its
// registers grow with the group size G (G query rows per lane), so the target
// drops for large groups rather than spill.  A mixed / prefill workgroup holds
// 128 KB of LDS and 8 waves, so one fits a CU at 2 waves per SIMD.
template <int G>
struct Occupancy {
  static constexpr int kDecode = G <= 4 ? 4 : (G <= 8 ? 2 : 1);
  static constexpr int kMixed = G <= 8 ? 2 : 1;
};

// Decode launch shape: NW waves share one item.  Eight waves let one item
// cover up to eight KV heads, one wave each, so that a workgroup reads whole
// slot rows of every page (measured on MI355X: 6.9 TB/s for whole 32 KB pages
// against 6.5 TB/s when eight workgroups each read one head's 256-byte
// chunks).  G = 16 runs one wave per SIMD and so takes four waves.
template <int G>
struct DecodeShape {
  static constexpr int kWaves = G <= 8 ? 8 : 4;
  static constexpr int kWgsPerCu = Occupancy<G>::kDecode * 4 / kWaves;
};

template <typename T, int D, int DV, int G>
__global__ __launch_bounds__(DecodeShape<G>::kWaves* kWave) __attribute__((amdgpu_waves_per_eu(Occupancy<G>::kDecode)))
void decode_kernel(KernelArgs a) {
  constexpr int NW = DecodeShape<G>::kWaves;
  __shared__ float smem[NW * G * (DV + 3)];
  const int first = a.wg_first[blockIdx.x], last = a.wg_first[blockIdx.x + 1];
  int tid = threadIdx.x;
  for (int i = first; i < last; ++i) {
    const WorkItem it = a.items[i];
    if (it.kind == kEmpty) continue;
    if (i > first) __syncthreads();  // the previous item's waves are done with the LDS
    asm volatile("" : "+v"(tid));    // per-lane values are recomputed per item, not kept live
    decode_item<T, D, DV, G, NW, DecodeUnroll<G>::kValue>(a, it, smem, tid, a.heads_shift);
  }
}

// The decode body with kShortItemWaves waves per workgroup, for lists of short
// items (block-sparse attention: one kept block, tens of keys, per item).  Few
// waves give each wave several key blocks to pipeline and leave room for
// many workgroups per CU; the eight-wave shape would hand each wave a single
// block and then spend most of the item on its eight-wave combine.
template <typename T, int D, int DV, int G>
__global__ __launch_bounds__(kShortItemWaves* kWave) __attribute__((amdgpu_waves_per_eu(Occupancy<G>::kDecode)))
void decode_short_kernel(KernelArgs a) {
  constexpr int NW = kShortItemWaves;
  __shared__ float smem[NW * G * (DV + 3)];
  const int first = a.wg_first[blockIdx.x], last = a.wg_first[blockIdx.x + 1];
  int tid = threadIdx.x;
  for (int i = first; i < last; ++i) {
    const WorkItem it = a.items[i];
    if (it.kind == kEmpty) continue;
    if (i > first) __syncthreads();  // the previous item's waves are done with the LDS
    asm volatile("" : "+v"(tid));    // per-lane values are recomputed per item, not kept live
    decode_item<T, D, DV, G, NW, DecodeUnroll<G>::kValue>(a, it, smem, tid, a.heads_shift);
  }
}

// One launch for plans with prefill tiles: decode items and prefill tiles
// share the grid (packed decode + chunked prefill in one dispatch).
template <typename T, int D, int DV, int G>
struct MixedShape {
  // the 32x32x16 MFMA tile with its LDS DMA ring: D = Dv = 64 or 128,
  // D = 192 with Dv = 128 (four 40 KB stages fill the 160 KB of LDS), and
  // D = Dv = 256 in two passes of 128 output dims (three 48 KB stages)
  static constexpr bool kMfma = sizeof(T) == 2 && G <= kPrefillRows &&
                                ((D == DV && (D == 64 || D == 128 || D == 256)) || (D == 192 && DV == 128));
  static constexpr int kDecodeBytes = kPrefillWaves * G * (DV + 3) * 4;
  static constexpr int kPrefillBytes =
      kMfma ? PrefillSmem<(kMfma ? D : 64), (kMfma ? PrefillPass<D, DV>::kDims : 64)>::kBytes : 0;
  static constexpr int kBytes = kDecodeBytes > kPrefillBytes ? kDecodeBytes : kPrefillBytes;
};

template <typename T, int D, int DV, int G>
__global__ __launch_bounds__(kPrefillWaves* kWave) __attribute__((amdgpu_waves_per_eu(Occupancy<G>::kMixed)))
void mixed_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[MixedShape<T, D, DV, G>::kBytes];
  // plans with prefill tiles run one item per workgroup (wg_first[b] = b)
  const WorkItem it = a.items[blockIdx.x];
  if (it.kind == kEmpty) return;
  if (it.kind == kPrefill) {
    if constexpr (MixedShape<T, D, DV, G>::kMfma)
      prefill_item<T, D, DV, G>(a, it, smem);
    else
      prefill_item_by_queries<T, D, DV, G, kPrefillWaves, DecodeUnroll<G>::kValue>(a, it,
                                                                                  reinterpret_cast<float*>(smem));
  } else {
    decode_item<T, D, DV, G, kPrefillWaves, DecodeUnroll<G>::kValue>(a, it, reinterpret_cast<float*>(smem));
  }
}

// grid: (split rows, chunks of 256 outputs per row)
constexpr int kMergeThreads = 256;
template <typename T, int DV, int G, bool PARTIAL = false>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(KernelArgs a, const MergeItem* merges) {
  const MergeItem mi = merges[blockIdx.x];
  merge_row<T, DV, G, PARTIAL>(a, mi, blockIdx.y, gridDim.y);
}

namespace {

// One main-kernel launch; with timing events, through hipExtLaunchKernel so
// that the events carry the kernel's own start and end.
template <typename K>
hipError_t launch_main(K kernel, int n_wg, int threads, const KernelArgs& a, const MainEvents& ev,
                       hipStream_t stream) {
  if (n_wg <= 0) return hipSuccess;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, dim3(n_wg), dim3(threads), 0, stream, ev.start, ev.stop, 0, a);
  else
    hipLaunchKernelGGL(kernel, dim3(n_wg), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int DV, int G>
hipError_t launch_decode_t(const KernelArgs& a, int n_wg, const MergeItem*, int, const MainEvents& ev,
                           hipStream_t stream) {
  return launch_main(decode_kernel<T, D, DV, G>, n_wg, DecodeShape<G>::kWaves * kWave, a, ev, stream);
}

template <typename T, int D, int DV, int G>
hipError_t launch_short_t(const KernelArgs& a, int n_wg, const MergeItem*, int, const MainEvents& ev,
                          hipStream_t stream) {
  return launch_main(decode_short_kernel<T, D, DV, G>, n_wg, kShortItemWaves * kWave, a, ev, stream);
}

template <typename T, int D, int DV, int G>
hipError_t launch_mixed_t(const KernelArgs& a, int n_wg, const MergeItem*, int, const MainEvents& ev,
                          hipStream_t stream) {
  return launch_main(mixed_kernel<T, D, DV, G>, n_wg, kPrefillWaves * kWave, a, ev, stream);
}

template <typename T, int DV, int G, bool PARTIAL = false>
hipError_t launch_merge_t(const KernelArgs& a, int, const MergeItem* merges, int n_merges, const MainEvents&,
                          hipStream_t stream) {
  if (n_merges > 0) {
    const int chunks = (G * DV / 4 + kMergeThreads - 1) / kMergeThreads;
    hipLaunchKernelGGL((merge_kernel<T, DV, G, PARTIAL>), dim3(n_merges, chunks), dim3(kMergeThreads), 0, stream, a,
                       merges);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Group sizes of one translation unit: pick_g<Sel, T, D, DV, Gs...>(g).
template <template <typename, int, int, int> class Sel, typename T, int D, int DV, int... Gs>
LaunchFn pick_g(int g) {
  LaunchFn f = nullptr;
  ((g == Gs ? (f = Sel<T, D, DV, Gs>::fn, 0) : 0), ...);
  return f;
}

// (K, V) head sizes with kernels: equal sizes 64, 128, 256, and K 192 with
// V 128 (a 128-wide no-position part plus a 64-wide rotary part in the key).
template <template <typename, int, int, int> class Sel, typename T, int... Gs>
LaunchFn pick_d(int d, int dv, int g) {
  if (d == 64 && dv == 64) return pick_g<Sel, T, 64, 64, Gs...>(g);
  if (d == 128 && dv == 128) return pick_g<Sel, T, 128, 128, Gs...>(g);
  if (d == 256 && dv == 256) return pick_g<Sel, T, 256, 256, Gs...>(g);
  if (d == 192 && dv == 128) return pick_g<Sel, T, 192, 128, Gs...>(g);
  return nullptr;
}

template <template <typename, int, int, int> class Sel, int... Gs>
LaunchFn pick(int dtype, int d, int dv, int g) {
  if (dtype == 0) return pick_d<Sel, float, Gs...>(d, dv, g);
  if (dtype == 1) return pick_d<Sel, uint16_t, Gs...>(d, dv, g);
  if (dtype == 2) return pick_d<Sel, _Float16, Gs...>(d, dv, g);
  return nullptr;
}

template <typename T, int D, int DV, int G>
struct DecodeSel {
  static constexpr LaunchFn fn = launch_decode_t<T, D, DV, G>;
};

template <typename T, int D, int DV, int G>
struct ShortSel {
  static constexpr LaunchFn fn = launch_short_t<T, D, DV, G>;
};

template <typename T, int D, int DV, int G>
struct MixedSel {
  static constexpr LaunchFn fn = launch_mixed_t<T, D, DV, G>;
};
template <typename T, int D, int DV, int G>
struct MergeSel {  // depends on the output width only
  static constexpr LaunchFn fn = launch_merge_t<T, DV, G>;
};


// The launchers and launch shapes of one set of group sizes.
template <int... Gs>
bool gqa_family_lookup(int dtype, int d, int dv, int g, GqaFamily* out) {
  if (!((g == Gs) || ...)) return false;
  out->decode = pick<DecodeSel, Gs...>(dtype, d, dv, g);
  out->decode_short = pick<ShortSel, Gs...>(dtype, d, dv, g);
  out->mixed = pick<MixedSel, Gs...>(dtype, d, dv, g);
  out->merge = pick<MergeSel, Gs...>(dtype, d, dv, g);
  ((g == Gs ? (out->waves = DecodeShape<Gs>::kWaves, out->wgs_per_cu = DecodeShape<Gs>::kWgsPerCu, 0) : 0), ...);
  return true;
}

}  // namespace

}  // namespace pa
