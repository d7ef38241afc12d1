// Kernel entry points and their launchers.  Host code reaches the kernels
// only through the launch_* functions declared in pa_launch.h.
#include <hip/hip_ext.h>

#include "pa_decode.h"
#include "pa_launch.h"
#include "pa_mla.h"
#include "pa_prefill.h"
#include "pa_prefill16.h"

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

// One launch for plans with prefill tiles: decode items and prefill tiles
// share the grid (packed decode + chunked prefill in one dispatch).
template <typename T, int D, int DV, int G>
struct MixedShape {
  static constexpr bool kMfma = sizeof(T) == 2 && D == DV && (D == 64 || D == 128) && G <= kPrefillRows;
  // K and V rows of different widths, and D = Dv = 256: the 16x16x32 MFMA tile
  static constexpr bool kMfma16 =
      sizeof(T) == 2 && !kMfma && D % 64 == 0 && DV % 64 == 0 && (D != DV || D == 256) && G <= kPrefillRows;
  static constexpr int kDecodeBytes = kPrefillWaves * G * (DV + 3) * 4;
  static constexpr int kPrefillBytes =
      kMfma ? PrefillSmem<(D <= 128 ? D : 128)>::kBytes : (kMfma16 ? Prefill16Smem<D, DV>::kBytes : 0);
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
      prefill_item<T, D, G>(a, it, smem);
    else if constexpr (MixedShape<T, D, DV, G>::kMfma16)
      prefill16_item<T, D, DV, G>(a, it, smem);
    else
      prefill_item_by_queries<T, D, DV, G, kPrefillWaves, DecodeUnroll<G>::kValue>(a, it,
                                                                                  reinterpret_cast<float*>(smem));
  } else {
    decode_item<T, D, DV, G, kPrefillWaves, DecodeUnroll<G>::kValue>(a, it, reinterpret_cast<float*>(smem));
  }
}

// Absorbed MLA: decode items (one query, one key range) and, in plans that
// have them (PREFILL), chunked-prefill items (two queries, two waves each);
// a 72 KB LDS tile ring, two workgroups per CU.  Decode-only plans run the
// instantiation without the prefill body, whose 128 output registers per
// wave would otherwise set the register allocation of the decode body too.
template <typename T, bool PREFILL>
__global__ __launch_bounds__(kMlaWaves* kWave) __attribute__((amdgpu_waves_per_eu(2))) void mla_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[MlaSmem::kBytes];
  const int first = a.wg_first[blockIdx.x], last = a.wg_first[blockIdx.x + 1];
  int tid = threadIdx.x;
  for (int i = first; i < last; ++i) {
    const WorkItem it = a.items[i];
    if (it.kind == kEmpty) continue;
    if (i > first) __syncthreads();  // the previous item's waves are done with the LDS ring
    asm volatile("" : "+v"(tid));    // per-lane values are recomputed per item, not kept live
    if (PREFILL && it.kind == kPrefill)
      mla_item<T, PREFILL>(a, it, smem, tid);
    else
      mla_item<T, false, !PREFILL>(a, it, smem, tid);
  }
}

// grid: (split rows, chunks of 256 outputs per row)
constexpr int kMergeThreads = 256;
template <typename T, int DV, int G>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(KernelArgs a, const MergeItem* merges) {
  const MergeItem mi = merges[blockIdx.x];
  merge_row<T, DV, G>(a, mi, blockIdx.y, gridDim.y);
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

using LaunchFn = hipError_t (*)(const KernelArgs&, int, const MergeItem*, int, const MainEvents&, hipStream_t);

template <typename T, int D, int DV, int G>
hipError_t launch_decode_t(const KernelArgs& a, int n_wg, const MergeItem*, int, const MainEvents& ev,
                           hipStream_t stream) {
  return launch_main(decode_kernel<T, D, DV, G>, n_wg, DecodeShape<G>::kWaves * kWave, a, ev, stream);
}

template <typename T, int D, int DV, int G>
hipError_t launch_mixed_t(const KernelArgs& a, int n_wg, const MergeItem*, int, const MainEvents& ev,
                          hipStream_t stream) {
  return launch_main(mixed_kernel<T, D, DV, G>, n_wg, kPrefillWaves * kWave, a, ev, stream);
}

template <typename T, int DV, int G>
hipError_t launch_merge_t(const KernelArgs& a, int, const MergeItem* merges, int n_merges, const MainEvents&,
                          hipStream_t stream) {
  if (n_merges > 0) {
    const int chunks = (G * DV / 4 + kMergeThreads - 1) / kMergeThreads;
    hipLaunchKernelGGL((merge_kernel<T, DV, G>), dim3(n_merges, chunks), dim3(kMergeThreads), 0, stream, a, merges);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <template <typename, int, int, int> class Sel, typename T, int D, int DV>
LaunchFn pick_g(int g) {
  switch (g) {
    case 1: return Sel<T, D, DV, 1>::fn;
    case 2: return Sel<T, D, DV, 2>::fn;
    case 4: return Sel<T, D, DV, 4>::fn;
    case 8: return Sel<T, D, DV, 8>::fn;
    case 16: return Sel<T, D, DV, 16>::fn;
    default: return nullptr;
  }
}

// (K, V) head sizes with kernels: equal sizes 64, 128, 256, and K 192 with
// V 128 (a 128-wide no-position part plus a 64-wide rotary part in the key).
template <template <typename, int, int, int> class Sel, typename T>
LaunchFn pick_d(int d, int dv, int g) {
  if (d == 64 && dv == 64) return pick_g<Sel, T, 64, 64>(g);
  if (d == 128 && dv == 128) return pick_g<Sel, T, 128, 128>(g);
  if (d == 256 && dv == 256) return pick_g<Sel, T, 256, 256>(g);
  if (d == 192 && dv == 128) return pick_g<Sel, T, 192, 128>(g);
  return nullptr;
}

template <template <typename, int, int, int> class Sel>
LaunchFn pick(int dtype, int d, int dv, int g) {
  if (dtype == 0) return pick_d<Sel, float>(d, dv, g);
  if (dtype == 1) return pick_d<Sel, uint16_t>(d, dv, g);
  if (dtype == 2) return pick_d<Sel, _Float16>(d, dv, g);
  return nullptr;
}

template <typename T, int D, int DV, int G>
struct DecodeSel {
  static constexpr LaunchFn fn = launch_decode_t<T, D, DV, G>;
};

template <typename T, int D, int DV, int G>
struct MixedSel {
  static constexpr LaunchFn fn = launch_mixed_t<T, D, DV, G>;
};
template <typename T, int D, int DV, int G>
struct MergeSel {  // depends on the output width only
  static constexpr LaunchFn fn = launch_merge_t<T, DV, G>;
};

}  // namespace

bool gqa_supported(int dtype, int d, int dv, int g) { return pick<DecodeSel>(dtype, d, dv, g) != nullptr; }

bool prefill_supported(int dtype, int d, int dv, int g) { return pick<MixedSel>(dtype, d, dv, g) != nullptr; }

hipError_t launch_gqa_main(int dtype, int d, int dv, int g, bool has_prefill, const KernelArgs& a,
                           const MainEvents& ev, hipStream_t stream) {
  LaunchFn f = has_prefill ? pick<MixedSel>(dtype, d, dv, g) : pick<DecodeSel>(dtype, d, dv, g);
  return f ? f(a, a.n_wg, nullptr, 0, ev, stream) : hipErrorInvalidValue;
}

hipError_t launch_gqa_merge(int dtype, int d, int dv, int g, const KernelArgs& a, const MergeItem* merges,
                            int n_merges, hipStream_t stream) {
  LaunchFn f = pick<MergeSel>(dtype, d, dv, g);
  return f ? f(a, 0, merges, n_merges, MainEvents{}, stream) : hipErrorInvalidValue;
}

int decode_wgs_per_cu(int g) {
  switch (g) {
    case 1: return DecodeShape<1>::kWgsPerCu;
    case 2: return DecodeShape<2>::kWgsPerCu;
    case 4: return DecodeShape<4>::kWgsPerCu;
    case 8: return DecodeShape<8>::kWgsPerCu;
    case 16: return DecodeShape<16>::kWgsPerCu;
    default: return 1;
  }
}

int decode_waves(int g) {
  switch (g) {
    case 1: return DecodeShape<1>::kWaves;
    case 2: return DecodeShape<2>::kWaves;
    case 4: return DecodeShape<4>::kWaves;
    case 8: return DecodeShape<8>::kWaves;
    case 16: return DecodeShape<16>::kWaves;
    default: return 1;
  }
}

// two 4-wave workgroups per CU (72 KB of LDS each, waves_per_eu(2))
int mla_wgs_per_cu() { return 2; }

bool mla_supported(int dtype, int h, int r, int p) {
  return (dtype == 1 || dtype == 2) && h == kMlaHeads && r == kMlaRank && p == kMlaRope;
}

hipError_t launch_mla_main(int dtype, bool has_prefill, const KernelArgs& a, const MainEvents& ev,
                           hipStream_t stream) {
  constexpr int threads = kMlaWaves * kWave;
  if (dtype == 1 && has_prefill) return launch_main(mla_kernel<uint16_t, true>, a.n_wg, threads, a, ev, stream);
  if (dtype == 1) return launch_main(mla_kernel<uint16_t, false>, a.n_wg, threads, a, ev, stream);
  if (dtype == 2 && has_prefill) return launch_main(mla_kernel<_Float16, true>, a.n_wg, threads, a, ev, stream);
  if (dtype == 2) return launch_main(mla_kernel<_Float16, false>, a.n_wg, threads, a, ev, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mla_merge(int dtype, const KernelArgs& a, const MergeItem* merges, int n_merges,
                            hipStream_t stream) {
  if (dtype == 1) return launch_merge_t<uint16_t, kMlaRank, kMlaHeads>(a, 0, merges, n_merges, MainEvents{}, stream);
  if (dtype == 2) return launch_merge_t<_Float16, kMlaRank, kMlaHeads>(a, 0, merges, n_merges, MainEvents{}, stream);
  return hipErrorInvalidValue;
}


}  // namespace pa
