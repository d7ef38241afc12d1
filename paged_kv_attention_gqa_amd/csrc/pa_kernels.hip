// Kernel entry points of the absorbed-MLA path, the GQA kernels of group sizes
// 1, 2, 4, 8 and 16 (templates in pa_gqa_kernels.h), and the dispatchers that
// host code reaches through pa_launch.h.
#include "pa_gqa_kernels.h"
#include "pa_mla.h"

namespace pa {

static_assert(kMlaHeads == kMlaGroupHeads, "an MLA work item covers one head group");
static_assert(kGenericUnitHeads == kMlaGroupHeads, "MLA plans serve both MLA kernels");

bool gqa_family_pow2(int dtype, int d, int dv, int g, GqaFamily* out) {
  return gqa_family_lookup<1, 2, 4, 8, 16>(dtype, d, dv, g, out);
}

// Absorbed MLA: decode items (one query and head group, one key range) and,
// in plans that have them (PREFILL), chunked-prefill items (two queries of
// one head group, two waves each);
// a 72 KB LDS tile ring, two workgroups per CU.  Decode-only plans run the
// instantiation without the prefill body, whose 128 output registers per
// wave would otherwise set the register allocation of the decode body too.
//
// NG = 2 (decode-only plans of more than one head group): each decode item
// takes two head groups of 16 heads, sharing the tile reads (80 KB of LDS).
template <typename T, bool PREFILL, int NG = 1>
__global__ __launch_bounds__(kMlaWaves* kWave) __attribute__((amdgpu_waves_per_eu(2))) void mla_kernel(KernelArgs a) {
  static_assert(NG == 1 || !PREFILL, "head-group pairs on decode-only plans");
  __shared__ __attribute__((aligned(16))) char smem[MlaSmem<NG>::kBytes];
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
      mla_item<T, false, !PREFILL, NG>(a, it, smem, tid);
  }
}

namespace {

// The kernels of group size g: the powers of two here, the other sizes in
// pa_kernels_g.hip.
bool gqa_family(int dtype, int d, int dv, int g, GqaFamily* f) {
  return gqa_family_pow2(dtype, d, dv, g, f) || gqa_family_other(dtype, d, dv, g, f);
}

}  // namespace

bool gqa_supported(int dtype, int d, int dv, int g) {
  GqaFamily f;
  return gqa_family(dtype, d, dv, g, &f) && f.decode != nullptr;
}

bool prefill_supported(int dtype, int d, int dv, int g) {
  GqaFamily f;
  return gqa_family(dtype, d, dv, g, &f) && f.mixed != nullptr;
}

hipError_t launch_gqa_main(int dtype, int d, int dv, int g, bool has_prefill, const KernelArgs& a,
                           const MainEvents& ev, hipStream_t stream) {
  GqaFamily f;
  if (!gqa_family(dtype, d, dv, g, &f)) return hipErrorInvalidValue;
  LaunchFn fn = has_prefill ? f.mixed : f.decode;
  return fn ? fn(a, a.n_wg, nullptr, 0, ev, stream) : hipErrorInvalidValue;
}

hipError_t launch_gqa_short(int dtype, int d, int dv, int g, const KernelArgs& a, hipStream_t stream) {
  GqaFamily f;
  if (!gqa_family(dtype, d, dv, g, &f) || !f.decode_short) return hipErrorInvalidValue;
  return f.decode_short(a, a.n_wg, nullptr, 0, MainEvents{}, stream);
}

hipError_t launch_gqa_merge(int dtype, int d, int dv, int g, const KernelArgs& a, const MergeItem* merges,
                            int n_merges, hipStream_t stream) {
  GqaFamily f;
  if (!gqa_family(dtype, d, dv, g, &f) || !f.merge) return hipErrorInvalidValue;
  return f.merge(a, 0, merges, n_merges, MainEvents{}, stream);
}

int decode_wgs_per_cu(int g) {
  GqaFamily f;
  return gqa_family(1, 128, 128, g, &f) ? f.wgs_per_cu : 1;
}

int decode_waves(int g) {
  GqaFamily f;
  return gqa_family(1, 128, 128, g, &f) ? f.waves : 1;
}

// two 4-wave workgroups per CU (72 KB of LDS each, waves_per_eu(2))
int mla_wgs_per_cu() { return 2; }

namespace {
bool mla_mfma_shape(int dtype, int r, int p) { return (dtype == 1 || dtype == 2) && r == kMlaRank && p == kMlaRope; }
// MLA on the vector kernel: one KV head (the latent), its H query heads in
// units of 16, the value the latent itself
GenericShape mla_generic_shape(const KernelArgs& a, int r, int p) {
  return GenericShape{r, p, r, a.hq, (a.hq + kMlaGroupHeads - 1) / kMlaGroupHeads, kMlaGroupHeads,
                      1 << a.heads_shift, 1};
}
}  // namespace

bool mla_supported(int dtype, int h, int r, int p) {
  return dtype >= 0 && dtype <= 2 && h >= 1 && r >= 1 && r <= kMlaMaxRank && p >= 1 && p <= kMlaMaxRope;
}

bool mla_bwd_supported(int dtype, int h, int r, int p) { return h >= 1 && mla_mfma_shape(dtype, r, p); }

hipError_t launch_mla_main(int dtype, int r, int p, bool has_prefill, const KernelArgs& a, const MainEvents& ev,
                           hipStream_t stream) {
  if (!mla_mfma_shape(dtype, r, p)) return launch_generic(dtype, mla_generic_shape(a, r, p), a, ev, stream);
  constexpr int threads = kMlaWaves * kWave;
  // decode-only plans of several head groups pair them (heads_shift 1)
  const bool pairs = !has_prefill && a.heads_shift == 1;
  if (dtype == 1 && has_prefill) return launch_main(mla_kernel<uint16_t, true>, a.n_wg, threads, a, ev, stream);
  if (dtype == 1 && pairs) return launch_main(mla_kernel<uint16_t, false, 2>, a.n_wg, threads, a, ev, stream);
  if (dtype == 1) return launch_main(mla_kernel<uint16_t, false>, a.n_wg, threads, a, ev, stream);
  if (dtype == 2 && has_prefill) return launch_main(mla_kernel<_Float16, true>, a.n_wg, threads, a, ev, stream);
  if (dtype == 2 && pairs) return launch_main(mla_kernel<_Float16, false, 2>, a.n_wg, threads, a, ev, stream);
  if (dtype == 2) return launch_main(mla_kernel<_Float16, false>, a.n_wg, threads, a, ev, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mla_merge(int dtype, int r, int p, const KernelArgs& a, const MergeItem* merges, int n_merges,
                            hipStream_t stream) {
  if (!mla_mfma_shape(dtype, r, p)) return launch_generic_merge(dtype, mla_generic_shape(a, r, p), a, merges, n_merges, stream);
  if (dtype == 1)
    return launch_merge_t<uint16_t, kMlaRank, kMlaHeads, true>(a, 0, merges, n_merges, MainEvents{}, stream);
  if (dtype == 2)
    return launch_merge_t<_Float16, kMlaRank, kMlaHeads, true>(a, 0, merges, n_merges, MainEvents{}, stream);
  return hipErrorInvalidValue;
}


}  // namespace pa
