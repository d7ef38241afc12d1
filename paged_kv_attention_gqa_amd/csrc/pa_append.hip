// Paged K/V append: the new keys and values of every packed query written
// into the pool slot of its absolute position (ruDNN 0.1.107 paged_attention
// `DevicePlan::append`: the cache write that precedes attention in a decode
// or prefill step; copy-on-write of shared caches is left to the caller).
//
// One 16-byte chunk per thread over [Q, heads, D + Dv]: row (i, h) of the new
// keys goes to pool row (slot_of[i], h), slot_of[i] = page * page_size +
// slot, from the plan.  Each chunk is read and written once: HBM-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.h"

namespace pa {

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void append_kernel(const u32x4_t* __restrict__ k_new,
                                                     const u32x4_t* __restrict__ v_new, u32x4_t* __restrict__ k_pool,
                                                     u32x4_t* __restrict__ v_pool,
                                                     const int32_t* __restrict__ slot_of, int64_t n_rows, int heads,
                                                     int kc, int vc) {
  // chunk index -> (row = query * heads + head, chunk c of the row's kc + vc)
  const int rc = kc + vc;
  const int64_t total = n_rows * rc;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / rc;
    const int c = (int)(idx - row * rc);
    const int64_t q = row / heads;
    const int h = (int)(row - q * heads);
    const int64_t dst_row = (int64_t)slot_of[q] * heads + h;
    if (c < kc)
      k_pool[dst_row * kc + c] = __builtin_nontemporal_load(k_new + row * kc + c);
    else
      v_pool[dst_row * vc + (c - kc)] = __builtin_nontemporal_load(v_new + row * vc + (c - kc));
  }
}

}  // namespace

hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* slot_of,
                         int64_t queries, int heads, int k_row_bytes, int v_row_bytes, int n_cu, hipStream_t stream) {
  const int64_t n_rows = queries * heads;
  const int kc = k_row_bytes / 16, vc = v_row_bytes / 16;
  const int64_t total = n_rows * (kc + vc);
  if (total == 0) return hipSuccess;
  // enough workgroups to fill the device several times over, each thread a
  // few chunks (grid-stride)
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < (int64_t)n_cu * 16 ? want : (int64_t)n_cu * 16);
  hipLaunchKernelGGL(append_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(k_new), reinterpret_cast<const u32x4_t*>(v_new),
                     reinterpret_cast<u32x4_t*>(k_pool), reinterpret_cast<u32x4_t*>(v_pool), slot_of, n_rows, heads,
                     kc, vc);
  return hipGetLastError();
}

}  // namespace pa
