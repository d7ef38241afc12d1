// Device-side building blocks shared by the paged-attention kernels (gfx950).
//
// Work is described by a flat list of WorkItem records built on the host from
// the schedule (sequence lengths, packed query offsets, absolute query
// positions, block tables) and uploaded once per plan.  One workgroup runs
// one item.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

// One unit of work.  Decode items cover one query, 2^KernelArgs::heads_shift
// consecutive KV heads and one contiguous range of that query's visible keys;
// prefill items cover up to a tile of consecutive queries of one sequence and
// one KV head.
struct WorkItem {
  int32_t kind;       // kDecode / kPrefill / kEmpty
  int32_t kvh;        // (first) KV head
  int32_t seq;        // sequence index (row of the block table)
  int32_t q_begin;    // first packed query
  int32_t q_count;    // number of queries (decode: 1)
  int32_t tok_begin;  // first logical key position visited (inclusive)
  int32_t tok_end;    // last logical key position visited (exclusive)
  int32_t slot;       // decode: split-partial slot of the first head (head kvh + i uses slot + i), or -1
                      // to write the output directly
};
constexpr int32_t kDecode = 0;
constexpr int32_t kPrefill = 1;
constexpr int32_t kEmpty = 2;  // padding in the dispatch order: the workgroup exits at once

// One split query row to combine: partials slot + j * stride, j < nsplit,
// hold the per-split statistics of (query q, KV head kvh).
struct MergeItem {
  int32_t q, kvh, slot, nsplit, stride;
};

// One unit of backward work.  dQ items: one query (q_end = q_begin + 1) and
// one KV head over that query's visible keys [tok_begin, tok_end); dQ tile
// items: up to kBwdQRows / G consecutive queries of one sequence and one KV
// head over the union of their visible keys.  dK/dV items: one block of keys
// [tok_begin, tok_end) of one sequence and KV head against the sequence's
// queries [q_begin, q_end).
struct BwdItem {
  int32_t seq, kvh;
  int32_t q_begin, q_end;
  int32_t tok_begin, tok_end;
};
constexpr int kBwdBlockKeys = 128;  // keys of one dK/dV item
constexpr int kMlaPrefillQueries = 2;  // queries of one absorbed-MLA chunked-prefill item (two waves each)
constexpr int kBwdQRows = 128;      // query rows (query, head of the group) of one dQ tile item

struct KernelArgs {
  const void* q;          // [Q, Hq, D]            (MLA: absorbed query [Q, H, R])
  const void* k;          // [pages, ps, Hkv, D]   (MLA: latent [pages, ps, 1, R])
  const void* v;          // [pages, ps, Hkv, Dv]  (MLA: latent)
  const void* qr;         // MLA only: position query [Q, H, P]
  const void* kr;         // MLA only: rotated position cache [pages, ps, 1, P]
  void* out;              // [Q, Hq, Dv]
  float* lse;             // [Q, Hq] or null
  float* ws_o;            // split partials: [slots, G, Dv] unnormalised sums
  float* ws_ml;           // split partials: [slots, G, 3] = (max in log2 units, sum, unrounded sum)
  const int32_t* block_table;  // [S, W]
  const int32_t* q_pos;        // [Q]
  const int32_t* seq_lens;     // [S]
  const WorkItem* items;
  int32_t n_items;
  const int32_t* wg_first;  // workgroup b runs items wg_first[b] .. wg_first[b + 1] - 1
  int32_t n_wg;             // workgroups of the main launch
  int32_t heads_shift;      // decode items of the decode launch cover 2^heads_shift KV heads
  int32_t table_width;
  int32_t page_shift;     // log2(page_size)
  int32_t hq, hkv;
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
  int32_t causal, window;
};

// ---------------------------------------------------------------------------
// Lane exchange.  DPP row operations stay inside a 16-lane row; crossing rows
// goes through ds_swizzle/bpermute (__shfl_xor).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // reverse within each 8-lane half row
constexpr int kDppMirror = 0x140;      // reverse within each 16-lane row

// Sum over aligned groups of N consecutive lanes (N = 1..64, power of two);
// every lane of the group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// group_sum over N values at once, one reduction step at a time across all
// values (independent DPP operations back to back).
template <int N, int COUNT>
__device__ __forceinline__ void group_sum_all(float* x) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int i = 0; i < COUNT; ++i) x[i] += dpp<kDppXor1>(x[i]);
  }
  if constexpr (N >= 4) {
#pragma unroll
    for (int i = 0; i < COUNT; ++i) x[i] += dpp<kDppXor2>(x[i]);
  }
  if constexpr (N >= 8) {
#pragma unroll
    for (int i = 0; i < COUNT; ++i) x[i] += dpp<kDppHalfMirror>(x[i]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < COUNT; ++i) x[i] += dpp<kDppMirror>(x[i]);
  }
  if constexpr (N >= 32) {
#pragma unroll
    for (int i = 0; i < COUNT; ++i) x[i] += __shfl_xor(x[i], 16);
  }
  if constexpr (N >= 64) {
#pragma unroll
    for (int i = 0; i < COUNT; ++i) x[i] += __shfl_xor(x[i], 32);
  }
}

// Max / sum of x over lanes i and i ^ 32 (v_permlane32_swap: a VALU lane
// exchange, no LDS round trip).  Both lanes of a pair get the same result.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over lanes i and i ^ 16 (v_permlane16_swap).
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32).  Results below the normal range
// flush to zero, which only affects softmax weights under 2^-126.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine across lanes whose index differs by a multiple of STRIDE (the
// other lanes of the same column), STRIDE * COUNT = 64.
template <int STRIDE>
__device__ __forceinline__ float column_max(float x) {
  for (int s = STRIDE; s < kWave; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float column_sum(float x) {
  for (int s = STRIDE; s < kWave; s <<= 1) x += __shfl_xor(x, s);
  return x;
}

// ---------------------------------------------------------------------------
// bf16 helpers (storage is raw 16-bit patterns).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  float2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs and an fp32 accumulator.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// ---------------------------------------------------------------------------
// 16-bit storage types: bf16 travels as raw uint16_t patterns, IEEE binary16
// (f16) as _Float16.  Pair16<T> works on two elements packed in one 32-bit
// word, element 0 in the low half; conversions from float round to nearest
// even.
// ---------------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

template <typename T>
struct Pair16;

template <>
struct Pair16<uint16_t> {  // bf16
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16(a, b); }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) { return dot2_bf16(a, b, c); }
};

template <>
struct Pair16<_Float16> {  // f16
  static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[0]; }
  static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[1]; }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    float2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2_t));
  }
  // v_dot2_f32_f16: a.lo*b.lo + a.hi*b.hi + c with an fp32 accumulator
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
  }
};

// (lo16(a), lo16(b)) and (hi16(a), hi16(b)): the same dimension of two keys.
__device__ __forceinline__ uint32_t interleave_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t interleave_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Wave-uniform read of plan metadata through the constant address space.
// The plan's device buffer is written only by its upload, never by a kernel,
// so the load may go through the scalar cache (s_load) and count against the
// scalar counter instead of the vector-memory counter.
typedef const __attribute__((address_space(4))) int32_t const_i32_t;
__device__ __forceinline__ int load_uniform(const int32_t* p, int idx) { return ((const_i32_t*)p)[idx]; }

// Wait until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt vmcnt(N); expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that leaves this wave's vector-memory operations in
// flight.  __syncthreads() opens with a workgroup release fence, which on
// gfx950 waits for every outstanding vector-memory operation (s_waitcnt
// vmcnt(0)) -- the LDS-DMA loads of the tiles being prefetched included --
// so a tile ring behind it keeps nothing in flight across the barrier.
// Here only LDS operations are waited for (ds_write before the barrier is
// visible after it); callers that publish LDS-DMA data wait for their own
// loads with wait_vmcnt first.  The "memory" clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace pa
