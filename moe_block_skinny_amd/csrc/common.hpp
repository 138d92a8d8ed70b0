// common.hpp -- device helpers shared by the gfx950 kernels of the decode
// MoE block: bf16 handling, 128-bit weight loads, dot products, wavefront
// reductions and the in-launch completion counters.
//
// Memory-ordering rule (the hazard the write-up's correctness section
// describes: a compiler hoisted an activation read above a synchronisation
// wait; the fix confined that load type to static weights):
//   * only weights, which no kernel of the library ever writes, are read with
//     plain or non-temporal loads;
//   * anything produced inside the same launch by another workgroup
//     (split-K partials, router logits) is read after an acquire fence with
//     relaxed agent-scope atomic loads, which the compiler can neither hoist
//     above the fence nor serve from a non-coherent cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> f32 ---------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// ---- element traits ------------------------------------------------------
// One 128-bit load holds VEC elements: 8 bf16 or 4 fp32.

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int VEC = 4; };
template <> struct Elem<bf16_t> { static constexpr int VEC = 8; };

__device__ __forceinline__ u32x4 ld128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load for weights only: they are read once per call, so keep them
// from displacing the activations and partial sums in the caches.
__device__ __forceinline__ u32x4 ld128_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A 32-bit word as two bf16.  Takes the word by value: bit-casting an
// ext-vector element subscript directly is miscompiled (always element 0).
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// sum_e w[e] * x[e] over one 128-bit chunk, accumulated into acc.
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 x, float acc, bf16_t) {
  const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  const uint32_t x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc, false);
  return acc;
}
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 x, float acc, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_fmaf(__uint_as_float(w[i]), __uint_as_float(x[i]), acc);
  return acc;
}

// Weight chunk (bf16 or fp32) against fp32 activations xs[0..VEC).
__device__ __forceinline__ float dot_chunk_f32x(u32x4 w, const float* xs, float acc, bf16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf(bf16_lo(w[i]), xs[2 * i], acc);
    acc = __builtin_fmaf(bf16_hi(w[i]), xs[2 * i + 1], acc);
  }
  return acc;
}
__device__ __forceinline__ float dot_chunk_f32x(u32x4 w, const float* xs, float acc, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(__uint_as_float(w[i]), xs[i], acc);
  return acc;
}

// ---- wavefront reductions -------------------------------------------------

// Sum over aligned groups of L lanes (L a power of two <= 64); every lane of
// the group ends with the group's sum.  Butterfly order is fixed, so the
// result is deterministic.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint64_t o2 = __shfl_xor(v, o, kWave);
    v = o2 > v ? o2 : v;
  }
  return v;
}

// ---- vector-ALU streaming core ---------------------------------------------

// One wave: R weight rows (row pointers wr[r], each row K-contiguous) against
// up to MB activation rows (xr[t], t < m), over 128-bit chunks [c0, c1) of K.
// Lane q takes chunks c0+q, c0+q+64, ...; U chunks per lane are in flight per
// row before any arithmetic.  Results are summed over the wave (fixed
// butterfly order), so every lane ends with all R x MB dot products.
template <typename T, int R, int MB, int U>
__device__ __forceinline__ void valu_dot(const T* const (&wr)[R], const T* const (&xr)[MB], int m,
                                         int c0, int c1, float (&acc)[R][MB]) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < MB; ++t) acc[r][t] = 0.f;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int c = c0 + lane; c < c1; c += 64 * U) {
    u32x4 wv[U][R], xv[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cc = c + 64 * u;
      const bool ok = cc < c1;
#pragma unroll
      for (int r = 0; r < R; ++r) wv[u][r] = ok ? ld128_stream(wr[r] + (size_t)cc * VEC) : zero;
#pragma unroll
      for (int t = 0; t < MB; ++t) xv[u][t] = (ok && t < m) ? ld128(xr[t] + (size_t)cc * VEC) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MB; ++t) acc[r][t] = dot_chunk(wv[u][r], xv[u][t], acc[r][t], T());
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < MB; ++t) acc[r][t] = group_sum<64>(acc[r][t]);
}

// Lane `lane` picks acc[t == lane]: spreads MB results over the first lanes.
template <int MB>
__device__ __forceinline__ float pick_lane(const float (&v)[MB], int lane) {
  float r = 0.f;
#pragma unroll
  for (int t = 0; t < MB; ++t)
    if (t == lane) r = v[t];
  return r;
}

// ---- cross-workgroup completion counters ---------------------------------

// Called by every thread of a workgroup after it stored its results.  Returns
// true in the workgroup that arrives last of `expected` on `counter`, which
// also resets the counter to zero for the next launch.  Every thread's
// release fence publishes its own stores at device scope before the barrier;
// the acquire fence in the last workgroup makes every other workgroup's
// stores visible to it.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* lds_flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    int last = (old == expected - 1u);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  const bool last = *lds_flag != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Coherent read of a value another workgroup of this launch produced.
__device__ __forceinline__ float ld_shared_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_shared_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Orderable key of a logit: larger key <=> larger value (finite inputs;
// -0 is folded into +0 first), low word breaks ties toward the lower index.
__device__ __forceinline__ uint64_t topk_key(float v, int idx) {
  v = v + 0.0f;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return (int)(0xffffffffu - (uint32_t)key);
}

__device__ __forceinline__ float silu(float z) {
  return z / (1.0f + __expf(-z));
}

}  // namespace moe
