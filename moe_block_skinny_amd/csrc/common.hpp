// common.hpp -- device helpers shared by the gfx950 kernels of the decode
// MoE block: bf16 handling, 128-bit weight loads, dot products, wavefront
// reductions and the in-launch completion counters.
//
// Memory-ordering rule (the hazard the write-up's correctness section
// describes: a compiler hoisted an activation read above a synchronisation
// wait; the fix confined that load type to static weights):
//   * only weights, which no kernel of the library ever writes, are read with
//     plain or non-temporal loads;
//   * anything produced inside the same launch by another workgroup (router
//     logits, K-slice partial sums, top-k ids, h in the fused block) is
//     stored device-coherent (st_coherent*) and read with device-coherent
//     loads (ld_coherent*) only after a completion counter or grid barrier
//     (arrive_last, grid_wait) has seen every producer arrive; their
//     acquire fence keeps the compiler from hoisting a load above the wait.
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
// fp32 activations as bf16 pairs: hi = RNE(x), lo = RNE(x - hi), so x =
// hi + lo to about 16 significant bits.  Elements 2i and 2i+1 go to the low
// and high halves of word i, as in a bf16 weight chunk.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const bf16_t ha = f32_to_bf16(a), hb = f32_to_bf16(b);
  const bf16_t la = f32_to_bf16(a - bf16_to_f32(ha)), lb = f32_to_bf16(b - bf16_to_f32(hb));
  hi = (uint32_t)ha | ((uint32_t)hb << 16);
  lo = (uint32_t)la | ((uint32_t)lb << 16);
}
// bf16 weight chunk against an activation chunk given as hi/lo bf16 pairs:
// the hi terms first, then the lo terms.
__device__ __forceinline__ float dot_chunk_hilo(u32x4 w, u32x4 hi, u32x4 lo) {
  return dot_chunk(w, lo, dot_chunk(w, hi, 0.f, bf16_t()), bf16_t());
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

// DPP move of a float (CTRL: a DPP lane-permutation control).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over each 16-lane row, left in every lane of the row: xor 1, xor 2
// (quad permutes), then half-mirror and mirror, which pair the quads and the
// half-rows once every quad is uniform.  Fixed order, so deterministic.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

// Sum over aligned groups of L lanes (L = 16, 32 or 64), valid in every lane
// of its group: DPP within rows, then the row sums are read out (readlane)
// and added in fixed order.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  v = row_sum16(v);
  if constexpr (L == 16) {
    return v;
  } else if constexpr (L == 32) {
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
  } else {
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
  }
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

// Workgroup barrier for LDS exchange only: this wave's LDS accesses are
// complete, then s_barrier.  Unlike __syncthreads it does not wait for the
// wave's global loads in flight (prefetches stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- cross-workgroup completion counters ---------------------------------

// Called by every thread of a workgroup after it stored its results, which
// other workgroups read, with st_coherent (below).  Returns true in the
// workgroup that arrives last of `expected` on `counter`, which also resets
// the counter to zero for the next launch.  Each wave first waits until its
// stores are complete (device-coherent stores: visible to every XCD); then
// thread 0 counts the arrival with a relaxed atomic -- no L2 write-back,
// which every XCD would serialise across its workgroups -- and only the last
// workgroup acquires (invalidates its caches, once, by thread 0; the barrier
// orders the other waves' loads after it) before it reads what the others
// wrote.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == expected - 1u);
    if (last) {
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __builtin_amdgcn_s_waitcnt(0);
    }
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// Store of a value that workgroups of the same launch on other XCDs will
// read: a device-coherent store (relaxed agent-scope atomic; on this GPU a
// store that writes through this XCD's L2), complete at device scope once
// the storing wave's memory counter has drained.  Publishing such values
// then needs no L2 write-back (buffer_wbl2), which every XCD serialises
// across its workgroups (a few hundred ns each).
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent16b(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads of values that other workgroups of the same launch stored with the
// stores above.  Device-coherent loads (the same cache policy as a relaxed
// agent-scope atomic load): a line this XCD's L2 still holds from before
// the producers wrote it -- e.g. from an earlier launch over the same
// workspace -- is not returned stale, which an acquire by one thread does
// not guarantee for every line (observed: a stale K-slice partial).
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coherent_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wide device-coherent loads and stores: raw buffer loads / stores with the
// sc1 cache policy (the compiler tracks them like any memory access, waits
// and hazards included), at a byte offset from the base of a buffer that
// covers 2 GB (offsets past it read 0 and write nothing).  Each write-through
// is a partial-line write at the memory side, so fewer, wider stores move
// fewer bytes.
typedef __amdgpu_buffer_rsrc_t coherent_rsrc_t;
__device__ __forceinline__ coherent_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int kCachePolicySc1 = 16;   // sc1: coherent at device scope
__device__ __forceinline__ u32x4 ld_coherent4(coherent_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void st_coherent4(coherent_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCachePolicySc1);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_coherent8(coherent_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCachePolicySc1);
}

// Grid-wide barrier in two halves, for a launch whose workgroups are all
// resident at once.  Words in caller memory, zero before the first use: a
// count, and one flag word per workgroup, kFlagStride words apart (each on a
// line of its own: many workgroups polling one line would queue behind each
// other at the memory side).
// grid_arrive: every wave waits until its stores are complete (the values
// other workgroups read are st_coherent stores, so complete means visible
// at device scope), then thread 0 counts the workgroup on `count` with a
// relaxed atomic and returns the workgroup's flag read before arriving.  The
// workgroup that arrives last of `expected` saw every other arrival, each
// made after that workgroup's stores completed; it resets the count and
// stores flag + 1 into every workgroup's flag.
// grid_wait: thread 0 polls its flag until it moves on, then acquires
// (invalidating this compute unit's L1 and the XCD's L2 lines that might
// hold stale copies) and waits for that to finish; the barrier after it
// orders the other waves' loads after the invalidate (they share those
// caches; one invalidate per wave would be paid 16 times per workgroup).
// Work placed between the halves overlaps the wait.  The count returns to
// zero after every barrier.  A wait gives up after spin_limit polls and sets
// *status to 1, so no wave is left spinning.
constexpr int kFlagStride = 32;   // 128 bytes

__device__ __forceinline__ uint32_t grid_arrive(uint32_t* count, uint32_t* flags, uint32_t expected, int* s_last) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* mine = flags + (size_t)blockIdx.x * kFlagStride;
  uint32_t g = 0u;
  if (threadIdx.x == 0) {
    g = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t old = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == expected - 1u;
    if (last) __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last[0] = last ? 1 : 0;
    s_last[1] = (int)g;
  }
  __syncthreads();
  if (s_last[0] && threadIdx.x < 64) {
    const uint32_t next = (uint32_t)s_last[1] + 1u;
    for (uint32_t i = threadIdx.x; i < gridDim.x; i += 64)
      __hip_atomic_store(flags + (size_t)i * kFlagStride, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return g;
}

__device__ __forceinline__ void grid_wait(const uint32_t* flags, uint32_t g0, int spin_limit, uint32_t* status) {
  if (threadIdx.x == 0) {
    const uint32_t* mine = flags + (size_t)blockIdx.x * kFlagStride;
    for (int n = 0; __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0; ++n) {
      if (n >= spin_limit) {
        __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
}


// Orderable 32-bit key of a logit: larger key <=> larger value (finite
// inputs; -0 is folded into +0 first), so equal keys are equal logits.
// Every finite value maps above 0, which marks "no candidate".
__device__ __forceinline__ uint32_t ord_key(float v) {
  v = v + 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave-wide max of a 32-bit key, uniform result: DPP within rows, then the
// four row maxima by readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));
  return mx(mx((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
            mx((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Wave-wide bitwise OR, uniform result (the same DPP steps as wave_max_u32).
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) | (uint32_t)__builtin_amdgcn_readlane((int)v, 16) |
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) | (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Wave-wide bitwise XOR, uniform result (the same DPP steps as wave_max_u32).
__device__ __forceinline__ uint32_t wave_xor_u32(uint32_t v) {
  v ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
  v ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);
  v ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false);
  v ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) ^ (uint32_t)__builtin_amdgcn_readlane((int)v, 16) ^
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) ^ (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Inclusive prefix sum over the 64 lanes of a wave (classic DPP scan:
// row_shr 1, 2, 4, 8, then row_bcast15 and row_bcast31 carry row totals).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

__device__ __forceinline__ float silu(float z) {
  return z / (1.0f + __expf(-z));
}

// ---- per-workgroup clock stamps (instrumented build) ----------------------
// Built with -DMOE_STAMPS (libmoe_skinny_stamps.so, `bench.py --timeline`),
// thread 0 of workgroup g < kStampWGs of a stamped kernel writes the 100 MHz
// constant clock (s_memrealtime) or a value to slot s of row g of that
// kernel's table: a launch's timeline per workgroup, without a profiler.
// Every translation unit holds its own tables; moe_stamps_route (skinny.hip)
// and moe_stamps_expert (expert.hip) copy or clear them.  Without
// MOE_STAMPS the macros are empty and no table exists.
constexpr int kStampWGs = 1024, kStampSlots = 8;
enum StampKernel { ST_ROUTE = 0, ST_FINISH = 1, ST_UP = 2, ST_DOWN = 3, ST_KERNELS = 4 };
#ifdef MOE_STAMPS
static __device__ unsigned long long g_stamps[ST_KERNELS * kStampWGs * kStampSlots];
__device__ __forceinline__ unsigned long long* stamp_cell(int k, int slot) {
  return &g_stamps[((size_t)k * kStampWGs + blockIdx.x) * kStampSlots + slot];
}
#define MOE_STAMP_VAL(k, slot, v)                                                        \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kStampWGs) *stamp_cell((k), (slot)) = \
        (unsigned long long)(v);                                                          \
  } while (0)
#define MOE_STAMP(k, slot) MOE_STAMP_VAL((k), (slot), __builtin_amdgcn_s_memrealtime())
// the CU the workgroup runs on: HW_ID (wave, SIMD, CU, shader array and
// engine ids) in the low word, XCC_ID in the high word
#define MOE_STAMP_CU(k, slot)                                                                          \
  MOE_STAMP_VAL((k), (slot), (unsigned long long)__builtin_amdgcn_s_getreg((31 << 11) | 4) |           \
                                 ((unsigned long long)__builtin_amdgcn_s_getreg((15 << 11) | 20) << 32))
#else
#define MOE_STAMP_VAL(k, slot, v) \
  do {                            \
  } while (0)
#define MOE_STAMP(k, slot) MOE_STAMP_VAL(k, slot, 0)
#define MOE_STAMP_CU(k, slot) MOE_STAMP_VAL(k, slot, 0)
#endif

}  // namespace moe
