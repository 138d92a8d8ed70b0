// mfma_core.hpp -- the matrix-core product of 64 weight rows (4 waves x 16
// rows, the A operand of v_mfma_f32_16x16x32_bf16) with up to 64 activation
// rows (NT tiles of 16 tokens, the B operand) over a range of K steps of 32.
// Used by the dense skinny product and by the experts' gate/up once a batch
// x rows is a dense contraction.
//
// Source: "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §1 (the kernel
// shape follows the batch: matrix cores only once the product is a real
// contraction) and part 1 §4 (small-batch decode is bound by weight reads).
//
// The activation rows pass through LDS in chunks of kChunk steps: the
// workgroup loads each chunk once with coalesced 128-bit loads and all four
// waves read it as their B operand (per-wave loads of a 16-token tile would
// touch 16 cache lines per instruction and move NT times the weight bytes
// again through the L1 path).  Every load is issued unconditionally from a
// clamped address, so the compiler never waits for all loads in flight at a
// branch.  Barriers order LDS only.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMfmaRows = 64;
constexpr unsigned kSlotStride = 256;   // CUs: workgroups g and g + 256 share one
constexpr int kMfmaWaves = 4;
constexpr int kChunk = 8;                   // 32-steps per LDS chunk
constexpr int kXRow = kChunk * 64 + 16;     // bytes per token row in LDS (padded)

template <int NT, int U = 2>
struct MfmaX {
  static constexpr int kPieces = NT * 16 * kChunk * 4;                  // 16-byte pieces per chunk
  static constexpr int kPerThread = kPieces / (kMfmaWaves * 64);
  static_assert(kPieces % (kMfmaWaves * 64) == 0, "whole pieces per thread");
  static constexpr int kBufBytes = NT * 16 * kXRow;                     // one chunk of activations
  static constexpr int kLdsBytes = U * kBufBytes;                       // U chunks per iteration
};

// Weight rows of a wave, as mfma_rows takes them: this lane's row of rows
// 0-7 (lane%8) and of rows 8-15, at element offset 8*(lane/8).
__device__ __forceinline__ int mfma_row_a() { return threadIdx.x & 7; }
__device__ __forceinline__ int mfma_row_b() { return 8 + (threadIdx.x & 7); }
__device__ __forceinline__ int mfma_col_off() { return ((threadIdx.x & 63) >> 3) * 8; }

// Token of this thread's i-th activation piece (pieces p = tid + 256 i of a
// chunk: token p / (4 kChunk), piece p % (4 kChunk)).
template <int NT>
__device__ __forceinline__ int mfma_piece_token(int i) {
  return (int)(threadIdx.x + i * kMfmaWaves * 64) / (4 * kChunk);
}

// acc[nt] += W[16 rows of this wave] . X[tokens nt*16 .. +15]^T over steps
// s0 .. s1-1 (s0 < s1).
//
// Weight loads move whole 128-byte lines: per pair of steps (64 elements)
// one instruction loads rows 0-7 of the wave (lane l: row l%8, elements
// 8*(l/8) .. +7 of the pair) and one rows 8-15.  The MFMA A operand wants
// lane l = R + 16 g to hold row R; so the first step of the pair takes K
// positions 16g .. 16g+7 of the 64 and the second 16g+8 .. 16g+15, which
// lane l holds directly for rows R < 8 (first step) and R >= 8 (second
// step), and lane l -+ 8 holds otherwise: a DPP row shift by 8.  The
// activations in LDS are read with the same K positions.  (Loading 16 rows
// x 64 bytes per instruction touched every line twice and cost ~3 us on the
// dense product.)
//
// wa / wb: this lane's row (lane%8) of the wave's rows 0-7 / 8-15, already
// offset by 8*(lane/8) elements; read only when oka / okb.  xrow[i]:
// activation row of this thread's i-th piece token, read only when xok[i]
// (else zeros go to LDS).  X rows and W rows hold K = 32 * (steps of the
// whole row) elements; steps index both.
//
// The work is cut in stages of U chunks (U * kChunk steps).  A stage's
// loads are issued unconditionally: steps past s1 read a cached activation
// row (weights) or the last step again (activations), and hold zero
// weights and activations when multiplied, so every chunk is multiplied
// whole, without a branch per step.

// Activations of the stage at step c (clamped into range).
template <int NT, int U>
__device__ __forceinline__ void mfma_issue_x(const bf16_t* const (&xrow)[MfmaX<NT>::kPerThread], int c, int s1,
                                             u32x4 (&xv)[U][MfmaX<NT>::kPerThread]) {
  constexpr int PPT = MfmaX<NT>::kPerThread;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int q = (tid + i * kMfmaWaves * 64) % (4 * kChunk);
      const int j = c + u * kChunk + q / 4;
      const int jc = j < s1 ? j : s1 - 1;
      xv[u][i] = ld128(xrow[i] + (size_t)jc * 32 + (q & 3) * 8);
    }
}

// Weights of the stage at step c (a lane whose step is past s1 reads the
// cached row `spare`).
template <int U>
__device__ __forceinline__ void mfma_issue_w(const bf16_t* wa, const bf16_t* wb, const bf16_t* spare, int c, int s1,
                                             u32x4 (&va)[U][kChunk / 2], u32x4 (&vb)[U][kChunk / 2]) {
  const int hi_step = (threadIdx.x & 63) >> 5;   // lanes 32-63 hold the pair's second step
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int p = 0; p < kChunk / 2; ++p) {
      const int j = c + u * kChunk + 2 * p;
      const bool in = j + hi_step < s1;
      va[u][p] = ld128_stream(in ? wa + (size_t)j * 32 : spare);
      vb[u][p] = ld128_stream(in ? wb + (size_t)j * 32 : spare);
    }
}

// The stage's activations into the LDS buffer `buf` (U chunks); zeros for
// tokens past the batch and steps past s1.
template <int NT, int U>
__device__ __forceinline__ void mfma_store_x(const u32x4 (&xv)[U][MfmaX<NT>::kPerThread],
                                             const bool (&xok)[MfmaX<NT>::kPerThread], int c, int s1,
                                             unsigned char* buf) {
  constexpr int PPT = MfmaX<NT>::kPerThread;
  const int tid = threadIdx.x;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pc = tid + i * kMfmaWaves * 64;
      const int t = pc / (4 * kChunk), q = pc % (4 * kChunk);
      const bool ok = xok[i] && c + u * kChunk + q / 4 < s1;
      *reinterpret_cast<u32x4*>(buf + u * MfmaX<NT>::kBufBytes + t * kXRow + q * 16) = ok ? xv[u][i] : zero;
    }
}

// The stage's products: weights in registers, activations from `buf`.
template <int NT, int U>
__device__ __forceinline__ void mfma_compute(const u32x4 (&va)[U][kChunk / 2], const u32x4 (&vb)[U][kChunk / 2],
                                             bool oka, bool okb, int c, int s1, const unsigned char* buf,
                                             f32x4 (&acc)[NT]) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const bool low = row < 8;
  const int hi_step = lane >> 5;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int p = 0; p < kChunk / 2; ++p) {
      const bool in = c + u * kChunk + 2 * p + hi_step < s1;
      const u32x4 a = (in && oka) ? va[u][p] : zero;
      const u32x4 b = (in && okb) ? vb[u][p] : zero;
      u32x4 ev, od;   // A operands of the pair's first and second step
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b_up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b[e], 0x118, 0xf, 0xf, false);  // row_shr:8
        const uint32_t a_dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a[e], 0x108, 0xf, 0xf, false);  // row_shl:8
        ev[e] = low ? a[e] : b_up;
        od[e] = low ? a_dn : b[e];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const unsigned char* xb = buf + u * MfmaX<NT>::kBufBytes + (nt * 16 + row) * kXRow + p * 128 + kq * 32;
        const u32x4 xe = *reinterpret_cast<const u32x4*>(xb);
        const u32x4 xo = *reinterpret_cast<const u32x4*>(xb + 16);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ev),
                                                          __builtin_bit_cast(bf16x8, xe), acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, od),
                                                          __builtin_bit_cast(bf16x8, xo), acc[nt], 0, 0, 0);
      }
    }
}

// One stage in flight at a time: each iteration requests the activations
// and then the weights of its stage before waiting for any of them, and
// leaves nothing in flight across the loop's back edge (a load still in
// flight there made the compiler copy its registers at the back edge and
// wait for every load).  s_x: MfmaX<NT, U>::kLdsBytes.
template <int NT, int U>
__device__ __forceinline__ void mfma_rows(const bf16_t* wa, bool oka, const bf16_t* wb, bool okb,
                                          const bf16_t* const (&xrow)[MfmaX<NT>::kPerThread],
                                          const bool (&xok)[MfmaX<NT>::kPerThread], int s0, int s1,
                                          unsigned char* s_x, f32x4 (&acc)[NT]) {
  constexpr int PPT = MfmaX<NT>::kPerThread;
  constexpr int NP = kChunk / 2;
  s0 = __builtin_amdgcn_readfirstlane(s0);
  s1 = __builtin_amdgcn_readfirstlane(s1);
  for (int c = s0; c < s1; c += U * kChunk) {
    u32x4 xv[U][PPT], va[U][NP], vb[U][NP];
    mfma_issue_x<NT, U>(xrow, c, s1, xv);
    __builtin_amdgcn_sched_barrier(0);   // activations first: the LDS stores wait only for them
    mfma_issue_w<U>(wa, wb, xrow[0], c, s1, va, vb);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();              // the previous iteration's LDS reads are done
    __builtin_amdgcn_sched_barrier(0);
    mfma_store_x<NT, U>(xv, xok, c, s1, s_x);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);   // no weight use above the barrier (it would wait there)
    mfma_compute<NT, U>(va, vb, oka, okb, c, s1, s_x, acc);
  }
}

// Two stages in flight: the loads of stage i+1 are requested before the
// products of stage i, whose weights sit in the other register set and
// whose activations sit in the other LDS buffer.  Unrolled by two so each
// register set keeps its registers across the back edge (the set in
// flight there is the one the next iteration multiplies first).  One
// barrier per stage: it publishes the stage's activations and retires the
// reads of the buffer the next stores overwrite.
// s_x: 2 * MfmaX<NT, U>::kLdsBytes.  TURNS: a grid of two workgroups per
// CU, which take turns at the higher wave priority (below).
template <int NT, int U, bool TURNS = false>
__device__ __forceinline__ void mfma_rows_db(const bf16_t* wa, bool oka, const bf16_t* wb, bool okb,
                                             const bf16_t* const (&xrow)[MfmaX<NT>::kPerThread],
                                             const bool (&xok)[MfmaX<NT>::kPerThread], int s0, int s1,
                                             unsigned char* s_x, f32x4 (&acc)[NT]) {
  constexpr int PPT = MfmaX<NT>::kPerThread;
  constexpr int NP = kChunk / 2;
  constexpr int G = U * kChunk;
  s0 = __builtin_amdgcn_readfirstlane(s0);
  s1 = __builtin_amdgcn_readfirstlane(s1);
  unsigned char* buf0 = s_x;
  unsigned char* buf1 = s_x + MfmaX<NT, U>::kLdsBytes;
  u32x4 xv[U][PPT], va0[U][NP], vb0[U][NP], va1[U][NP], vb1[U][NP];
  mfma_issue_x<NT, U>(xrow, s0, s1, xv);
  __builtin_amdgcn_sched_barrier(0);
  mfma_issue_w<U>(wa, wb, xrow[0], s0, s1, va0, vb0);
  __builtin_amdgcn_sched_barrier(0);
  mfma_store_x<NT, U>(xv, xok, s0, s1, buf0);
  __builtin_amdgcn_sched_barrier(0);
  for (int c = s0;; c += 2 * G) {
    // the two workgroups of a CU (g and g + kSlotStride) take turns at the
    // higher wave priority, a double stage each: left to age order the CU
    // serves the older one first and the younger then streams alone at a
    // lower rate (clock stamps at batch 64: identical tiles took 54 us on
    // the first and 67 us on the second; with the turns the block took 133
    // instead of 134.8 us)
    if constexpr (TURNS) {
      if (((c - s0) / (2 * G) + (blockIdx.x >= kSlotStride ? 1 : 0)) & 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    mfma_issue_x<NT, U>(xrow, c + G, s1, xv);
    __builtin_amdgcn_sched_barrier(0);
    mfma_issue_w<U>(wa, wb, xrow[0], c + G, s1, va1, vb1);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfma_compute<NT, U>(va0, vb0, oka, okb, c, s1, buf0, acc);
    __builtin_amdgcn_sched_barrier(0);
    mfma_store_x<NT, U>(xv, xok, c + G, s1, buf1);
    __builtin_amdgcn_sched_barrier(0);
    if (c + G >= s1) break;
    mfma_issue_x<NT, U>(xrow, c + 2 * G, s1, xv);
    __builtin_amdgcn_sched_barrier(0);
    mfma_issue_w<U>(wa, wb, xrow[0], c + 2 * G, s1, va0, vb0);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfma_compute<NT, U>(va1, vb1, oka, okb, c + G, s1, buf1, acc);
    __builtin_amdgcn_sched_barrier(0);
    mfma_store_x<NT, U>(xv, xok, c + 2 * G, s1, buf0);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 * G >= s1) break;
  }
}

}  // namespace moe
