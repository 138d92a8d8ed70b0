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

// Token of this thread's i-th activation piece (pieces p = tid + 256 i of a
// chunk: token p / (4 kChunk), piece p % (4 kChunk)).
template <int NT>
__device__ __forceinline__ int mfma_piece_token(int i) {
  return (int)(threadIdx.x + i * kMfmaWaves * 64) / (4 * kChunk);
}

// acc[nt] += W[16 rows of this wave] . X[tokens nt*16 .. +15]^T over steps
// s0 .. s1-1 (s0 < s1).  wr: this lane's weight row (row lane%16 of the
// wave's 16), already offset by (lane/16)*8 elements, read only when wok.
// xrow[i]: activation row of this thread's i-th piece token, read only when
// xok[i] (else zeros go to LDS).  X rows and W rows hold K = 32 * (steps of
// the whole row) elements; steps index both.  s_x: MfmaX<NT, U>::kLdsBytes.
//
// Each iteration requests the activations and then the weights of U chunks
// before waiting for any of them, so a wave keeps U * 8 KB of weights in
// flight, and leaves nothing in flight
// across the loop's back edge (a load still in flight there made the
// compiler copy its registers at the back edge and wait for every load).
// Chunks past s1 hold zero activations (weight loads from a cached row), so
// every chunk is multiplied whole, without a branch per step.
template <int NT, int U>
__device__ __forceinline__ void mfma_rows(const bf16_t* wr, bool wok, const bf16_t* const (&xrow)[MfmaX<NT>::kPerThread],
                                          const bool (&xok)[MfmaX<NT>::kPerThread], int s0, int s1,
                                          unsigned char* s_x, f32x4 (&acc)[NT]) {
  constexpr int PPT = MfmaX<NT>::kPerThread;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  s0 = __builtin_amdgcn_readfirstlane(s0);
  s1 = __builtin_amdgcn_readfirstlane(s1);
  for (int c = s0; c < s1; c += U * kChunk) {
    u32x4 xv[U][PPT], wv[U][kChunk];
    // activations of the iteration's chunks (clamped into range) ...
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int q = (tid + i * kMfmaWaves * 64) % (4 * kChunk);
        const int j = c + u * kChunk + q / 4;
        const int jc = j < s1 ? j : s1 - 1;
        xv[u][i] = ld128(xrow[i] + (size_t)jc * 32 + (q & 3) * 8);
      }
    __builtin_amdgcn_sched_barrier(0);   // activations first: st_x waits only for them
    // ... then the weights (steps past s1: a cached activation row)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int v = 0; v < kChunk; ++v) {
        const int j = c + u * kChunk + v;
        wv[u][v] = ld128_stream(j < s1 ? wr + (size_t)j * 32 : xrow[0]);
      }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();              // the previous iteration's LDS reads are done
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + i * kMfmaWaves * 64;
        const int t = pc / (4 * kChunk), q = pc % (4 * kChunk);
        const bool ok = xok[i] && c + u * kChunk + q / 4 < s1;
        *reinterpret_cast<u32x4*>(s_x + u * MfmaX<NT>::kBufBytes + t * kXRow + q * 16) = ok ? xv[u][i] : zero;
      }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);   // no weight use above the barrier (it would wait there)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int v = 0; v < kChunk; ++v) {
        const bool ok = wok && c + u * kChunk + v < s1;
        const u32x4 av = ok ? wv[u][v] : zero;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x4 bv = *reinterpret_cast<const u32x4*>(s_x + u * MfmaX<NT>::kBufBytes + (nt * 16 + row) * kXRow +
                                                           (v * 4 + kq) * 16);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                            __builtin_bit_cast(bf16x8, bv), acc[nt], 0, 0, 0);
        }
      }
  }
}

}  // namespace moe
