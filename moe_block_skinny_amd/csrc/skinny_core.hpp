// skinny_core.hpp -- the vector-ALU skinny product of a row block: RB
// weight rows over all of K for up to MB activation rows, with the whole
// workgroup (its waves split K and meet in LDS in fixed wave order), and
// the epilogue that stores a result or turns it into a router logit.  Used
// by the skinny kernels and by the fused block kernel, which therefore give
// identical bits.
//
// Source: "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §1 (a
// small-matrix kernel at batch 1-2, split-K at larger batch) and part 1 §3
// (router scores per token).
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace moe {

// Weight row n of the product (clamped to N - 1): a router or dense row, or,
// from E = N - L on, a row of the latent input projection.
template <typename T>
__device__ __forceinline__ const T* product_row(const SkinnyLaunch& a, int n) {
  n = n < a.N ? n : a.N - 1;
  const int E = a.N - a.L;
  return n < E ? reinterpret_cast<const T*>(a.W) + (size_t)n * a.K
               : reinterpret_cast<const T*>(a.Wlat) + (size_t)(n - E) * a.K;
}

// Result (t, n) of the product: a router logit (+ bias), a latent projection
// value, or a stored value.
__device__ __forceinline__ void finish_value(const SkinnyLaunch& a, int t, int n, float v) {
  const int E = a.N - a.L;
  if (a.router && n >= E) {
    const size_t o = (size_t)t * a.L + (n - E);
    if (a.latent_bf16) reinterpret_cast<bf16_t*>(a.latent_out)[o] = f32_to_bf16(v);
    else reinterpret_cast<float*>(a.latent_out)[o] = v;
  } else if (a.router) {
    if (a.bias) v += a.bias[(size_t)t * a.bias_ld + n];
    st_coherent(&a.logits[(size_t)t * E + n], v);   // read by other workgroups of the launch
    if (a.logits_out) a.logits_out[(size_t)t * E + n] = v;
  } else {
    const size_t o = (size_t)t * a.N + n;
    // the residual is read and the result stored by the same thread, so Y
    // may be R itself (an in-place residual update)
    if (a.R) v += a.bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.R)[o]) : reinterpret_cast<const float*>(a.R)[o];
    if (a.y_bf16) reinterpret_cast<bf16_t*>(a.Y)[o] = f32_to_bf16(v);
    else reinterpret_cast<float*>(a.Y)[o] = v;
  }
}

// Rows n0 .. n0 + RB - 1, all K, with the whole workgroup.  Wave w takes the
// 64-chunk blocks w, w + NW, w + 2 NW, ... of every row (one 1 KB segment per
// row per load instruction); U blocks per lane are in flight.  s_red holds
// NW * RB * MB floats.  Ends after a barrier; threads < RB * MB finish one
// value each.
template <typename T, int RB, int MB, int U>
__device__ __forceinline__ void valu_rows(const SkinnyLaunch& a, int n0, float* s_red) {
  constexpr int VEC = Elem<T>::VEC;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const T* X = reinterpret_cast<const T*>(a.X);
  const T* wr[RB];
  const T* xr[MB];
#pragma unroll
  for (int r = 0; r < RB; ++r) wr[r] = product_row<T>(a, n0 + r);
#pragma unroll
  for (int t = 0; t < MB; ++t) xr[t] = X + (size_t)(t < a.M ? t : 0) * a.K;
  const int C = a.K / VEC;
  float acc[RB][MB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int t = 0; t < MB; ++t) acc[r][t] = 0.f;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int blk = wave; blk * 64 < C; blk += nw * U) {
    u32x4 wv[U][RB], xv[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (blk + u * nw) * 64 + lane;
      const bool ok = c < C;
#pragma unroll
      for (int r = 0; r < RB; ++r) wv[u][r] = ok ? ld128_stream(wr[r] + (size_t)c * VEC) : zero;
#pragma unroll
      for (int t = 0; t < MB; ++t) xv[u][t] = (ok && t < a.M) ? ld128(xr[t] + (size_t)c * VEC) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MB; ++t) acc[r][t] = dot_chunk(wv[u][r], xv[u][t], acc[r][t], T());
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      const float v = group_sum<64>(acc[r][t]);
      if (lane == 0) s_red[(wave * RB + r) * MB + t] = v;
    }
  __syncthreads();
  if (threadIdx.x < RB * MB) {
    const int r = threadIdx.x / MB, t = threadIdx.x % MB, n = n0 + r;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += s_red[(w * RB + r) * MB + t];
    if (n < a.N && t < a.M) finish_value(a, t, n, v);
  }
}

// valu_rows<T, RB, MB, U> of a workgroup of NV waves, computed by one of NR
// waves (NV a multiple of NR) with the same bits: wave w plays waves w,
// w + NR, w + 2 NR, ...; each played wave keeps its own sums over its own
// blocks in its own order, is reduced on its own, and the NV sums meet in
// LDS in wave order as in valu_rows.  The played waves' loads of one block
// group go out together.  Rows n0 .. n0 + RB - 1 of W [N][K] against the M
// rows of X [M][K]; fin(t, n, v) takes each result (threads < RB * MB).
// s_red holds NV * RB * MB floats.  Ends after a barrier.
struct RowsSrc {
  const void* X;
  const void* W;
  int M, N, K;
};

template <typename T, int RB, int MB, int U, int NV, int NR, typename Fin>
__device__ __forceinline__ void valu_rows_as(const RowsSrc& s, int n0, float* s_red, Fin&& fin) {
  static_assert(NV % NR == 0, "whole played waves per wave");
  constexpr int VEC = Elem<T>::VEC;
  constexpr int J = NV / NR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const T* X = reinterpret_cast<const T*>(s.X);
  const T* wr[RB];
  const T* xr[MB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
    wr[r] = reinterpret_cast<const T*>(s.W) + (size_t)(n0 + r < s.N ? n0 + r : s.N - 1) * s.K;
#pragma unroll
  for (int t = 0; t < MB; ++t) xr[t] = X + (size_t)(t < s.M ? t : 0) * s.K;
  const int C = s.K / VEC;
  float acc[J][RB][MB];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int t = 0; t < MB; ++t) acc[j][r][t] = 0.f;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // played wave v = wave + NR j takes blocks v + base + u NV (base = 0,
  // NV U, ...; u < U), as wave v of valu_rows; a block group none of this
  // wave's played waves has is skipped (a played wave past the range adds
  // zero products, which leave its sums as they are)
  for (int base = 0; (wave + base) * 64 < C; base += NV * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((wave + base + u * NV) * 64 >= C) break;
      u32x4 wv[J][RB], xv[J][MB];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = (wave + NR * j + base + u * NV) * 64 + lane;
        const bool ok = c < C;
#pragma unroll
        for (int r = 0; r < RB; ++r) wv[j][r] = ok ? ld128_stream(wr[r] + (size_t)c * VEC) : zero;
#pragma unroll
        for (int t = 0; t < MB; ++t) xv[j][t] = (ok && t < s.M) ? ld128(xr[t] + (size_t)c * VEC) : zero;
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int t = 0; t < MB; ++t) acc[j][r][t] = dot_chunk(wv[j][r], xv[j][t], acc[j][r][t], T());
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        const float v = group_sum<64>(acc[j][r][t]);
        if (lane == 0) s_red[((wave + NR * j) * RB + r) * MB + t] = v;
      }
  __syncthreads();
  if (threadIdx.x < RB * MB) {
    const int r = threadIdx.x / MB, t = threadIdx.x % MB, n = n0 + r;
    float v = 0.f;
    for (int w = 0; w < NV; ++w) v += s_red[(w * RB + r) * MB + t];
    if (n < s.N && t < s.M) fin(t, n, v);
  }
}

}  // namespace moe
