// skinny.hip -- skinny products Y = X . W^T with few activation rows, used
// for the dense attention input projection and for router scoring, plus the
// router's top-k selection, gate weights and token->expert plan.
//
// Sources (web pages on the Kimi K3 specialised decode path):
//   [WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §1
//     (tuning shapes to the workload): a small-matrix kernel at batch 1-2,
//     split-K at larger batch to spread the product over more GPU workers,
//     launches sized to fill the GPU; part 1 §3 (MoE scheduling): router
//     scores per token before the experts run; part 1 §4: small-batch decode
//     is bound by reading weights from memory.
//   [AREX] "vLLM 宣布 Kimi K3 在 GB300 NVL72 上实现 batch 1 解码 842
//     tokens/s", section "每层从 23 个内核减到 13 个" (same kernel choice).
//
// Three kernel shapes, all streaming every weight byte exactly once with
// 128-bit loads (one 1 KB row segment per wave instruction):
//   gemv   : M <= 2 activation rows; a workgroup owns 2 weight rows, its
//            waves split K, v_dot2_f32_bf16 (or fp32 FMA) accumulates.
//   splitk : M <= 8; a workgroup owns 4 weight rows, so each activation chunk
//            a lane loads is reused 4 times; its waves split K.
//   mfma   : M <= 64 (bf16); v_mfma_f32_16x16x32_bf16 with 16 weight rows as
//            the A operand and up to four 16-token tiles as B, used once
//            batch x rows is a dense contraction; its waves split K.
// Split-K stays inside the workgroup: each wave reduces its lanes, the waves
// meet in LDS and are summed in fixed wave order, so results are
// deterministic and no partial sum ever goes through global memory (a
// device-wide fence on this GPU writes back and invalidates the L2 of every
// XCD, far dearer than an LDS exchange).  The number of waves per workgroup
// is chosen on the host so that a launch has ~1.5k waves in flight.
// In router mode every workgroup arrives once on a completion counter; the
// last one selects the top-k experts per token, computes their softmax
// weights and builds the plan.

#include "common.hpp"
#include "expert_core.hpp"
#include "internal.hpp"

namespace moe {


// ---- epilogue ---------------------------------------------------------------

__device__ __forceinline__ void finish_value(const SkinnyLaunch& a, int t, int n, float v) {
  if (a.router) {
    if (a.bias) v += a.bias[(size_t)t * a.bias_ld + n];
    a.logits[(size_t)t * a.N + n] = v;
    if (a.logits_out) a.logits_out[(size_t)t * a.N + n] = v;
  } else if (a.y_bf16) {
    reinterpret_cast<bf16_t*>(a.Y)[(size_t)t * a.N + n] = f32_to_bf16(v);
  } else {
    reinterpret_cast<float*>(a.Y)[(size_t)t * a.N + n] = v;
  }
}

// ---- router finish: top-k, weights, plan (one workgroup) ------------------

// Top-k of every token: waves take tokens wave, wave + nw, ..., with the
// logits of four tokens loaded before any is used (one memory round trip
// per group); ids and weights go to LDS and to the caller's arrays.
__device__ __forceinline__ void topk_tokens(const SkinnyLaunch& a, TopkScratch* s_tk, int32_t* s_ids, float* s_w) {
  constexpr int QB = 4;
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
  const int E = a.N, M = a.M, k = a.k;
  for (int t0 = wave; t0 < M; t0 += nw * QB) {
    float lv[QB][kNI];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int t = t0 + nw * q;
      load_logit_row(a.logits, t < M ? t : M - 1, E, lv[q]);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int t = t0 + nw * q;
      if (t < M)
        topk_wave(lv[q], E, k, s_tk[wave], s_ids + t * k, s_w + t * k, a.topk_ids + (size_t)t * k,
                  a.topk_w + (size_t)t * k);
    }
  }
}

__device__ __forceinline__ void route_finish(const SkinnyLaunch& a) {
  __shared__ int32_t s_ids[kMaxB * kMaxK];
  __shared__ float s_w[kMaxB * kMaxK];
  __shared__ TopkScratch s_tk[16];
  __shared__ unsigned long long s_mask[kMaxE];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_act[kMaxE];
  __shared__ int s_n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int M = a.M, E = a.N, k = a.k, nslot = M * k;

  topk_tokens(a, s_tk, s_ids, s_w);
  __syncthreads();
  if (nslot <= 64) {  // one wave sorts the slots
    if (wave == 0) plan_wave(s_ids, nslot, E, reinterpret_cast<int*>(s_tk), a.plan, nullptr);
    return;
  }
  for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();
  // bit t of s_mask[e] is set when token t selected expert e (B <= 64)
  for (int s = tid; s < nslot; s += blockDim.x) atomicOr(&s_mask[s_ids[s]], 1ull << (s / k));
  __syncthreads();
  // exclusive prefix sums over experts of slot counts and of "is active",
  // packed in one int (counts <= 1024 in the low half, actives <= 512 in
  // the high half): a DPP scan per wave, wave totals through LDS.
  __shared__ int s_wtot[16];
  const int nwv = (E + 63) >> 6;
  int incl = 0, packed = 0;
  if (tid < nwv * 64) {
    const int c = tid < E ? __popcll(s_mask[tid]) : 0;
    packed = c | ((c > 0 ? 1 : 0) << 16);
    incl = wave_incl_scan(packed);
    if (lane == 63) s_wtot[wave] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wtot[w];
    const int ex = base + incl - packed;
    s_cnt[tid] = ex & 0xffff;
    s_act[tid] = ex >> 16;
  }
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < nwv; ++w) tot += s_wtot[w];
    s_n = tot >> 16;
  }
  __syncthreads();
  const int n = s_n;
  const int maxa = nslot < E ? nslot : E;
  int32_t* active = a.plan + 1;
  int32_t* offs = a.plan + 1 + maxa;
  int32_t* slots = a.plan + 2 + 2 * maxa;
  if (tid == 0) a.plan[0] = n;
  for (int e = tid; e < E; e += blockDim.x)
    if (s_mask[e]) { active[s_act[e]] = e; offs[s_act[e]] = s_cnt[e]; }
  for (int i = n + tid; i < maxa; i += blockDim.x) active[i] = -1;
  for (int i = n + tid; i <= maxa; i += blockDim.x) offs[i] = nslot;
  for (int s = tid; s < nslot; s += blockDim.x) {
    int e = s_ids[s], t = s / k;
    unsigned long long below = (t == 0) ? 0ull : (s_mask[e] & ((1ull << t) - 1ull));
    slots[s_cnt[e] + __popcll(below)] = s;
  }
}

// Router tail: every router workgroup arrives once; the last runs the finish.
__device__ __forceinline__ void router_tail(const SkinnyLaunch& a) {
  __shared__ int s_flag;
  if (!a.router || !a.finish) return;
  if (!arrive_last(a.done_counter, (uint32_t)a.router_wgs, &s_flag)) return;
  route_finish(a);
}

// ---- vector-ALU kernels (gemv / splitk) ----------------------------------

// Workgroup: RB weight rows starting at blockIdx.x * RB, all K.  Wave w
// takes the 64-chunk blocks w, w + NW, w + 2 NW, ... of every row (one 1 KB
// segment per row per load instruction); U blocks per lane are in flight.
template <typename T, int RB, int MB, int U, bool ROUTER>
__global__ __launch_bounds__(1024) void skinny_valu_kernel(SkinnyLaunch a) {
  constexpr int VEC = Elem<T>::VEC;
  __shared__ float s_red[16 * RB * MB];
  if (ROUTER && (int)blockIdx.x >= a.router_wgs) {  // shared expert gate/up
    shared_up_task<T, kPathValu>(a.ex, blockIdx.x - a.router_wgs, s_red);
    return;
  }
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * RB;
  const T* W = reinterpret_cast<const T*>(a.W);
  const T* X = reinterpret_cast<const T*>(a.X);
  const T* wr[RB];
  const T* xr[MB];
#pragma unroll
  for (int r = 0; r < RB; ++r) wr[r] = W + (size_t)(n0 + r < a.N ? n0 + r : a.N - 1) * a.K;
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
  if constexpr (ROUTER) router_tail(a);
}

// ---- MFMA kernel (bf16) --------------------------------------------------

// Workgroup: 16 weight rows (A operand: lane l holds row l%16, K elements
// 8*(l/16) .. +7 of each 32-wide step) against NT tiles of 16 activation
// rows (B operand: lane l holds token l%16 of the tile, same K elements).
// Wave w takes the 4-step blocks w, w + NW, ... (128 K elements per row, 256
// contiguous bytes, over four back-to-back loads).  The accumulator of tile
// nt holds, in lane l, rows 4*(l/16)+i, token l%16.
template <int NT, bool ROUTER>
__global__ __launch_bounds__(512) void skinny_mfma_kernel(SkinnyLaunch a) {
  constexpr int SB = 4;  // K steps per block
  extern __shared__ float s_dyn[];  // [NW][NT][64][4]
  if (ROUTER && (int)blockIdx.x >= a.router_wgs) {  // shared expert gate/up
    shared_up_task<bf16_t, kPathMfma>(a.ex, blockIdx.x - a.router_wgs, s_dyn);
    return;
  }
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int J = a.K / 32;
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.W);
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  const bf16_t* wr = W + (size_t)(n0 + row < a.N ? n0 + row : a.N - 1) * a.K;
  const bf16_t* xr[NT];
  bool xok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tok = nt * 16 + row;
    xok[nt] = tok < a.M;
    xr[nt] = X + (size_t)(xok[nt] ? tok : 0) * a.K;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_kloop<NT, SB>(wr, n0 + row < a.N, xr, xok, kq, J, wave, nw, acc);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_dyn[((wave * NT + nt) * 64 + lane) * 4 + i] = acc[nt][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < NT * 256; idx += blockDim.x) {
    const int nt = idx >> 8, l = (idx >> 2) & 63, i = idx & 3;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += s_dyn[((w * NT + nt) * 64 + l) * 4 + i];
    const int n = n0 + 4 * (l >> 4) + i, t = nt * 16 + (l & 15);
    if (n < a.N && t < a.M) finish_value(a, t, n, v);
  }
  if constexpr (ROUTER) router_tail(a);
}

// ---- host side -----------------------------------------------------------

int skinny_rows_per_block(int variant, int router) {
  if (variant == VAR_MFMA) return 16;
  if (router || variant == VAR_SPLITK) return 4;
  return 2;
}

// Waves per workgroup (the in-workgroup K split): enough for ~1536 waves per
// launch, at most 16, and no wave with less than one 1 KB block per row.
// The router takes 16 waves outright: it has few rows, and each of its
// workgroups pays one device-scope release on the completion counter.
int skinny_default_splits(int variant, int bf16, int M, int N, int K, int router) {
  // The router's finish needs one thread per expert (E <= 512): its
  // workgroups always have 16 waves (vector) or 8 (MFMA); waves beyond the
  // K range just idle through the product.
  if (router) return variant == VAR_MFMA ? 8 : 16;
  const int rows = skinny_rows_per_block(variant, router);
  const int nwg = (N + rows - 1) / rows;
  int nw = (1536 + nwg - 1) / nwg;
  int maxw = variant == VAR_MFMA ? (K / 32) / 4 : (K / (bf16 ? 8 : 4)) / 64;
  if (maxw > (variant == VAR_MFMA ? 8 : 16)) maxw = variant == VAR_MFMA ? 8 : 16;
  if (variant == VAR_MFMA) {
    // dynamic LDS nw * nt KB plus the router's static LDS within 64 KB
    const int nt = (M + 15) / 16;
    if (maxw > 40 / nt) maxw = 40 / nt;
  }
  if (maxw < 1) maxw = 1;
  if (nw > maxw) nw = maxw;
  if (nw < 1) nw = 1;
  return nw;
}

// Shared-expert gate/up workgroups appended to the router grid: the vector
// shape takes one pair per wave, the MFMA shape four pairs per workgroup.
int shared_up_tiles_host(const ExpertLaunch& ex, int nw) {
  const bool mfma = expert_paths(ex.bf16, ex.force, ex.B) != kPathValu;
  const int pp = nw / 2;
  return mfma ? (ex.Is + kUpPairsMfma - 1) / kUpPairsMfma : (ex.Is + pp - 1) / pp;
}

// Router launches take the instantiation with the router's finish and side
// job compiled in (and their LDS); plain products the one without.
template <typename K>
static void launch_as(const SkinnyLaunch& a, K router_kernel, K plain_kernel, dim3 grid, dim3 block, size_t lds,
                      hipStream_t st) {
  if (a.router) launch(K_ROUTE, router_kernel, grid, block, (uint32_t)lds, st, a);
  else launch(K_SKINNY, plain_kernel, grid, block, (uint32_t)lds, st, a);
}

hipError_t launch_skinny(const SkinnyLaunch& a0, hipStream_t st, char* desc, size_t desc_len) {
  SkinnyLaunch a = a0;
  const int rows = skinny_rows_per_block(a.variant, a.router);
  const int nwg = (a.N + rows - 1) / rows;
  const int nw = a.S;
  a.router_wgs = nwg;
  const int extra = (a.router && a.ex.Ws13) ? shared_up_tiles_host(a.ex, nw) : 0;
  a.shared_tiles = extra;
  dim3 grid((unsigned)(nwg + extra)), block((unsigned)(64 * nw));
  const char* name = "?";
  if (a.variant == VAR_MFMA) {
    const int nt = (a.M + 15) / 16;
    const size_t lds = (size_t)nw * nt * 256 * sizeof(float);
    switch (nt) {
      case 1: launch_as(a, skinny_mfma_kernel<1, true>, skinny_mfma_kernel<1, false>, grid, block, lds, st); break;
      case 2: launch_as(a, skinny_mfma_kernel<2, true>, skinny_mfma_kernel<2, false>, grid, block, lds, st); break;
      case 3: launch_as(a, skinny_mfma_kernel<3, true>, skinny_mfma_kernel<3, false>, grid, block, lds, st); break;
      default: launch_as(a, skinny_mfma_kernel<4, true>, skinny_mfma_kernel<4, false>, grid, block, lds, st); break;
    }
    name = "mfma";
  } else if (a.router) {
    name = a.variant == VAR_SPLITK ? "splitk" : "gemv";
    if (a.bf16) {
      if (a.M <= 1) launch(K_ROUTE, skinny_valu_kernel<bf16_t, 4, 1, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 2) launch(K_ROUTE, skinny_valu_kernel<bf16_t, 4, 2, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 4) launch(K_ROUTE, skinny_valu_kernel<bf16_t, 4, 4, 2, true>, grid, block, 0, st, a);
      else launch(K_ROUTE, skinny_valu_kernel<bf16_t, 4, 8, 1, true>, grid, block, 0, st, a);
    } else {
      if (a.M <= 1) launch(K_ROUTE, skinny_valu_kernel<float, 4, 1, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 2) launch(K_ROUTE, skinny_valu_kernel<float, 4, 2, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 4) launch(K_ROUTE, skinny_valu_kernel<float, 4, 4, 2, true>, grid, block, 0, st, a);
      else launch(K_ROUTE, skinny_valu_kernel<float, 4, 8, 1, true>, grid, block, 0, st, a);
    }
  } else if (a.variant == VAR_SPLITK) {
    if (a.bf16) {
      if (a.M <= 4) launch(K_SKINNY, skinny_valu_kernel<bf16_t, 4, 4, 2, false>, grid, block, 0, st, a);
      else launch(K_SKINNY, skinny_valu_kernel<bf16_t, 4, 8, 1, false>, grid, block, 0, st, a);
    } else {
      if (a.M <= 4) launch(K_SKINNY, skinny_valu_kernel<float, 4, 4, 2, false>, grid, block, 0, st, a);
      else launch(K_SKINNY, skinny_valu_kernel<float, 4, 8, 1, false>, grid, block, 0, st, a);
    }
    name = "splitk";
  } else {
    if (a.bf16) {
      if (a.M <= 1) launch(K_SKINNY, skinny_valu_kernel<bf16_t, 2, 1, 4, false>, grid, block, 0, st, a);
      else launch(K_SKINNY, skinny_valu_kernel<bf16_t, 2, 2, 4, false>, grid, block, 0, st, a);
    } else {
      if (a.M <= 1) launch(K_SKINNY, skinny_valu_kernel<float, 2, 1, 4, false>, grid, block, 0, st, a);
      else launch(K_SKINNY, skinny_valu_kernel<float, 2, 2, 4, false>, grid, block, 0, st, a);
    }
    name = "gemv";
  }
  if (desc)
    snprintf(desc, desc_len, "%s M=%d N=%d K=%d waves/wg=%d grid=%d%s%s", name, a.M, a.N, a.K, nw, nwg,
             extra ? " +shared gate/up" : "", a.router && !a.finish ? " logits-only" : "");
  return hipGetLastError();
}

}  // namespace moe
