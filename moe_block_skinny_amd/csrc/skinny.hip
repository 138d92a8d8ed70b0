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
//   gemv   : M <= 2 activation rows; a wave owns 2 weight rows over a K range,
//            the 64 lanes split K, v_dot2_f32_bf16 (or fp32 FMA) accumulates,
//            one butterfly reduction at the end.
//   splitk : M <= 8; a wave owns 4 weight rows so each activation chunk it
//            loads is reused 4 times.
//   mfma   : M <= 64 (bf16); v_mfma_f32_16x16x32_bf16 with 16 weight rows as
//            the A operand and up to four 16-token tiles as B, used once
//            batch x rows is a dense contraction.
// Every shape may split K over S workgroups.  Split partials go to an fp32
// workspace and the last workgroup of each row block (completion counter)
// sums them in fixed split order, so results are deterministic.
// In router mode the last row block to finish also selects the top-k
// experts per token, computes their softmax weights and builds the plan.

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kNW = 4;  // waves per workgroup

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

__device__ __forceinline__ void emit(const SkinnyLaunch& a, int s, int t, int n, float v) {
  if (a.S > 1)
    a.partial[((size_t)s * a.M + t) * a.N + n] = v;
  else
    finish_value(a, t, n, v);
}

// ---- router finish: top-k, weights, plan (one workgroup) ------------------

constexpr int kMaxE = 512;
constexpr int kMaxK = 16;
constexpr int kMaxB = 64;

// One wave selects token t's top-k.  Keys order by fp32 logit, then by lower
// expert index; k rounds of a wave-wide max each remove one winner.
__device__ void topk_token(const SkinnyLaunch& a, int t, int* s_ids) {
  const int lane = threadIdx.x & 63;
  const int E = a.N, k = a.k;
  uint64_t key[kMaxE / 64];
#pragma unroll
  for (int i = 0; i < kMaxE / 64; ++i) {
    int e = lane + 64 * i;
    key[i] = e < E ? topk_key(ld_shared_f32(&a.logits[(size_t)t * E + e]), e) : 0ull;
  }
  int sel_e[kMaxK];
  float sel_v[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    sel_e[j] = 0x7fffffff;
    sel_v[j] = 0.f;
    if (j < k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kMaxE / 64; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      int e = key_index(best);
      sel_e[j] = e;
      sel_v[j] = key_value(best);
#pragma unroll
      for (int i = 0; i < kMaxE / 64; ++i)
        if (lane + 64 * i == e) key[i] = 0ull;
    }
  }
  // softmax over the selection; sel_v[0] is the largest selected logit
  const float m = sel_v[0];
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) z += expf(sel_v[j] - m);
  int my_e = 0x7fffffff;
  float my_v = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j == lane) { my_e = sel_e[j]; my_v = sel_v[j]; }
  if (lane < k) {
    int pos = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && sel_e[j] < my_e) ++pos;
    a.topk_ids[(size_t)t * k + pos] = my_e;
    a.topk_w[(size_t)t * k + pos] = expf(my_v - m) / z;
    s_ids[t * k + pos] = my_e;
  }
}

__device__ void route_finish(const SkinnyLaunch& a) {
  __shared__ int s_ids[kMaxB * kMaxK];
  __shared__ unsigned long long s_mask[kMaxE];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_act[kMaxE];
  __shared__ int s_n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int M = a.M, E = a.N, k = a.k, nslot = M * k;

  for (int t = wave; t < M; t += kNW) topk_token(a, t, s_ids);
  for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();
  // bit t of s_mask[e] is set when token t selected expert e (B <= 64)
  for (int s = tid; s < nslot; s += blockDim.x) atomicOr(&s_mask[s_ids[s]], 1ull << (s / k));
  __syncthreads();
  if (wave == 0) {
    // exclusive prefix sums over experts of slot counts and of "is active"
    int c[kMaxE / 64], act[kMaxE / 64], cs = 0, as = 0;
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
      int e = lane * (kMaxE / 64) + i;
      c[i] = e < E ? __popcll(s_mask[e]) : 0;
      act[i] = c[i] > 0;
      cs += c[i];
      as += act[i];
    }
    int ci = cs, ai = as;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int yc = __shfl_up(ci, o, 64), ya = __shfl_up(ai, o, 64);
      if (lane >= o) { ci += yc; ai += ya; }
    }
    int ce = ci - cs, ae = ai - as;
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
      int e = lane * (kMaxE / 64) + i;
      if (e < E) { s_cnt[e] = ce; s_act[e] = ae; }
      ce += c[i];
      ae += act[i];
    }
    if (lane == 63) s_n = ai;
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

// Shared tail of every skinny kernel: split-K reduction by the last
// workgroup of the row block, then (router) the route finish by the last row
// block.  rows_pb = rows per row block, nrb = row blocks.
__device__ __forceinline__ void skinny_tail(const SkinnyLaunch& a, int rb, int rows_pb, int nrb) {
  __shared__ int s_flag;
  if (a.S > 1) {
    if (!arrive_last(&a.rb_counter[rb], (uint32_t)a.S, &s_flag)) return;
    const int n_lo = rb * rows_pb;
    for (int idx = threadIdx.x; idx < rows_pb * a.M; idx += blockDim.x) {
      int t = idx / rows_pb, n = n_lo + idx % rows_pb;
      if (n >= a.N) continue;
      float v = 0.f;
      for (int s = 0; s < a.S; ++s) v += ld_shared_f32(&a.partial[((size_t)s * a.M + t) * a.N + n]);
      finish_value(a, t, n, v);
    }
  }
  if (a.router) {
    if (!arrive_last(a.done_counter, (uint32_t)nrb, &s_flag)) return;
    route_finish(a);
  }
}

// ---- vector-ALU kernels (gemv / splitk) ----------------------------------

template <typename T, int R, int MB>
__global__ __launch_bounds__(256) void skinny_valu_kernel(SkinnyLaunch a) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int U = MB <= 2 ? 4 : 2;
  const int rows_pb = kNW * R;
  const int nrb = (a.N + rows_pb - 1) / rows_pb;
  const int rb = blockIdx.x % nrb, s = blockIdx.x / nrb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = rb * rows_pb + wave * R;
  const int C = a.K / VEC;
  const int c0 = (int)((long long)s * C / a.S), c1 = (int)((long long)(s + 1) * C / a.S);
  const T* W = reinterpret_cast<const T*>(a.W);
  const T* X = reinterpret_cast<const T*>(a.X);
  const T* wr[R];
  const T* xr[MB];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = W + (size_t)(n0 + r < a.N ? n0 + r : a.N - 1) * a.K;
#pragma unroll
  for (int t = 0; t < MB; ++t) xr[t] = X + (size_t)(t < a.M ? t : 0) * a.K;
  float acc[R][MB];
  valu_dot<T, R, MB, U>(wr, xr, a.M, c0, c1, acc);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = n0 + r;
    const float v = pick_lane<MB>(acc[r], lane);
    if (n < a.N && lane < a.M && lane < MB) emit(a, s, lane, n, v);
  }
  skinny_tail(a, rb, rows_pb, nrb);
}

// ---- MFMA kernel (bf16) --------------------------------------------------

// A wave: 16 weight rows (A operand: lane l holds row l%16, K elements
// 8*(l/16) .. +7 of each 32-wide step) against NT tiles of 16 activation
// rows (B operand: lane l holds token l%16 of the tile, same K elements).
// The accumulator of tile nt holds, in lane l, rows 4*(l/16)+i, token l%16.
template <int NT>
__global__ __launch_bounds__(256) void skinny_mfma_kernel(SkinnyLaunch a) {
  constexpr int U = NT <= 2 ? 4 : 2;
  const int rows_pb = kNW * 16;
  const int nrb = (a.N + rows_pb - 1) / rows_pb;
  const int rb = blockIdx.x % nrb, s = blockIdx.x / nrb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const int n0 = rb * rows_pb + wave * 16;
  const int J = a.K / 32;
  const int j0 = (int)((long long)s * J / a.S), j1 = (int)((long long)(s + 1) * J / a.S);
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.W);
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  const bf16_t* wr = W + (size_t)(n0 + row < a.N ? n0 + row : a.N - 1) * a.K;
  const bf16_t* xr[NT];
  bool xok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int tok = nt * 16 + row;
    xok[nt] = tok < a.M;
    xr[nt] = X + (size_t)(xok[nt] ? tok : 0) * a.K;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int j = j0; j < j1; j += U) {
    u32x4 av[U], bv[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u;
      const bool ok = jj < j1;
      const size_t off = (size_t)(jj * 4 + kq) * 8;
      av[u] = ok ? ld128_stream(wr + off) : zero;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bv[u][nt] = (ok && xok[nt]) ? ld128(xr[nt] + off) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                          __builtin_bit_cast(bf16x8, bv[u][nt]),
                                                          acc[nt], 0, 0, 0);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 4 * kq + i, t = nt * 16 + row;
      if (n < a.N && t < a.M) emit(a, s, t, n, acc[nt][i]);
    }
  skinny_tail(a, rb, rows_pb, nrb);
}

// ---- host side -----------------------------------------------------------

int skinny_rows_per_block(int variant, int bf16, int M) {
  (void)bf16;
  (void)M;
  if (variant == VAR_MFMA) return kNW * 16;
  if (variant == VAR_SPLITK) return kNW * 4;
  return kNW * 2;
}

// Enough workgroups to keep every CU streaming (about 4 per CU), but no
// split thinner than two 1 KB loads per lane.
int skinny_default_splits(int variant, int bf16, int M, int N, int K) {
  const int rows_pb = skinny_rows_per_block(variant, bf16, M);
  const int nrb = (N + rows_pb - 1) / rows_pb;
  const int target = 1024;
  int S = (target + nrb - 1) / nrb;
  const int vec = bf16 ? 8 : 4;
  const int chunks = K / vec;
  int smax = chunks / (64 * 2);
  if (variant == VAR_MFMA) smax = (K / 32) / 8;
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  return S;
}

hipError_t launch_skinny(const SkinnyLaunch& a, hipStream_t st, char* desc, size_t desc_len) {
  const int rows_pb = skinny_rows_per_block(a.variant, a.bf16, a.M);
  const int nrb = (a.N + rows_pb - 1) / rows_pb;
  dim3 grid((unsigned)(nrb * a.S)), block(256);
  const char* name = "?";
  if (a.variant == VAR_MFMA) {
    const int nt = (a.M + 15) / 16;
    switch (nt) {
      case 1: hipLaunchKernelGGL(skinny_mfma_kernel<1>, grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL(skinny_mfma_kernel<2>, grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL(skinny_mfma_kernel<3>, grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL(skinny_mfma_kernel<4>, grid, block, 0, st, a); break;
    }
    name = "mfma";
  } else if (a.variant == VAR_SPLITK) {
    if (a.bf16) {
      if (a.M <= 4) hipLaunchKernelGGL((skinny_valu_kernel<bf16_t, 4, 4>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((skinny_valu_kernel<bf16_t, 4, 8>), grid, block, 0, st, a);
    } else {
      if (a.M <= 4) hipLaunchKernelGGL((skinny_valu_kernel<float, 4, 4>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((skinny_valu_kernel<float, 4, 8>), grid, block, 0, st, a);
    }
    name = "splitk";
  } else {
    if (a.bf16) {
      if (a.M <= 1) hipLaunchKernelGGL((skinny_valu_kernel<bf16_t, 2, 1>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((skinny_valu_kernel<bf16_t, 2, 2>), grid, block, 0, st, a);
    } else {
      if (a.M <= 1) hipLaunchKernelGGL((skinny_valu_kernel<float, 2, 1>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((skinny_valu_kernel<float, 2, 2>), grid, block, 0, st, a);
    }
    name = "gemv";
  }
  if (desc) snprintf(desc, desc_len, "%s M=%d N=%d K=%d S=%d grid=%d", name, a.M, a.N, a.K, a.S, nrb * a.S);
  return hipGetLastError();
}

}  // namespace moe
