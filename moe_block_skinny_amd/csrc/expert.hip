// expert.hip -- routed and shared experts of the decode MoE block, and the
// weighted combine.
//
// Sources (web pages on the Kimi K3 specialised decode path):
//   [WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §3
//     (MoE scheduling): routed experts run after routing, a shared expert
//     runs for every token; part 1 §1: batch-shaped kernel choice; part 1 §4:
//     small-batch decode is bound by reading weights.  Part 3 §4 (measuring
//     performance): which experts are selected decides which weights are read.
//   [AICODER] "2.8 万亿参数 Kimi K3 单请求飙至 842 tok/s！...", section
//     "架构亮点与底层机制" (MoE gating and expert GEMM).
//
// Expert e computes h = silu(x . Wg^T) * (x . Wu^T), y = h . W2^T, with
// silu(z) = z / (1 + exp(-z)); W13[e] is [2I][d] (gate rows, then up rows),
// W2[e] is [d][I].  The routing plan lists each selected expert once with
// the slots (token t, choice j) that picked it, so each selected expert's
// weights are streamed exactly once however many tokens chose it; experts no
// token chose are never touched.  The shared expert is one more entry that
// every token uses.
//
// Kernel shape follows the expert's token count m:
//   m <= 8 : vector ALU.  Gate/up: one wave per (gate row i, up row I+i)
//            pair over the whole of d, so SwiGLU happens in registers.
//            Down: a few lanes per W2 row (I is short), several rows per lane.
//   m > 8  : MFMA 16x16x32 bf16.  Gate/up: a 16-row A tile holding 4 gate +
//            4 up rows, the four waves of the workgroup split d and reduce
//            through LDS.  Down: 16 W2 rows per wave; h (fp32) enters the
//            MFMA as a bf16 hi/lo pair so it keeps ~16 mantissa bits.
// Both kernels are persistent: the grid is sized for the largest possible
// plan and every workgroup walks the (expert, tile) tasks of the actual plan.

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kUpPairs = 4;     // gate/up row pairs per up task (one per wave)
constexpr int kDownRows = 64;   // W2 rows per down task (16 per wave)
constexpr int kMaxTok = 64;

// Decoded view of a plan entry: expert a (a == n: the shared expert).
struct ExpertView {
  int m;                 // tokens
  int I;                 // intermediate size of this expert
  const void* W13;       // [2I][d]
  const void* W2;        // [d][I]
  int slot0;             // first plan slot (routed) or -1 (shared)
};

struct PlanView {
  int n, maxa;
  const int32_t* active;
  const int32_t* offs;
  const int32_t* slots;
};

__device__ __forceinline__ PlanView plan_view(const ExpertLaunch& a) {
  PlanView p;
  const int nslot = a.B * a.k;
  p.maxa = nslot < a.E ? nslot : a.E;
  p.n = a.plan[0];
  p.active = a.plan + 1;
  p.offs = a.plan + 1 + p.maxa;
  p.slots = a.plan + 2 + 2 * p.maxa;
  return p;
}

template <typename T>
__device__ __forceinline__ ExpertView expert_view(const ExpertLaunch& a, const PlanView& p, int e_idx) {
  ExpertView v;
  if (e_idx < p.n) {
    const int e = p.active[e_idx];
    v.m = p.offs[e_idx + 1] - p.offs[e_idx];
    v.I = a.I;
    v.W13 = reinterpret_cast<const T*>(a.W13) + (size_t)e * 2 * a.I * a.d;
    v.W2 = reinterpret_cast<const T*>(a.W2) + (size_t)e * a.d * a.I;
    v.slot0 = p.offs[e_idx];
  } else {
    v.m = a.B;
    v.I = a.Is;
    v.W13 = a.Ws13;
    v.W2 = a.Ws2;
    v.slot0 = -1;
  }
  return v;
}

// Token index and h row of the i-th token of an expert.
__device__ __forceinline__ void token_of(const ExpertLaunch& a, const PlanView& p, const ExpertView& v,
                                         int i, int& tok, int& hrow) {
  if (v.slot0 >= 0) {
    const int s = p.slots[v.slot0 + i];
    tok = s / a.k;
    hrow = s;
  } else {
    tok = i;
    hrow = a.B * a.k + i;
  }
}

// Task walk shared by both expert kernels: routed experts first (tiles_r
// tasks each), then the shared expert (tiles_s tasks).
__device__ __forceinline__ int total_tasks(const ExpertLaunch& a, const PlanView& p, int tiles_r, int tiles_s) {
  return p.n * tiles_r + (a.Ws13 ? tiles_s : 0);
}
__device__ __forceinline__ void task_of(const PlanView& p, int task, int tiles_r, int& e_idx, int& tile) {
  if (task < p.n * tiles_r) {
    e_idx = task / tiles_r;
    tile = task % tiles_r;
  } else {
    e_idx = p.n;
    tile = task - p.n * tiles_r;
  }
}

__device__ __forceinline__ bool use_mfma(const ExpertLaunch& a, int m) {
  if (!a.bf16) return false;
  if (a.force == VAR_MFMA) return true;
  if (a.force == VAR_GEMV) return false;
  return m > 8;
}

// ---- gate/up + SwiGLU --------------------------------------------------------

template <typename T, int MB>
__device__ void up_valu(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int tile) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int U = MB <= 2 ? 4 : 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = tile * kUpPairs + wave;
  if (i >= v.I) return;
  const T* W13 = reinterpret_cast<const T*>(v.W13);
  const T* X = reinterpret_cast<const T*>(a.X);
  const T* wr[2] = {W13 + (size_t)i * a.d, W13 + (size_t)(v.I + i) * a.d};
  const T* xr[MB];
  int hrow[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) {
    int tok = 0, hr = 0;
    if (t < v.m) token_of(a, p, v, t, tok, hr);
    xr[t] = X + (size_t)tok * a.d;
    hrow[t] = hr;
  }
  float acc[2][MB];
  valu_dot<T, 2, MB, U>(wr, xr, v.m, 0, a.d / VEC, acc);
  if (lane < v.m) {
    const float g = pick_lane<MB>(acc[0], lane), u = pick_lane<MB>(acc[1], lane);
    int hr = 0;
#pragma unroll
    for (int t = 0; t < MB; ++t)
      if (t == lane) hr = hrow[t];
    a.h[(size_t)hr * a.hld + i] = silu(g) * u;
  }
}

template <typename T>
__device__ void up_valu_dispatch(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int tile) {
  if (v.m <= 1) up_valu<T, 1>(a, p, v, tile);
  else if (v.m <= 2) up_valu<T, 2>(a, p, v, tile);
  else if (v.m <= 4) up_valu<T, 4>(a, p, v, tile);
  else up_valu<T, 8>(a, p, v, tile);
}

// A tile: lanes with row%16 in 0..3 load gate rows i0..i0+3, 4..7 load up
// rows, 8..15 stay zero.  Wave w covers the w-th quarter of the K steps.
template <int NT>
__device__ void up_mfma(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int tile,
                        float* s_red /* [4][NT][64][4] */) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const int i0 = tile * kUpPairs;
  const bf16_t* W13 = reinterpret_cast<const bf16_t*>(v.W13);
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  int wrow = -1;
  if (row < 4 && i0 + row < v.I) wrow = i0 + row;
  else if (row >= 4 && row < 8 && i0 + row - 4 < v.I) wrow = v.I + i0 + row - 4;
  const bf16_t* wr = W13 + (size_t)(wrow >= 0 ? wrow : 0) * a.d;
  const bf16_t* xr[NT];
  bool xok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int ti = nt * 16 + row;
    int tok = 0, hr = 0;
    xok[nt] = ti < v.m;
    if (xok[nt]) token_of(a, p, v, ti, tok, hr);
    xr[nt] = X + (size_t)tok * a.d;
  }
  const int J = a.d / 32;
  const int j0 = wave * J / 4, j1 = (wave + 1) * J / 4;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int U = 4;
  for (int j = j0; j < j1; j += U) {
    u32x4 av[U], bv[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u;
      const bool ok = jj < j1;
      const size_t off = (size_t)(jj * 4 + kq) * 8;
      av[u] = (ok && wrow >= 0) ? ld128_stream(wr + off) : zero;
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
    for (int q = 0; q < 4; ++q) s_red[((wave * NT + nt) * 64 + lane) * 4 + q] = acc[nt][q];
  __syncthreads();
  // thread (q, t): pair i0+q, token t.  Gate sums sit in lanes 0..15 (rows
  // 0..3), up sums in lanes 16..31 (rows 4..7) of each wave's tile.
  const int q = threadIdx.x >> 6, t = threadIdx.x & 63;
  if (t < v.m && i0 + q < v.I) {
    const int nt = t >> 4, l = t & 15;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      g += s_red[((w * NT + nt) * 64 + l) * 4 + q];
      u += s_red[((w * NT + nt) * 64 + 16 + l) * 4 + q];
    }
    int tok, hr;
    token_of(a, p, v, t, tok, hr);
    a.h[(size_t)hr * a.hld + i0 + q] = silu(g) * u;
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(256) void expert_up_kernel(ExpertLaunch a) {
  __shared__ float s_red[4 * 4 * 64 * 4];
  const PlanView p = plan_view(a);
  const int tiles_r = (a.I + kUpPairs - 1) / kUpPairs;
  const int tiles_s = (a.Is + kUpPairs - 1) / kUpPairs;
  const int total = total_tasks(a, p, tiles_r, tiles_s);
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    int e_idx, tile;
    task_of(p, task, tiles_r, e_idx, tile);
    const ExpertView v = expert_view<T>(a, p, e_idx);
    if (use_mfma(a, v.m)) {
      if constexpr (sizeof(T) == 2) {
        const int nt = (v.m + 15) / 16;
        if (nt <= 1) up_mfma<1>(a, p, v, tile, s_red);
        else if (nt == 2) up_mfma<2>(a, p, v, tile, s_red);
        else if (nt == 3) up_mfma<3>(a, p, v, tile, s_red);
        else up_mfma<4>(a, p, v, tile, s_red);
      }
    } else {
      up_valu_dispatch<T>(a, p, v, tile);
    }
  }
}

// ---- down projection ---------------------------------------------------------

// Yslot row for token index i of expert v.
__device__ __forceinline__ float* yslot_row(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int i) {
  int t, slot_j;
  if (v.slot0 >= 0) {
    const int s = p.slots[v.slot0 + i];
    t = s / a.k;
    slot_j = s % a.k;
  } else {
    t = i;
    slot_j = a.k;
  }
  return a.Yslot + ((size_t)t * (a.k + 1) + slot_j) * a.d;
}

// L lanes per W2 row (L*VEC >= I), P = 64/L rows per load instruction, R
// rows per lane: a wave covers 16 rows.
template <typename T, int L>
__device__ void down_valu(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int tile) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int P = 64 / L;
  constexpr int R = 16 / P;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane % L, g = lane / L;
  const bool cok = c * VEC < v.I;
  const int rbase = tile * kDownRows + wave * 16 + g;
  const T* W2 = reinterpret_cast<const T*>(v.W2);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = rbase + P * r;
    wv[r] = (cok && row < a.d) ? ld128_stream(W2 + (size_t)row * v.I + (size_t)c * VEC) : zero;
  }
  // one token at a time: R dot products, reduce over the L lanes, store
  for (int t = 0; t < v.m; ++t) {
    int tok, hr;
    token_of(a, p, v, t, tok, hr);
    float xs[VEC];
    const float* hp = a.h + (size_t)hr * a.hld + (size_t)(cok ? c * VEC : 0);
#pragma unroll
    for (int e = 0; e < VEC; ++e) xs[e] = cok ? hp[e] : 0.f;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum<L>(dot_chunk_f32x(wv[r], xs, 0.f, T()));
    if (c == 0) {
      float* y = yslot_row(a, p, v, t);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = rbase + P * r;
        if (row < a.d) y[row] = acc[r];
      }
    }
  }
}

// 16 W2 rows per wave, full I in 32-wide steps; h enters as hi + lo bf16.
template <int NT>
__device__ void down_mfma(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int tile) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const int r0 = tile * kDownRows + wave * 16;
  const bf16_t* W2 = reinterpret_cast<const bf16_t*>(v.W2);
  const bf16_t* wr = W2 + (size_t)(r0 + row < a.d ? r0 + row : a.d - 1) * v.I;
  const float* hr_[NT];
  bool ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int ti = nt * 16 + row;
    int tok = 0, hr = 0;
    ok[nt] = ti < v.m;
    if (ok[nt]) token_of(a, p, v, ti, tok, hr);
    hr_[nt] = a.h + (size_t)hr * a.hld;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int J = v.I / 32;
  for (int j = 0; j < J; ++j) {
    const size_t off = (size_t)(j * 4 + kq) * 8;
    const u32x4 av = ld128_stream(wr + off);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
      if (ok[nt]) {
        const f32x4 h0 = *reinterpret_cast<const f32x4*>(hr_[nt] + off);
        const f32x4 h1 = *reinterpret_cast<const f32x4*>(hr_[nt] + off + 4);
        float hv[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16_t a0 = f32_to_bf16(hv[2 * e]), a1 = f32_to_bf16(hv[2 * e + 1]);
          const bf16_t b0 = f32_to_bf16(hv[2 * e] - bf16_to_f32(a0));
          const bf16_t b1 = f32_to_bf16(hv[2 * e + 1] - bf16_to_f32(a1));
          hi[e] = (uint32_t)a0 | ((uint32_t)a1 << 16);
          lo[e] = (uint32_t)b0 | ((uint32_t)b1 << 16);
        }
      }
      const u32x4 hv4 = {hi[0], hi[1], hi[2], hi[3]}, lv4 = {lo[0], lo[1], lo[2], lo[3]};
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                        __builtin_bit_cast(bf16x8, hv4), acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                        __builtin_bit_cast(bf16x8, lv4), acc[nt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int ti = nt * 16 + row;
    if (ti < v.m) {
      float* y = yslot_row(a, p, v, ti);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * kq + i;
        if (r < a.d) y[r] = acc[nt][i];
      }
    }
  }
}

template <typename T>
__device__ void down_valu_dispatch(const ExpertLaunch& a, const PlanView& p, const ExpertView& v, int tile) {
  constexpr int VEC = Elem<T>::VEC;
  const int chunks = v.I / VEC;
  if (chunks <= 16) down_valu<T, 16>(a, p, v, tile);
  else if (chunks <= 32) down_valu<T, 32>(a, p, v, tile);
  else down_valu<T, 64>(a, p, v, tile);
}

template <typename T>
__global__ __launch_bounds__(256) void expert_down_kernel(ExpertLaunch a) {
  const PlanView p = plan_view(a);
  const int tiles = (a.d + kDownRows - 1) / kDownRows;
  const int total = total_tasks(a, p, tiles, tiles);
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    int e_idx, tile;
    task_of(p, task, tiles, e_idx, tile);
    const ExpertView v = expert_view<T>(a, p, e_idx);
    if (use_mfma(a, v.m)) {
      if constexpr (sizeof(T) == 2) {
        const int nt = (v.m + 15) / 16;
        if (nt <= 1) down_mfma<1>(a, p, v, tile);
        else if (nt == 2) down_mfma<2>(a, p, v, tile);
        else if (nt == 3) down_mfma<3>(a, p, v, tile);
        else down_mfma<4>(a, p, v, tile);
      }
    } else {
      down_valu_dispatch<T>(a, p, v, tile);
    }
  }
}

// ---- combine -------------------------------------------------------------------

// out[t][r] = sum_j w[t][j] * Yslot[t][j][r] (j ascending = ascending expert
// id), then + Yslot[t][k][r] for the shared expert; fp32, fixed order.
__global__ __launch_bounds__(256) void combine_kernel(CombineLaunch a) {
  const size_t n = (size_t)a.B * a.d;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(idx / a.d), r = (int)(idx % a.d);
    const float* ys = a.Yslot + (size_t)t * (a.k + 1) * a.d + r;
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) acc = __builtin_fmaf(a.topk_w[(size_t)t * a.k + j], ys[(size_t)j * a.d], acc);
    if (a.has_shared) acc += ys[(size_t)a.k * a.d];
    if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[idx] = f32_to_bf16(acc);
    else reinterpret_cast<float*>(a.out)[idx] = acc;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---- host side ---------------------------------------------------------------

static int max_tasks(const ExpertLaunch& a, int tiles_r, int tiles_s) {
  const int nslot = a.B * a.k;
  const int maxa = nslot < a.E ? nslot : a.E;
  return maxa * tiles_r + (a.Ws13 ? tiles_s : 0);
}

static const int kMaxResidentWG = 256 * 8;

hipError_t launch_expert_up(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len) {
  const int tiles_r = (a.I + kUpPairs - 1) / kUpPairs;
  const int tiles_s = (a.Is + kUpPairs - 1) / kUpPairs;
  int g = max_tasks(a, tiles_r, tiles_s);
  if (g > kMaxResidentWG) g = kMaxResidentWG;
  if (g < 1) g = 1;
  if (a.bf16) hipLaunchKernelGGL(expert_up_kernel<bf16_t>, dim3(g), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(expert_up_kernel<float>, dim3(g), dim3(256), 0, st, a);
  if (desc) snprintf(desc, desc_len, "up grid=%d force=%d", g, a.force);
  return hipGetLastError();
}

hipError_t launch_expert_down(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len) {
  const int tiles = (a.d + kDownRows - 1) / kDownRows;
  int g = max_tasks(a, tiles, tiles);
  if (g > kMaxResidentWG) g = kMaxResidentWG;
  if (g < 1) g = 1;
  if (a.bf16) hipLaunchKernelGGL(expert_down_kernel<bf16_t>, dim3(g), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(expert_down_kernel<float>, dim3(g), dim3(256), 0, st, a);
  if (desc) snprintf(desc, desc_len, "down grid=%d force=%d", g, a.force);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.d;
  int g = (int)((n + 255) / 256);
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(combine_kernel, dim3(g), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  int g = (int)((words + 255) / 256);
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(g), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace moe
