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
//   rows   : the dense product at M = 2..8 (bf16, K <= 8192); a workgroup
//            owns 12 weight rows over all of K, one 16-byte chunk of K per
//            thread, so every activation chunk serves 12 rows and no
//            partial sum leaves the workgroup.
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
#include "skinny_core.hpp"

namespace moe {


// ---- router finish: top-k, weights, plan (one workgroup) ------------------

// Top-k of every token: waves take tokens wave, wave + nw, ..., with the
// logits of four tokens loaded before any is used (one memory round trip
// per group); ids and weights go to LDS and to the caller's arrays.

template <int NTK>
__device__ __forceinline__ void topk_tokens(const SkinnyLaunch& a, TopkScratch* s_tk, int32_t* s_ids, float* s_w) {
  constexpr int QB = 4;
  const int nw = (blockDim.x >> 6) < NTK ? (blockDim.x >> 6) : NTK;
  const int wave = threadIdx.x >> 6;
  if (wave >= nw) return;
  const int E = a.N - a.L, M = a.M, k = a.k;
  for (int t0 = wave; t0 < M; t0 += nw * QB) {
    float lv[QB][kNI];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int t = t0 + nw * q;
      load_logit_row<true>(a.logits, t < M ? t : M - 1, E, lv[q]);
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

// The routing plan of all M*k slots from their expert ids (s_ids, LDS), by
// the whole workgroup, into a.plan.
__device__ __forceinline__ void route_plan(const SkinnyLaunch& a, const int32_t* s_ids) {
  __shared__ PlanScratch s_ps;
  plan_block(s_ids, a.M * a.k, a.k, a.N - a.L, a.plan, nullptr, s_ps);
}

// Top-k of every token and the plan, by one workgroup.  NTK: waves that
// select (each holds a TopkScratch in LDS).
template <int NTK>
__device__ __forceinline__ void route_finish(const SkinnyLaunch& a) {
  __shared__ int32_t s_ids[kMaxB * kMaxK];
  __shared__ float s_w[kMaxB * kMaxK];
  __shared__ TopkScratch s_tk[NTK];
  topk_tokens<NTK>(a, s_tk, s_ids, s_w);
  __syncthreads();
  route_plan(a, s_ids);
}

// Router tail: every router workgroup arrives once; the last runs the finish.
__device__ __forceinline__ void router_tail(const SkinnyLaunch& a) {
  __shared__ int s_flag;
  if (!a.router || !a.finish) return;
  if (!arrive_last(a.done_counter, (uint32_t)a.router_arrivals, &s_flag)) return;
  route_finish<kTopkWaves>(a);
}

// The finish as a launch of its own, after the MFMA router product, whose
// workgroups store the partial sums of their K slices: one workgroup per
// token; its four waves each add a quarter of the slices (all of a wave's
// partials requested at once, 16-byte loads, 4 experts per lane), wave 0 adds
// the four quarters in wave order (the same order in every run), adds the
// bias, selects the top-k and stores ids and weights (device-coherent).
// Unless the gate/up launch builds the plan, every workgroup then arrives
// and the last one reads every token's ids and builds the plan.
constexpr int kFinishWaves = 4;
constexpr int kFinishSlices = 8;   // partials per wave requested together
__global__ __launch_bounds__(kFinishWaves * 64) void route_finish_kernel(SkinnyLaunch a) {
  __shared__ TopkScratch s_tk[1];
  __shared__ int32_t s_ids[kMaxB * kMaxK];
  __shared__ float s_w[kMaxB * kMaxK];
  __shared__ __align__(16) float s_lg[kFinishWaves][kMaxE];
  __shared__ int s_last;
  MOE_STAMP(ST_FINISH, 0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int E = a.N - a.L, k = a.k;   // router rows; the partial rows hold all N
  float lv[kNI];
  // wave 0's bias values, requested with the partial sums (requested after
  // the sums, they cost one more memory round trip: 1.2 us at batch 64)
  float bv[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    const int e = lane + 64 * i;
    bv[i] = (wave == 0 && a.bias && e < E) ? a.bias[(size_t)t * a.bias_ld + e] : 0.f;
  }
  if ((E & 3) == 0) {
    // wave w: slices [q0, q1); lane l: experts 4l .. 4l+3 and 256 + 4l .. +3
    constexpr int NV = kMaxE / 256;
    const int per = (a.ks_n + kFinishWaves - 1) / kFinishWaves;
    const int q0 = wave * per, q1 = q0 + per < a.ks_n ? q0 + per : a.ks_n;
    const int nv4 = E >> 2;
    f32x4 sum[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) sum[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int qb = q0; qb < q1; qb += kFinishSlices) {
      f32x4 pv[kFinishSlices][NV];
#pragma unroll
      for (int q = 0; q < kFinishSlices; ++q) {
        const int qc = qb + q < q1 ? qb + q : q1 - 1;
        const f32x4* row = reinterpret_cast<const f32x4*>(a.part + ((size_t)qc * a.M + t) * a.N);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int j = lane + 64 * v;
          pv[q][v] = row[j < nv4 ? j : nv4 - 1];
        }
      }
#pragma unroll
      for (int q = 0; q < kFinishSlices; ++q)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (qb + q < q1) sum[v] += pv[q][v];
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int j = lane + 64 * v;
      if (j < nv4) *reinterpret_cast<f32x4*>(&s_lg[wave][4 * j]) = sum[v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        const int e = lane + 64 * i;
        const int ec = e < E ? e : E - 1;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kFinishWaves; ++w) v += s_lg[w][ec];
        lv[i] = v;
      }
    }
  } else if (wave == 0) {
#pragma unroll
    for (int i = 0; i < kNI; ++i) lv[i] = 0.f;
    for (int q = 0; q < a.ks_n; ++q)
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        const int e = lane + 64 * i;
        lv[i] += a.part[((size_t)q * a.M + t) * a.N + (e < E ? e : E - 1)];
      }
  }
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        if (a.bias) lv[i] += bv[i];
        a.logits[(size_t)t * E + e] = lv[i];
        if (a.logits_out) a.logits_out[(size_t)t * E + e] = lv[i];
      }
    }
    topk_wave(lv, E, k, s_tk[0], s_ids + t * k, s_w + t * k, a.topk_ids + (size_t)t * k,
              a.topk_w + (size_t)t * k);
  }
  if (a.L) {
    // the latent projection columns E .. N-1 of this token: every slice's
    // partials of 4 columns per thread, requested per group of slices, added
    // in slice order (E and L multiples of 4)
    for (int c = 4 * (int)threadIdx.x; c < a.L; c += 4 * (int)blockDim.x) {
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      for (int qb = 0; qb < a.ks_n; qb += kFinishSlices) {
        f32x4 pv[kFinishSlices];
#pragma unroll
        for (int q = 0; q < kFinishSlices; ++q) {
          const int qc = qb + q < a.ks_n ? qb + q : a.ks_n - 1;
          pv[q] = *reinterpret_cast<const f32x4*>(a.part + ((size_t)qc * a.M + t) * a.N + E + c);
        }
#pragma unroll
        for (int q = 0; q < kFinishSlices; ++q)
          if (qb + q < a.ks_n) sum += pv[q];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) finish_value(a, t, E + c + i, sum[i]);
    }
  }
  MOE_STAMP(ST_FINISH, 1);
  if (a.plan_by_consumer) return;   // the gate/up launch builds the plan from the ids
  if (!arrive_last(a.done_counter, gridDim.x, &s_last)) return;
  {
    // every token's ids, all requested before any is stored
    constexpr int PER = kMaxB * kMaxK / (kFinishWaves * 64);
    int32_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = threadIdx.x + j * kFinishWaves * 64;
      v[j] = ld_coherent_i32(a.topk_ids + (i < a.M * k ? i : 0));
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = threadIdx.x + j * kFinishWaves * 64;
      if (i < a.M * k) s_ids[i] = v[j];
    }
  }
  __syncthreads();
  route_plan(a, s_ids);
}

// ---- vector-ALU kernels (gemv / splitk) ----------------------------------

// Router rows per workgroup: E = 384 router rows spread over 192 compute
// units (one 16-wave workgroup each).  A compute unit keeps only so many
// loads in flight, so a launch that leaves CUs idle streams proportionally
// slower: with 4 rows per workgroup the 96 workgroups took ~3x the time of
// one memory round trip.
constexpr int kRouterRows = 2;

// Workgroup: RB weight rows starting at blockIdx.x * RB (valu_rows).
template <typename T, int RB, int MB, int U, bool ROUTER>
__global__ __launch_bounds__(1024) void skinny_valu_kernel(SkinnyLaunch a) {
  // the product's wave partials, or the shared gate/up's pair exchange
  // (8 pair slots of 2 x kPartStride floats)
  __shared__ float s_red[16 * RB * MB > 16 * kPartStride ? 16 * RB * MB : 16 * kPartStride];
  if (ROUTER) MOE_STAMP(ST_ROUTE, 0);
  if (ROUTER && a.clear && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.clear_n; i += blockDim.x) a.clear[i] = 0;
  if (ROUTER && (int)blockIdx.x >= a.router_wgs) {  // shared expert gate/up
    shared_up_task<T>(a.ex, blockIdx.x - a.router_wgs, s_red);
    return;
  }
  valu_rows<T, RB, MB, U>(a, blockIdx.x * RB, s_red);
  if constexpr (ROUTER) MOE_STAMP(ST_ROUTE, 1);
  if constexpr (ROUTER) router_tail(a);
}

// ---- rows kernel (bf16, few tokens, K <= 8192) -----------------------------

// A workgroup owns kRowsGroups x RPP weight rows over all of K; thread j
// takes the 16-byte chunk j of K (K / 8 threads).  Its activation chunks
// (MB tokens) are requested once and serve every row, so the activations
// cost 8 x MB bytes per 16 x RPP x kRowsGroups bytes of weights, and no
// partial sum leaves the workgroup: no K slices, no arrival counter, no
// reduction tail.  The rows go RPP at a time; the next group's weights are
// requested before the current group's products.  A group's RPP x MB sums
// are reduced across the wave by halving exchanges (each step keeps half
// the values and adds the partner lane's other half, so after log2(V)
// steps lane l holds sum V-index l >> (6 - log2 V)), finished by
// exchanges over the remaining lane bits; the waves meet in LDS and are
// added in wave order (deterministic).
constexpr int kRowsGroups = 3;

// Lane exchanges of the halving steps.  Over 32 and 16 lanes: the swaps
// of gfx950 (v_permlane32_swap: lanes 32-63 of the first operand trade
// places with lanes 0-31 of the second; v_permlane16_swap: the odd 16-lane
// rows of the first with the even rows of the second), so that lo + hi
// afterwards holds, in a lower lane, its lo plus its partner's lo and, in
// an upper lane, its hi plus its partner's hi.  Within a row: DPP
// (mirror, half-mirror, quad permutes), pairing lane i with a lane that
// differs in bit log2(M) and holds the same sums so far.
template <int M>
__device__ __forceinline__ float swap_halves_sum(float lo, float hi) {
  const unsigned a = __builtin_bit_cast(unsigned, lo), b = __builtin_bit_cast(unsigned, hi);
  unsigned x, y;
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    x = r[0];
    y = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    x = r[0];
    y = r[1];
  }
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
template <int M>
__device__ __forceinline__ float in_row_partner(float v) {
  static_assert(M == 8 || M == 4 || M == 2 || M == 1, "in-row masks");
  if constexpr (M == 8) return dpp_f32<0x140>(v);        // row_mirror: i <-> 15 - i
  else if constexpr (M == 4) return dpp_f32<0x141>(v);   // row_half_mirror: i <-> 7 - i
  else if constexpr (M == 2) return dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  else return dpp_f32<0xB1>(v);                          // quad_perm [1,0,3,2]
}

// One halving step over mask M on the first N of v's values (a lane with
// bit M keeps the upper half), then the next steps; all indices are
// compile-time constants.
template <int N, int M, int V>
__device__ __forceinline__ void halve(float (&v)[V], int lane) {
  if constexpr (N > 1) {
    if constexpr (M >= 16) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) v[i] = swap_halves_sum<M>(v[i], v[i + N / 2]);
    } else {
      const bool upper = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const float give = upper ? v[i] : v[i + N / 2];
        const float keep = upper ? v[i + N / 2] : v[i];
        v[i] = keep + in_row_partner<M>(give);
      }
    }
    halve<N / 2, M / 2>(v, lane);
  }
}

// The halving steps over masks M0, M0 / 2, ... for V values (V <= 2 M0,
// both powers of two), then sums of the one value left over the lower
// masks.  (The first step over mask 32 is taken with the products.)
template <int V, int M0>
__device__ __forceinline__ float halving_sum(float (&v)[V]) {
  static_assert(V >= 1 && V <= 2 * M0 && (V & (V - 1)) == 0, "V a power of two <= 2 M0");
  static_assert(M0 <= 16, "the in-row sums below take masks up to 8");
  halve<V, M0>(v, threadIdx.x & 63);
  float r = v[0];
  if constexpr (M0 / V >= 8) r += in_row_partner<8>(r);
  if constexpr (M0 / V >= 4) r += in_row_partner<4>(r);
  if constexpr (M0 / V >= 2) r += in_row_partner<2>(r);
  if constexpr (M0 / V >= 1) r += in_row_partner<1>(r);
  return r;
}

// NG groups of RPP rows; ALL: every group's weights requested before the
// first products (NG register sets) instead of the next group's during the
// current products (two sets in turns).
template <int MB, int RPP, int NG = kRowsGroups, bool ALL = false>
__global__ __launch_bounds__(1024) void skinny_rows_kernel(SkinnyLaunch a) {
  static_assert(RPP * NG == 4 * kRowsGroups, "12 rows per workgroup");
  static_assert(RPP >= 2 && (RPP & (RPP - 1)) == 0, "row pairs for the first halving step");
  constexpr int V = RPP * MB;
  constexpr int SH = V == 64 ? 0 : (V == 32 ? 1 : (V == 16 ? 2 : (V == 8 ? 3 : (V == 4 ? 4 : (V == 2 ? 5 : 6)))));
  __shared__ float s_w[16][NG * V];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int n0 = blockIdx.x * (RPP * NG);
  const int C = a.K / 8;
  const bool live = (int)threadIdx.x < C;
  const int c = live ? (int)threadIdx.x : C - 1;   // a lane past K: zero activations
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  u32x4 xv[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) xv[t] = ld128(X + (size_t)(t < a.M ? t : 0) * a.K + (size_t)c * 8);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int NB = ALL ? NG : 2;   // weight register sets: every group's, or two in turns
  u32x4 wv[NB][RPP];
#pragma unroll
  for (int g = 0; g < (ALL ? NG : 1); ++g)
#pragma unroll
    for (int r = 0; r < RPP; ++r) wv[g][r] = ld128_stream(product_row<bf16_t>(a, n0 + g * RPP + r) + (size_t)c * 8);
  __builtin_amdgcn_sched_barrier(0);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  bool xz = false;   // activations zeroed past K (once, at their first use)
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (!ALL && g + 1 < NG) {
#pragma unroll
      for (int r = 0; r < RPP; ++r)
        wv[(g + 1) % NB][r] = ld128_stream(product_row<bf16_t>(a, n0 + (g + 1) * RPP + r) + (size_t)c * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    // products of rows r and r + RPP / 2 and the first halving step (mask
    // 32) together, so that only half the sums are live at once
    if (!xz) {
#pragma unroll
      for (int t = 0; t < MB; ++t) xv[t] = live ? xv[t] : zero;
      xz = true;
    }
    float h[V / 2];
#pragma unroll
    for (int r = 0; r < RPP / 2; ++r) {
      const u32x4 wl = wv[g % NB][r];
      const u32x4 wh = wv[g % NB][r + RPP / 2];
#pragma unroll
      for (int t = 0; t < MB; ++t)
        h[r * MB + t] = swap_halves_sum<32>(dot_chunk(wl, xv[t], 0.f, bf16_t()), dot_chunk(wh, xv[t], 0.f, bf16_t()));
    }
    const float v = halving_sum<V / 2, 16>(h);
    if ((lane & ((1 << SH) - 1)) == 0) s_w[wave][g * V + (lane >> SH)] = v;
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  // (a loop: a workgroup of one wave has fewer threads than results)
  for (int i = threadIdx.x; i < NG * V; i += blockDim.x) {
    const int g = i / V, j = i % V;
    const int n = n0 + g * RPP + j / MB, t = j % MB;
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += s_w[w][i];
    if (n < a.N && t < a.M) finish_value(a, t, n, sum);
  }
}

// ---- MFMA kernel (bf16) --------------------------------------------------

// Workgroup of 4 waves = 64 weight rows (wave w: rows n0 + 16 w .. + 15)
// over one K slice (blockIdx -> row group, slice), by mfma_rows
// (mfma_core.hpp: activation chunks staged through LDS, double-buffered
// weights).  With several slices the workgroups store fp32 partial sums
// [slice][M][N]; the last of a row group's slices to arrive adds them in
// slice order (deterministic).
constexpr int kMaxSlices = 32;
constexpr int kSliceGroup = 8;   // partial sums requested together by the last slice
constexpr int kMaxPartialBytes = 128 * 1024;   // partials one last slice reads

void skinny_mfma_slices(int M, int N, int K, int* ks_n, int* ks_steps) {
  const int rg = (N + kMfmaRows - 1) / kMfmaRows;
  const int J = K / 32;
  const int nchunk = (J + kChunk - 1) / kChunk;
  int ks = 256 / rg;                         // one workgroup per CU (two per
  if (ks > kMaxSlices) ks = kMaxSlices;      // CU measured slower);
                                             // the cap bounds the partial traffic
                                             // (small N, e.g. the router: many
                                             // slices, so every CU streams)
  if (ks > nchunk) ks = nchunk;
  // the last slice of a row group reads every slice's partial tile (64 rows
  // x 16 NT tokens x 4 bytes): at most kMaxPartialBytes, so the reduction
  // tail stays one or two memory round trips (the 384-row router at batch
  // 64 with 28 slices spent ~10 us reading 458 KB in one workgroup)
  const int nt = (M + 15) / 16;
  const int ks_cap = kMaxPartialBytes / (kMfmaRows * 16 * nt * 4);
  if (ks > ks_cap) ks = ks_cap;
  if (ks < 1) ks = 1;
  const int chunks = (nchunk + ks - 1) / ks;
  *ks_steps = chunks * kChunk;
  *ks_n = (J + *ks_steps - 1) / *ks_steps;
}

// K slices of the MFMA router: enough 64-row x K-slice workgroups to put
// one on most compute units, one LDS chunk (8 steps) each at E = 384, d =
// 7168; nothing is reduced inside the launch (the finish launch adds the
// slices), so the partial traffic only has to stay below the weight bytes:
// [slices][M][N] fp32 against N x K bf16, i.e. slices x M x 2 < K.
void router_mfma_slices(int M, int N, int K, int* ks_n, int* ks_steps) {
  const int rg = (N + kMfmaRows - 1) / kMfmaRows;
  const int J = K / 32;
  const int nchunk = (J + kChunk - 1) / kChunk;
  int ks = 256 / rg;
  if (ks > nchunk) ks = nchunk;
  const int cap = K / (2 * (M > 0 ? M : 1));
  if (ks > cap) ks = cap;
  if (ks < 1) ks = 1;
  const int chunks = (nchunk + ks - 1) / ks;
  *ks_steps = chunks * kChunk;
  *ks_n = (J + *ks_steps - 1) / *ks_steps;
}

template <int NT, bool ROUTER>
__global__ __launch_bounds__(kMfmaWaves * 64) void skinny_mfma_kernel(SkinnyLaunch a) {
  constexpr int U = 1;
  __shared__ __align__(16) unsigned char s_x[2 * MfmaX<NT, U>::kLdsBytes];
  constexpr int PPT = MfmaX<NT>::kPerThread;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = lane & 15, kq = lane >> 4;
  if (ROUTER) MOE_STAMP(ST_ROUTE, 0);
  const int rgi = blockIdx.x / a.ks_n, ks = blockIdx.x % a.ks_n;
  const int n0 = rgi * kMfmaRows + wave * 16;
  const int J = a.K / 32;
  const int s0 = ks * a.ks_steps;
  const int s1 = s0 + a.ks_steps < J ? s0 + a.ks_steps : J;
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  const int ra = n0 + mfma_row_a(), rb = n0 + mfma_row_b();
  const bool oka = ra < a.N, okb = rb < a.N;
  const bf16_t* wa = product_row<bf16_t>(a, ra) + mfma_col_off();
  const bf16_t* wb = product_row<bf16_t>(a, rb) + mfma_col_off();
  const bf16_t* xrow[PPT];
  bool xok[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int t = mfma_piece_token<NT>(i);
    xok[i] = t < a.M;
    xrow[i] = X + (size_t)(xok[i] ? t : 0) * a.K;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_rows_db<NT, U>(wa, oka, wb, okb, xrow, xok, s0, s1, s_x, acc);
  if (ROUTER && a.defer) {
    // partial sums [slice][M][N] for the finish launch (a later launch: plain
    // stores); a lane's 4 values are 4 consecutive rows of one token
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 4 * kq, t = nt * 16 + row;
      float* dst = &a.part[((size_t)ks * a.M + t) * a.N + n];
      if ((a.N & 3) == 0 && t < a.M && n + 3 < a.N) {
        *reinterpret_cast<f32x4*>(dst) = acc[nt];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < a.N && t < a.M) dst[i] = acc[nt][i];
      }
    }
    MOE_STAMP(ST_ROUTE, 1);
    return;
  }
  if (a.ks_n == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 4 * kq + i, t = nt * 16 + row;
        if (n < a.N && t < a.M) finish_value(a, t, n, acc[nt][i]);
      }
  } else {
    // partial sums [slice][M][N]: a lane's 4 values are 4 consecutive rows
    // of one token, stored in one 16-byte device-coherent store
    const bool vec = (a.N & 3) == 0;
    const coherent_rsrc_t prs = coherent_rsrc(a.part);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 4 * kq, t = nt * 16 + row;
      float* dst = &a.part[((size_t)ks * a.M + t) * a.N + n];
      if (vec && t < a.M && n + 3 < a.N) {
        st_coherent4(prs, (uint32_t)((((size_t)ks * a.M + t) * a.N + n) * 4), __builtin_bit_cast(u32x4, acc[nt]));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < a.N && t < a.M) st_coherent(dst + i, acc[nt][i]);
      }
    }
    __shared__ int s_last;
    if (!arrive_last(a.rg_counter + rgi, (uint32_t)a.ks_n, &s_last)) return;
    // the last slice of the row group adds the partials in slice order:
    // thread tid takes 4 consecutive rows of one token at positions tid,
    // tid + 256, ... (NT of them: 64 rows x 16 NT tokens); the partials of
    // kSliceGroup slices for all its positions are requested before any is
    // added (one memory round trip per group of slices)
    const int nb = rgi * kMfmaRows;
    f32x4 sum[NT];
#pragma unroll
    for (int p = 0; p < NT; ++p) sum[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < a.ks_n; q0 += kSliceGroup) {
      f32x4 pv[NT][kSliceGroup];
#pragma unroll
      for (int p = 0; p < NT; ++p) {
        const int idx = (tid + p * kMfmaWaves * 64) * 4;
        const int t = idx / kMfmaRows, n = nb + idx % kMfmaRows;
        const bool ok = vec && t < a.M && n + 3 < a.N;
#pragma unroll
        for (int q = 0; q < kSliceGroup; ++q) {
          const int qc = q0 + q < a.ks_n ? q0 + q : 0;
          pv[p][q] = __builtin_bit_cast(
              f32x4, ld_coherent4(prs, (uint32_t)((((size_t)qc * a.M + (ok ? t : 0)) * a.N + (ok ? n : 0)) * 4)));
        }
      }
#pragma unroll
      for (int p = 0; p < NT; ++p)
#pragma unroll
        for (int q = 0; q < kSliceGroup; ++q)
          if (q0 + q < a.ks_n) sum[p] += pv[p][q];
    }
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      const int idx = (tid + p * kMfmaWaves * 64) * 4;
      const int t = idx / kMfmaRows, n = nb + idx % kMfmaRows;
      if (t >= a.M || n >= a.N) continue;
      if (vec && n + 3 < a.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) finish_value(a, t, n + i, sum[p][i]);
      } else {
        for (int i = 0; i < 4 && n + i < a.N; ++i) {
          float v = 0.f;
          for (int q = 0; q < a.ks_n; ++q) v += ld_coherent(&a.part[((size_t)q * a.M + t) * a.N + n + i]);
          finish_value(a, t, n + i, v);
        }
      }
    }
  }
}

// Router with latent rows on the vector shape: 4 rows per 8-wave workgroup,
// so that with the router kernel's register count (one 16-wave or two
// 8-wave workgroups per compute unit) the E + L rows (1408 at E = 384, L =
// 1024) run in one round of resident workgroups: two rows per 16-wave
// workgroup took three rounds, and the merged product was slower than the
// router and the latent product launched apart.
constexpr int kRouterLatentRows = 4;
constexpr int kRouterLatentWaves = 8;

int skinny_rows_per_block(int variant, int router) {
  if (variant == VAR_MFMA) return kMfmaRows;
  if (router == 2) return kRouterLatentRows;
  if (router) return kRouterRows;
  if (variant == VAR_SPLITK) return 4;
  if (variant == VAR_ROWS) return 4 * kRowsGroups;
  return 2;
}
int skinny_default_splits(int variant, int bf16, int M, int N, int K, int router) {
  (void)M;
  if (variant == VAR_MFMA) return kMfmaWaves;
  if (variant == VAR_ROWS) return (K / 8 + 63) / 64;   // one 16-byte chunk of K per thread
  // The router's workgroups have 16 waves (the finish is shared among them);
  // waves beyond the K range just idle through the product.
  if (router) return 16;
  const int rows = skinny_rows_per_block(variant, router);
  const int nwg = (N + rows - 1) / rows;
  // waves per launch: ~12 per CU for the small-matrix shape (two per
  // workgroup at N = 3072: 9.4 -> 8.9 us at B = 1), ~6 for split-K (more
  // made it slower: its activation loads already match the weight loads)
  const int target = variant == VAR_GEMV ? 3072 : 1536;
  int nw = (target + nwg - 1) / nwg;
  int maxw = (K / (bf16 ? 8 : 4)) / 64;
  if (maxw > 16) maxw = 16;
  if (maxw < 1) maxw = 1;
  if (nw > maxw) nw = maxw;
  if (nw < 1) nw = 1;
  return nw;
}
int shared_up_tiles_host(const ExpertLaunch& ex, int nw) {
  const int pp = nw / 2;
  return (ex.Is + pp - 1) / pp;
}

hipError_t launch_skinny(const SkinnyLaunch& a0, hipStream_t st, char* desc, size_t desc_len) {
  SkinnyLaunch a = a0;
  const bool latent_rows = a.router && a.L > 0 && a.variant != VAR_MFMA;
  const int rows = skinny_rows_per_block(a.variant, latent_rows ? 2 : a.router);
  const int nrg = (a.N + rows - 1) / rows;
  if (latent_rows) a.S = kRouterLatentWaves;
  const int nw = a.S;
  if (a.variant == VAR_MFMA) {
    if (a.router && a.finish) router_mfma_slices(a.M, a.N, a.K, &a.ks_n, &a.ks_steps);
    else skinny_mfma_slices(a.M, a.N, a.K, &a.ks_n, &a.ks_steps);
  } else {
    a.ks_n = 1;
    a.ks_steps = 0;
  }
  const int nwg = nrg * a.ks_n;
  a.router_wgs = nwg;
  a.router_arrivals = nrg;
  // the shared expert's gate/up rides a vector router launch (vector shape)
  const int extra = (a.router && a.ex.Ws13 && a.variant != VAR_MFMA) ? shared_up_tiles_host(a.ex, nw) : 0;
  a.shared_tiles = extra;
  dim3 grid((unsigned)(nwg + extra)), block((unsigned)(64 * nw));
  const char* name = "?";
  if (a.variant == VAR_MFMA) {
    if ((a.ks_n > 1 || (a.router && a.finish)) && (!a.part || !a.rg_counter)) return hipErrorInvalidValue;
    const int nt = (a.M + 15) / 16;
    const size_t lds = 0;
    // router with finish: the product launch stores logits only, then the
    // finish launch selects; with the profiling hook armed the product's
    // dispatch records the start event and the finish's the stop event
    const bool split = a.router && a.finish;
    SkinnyLaunch p = a;
    if (split) {
      p.finish = 0;
      p.defer = 1;
    }
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool prof = a.router && profile_events_for(K_ROUTE, &e0, &e1);
    auto go = [&](auto rk, auto pk) {
      if (!a.router) launch(K_SKINNY, pk, grid, block, (uint32_t)lds, st, p);
      else if (prof) hipExtLaunchKernelGGL(rk, grid, block, lds, st, e0, split ? nullptr : e1, 0u, p);
      else hipLaunchKernelGGL(rk, grid, block, lds, st, p);
    };
    switch (nt) {
      case 1: go(skinny_mfma_kernel<1, true>, skinny_mfma_kernel<1, false>); break;
      case 2: go(skinny_mfma_kernel<2, true>, skinny_mfma_kernel<2, false>); break;
      case 3: go(skinny_mfma_kernel<3, true>, skinny_mfma_kernel<3, false>); break;
      default: go(skinny_mfma_kernel<4, true>, skinny_mfma_kernel<4, false>); break;
    }
    if (split) {
      const dim3 fg((unsigned)a.M);   // one workgroup per token
      if (prof) hipExtLaunchKernelGGL(route_finish_kernel, fg, dim3(kFinishWaves * 64), 0, st, nullptr, e1, 0u, a);
      else hipLaunchKernelGGL(route_finish_kernel, fg, dim3(kFinishWaves * 64), 0, st, a);
    }
    name = split ? "mfma + finish launch" : "mfma";
  } else if (latent_rows) {
    name = a.variant == VAR_SPLITK ? "splitk" : "gemv";
    constexpr int RL = kRouterLatentRows;
    if (a.bf16) {
      if (a.M <= 1) launch(K_ROUTE, skinny_valu_kernel<bf16_t, RL, 1, 2, true>, grid, block, 0, st, a);
      else if (a.M <= 2) launch(K_ROUTE, skinny_valu_kernel<bf16_t, RL, 2, 2, true>, grid, block, 0, st, a);
      else if (a.M <= 4) launch(K_ROUTE, skinny_valu_kernel<bf16_t, RL, 4, 1, true>, grid, block, 0, st, a);
      else launch(K_ROUTE, skinny_valu_kernel<bf16_t, RL, 8, 1, true>, grid, block, 0, st, a);
    } else {
      if (a.M <= 1) launch(K_ROUTE, skinny_valu_kernel<float, RL, 1, 2, true>, grid, block, 0, st, a);
      else if (a.M <= 2) launch(K_ROUTE, skinny_valu_kernel<float, RL, 2, 2, true>, grid, block, 0, st, a);
      else if (a.M <= 4) launch(K_ROUTE, skinny_valu_kernel<float, RL, 4, 1, true>, grid, block, 0, st, a);
      else launch(K_ROUTE, skinny_valu_kernel<float, RL, 8, 1, true>, grid, block, 0, st, a);
    }
  } else if (a.router) {
    name = a.variant == VAR_SPLITK ? "splitk" : "gemv";
    if (a.bf16) {
      if (a.M <= 1) launch(K_ROUTE, skinny_valu_kernel<bf16_t, kRouterRows, 1, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 2) launch(K_ROUTE, skinny_valu_kernel<bf16_t, kRouterRows, 2, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 4) launch(K_ROUTE, skinny_valu_kernel<bf16_t, kRouterRows, 4, 2, true>, grid, block, 0, st, a);
      else launch(K_ROUTE, skinny_valu_kernel<bf16_t, kRouterRows, 8, 1, true>, grid, block, 0, st, a);
    } else {
      if (a.M <= 1) launch(K_ROUTE, skinny_valu_kernel<float, kRouterRows, 1, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 2) launch(K_ROUTE, skinny_valu_kernel<float, kRouterRows, 2, 4, true>, grid, block, 0, st, a);
      else if (a.M <= 4) launch(K_ROUTE, skinny_valu_kernel<float, kRouterRows, 4, 2, true>, grid, block, 0, st, a);
      else launch(K_ROUTE, skinny_valu_kernel<float, kRouterRows, 8, 1, true>, grid, block, 0, st, a);
    }
  } else if (a.variant == VAR_ROWS) {
    if (!a.bf16 || a.router || a.K % 8 || a.K / 8 > 1024 || a.M > 8) return hipErrorInvalidValue;
    if (a.M <= 1) launch(K_SKINNY, skinny_rows_kernel<1, 4>, grid, block, 0, st, a);
    else if (a.M <= 2) launch(K_SKINNY, skinny_rows_kernel<2, 4>, grid, block, 0, st, a);
    else if (a.M <= 4) launch(K_SKINNY, skinny_rows_kernel<4, 4>, grid, block, 0, st, a);
    // 5..8 tokens: every group's weights requested up front (ALL): the
    // products of the last group, which follow the last weight bytes, are
    // the part the stream cannot hide (dense B = 8 11.3 -> 11.1 us, output
    // projection 14.2 -> 13.5 us, same box; 6 groups of 2 rows: 11.2 /
    // 13.7 us)
    else launch(K_SKINNY, skinny_rows_kernel<8, 4, kRowsGroups, true>, grid, block, 0, st, a);
    name = "rows";
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
    snprintf(desc, desc_len, "%s M=%d N=%d K=%d waves/wg=%d grid=%d%s%s%s", name, a.M, a.N, a.K, nw, nwg,
             a.ks_n > 1 ? " k-slices" : "", extra ? " +shared gate/up" : "",
             a.router && !a.finish ? " logits-only" : "");
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_STAMPS
// Instrumented build: copy (out != null) or clear the clock stamps of this
// file's kernels (the router launches and the router's finish launch).
extern "C" int moe_stamps_route(void* out, int clear) {
  static unsigned long long zeros[moe::ST_KERNELS * moe::kStampWGs * moe::kStampSlots];
  if (clear) return (int)hipMemcpyToSymbol(HIP_SYMBOL(moe::g_stamps), zeros, sizeof zeros);
  return (int)hipMemcpyFromSymbol(out, HIP_SYMBOL(moe::g_stamps), sizeof zeros);
}
#endif
