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
// Kernel shape follows the expert's token count m (expert_core.hpp).
// Kernels:
//   expert_up_kernel           gate/up + SwiGLU -> h, tasks (entry, 4 pairs);
//   expert_down_kernel         down -> per-slot outputs Yslot in HBM, tasks
//                              (entry, 64 rows);
//   expert_down_combine_kernel down + weighted combine -> out: a workgroup
//                              owns 16 output rows, its waves take the
//                              entries in turn and park the per-slot outputs
//                              in an LDS tile, then the tile is combined in
//                              the same order as combine_kernel (so the two
//                              routes give identical bits);
//   combine_kernel             out = sum_j w_j Yslot_j (+ Yslot_k).
// The first two are persistent: the grid is sized for the largest possible
// plan and every workgroup walks the tasks of the actual plan, which it
// first copies into LDS.  No kernel waits on another workgroup.

#include "common.hpp"
#include "expert_core.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kDownRows = 64;   // W2 rows per unfused down task (16 per wave)

__device__ __forceinline__ int entries(const ExpertLaunch& a, const PlanView& p, bool with_shared) {
  return p.n + ((with_shared && a.Ws13) ? 1 : 0);
}

// ---- gate/up + SwiGLU --------------------------------------------------------

// Vector-only instantiations: tasks (entry, 2 pairs), 4 waves, waves w and
// w + 2 take the two halves of d for pair w (more loads in flight per pair
// at no register cost).  With MFMA entries: an entry with more than 8 tokens
// has tasks of 32 pairs (64 weight rows, up_mfma), the others tasks of 2
// pairs as above; every workgroup lists the tasks per entry in LDS (a
// prefix over the plan) and walks them.
constexpr int kUpWaves = 4;
constexpr int kUpAllMfmaTasks = 256;   // one 64-row task per compute unit
constexpr unsigned kUpCUs = 256;       // workgroups g and g + 256 share a CU
constexpr int kUpPairsValu = 2;

template <typename T, int PATHS>
__global__ __launch_bounds__(kUpWaves * 64, PATHS == kPathValu ? 4 : 2) void expert_up_kernel(ExpertLaunch a) {
  constexpr int PPT = kUpPairsValu;
  __shared__ int32_t s_plan[kMaxPlanWords];
  __shared__ float s_red[PPT * 2 * kPartStride];
  const int wave = threadIdx.x >> 6;
  const int tiles_r = (a.I + PPT - 1) / PPT;
  const int tiles_s = (a.Ws13 && !a.skip_shared) ? (a.Is + PPT - 1) / PPT : 0;
  // stamps (instrumented build): 0 start; 1 router rows scored or shared
  // tiles done (vector shape), plan built (matrix shape); 2 plan ready
  // (vector), tasks listed (matrix); 3 first routed task done; 4 end;
  // 5 routed tasks | shared tasks << 16; 6 first matrix task: tokens |
  // cut << 16 | slice << 17 | shared << 20; 7 the CU
  MOE_STAMP(ST_UP, 0);
  MOE_STAMP_CU(ST_UP, 7);
  [[maybe_unused]] int n_routed = 0, n_shared = 0;
  if constexpr (PATHS == kPathValu) {
    // With the router rows in this launch, its first router_wgs workgroups
    // score them and leave; the others are the gate/up workgroups
    if (a.router_wgs && (int)blockIdx.x < a.router_wgs) {
      __shared__ float s_rr[kRouterPlayedWaves * kRouterRowsInUp * 2];
      router_rows_in_up<T, kUpWaves>(a, blockIdx.x, s_rr);
      MOE_STAMP(ST_UP, 1);
      return;
    }
    const int G = (int)gridDim.x - a.router_wgs;   // gate/up workgroups
    // Tasks: with routing here, the shared expert's tiles first -- they
    // need no plan and keep HBM busy while the routed workgroups select (and,
    // with the router rows here, while those are scored) -- then the routed
    // tiles; otherwise the routed tiles, then the shared ones.
    const bool here = a.logits != nullptr || a.lkeys != nullptr;
    PlanView p;
    int task0 = (int)blockIdx.x - a.router_wgs;
    if (here) {
      __shared__ TopkScratch s_tk[kUpWaves];
      __shared__ int32_t s_ids[64];
      __shared__ float s_w[64];
      // per-token selection: this workgroup's token first (before its
      // shared tiles), the wait for every token's after them
      if (a.ready) select_own_token(a, s_tk, s_ids, s_w);
      // with the router rows here, a workgroup that has no shared tile would
      // poll the keys for the ~2 us the router workgroups take, and its
      // loads would only queue with theirs: it sleeps ~1.8 us first (64 x
      // 64 cycles; polling from the start cost ~0.5 us at batch 1)
      if (a.lkeys && task0 >= tiles_s) __builtin_amdgcn_s_sleep(64);
      for (; task0 < tiles_s; task0 += G) {
        up_valu_dispatch<T, 2>(a, nullptr, shared_view(a), task0 * PPT + wave % PPT, wave / PPT, wave % PPT, s_red);
        __syncthreads();
        ++n_shared;
      }
      MOE_STAMP(ST_UP, 1);
      p = a.ready ? wait_token_plan(a, s_plan, s_tk, s_ids) : route_here<false, 1>(a, s_plan, s_tk, s_ids, s_w);
    } else {
      p = stage_plan(a, s_plan);
    }
    MOE_STAMP(ST_UP, 2);
    const int first = here ? tiles_s : 0;                    // first routed task
    const int total = first + p.n * tiles_r + (here ? 0 : tiles_s);
    // the four workgroups of a CU (g, g + 256, g + 512, g + 768) rotate
    // through the wave priorities, one task at a time, so the CU does not
    // serve them strictly by age (at batch 8 the first slot's workgroups
    // streamed their tasks 1.65x as fast as the fourth's; rotated, the
    // block took 75.3 instead of 76.0 us)
    int turn = (int)(blockIdx.x / kUpCUs);
    for (int task = task0; task < total; task += G) {
      switch (turn++ & 3) {
        case 0: __builtin_amdgcn_s_setprio(3); break;
        case 1: __builtin_amdgcn_s_setprio(2); break;
        case 2: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
      }
      const int rt = task - first;
      const bool routed = rt < p.n * tiles_r;
      const ExpertView v = routed ? expert_view<T>(a, p, rt / tiles_r) : shared_view(a);
      const int tile = routed ? rt % tiles_r : rt - p.n * tiles_r;
      up_valu_dispatch<T, 2>(a, p.slots, v, tile * PPT + wave % PPT, wave / PPT, wave % PPT, s_red);
      __syncthreads();  // s_red is reused by the next task
      if (n_routed++ == 0) MOE_STAMP(ST_UP, 3);
    }
  } else {
    __shared__ __align__(16) unsigned char s_x[MfmaX<4, kUpMfmaChunks>::kLdsBytes];
    __shared__ int s_tstart[kMaxE + 2];
    static_assert(sizeof(s_x) >= kPlanFromIdsBytes, "plan scratch fits the activation buffer");
    const PlanView p = a.ids_in ? plan_from_ids(a, s_plan, s_x) : stage_plan(a, s_plan);
    MOE_STAMP(ST_UP, 1);
    const int ne = p.n + (tiles_s > 0 ? 1 : 0);   // routed entries, then the shared one
    const int tiles_m = (a.I + kUpPairsMfma - 1) / kUpPairsMfma;
    const int tiles_ms = (a.Is + kUpPairsMfma - 1) / kUpPairsMfma;
    // Every entry takes the matrix shape once the routed entries alone make
    // a 64-row task per compute unit: the vector shape re-reads the entry's
    // activations (m rows of d) for every 4 weight rows, so at up to 8
    // tokens it moves up to twice its weight bytes again and streams at
    // about 2/3 the matrix shape's rate per workgroup (batch 64: ~34 such
    // entries made ~4300 vector tasks, 120 us); below that count the small
    // vector tasks are needed to spread the entries over the compute units.
    const bool all_mfma = PATHS == kPathBoth && p.n * tiles_m >= kUpAllMfmaTasks;
    auto mfma_entry = [&](int m) { return all_mfma || use_mfma<PATHS>(m); };
    // Tiles of entries with more than 16 tokens take longest (their
    // activations are staged in several 16-token tiles per K step): the
    // tiles of entries with at least smin token tiles are cut in two K
    // slices on two workgroups, the later of which adds the halves and
    // applies SwiGLU.  smin is the smallest of 2, 3, 4 for which the grid
    // still gives every task a workgroup of its own (0: no cut), so the
    // heaviest entries are cut first when not all can be.  s_tstart[e]:
    // first task of entry e; s_pbase[e] / s_cbase[e]: its first partial
    // block (4 KB units) and tile counter (cut entries); one wave, 64
    // entries per pass.
    constexpr int kSplit = 2;
    __shared__ unsigned short s_pbase[kMaxE + 2];
    __shared__ unsigned short s_cbase[kMaxE + 2];
    __shared__ int s_use_split;
    auto entry_tasks = [&](int e, int smin, int& pn, int& cn) {
      const bool sh = e >= p.n;
      const int m = sh ? a.B : p.offs[e + 1] - p.offs[e];
      pn = cn = 0;
      if (!mfma_entry(m)) return sh ? tiles_s : tiles_r;
      const int tiles = sh ? tiles_ms : tiles_m;
      if (smin && (m + 15) / 16 >= smin) {
        cn = tiles;
        pn = tiles * kSplit * ((m + 15) / 16);
        return tiles * kSplit;
      }
      return tiles;
    };
    if (wave == 0) {
      const int lane = threadIdx.x & 63;
      // tasks uncut (t1), and with the entries of >= 2, 3, 4 token tiles cut
      int t1 = 0, t2 = 0, t3 = 0, t4 = 0;
      if (a.up_part) {
        for (int e0 = 0; e0 < ne; e0 += 64) {
          const int e = e0 + lane;
          int pn, cn, n = 0, x = 0, nt = 0;
          if (e < ne) {
            n = entry_tasks(e, 0, pn, cn);
            const int m = e >= p.n ? a.B : p.offs[e + 1] - p.offs[e];
            if (mfma_entry(m)) {
              x = e >= p.n ? tiles_ms : tiles_m;   // a cut adds one task per tile
              nt = (m + 15) / 16;
            }
          }
          t1 += __builtin_amdgcn_readlane(wave_incl_scan(n), 63);
          t2 += __builtin_amdgcn_readlane(wave_incl_scan(nt >= 2 ? x : 0), 63);
          t3 += __builtin_amdgcn_readlane(wave_incl_scan(nt >= 3 ? x : 0), 63);
          t4 += __builtin_amdgcn_readlane(wave_incl_scan(nt >= 4 ? x : 0), 63);
        }
      }
      const int G = (int)gridDim.x;
      const int split = !a.up_part ? 0 : (t1 + t2 <= G ? 2 : (t1 + t3 <= G ? 3 : (t1 + t4 <= G ? 4 : 0)));
      int base = 0, pb = 0, cb = 0;
      for (int e0 = 0; e0 < ne; e0 += 64) {
        const int e = e0 + lane;
        int pn = 0, cn = 0;
        const int n = e < ne ? entry_tasks(e, split, pn, cn) : 0;
        const int incl = wave_incl_scan(n), pincl = wave_incl_scan(pn), cincl = wave_incl_scan(cn);
        if (e < ne) {
          s_tstart[e] = base + incl - n;
          s_pbase[e] = (unsigned short)(pb + pincl - pn);
          s_cbase[e] = (unsigned short)(cb + cincl - cn);
        }
        base += __builtin_amdgcn_readlane(incl, 63);
        pb += __builtin_amdgcn_readlane(pincl, 63);
        cb += __builtin_amdgcn_readlane(cincl, 63);
      }
      if (lane == 0) {
        s_tstart[ne] = base;
        s_use_split = split;
      }
    }
    __syncthreads();
    const int total = s_tstart[ne];
    const int smin = s_use_split;
    MOE_STAMP(ST_UP, 2);
    const int J = a.d / 32, nch = (J + kChunk - 1) / kChunk;
    for (int task = blockIdx.x; task < total; task += gridDim.x) {
      // entry of the task: the last e with s_tstart[e] <= task
      int lo = 0, hi = ne - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tstart[mid] <= task) lo = mid;
        else hi = mid - 1;
      }
      const int e = wave_uniform(lo);
      const ExpertView v = e < p.n ? expert_view<T>(a, p, e) : shared_view(a);
      const int local = task - s_tstart[e];
      if (mfma_entry(v.m)) {
        UpSlice sl = {0, J, 0, 1, nullptr, nullptr};
        int tile = local;
        if (smin && (v.m + 15) / 16 >= smin) {
          const int q = local % kSplit, nt = (v.m + 15) / 16;
          tile = local / kSplit;
          sl.s0 = (q * nch / kSplit) * kChunk;
          sl.s1 = ((q + 1) * nch / kSplit) * kChunk;
          if (sl.s1 > J) sl.s1 = J;
          sl.slice = q;
          sl.split = kSplit;
          sl.part = a.up_part + (size_t)(s_pbase[e] + tile * kSplit * nt) * (kMfmaWaves * 64 * 4);
          sl.counter = a.up_counter + s_cbase[e] + tile;
        }
        up_mfma_dispatch<T>(a, p.slots, v, tile * kUpPairsMfma, s_x, sl);
        if (n_routed == 0)
          MOE_STAMP_VAL(ST_UP, 6, v.m | (sl.split > 1) << 16 | sl.slice << 17 | (e >= p.n) << 20);
      } else {
        up_valu_dispatch<T, 2>(a, p.slots, v, local * PPT + wave % PPT, wave / PPT, wave % PPT, s_red);
      }
      __syncthreads();  // s_red / s_x are reused by the next task
      if (n_routed++ == 0) MOE_STAMP(ST_UP, 3);
    }
  }
  MOE_STAMP(ST_UP, 4);
  MOE_STAMP_VAL(ST_UP, 5, n_routed | n_shared << 16);
}

// ---- down projection -> Yslot ----------------------------------------------

// Tasks (entry, 64-row tile of d), four waves of 16 rows.  A workgroup
// takes a contiguous range of the task list (entry-major), so it stages an
// entry's h once for all the tiles of that entry it holds.  MFMA entries
// (m > 8): each wave requests its W2 rows (all K steps) first, then the
// workgroup stages h (bf16 planes) in LDS and the waves multiply from it;
// vector entries: down_valu with h from global.  Per-slot outputs go to
// Yslot; combine_kernel adds them.
template <typename T, int PATHS>
__global__ __launch_bounds__(256) void expert_down_kernel(ExpertLaunch a) {
  __shared__ int32_t s_plan[kMaxPlanWords];
  __shared__ __align__(16) unsigned char s_h[PATHS == kPathValu ? 16 : kHLdsBytes];
  const PlanView p = stage_plan(a, s_plan);
  const int tiles = (a.d + kDownRows - 1) / kDownRows;
  const int total = entries(a, p, true) * tiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = (total + gridDim.x - 1) / gridDim.x;
  const int t0 = blockIdx.x * per, t1 = t0 + per < total ? t0 + per : total;
  const YSink sink = {a.Yslot, 0, 0, 0};
  int staged = -1;   // entry whose h sits in s_h
  for (int task = t0; task < t1; ++task) {
    const int e_idx = task / tiles, tile = task % tiles;
    const ExpertView v = wave_uniform(expert_view<T>(a, p, e_idx));
    const int r0 = tile * kDownRows + wave * 16;
    if constexpr (PATHS != kPathValu && sizeof(T) == 2) {
      if (use_mfma<PATHS>(v.m)) {
        constexpr int JM = kMaxInter / 32;
        const int J = wave_uniform(v.I / 32);
        u32x4 wv[JM];
        load_w2_operands(reinterpret_cast<const bf16_t*>(v.W2), v.I, r0, a.d, J, wv);
        if (staged != e_idx) {
          __syncthreads();   // the previous entry's h reads are done
          stage_h_entry(a, p.slots, v, s_h);
          staged = e_idx;
        }
        __syncthreads();
        const int nt = (v.m + 15) / 16;
        if (nt <= 1) down_mfma_lds<1>(a, p.slots, v, r0, wv, s_h);
        else if (nt == 2) down_mfma_lds<2>(a, p.slots, v, r0, wv, s_h);
        else if (nt == 3) down_mfma_lds<3>(a, p.slots, v, r0, wv, s_h);
        else down_mfma_lds<4>(a, p.slots, v, r0, wv, s_h);
        continue;
      }
    }
    down_dispatch<T, kPathValu>(a, p.slots, v, r0, sink);
  }
}

// ---- down projection + combine -> out ----------------------------------------

// RT output rows per workgroup: 32 on the vector-only path with short rows
// (I, Is <= 16 chunks: 8 loads per lane per entry, so the whole grid is
// resident at once), else 16 (one M tile per MFMA wave; the LDS tile stays
// within 36 KB at B=64).
// PAIRED (matrix shape, RT > 16): a.down_rows (17..32) rows per workgroup,
// 8 waves of 256 registers; one wave takes both 16-row halves of an entry
// (down_mfma_duo), so h of an entry crosses from L2 once per workgroup (per
// 16 rows it was the larger part of the launch's L2 traffic at batch 64;
// per 16-row half on a pair of waves the launch took 56.8 us at batch 64,
// one wave for both 51.2 us).
template <typename T, int PATHS, int RT, bool PIPE>
__global__ __launch_bounds__(PATHS == kPathValu ? 1024 : 512, (PATHS == kPathValu || RT > 16) ? 1 : 4)
void expert_down_combine_kernel(ExpertLaunch a) {
  constexpr bool PAIRED = !PIPE && RT > 16 && PATHS != kPathValu;
  // PIPE (vector shape, short rows, h fits in LDS): h is staged in LDS with
  // the plan and each wave prefetches its next entry's W2 rows
  // (down_valu_pipe)
  __shared__ int32_t s_plan[kMaxPlanWords];
  __shared__ float s_tw[kMaxB * kMaxK];
  extern __shared__ float s_dyn[];   // s_y [B*k + B][rt], then (PIPE) h [B*k + B][hld]
  const int rt = (PIPE || PAIRED) ? a.down_rows : RT;
  float* s_y = s_dyn;
  float* s_h = s_dyn + (size_t)(a.B * a.k + a.B) * rt;
  // stamps (instrumented build): 0 start, 1 staged, 2 products done, 3 end,
  // 7 the CU
  MOE_STAMP(ST_DOWN, 0);
  MOE_STAMP_CU(ST_DOWN, 7);
  // the router rows' keys of the gate/up launch, zero again for the next call
  if (a.lkeys) {
    const int n = a.B * a.E;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < kKeyCopies * n; i += gridDim.x * blockDim.x)
      a.lkeys[(i / n) * kKeyStride + i % n] = 0u;
  }
  // The gate weights, (PIPE) h and the plan are requested together, into
  // registers, and written to LDS once all have arrived: one memory round
  // trip before the first W2 request instead of one per array.  h goes to
  // LDS as stored (fp32, or for bf16 weights the hi and lo planes, which are
  // the word rows down_valu_pipe reads).
  constexpr int kTwRegs = 2, kHRegs = 4;
  const int ntw = a.B * a.k, n4 = PIPE ? (a.B * a.k + a.B) * a.hld / 4 : 0;
  const int nt_ = (int)blockDim.x;
  float twr[kTwRegs];
  f32x4 hr[kHRegs];
#pragma unroll
  for (int q = 0; q < kTwRegs; ++q) {
    const int i = threadIdx.x + q * nt_;
    twr[q] = a.topk_w[i < ntw ? i : 0];
  }
  if constexpr (PIPE) {
#pragma unroll
    for (int q = 0; q < kHRegs; ++q) {
      const int i = threadIdx.x + q * nt_;
      hr[q] = reinterpret_cast<const f32x4*>(a.h)[i < n4 ? i : 0];
    }
  }
  __shared__ int s_order[kMaxB * kMaxK + kMaxB];
  const PlanView p = stage_plan(a, s_plan);
#pragma unroll
  for (int q = 0; q < kTwRegs; ++q) {
    const int i = threadIdx.x + q * nt_;
    if (i < ntw) s_tw[i] = twr[q];
  }
  for (int i = threadIdx.x + kTwRegs * nt_; i < ntw; i += nt_) s_tw[i] = a.topk_w[i];
  if constexpr (PIPE) {
#pragma unroll
    for (int q = 0; q < kHRegs; ++q) {
      const int i = threadIdx.x + q * nt_;
      if (i < n4) reinterpret_cast<f32x4*>(s_h)[i] = hr[q];
    }
    for (int i = threadIdx.x + kHRegs * nt_; i < n4; i += nt_)
      reinterpret_cast<f32x4*>(s_h)[i] = reinterpret_cast<const f32x4*>(a.h)[i];
  }
  MOE_STAMP(ST_DOWN, 1);
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * rt;
  const YSink sink = {s_y, 1, r0, rt};
  const int ne = entries(a, p, a.y_shared == nullptr);   // the shared entry, unless computed elsewhere
  // entries by falling token count, dealt to the waves in snake order
  // (w, 2nw-1-w, 2nw+w, ...) so their token totals come out close
  __shared__ int s_next;
  if (wave == 0) {
    if constexpr (PAIRED) {
      order_entries_by_tiles(a, p, ne, s_order);
    } else if (ne <= nw) {
      // one entry per wave at most: the order only says which wave takes
      // which entry, and each entry writes its own rows of s_y
      for (int i = threadIdx.x; i < ne; i += 64) s_order[i] = i;
    } else {
      order_entries(a, p, ne, s_order);
    }
    if ((threadIdx.x & 63) == 0) s_next = nw;
  }
  __syncthreads();
  if constexpr (PIPE) {
    down_valu_pipe<T, RT>(a, p, ne, s_order, r0, rt, sink, s_h);
  } else if constexpr (PAIRED) {
    // entries in order: wave w starts with entry w and then claims the next
    // free one from an LDS counter, so the waves finish together whatever
    // each entry costs (a fixed deal of the entries left the last waves
    // ~20 us behind the first at batch 64).  An entry's outputs go to its
    // own rows of s_y, so the result does not depend on which wave takes
    // which entry.
    const int r_end = r0 + rt < a.d ? r0 + rt : a.d;
    for (int u = wave;;) {
      if (u >= ne) break;
      const ExpertView v = expert_view<T>(a, p, s_order[u]);
      const int nt = (v.m + 15) / 16;
      if (nt <= 1) down_mfma_duo<1>(a, p.slots, v, r0, sink, r_end);
      else if (nt == 2) down_mfma_duo<2>(a, p.slots, v, r0, sink, r_end);
      else if (nt == 3) down_mfma_duo<3>(a, p.slots, v, r0, sink, r_end);
      else down_mfma_duo<4>(a, p.slots, v, r0, sink, r_end);
      int nx = 0;
      if ((threadIdx.x & 63) == 0) nx = atomicAdd(&s_next, 1);
      u = __builtin_amdgcn_readfirstlane(nx);
    }
  } else {
    for (int j = 0;; ++j) {
      const int pos = j * nw + ((j & 1) ? nw - 1 - wave : wave);
      if (pos >= ne) break;
      down_dispatch<T, PATHS, RT>(a, p.slots, expert_view<T>(a, p, s_order[pos]), r0, sink);
    }
  }
  __syncthreads();
  MOE_STAMP(ST_DOWN, 2);
  const int has_shared = a.Ws13 ? 1 : 0;
  for (int idx = threadIdx.x; idx < a.B * rt; idx += blockDim.x) {
    const int t = idx / rt, r = idx % rt;
    if (r0 + r >= a.d) continue;
    const float v = combine_one(s_tw + t * a.k, a.k, has_shared, [&](int j) {
      if (j == a.k && a.y_shared) return a.y_shared[(size_t)t * a.d + r0 + r];
      return s_y[(j < a.k ? t * a.k + j : a.B * a.k + t) * rt + r];
    });
    const size_t o = (size_t)t * a.d + r0 + r;
    if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[o] = f32_to_bf16(v);
    else reinterpret_cast<float*>(a.out)[o] = v;
  }
  MOE_STAMP(ST_DOWN, 3);
}

// ---- the shared expert alone (side stream) ---------------------------------

// Gate/up + SwiGLU of the shared expert: tasks of 2 pairs on 4 waves (waves
// w and w + 2 take the two halves of d for pair w), the tasks and products
// of the shared tiles in expert_up_kernel, hence the same bits.
template <typename T>
__global__ __launch_bounds__(kUpWaves * 64) void shared_up_kernel(ExpertLaunch a) {
  constexpr int PPT = kUpPairsValu;
  __shared__ float s_red[PPT * 2 * kPartStride];
  const int wave = threadIdx.x >> 6;
  up_valu_dispatch<T, 2>(a, nullptr, shared_view(a), blockIdx.x * PPT + wave % PPT, wave / PPT, wave % PPT, s_red);
}

// Down projection of the shared expert: 64 output rows per workgroup, 16
// per wave (down_valu, the products of the block's vector down), into
// a.Yslot laid out [B][1][d] (a launch with k = 0).
template <typename T>
__global__ __launch_bounds__(256) void shared_down_kernel(ExpertLaunch a) {
  const int wave = threadIdx.x >> 6;
  const YSink sink = {a.Yslot, 0, 0, 0};
  down_dispatch<T, kPathValu>(a, nullptr, wave_uniform(shared_view(a)), blockIdx.x * kDownRows + wave * 16, sink);
}

// ---- combine -------------------------------------------------------------------

__global__ __launch_bounds__(256) void combine_kernel(CombineLaunch a) {
  const size_t n = (size_t)a.B * a.d;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(idx / a.d), r = (int)(idx % a.d);
    const float* ys = a.Yslot + (size_t)t * (a.k + 1) * a.d + r;
    const float v = combine_one(a.topk_w + (size_t)t * a.k, a.k, a.has_shared,
                                [&](int j) { return ys[(size_t)j * a.d]; });
    if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[idx] = f32_to_bf16(v);
    else reinterpret_cast<float*>(a.out)[idx] = v;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---- host side ---------------------------------------------------------------

static int max_entries(const ExpertLaunch& a) {
  const int nslot = a.B * a.k;
  return (nslot < a.E ? nslot : a.E) + (a.Ws13 ? 1 : 0);
}

static const int kCUs = 256;                   // compute units of an MI355X
static const int kMaxResidentWG = kCUs * 8;
static const size_t kMaxStagedH = 72 * 1024;   // h staged in LDS by the 32-row down+combine

hipError_t launch_expert_up(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len) {
  const int paths = expert_paths(a.bf16, a.force, a.B);
  const int tiles_r = (a.I + kUpPairsValu - 1) / kUpPairsValu;
  const int tiles_s = (a.Is + kUpPairsValu - 1) / kUpPairsValu;
  const int nslot = a.B * a.k;
  int g = (nslot < a.E ? nslot : a.E) * tiles_r + ((a.Ws13 && !a.skip_shared) ? tiles_s : 0);
  // vector shape: the whole grid resident at once (4 workgroups per CU), so
  // no workgroup stages the plan, or selects, after others have finished;
  // with MFMA tasks: two workgroups per CU, walking the task list
  const int cap = paths == kPathValu ? 4 * kCUs : 2 * kCUs;
  if (g > cap) g = cap;
  // with the per-token selection, workgroup t selects token t: at least B
  if (a.ready && g < a.B) g = a.B;
  // router workgroups ahead of the gate/up ones, the whole grid resident
  if (a.router_wgs && g > cap - a.router_wgs) g = cap - a.router_wgs;
  if (g < 1) g = 1;
  const dim3 grid(g + a.router_wgs), block(kUpWaves * 64);
  if (!a.bf16) launch(K_EXPERT_UP, (expert_up_kernel<float, kPathValu>), grid, block, 0, st, a);
  else if (paths == kPathValu) launch(K_EXPERT_UP, (expert_up_kernel<bf16_t, kPathValu>), grid, block, 0, st, a);
  else if (paths == kPathMfma) launch(K_EXPERT_UP, (expert_up_kernel<bf16_t, kPathMfma>), grid, block, 0, st, a);
  else launch(K_EXPERT_UP, (expert_up_kernel<bf16_t, kPathBoth>), grid, block, 0, st, a);
  if (desc)
    snprintf(desc, desc_len, "up grid=%d%s%s%s force=%d", g, a.skip_shared ? " routed-only" : "",
             a.router_wgs ? " +router rows" : "", (a.logits || a.lkeys) ? " +top-k/plan" : "", a.force);
  return hipGetLastError();
}

hipError_t launch_expert_down(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len) {
  // two 4-wave workgroups per CU, each a contiguous range of the tasks
  const int tiles = (a.d + kDownRows - 1) / kDownRows;
  int g = max_entries(a) * tiles;
  if (g > 2 * kCUs) g = 2 * kCUs;
  if (g < 1) g = 1;
  const int paths = expert_paths(a.bf16, a.force, a.B);
  if (!a.bf16) launch(K_EXPERT_DOWN, (expert_down_kernel<float, kPathValu>), dim3(g), dim3(256), 0, st, a);
  else if (paths == kPathValu) launch(K_EXPERT_DOWN, (expert_down_kernel<bf16_t, kPathValu>), dim3(g), dim3(256), 0, st, a);
  else if (paths == kPathMfma) launch(K_EXPERT_DOWN, (expert_down_kernel<bf16_t, kPathMfma>), dim3(g), dim3(256), 0, st, a);
  else launch(K_EXPERT_DOWN, (expert_down_kernel<bf16_t, kPathBoth>), dim3(g), dim3(256), 0, st, a);
  if (desc) snprintf(desc, desc_len, "down tasks grid=%d force=%d", g, a.force);
  return hipGetLastError();
}

hipError_t launch_expert_down_combine(const ExpertLaunch& a0, hipStream_t st, char* desc, size_t desc_len) {
  ExpertLaunch a = a0;
  const int paths = expert_paths(a.bf16, a.force, a.B);
  // the matrix-shape down reads h from the tiled copy the gate/up launch wrote
  if (paths != kPathValu && (!a.ht_hi || !a.ht_lo)) return hipErrorInvalidValue;
  const int vec = a.bf16 ? 8 : 4;
  const bool short_rows = a.I <= 16 * vec && (!a.Ws13 || a.Is <= 16 * vec);
  const size_t h_bytes = (size_t)(a.B * a.k + a.B) * a.hld * sizeof(float);
  // prefetching shape: one 16-wave workgroup per CU (its register count
  // allows no second), rows split evenly in multiples of 4, up to 28
  const int rt_pipe = 4 * ((a.d + 4 * kCUs - 1) / (4 * kCUs));
  const bool pipe = paths == kPathValu && short_rows && h_bytes <= kMaxStagedH && rt_pipe <= 28;
  int rt = 16;
  if (pipe) {
    rt = rt_pipe;
    a.down_rows = rt;
  }
  // matrix shape: rows split evenly over the compute units in multiples of
  // 4; above 16 one wave takes both 16-row halves of an entry (8 waves)
  const bool paired = !pipe && paths != kPathValu && a.bf16 && rt_pipe > 16 && rt_pipe <= 32;
  if (paired) {
    rt = rt_pipe;
    a.down_rows = rt;
  }
  const int g = (a.d + rt - 1) / rt;
  int nw = max_entries(a);
  const int maxw = paths == kPathValu ? 16 : 8;
  if (nw > maxw) nw = maxw;
  if (nw < 1) nw = 1;
  const size_t lds = (size_t)(a.B * a.k + a.B) * rt * sizeof(float) + (pipe ? h_bytes : 0);
  const dim3 grid(g), block(64 * nw);
  if (!a.bf16 && pipe) launch(K_EXPERT_DOWN, (expert_down_combine_kernel<float, kPathValu, 28, true>), grid, block, lds, st, a);
  else if (!a.bf16) launch(K_EXPERT_DOWN, (expert_down_combine_kernel<float, kPathValu, 16, false>), grid, block, lds, st, a);
  else if (pipe) launch(K_EXPERT_DOWN, (expert_down_combine_kernel<bf16_t, kPathValu, 28, true>), grid, block, lds, st, a);
  else if (paths == kPathValu) launch(K_EXPERT_DOWN, (expert_down_combine_kernel<bf16_t, kPathValu, 16, false>), grid, block, lds, st, a);
  // with the matrix shape allowed, every entry takes it, also one of one
  // token: an entry's W2 rows cost one round trip either way, the matrix
  // shape was no slower per entry at batch 64 (~6 us against ~7 us for 1-2
  // tokens, ~10-16 us for 3-8 on the vector shape), and the kernel holding
  // both shapes spilled 35 registers to scratch
  else if (paired) launch(K_EXPERT_DOWN, (expert_down_combine_kernel<bf16_t, kPathMfma, 32, false>), grid, block, lds, st, a);
  else launch(K_EXPERT_DOWN, (expert_down_combine_kernel<bf16_t, kPathMfma, 16, false>), grid, block, lds, st, a);
  if (desc)
    snprintf(desc, desc_len, "down+combine grid=%d rows/wg=%d waves/wg=%d%s force=%d", g, rt, nw,
             pipe ? " prefetch" : (paired ? " paired" : ""), a.force);
  return hipGetLastError();
}

hipError_t launch_shared_up(const ExpertLaunch& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.Is + kUpPairsValu - 1) / kUpPairsValu)), block(kUpWaves * 64);
  if (a.bf16) launch(K_EXPERT_UP, shared_up_kernel<bf16_t>, grid, block, 0, st, a);
  else launch(K_EXPERT_UP, shared_up_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_shared_down(const ExpertLaunch& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.d + kDownRows - 1) / kDownRows)), block(256);
  if (a.bf16) launch(K_NONE, shared_down_kernel<bf16_t>, grid, block, 0, st, a);
  else launch(K_NONE, shared_down_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.d;
  int g = (int)((n + 255) / 256);
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  launch(K_COMBINE, combine_kernel, dim3(g), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  int g = (int)((words + 255) / 256);
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  launch(K_NONE, fill_zero_kernel, dim3(g), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_STAMPS
// Instrumented build: copy (out != null) or clear the clock stamps of this
// file's kernels (the gate/up and down + combine launches).
extern "C" int moe_stamps_expert(void* out, int clear) {
  static unsigned long long zeros[moe::ST_KERNELS * moe::kStampWGs * moe::kStampSlots];
  if (clear) return (int)hipMemcpyToSymbol(HIP_SYMBOL(moe::g_stamps), zeros, sizeof zeros);
  return (int)hipMemcpyFromSymbol(out, HIP_SYMBOL(moe::g_stamps), sizeof zeros);
}
#endif
