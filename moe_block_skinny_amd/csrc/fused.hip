// fused.hip -- the whole decode MoE block in one launch, for small batch on
// the vector shape (B*k <= 64 slots, short expert rows).
//
// Sources (web pages on the Kimi K3 specialised decode path):
//   [WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §3 (MoE
//     scheduling: router scores, then the routed experts; a shared expert for
//     every token, overlapped with routing), part 1 §4 (small-batch decode is
//     bound by reading weights, so idle gaps between kernels cost bandwidth),
//     part 2 §1 (fewer launches per layer).
//   [AREX] "vLLM 宣布 Kimi K3 在 GB300 NVL72 上实现 batch 1 解码 842
//     tokens/s", section "每层从 23 个内核减到 13 个" (kernel count per layer).
//
// One workgroup of 16 waves per compute unit, all resident at once, runs the
// block's stages in order and meets the others at two grid-wide barriers:
//   1. router rows (2 per workgroup, whole workgroup) on the first
//      ceil(E/2) workgroups; every workgroup then arrives on the router
//      barrier; the shared expert's gate/up runs as 2-pair tasks of 4-wave
//      sub-groups on the other workgroups (it needs no routing);
//   2. wait for the router barrier; every workgroup selects the top-k of all
//      tokens from the logits and builds the plan in LDS (the last one also
//      stores ids, weights and plan for the caller);
//   3. the routed experts' gate/up + SwiGLU as 2-pair tasks, four sub-groups
//      of 4 waves per workgroup (tasks spread over all workgroups first);
//      arrive on the h barrier;
//   4. wait for it; stage h in LDS; the workgroup's ex.down_rows output rows
//      of every entry (down_valu_pipe), then the weighted combine of those
//      rows into out.
// Every product is the same device function, with the same split of the
// sums, as the three-launch schedule (router kernel, gate/up kernel,
// down+combine kernel), so the two schedules give identical bits.

#include "common.hpp"
#include "expert_core.hpp"
#include "internal.hpp"
#include "skinny_core.hpp"

namespace moe {

constexpr int kBlockWaves = 16;
constexpr int kSubWaves = 4;                      // waves of a gate/up sub-group
constexpr int kSubs = kBlockWaves / kSubWaves;    // sub-groups per workgroup
constexpr int kBlockRouterRows = 2;               // router rows per workgroup task
constexpr int kBlockMaxSlots = 64;                // B*k of the fused block
constexpr int kBlockPlanWords = 2 + 2 * kBlockMaxSlots + kBlockMaxSlots;
constexpr int kBlockDownRows = 28;                // most output rows per workgroup

// Gate/up task `task` of a sub-group (2 pairs, the 4 waves split each pair's
// d in two halves); a task past `total` (v.I = 0) only reaches the barrier.
template <typename T>
__device__ __forceinline__ void sub_up_task(const ExpertLaunch& a, const int32_t* slots, ExpertView v, int tile,
                                            bool ok, float* s_red) {
  const int wave = threadIdx.x >> 6;
  const int sub = wave / kSubWaves, sw = wave % kSubWaves;
  const int pin = sw & 1, half = sw >> 1;
  if (!ok) {
    v.I = 0;
    v.m = 0;
  }
  up_valu_dispatch<T, 2>(a, slots, v, (ok ? tile : 0) * 2 + pin, half, sub * 2 + pin, s_red);
  __syncthreads();   // s_red is reused by the next task
}

template <typename T, int MB, int U>
__global__ __launch_bounds__(kBlockWaves * 64) void moe_block_kernel(BlockLaunch f) {
  extern __shared__ __align__(16) float s_dyn[];   // top-k scratch; later s_y and h
  __shared__ float s_red[kBlockWaves * kBlockRouterRows * 8];
  __shared__ int32_t s_plan[kBlockPlanWords];
  __shared__ int32_t s_ids[kBlockMaxSlots];
  __shared__ float s_w[kBlockMaxSlots];
  __shared__ int s_order[kBlockMaxSlots + 1];
  const ExpertLaunch& a = f.ex;
  const int G = gridDim.x, b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int sub = wave / kSubWaves;

  // 1. router rows, arrival, shared gate/up
  for (int task = b; task < f.router_tasks; task += G) {
    valu_rows<T, kBlockRouterRows, MB, U>(f.r, task * kBlockRouterRows, s_red);
    __syncthreads();
  }
  __shared__ int s_last[2];
  const uint32_t g_r = grid_arrive(f.count + 0, f.flags_r, (uint32_t)G, s_last);
  {
    // sub-group slots counted from the last workgroup, which has no router task
    const int rb = G - 1 - b;
    for (int t0 = 0; t0 < f.shared_tasks; t0 += kSubs * G) {
      const int task = t0 + sub * G + rb;
      sub_up_task<T>(a, nullptr, shared_view(a), task, task < f.shared_tasks, s_red);
    }
  }

  // 2. top-k and plan of all tokens, in this workgroup's LDS
  grid_wait(f.flags_r, g_r, f.spin_limit, f.status);
  const PlanView p = route_here<true>(a, s_plan, reinterpret_cast<TopkScratch*>(s_dyn), s_ids, s_w);

  // 3. routed gate/up + SwiGLU
  {
    const int tiles = (a.I + 1) / 2;
    const int total = p.n * tiles;
    for (int t0 = 0; t0 < total; t0 += kSubs * G) {
      const int task = t0 + sub * G + b;
      const bool ok = task < total;
      sub_up_task<T>(a, p.slots, expert_view<T>(a, p, ok ? task / tiles : 0), ok ? task % tiles : 0, ok, s_red);
    }
  }
  const uint32_t g_h = grid_arrive(f.count + kFlagStride, f.flags_h, (uint32_t)G, s_last);

  // 4. down projection of this workgroup's rows, weighted combine
  grid_wait(f.flags_h, g_h, f.spin_limit, f.status);
  const int rt = a.down_rows;
  const int r0 = b * rt;
  if (r0 >= a.d) return;
  const int nrows = a.B * a.k + a.B;
  float* s_y = s_dyn;
  float* s_h = s_dyn + (size_t)nrows * rt;
  {
    // h to LDS as stored (fp32, or for bf16 weights the hi and lo planes,
    // which are the word rows down_valu_pipe reads)
    const int n4 = nrows * a.hld / 4;
    const coherent_rsrc_t hrs = coherent_rsrc(a.h);   // written by other workgroups of this launch
    for (int i = threadIdx.x; i < n4; i += blockDim.x)
      reinterpret_cast<u32x4*>(s_h)[i] = ld_coherent4(hrs, (uint32_t)i * 16u);
  }
  const int ne = p.n + (a.Ws13 ? 1 : 0);
  if (wave == 0) order_entries(a, p, ne, s_order);
  __syncthreads();
  const YSink sink = {s_y, 1, r0, rt};
  down_valu_pipe<T, kBlockDownRows>(a, p, ne, s_order, r0, rt, sink, s_h);
  __syncthreads();
  const int has_shared = a.Ws13 ? 1 : 0;
  for (int idx = threadIdx.x; idx < a.B * rt; idx += blockDim.x) {
    const int t = idx / rt, r = idx % rt;
    if (r0 + r >= a.d) continue;
    const float acc = combine_one(s_w + t * a.k, a.k, has_shared, [&](int j) {
      return s_y[(j < a.k ? t * a.k + j : a.B * a.k + t) * rt + r];
    });
    const size_t o = (size_t)t * a.d + r0 + r;
    if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[o] = f32_to_bf16(acc);
    else reinterpret_cast<float*>(a.out)[o] = acc;
  }
}

// ---- host side ---------------------------------------------------------------

static size_t block_lds(const ExpertLaunch& ex, int rt) {
  const size_t nrows = (size_t)ex.B * ex.k + ex.B;
  const size_t down = nrows * rt * sizeof(float) + nrows * ex.hld * sizeof(float);
  const size_t topk = (size_t)kTopkWaves * sizeof(TopkScratch);
  return down > topk ? down : topk;
}

template <typename T>
static void* block_kernel_for(int B) {
  if (B <= 1) return reinterpret_cast<void*>(moe_block_kernel<T, 1, 4>);
  if (B <= 2) return reinterpret_cast<void*>(moe_block_kernel<T, 2, 4>);
  if (B <= 4) return reinterpret_cast<void*>(moe_block_kernel<T, 4, 2>);
  return reinterpret_cast<void*>(moe_block_kernel<T, 8, 1>);
}

// Compute units of the current device, and whether one workgroup of the
// fused kernel fits on each with `lds` bytes of dynamic LDS (cached per
// device and kernel for the largest LDS the launcher allows).
static constexpr size_t kBlockMaxLds = 96 * 1024;

static int fused_grid_for(void* kernel) {
  static int cache_dev[16][16];
  static void* cache_k[16][16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  for (int i = 0; i < 16; ++i) {
    if (cache_k[dev][i] == kernel) return cache_dev[dev][i];
    if (!cache_k[dev][i]) {
      int cus = 0, occ = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kernel),
                                                       kBlockWaves * 64, kBlockMaxLds) != hipSuccess)
        occ = 0;
      cache_dev[dev][i] = occ >= 1 ? cus : 0;
      cache_k[dev][i] = kernel;
      return cache_dev[dev][i];
    }
  }
  return 0;
}

int moe_block_fused_grid(const ExpertLaunch& ex, int bf16, int B) {
  void* k = bf16 ? block_kernel_for<bf16_t>(B) : block_kernel_for<float>(B);
  int G = fused_grid_for(k);
  if (G > kBlockMaxGrid) G = kBlockMaxGrid;
  if (G < 1) return 0;
  const int vec = bf16 ? 8 : 4;
  if (ex.B > 8 || ex.B * ex.k > kBlockMaxSlots) return 0;   // vector shape: at most 8 tokens per expert
  if (ex.I > 16 * vec || (ex.Ws13 && ex.Is > 16 * vec)) return 0;   // down_valu_pipe rows
  const int rt = 4 * ((ex.d + 4 * G - 1) / (4 * G));
  if (rt > kBlockDownRows) return 0;
  if (block_lds(ex, rt) > kBlockMaxLds) return 0;
  if ((ex.E + kBlockRouterRows - 1) / kBlockRouterRows > 4 * G) return 0;
  return G;
}

hipError_t launch_moe_block_fused(BlockLaunch& f, hipStream_t st, char* desc, size_t desc_len) {
  const int G = moe_block_fused_grid(f.ex, f.ex.bf16, f.ex.B);
  if (G < 1) return hipErrorInvalidValue;
  const int rt = 4 * ((f.ex.d + 4 * G - 1) / (4 * G));
  f.ex.down_rows = rt;
  f.router_tasks = (f.r.N + kBlockRouterRows - 1) / kBlockRouterRows;
  f.shared_tasks = f.ex.Ws13 ? (f.ex.Is + 1) / 2 : 0;
  if (f.spin_limit <= 0) f.spin_limit = 1 << 20;   // about a second of polling
  const size_t lds = block_lds(f.ex, rt);
  void* k = f.ex.bf16 ? block_kernel_for<bf16_t>(f.ex.B) : block_kernel_for<float>(f.ex.B);
  const dim3 grid(G), block(kBlockWaves * 64);
  // A cooperative launch: the runtime refuses it unless every workgroup of
  // the grid can be resident at once, which the two grid-wide barriers need
  // (a workgroup that never started would leave the others polling until
  // the spin limit, then reading logits and h that were never written).
  // With the profiling hook armed the events are recorded on the stream
  // around the launch (a cooperative dispatch takes no events itself).
  hipEvent_t e0 = nullptr, e1 = nullptr;
  void* args[] = {&f};
  const bool prof = profile_events_for(K_BLOCK, &e0, &e1);
  hipError_t err = hipSuccess;
  if (prof) err = hipEventRecord(e0, st);
  if (err == hipSuccess) err = hipLaunchCooperativeKernel(k, grid, block, args, (unsigned)lds, st);
  if (err == hipSuccess && prof) err = hipEventRecord(e1, st);
  if (desc)
    snprintf(desc, desc_len, "fused grid=%d waves/wg=%d router tasks=%d shared tasks=%d rows/wg=%d", G, kBlockWaves,
             f.router_tasks, f.shared_tasks, rt);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace moe
