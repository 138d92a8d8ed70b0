// internal.hpp -- host-side launch interface between the C-ABI layer
// (abi.cpp) and the kernel translation units.  Not part of the public API.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Variant { VAR_AUTO = 0, VAR_GEMV = 1, VAR_SPLITK = 2, VAR_MFMA = 3, VAR_ROWS = 4 };

// Router rows per workgroup when the router product runs inside the gate/up
// launch (ExpertLaunch::router_wgs), and the copies of the logit keys it
// stores: gate/up workgroup g polls copy g % kKeyCopies, kKeyStride words
// apart (B <= 2 tokens of E <= 512 experts each).
constexpr int kRouterRowsInUp = 2;
constexpr int kKeyCopies = 16;
constexpr int kKeyStride = 1024;

// Expert FFN stage over the routing plan.  h is fp32 [B*k + B][Imax]:
// routed slot s = t*k + j at row s, shared-expert token t at row B*k + t.
struct ExpertLaunch {
  int bf16;
  int B, d, E, k, I, Is;
  const void* X;            // [B][d]
  const int32_t* plan;
  const void* W13;          // [E][2I][d]
  const void* W2;           // [E][d][I]
  const void* Ws13;         // [2Is][d] or null
  const void* Ws2;          // [d][Is]
  float* h;                 // workspace
  // h of the matrix-shape down in 16-token tiles (hi plane, lo plane).  When
  // set, the gate/up launch writes h here instead of to the slot rows: an
  // entry's tile is 16 x hld bf16 in the order the matrix operand reads it,
  // so each K step of a tile is one contiguous 1 KB
  uint16_t* ht_hi;
  uint16_t* ht_lo;
  int hld;                  // row stride of h (max(I, Is))
  float* Yslot;             // [B][k+1][d]
  int force;                // VAR_AUTO, VAR_GEMV (vector path for all),
                            // VAR_MFMA (matrix path for all bf16 experts)
  int skip_shared;          // gate/up kernel: the shared expert is done elsewhere
  // fused down + combine
  const float* topk_w;      // [B][k]
  void* out;                // [B][d]
  int out_bf16;
  // routing inside the gate/up launch (fused block, B*k <= 64, vector
  // shape): router logits [B][E] with the bias added; the last workgroup
  // stores ids, weights (= topk_w) and the plan (= plan)
  const float* logits;
  int32_t* ids_out;
  float* w_out;
  int32_t* plan_out;
  // gate/up launch after a router finish that stored only ids [B][k]: every
  // workgroup builds the plan from them; the last also stores it (plan_out)
  const int32_t* ids_in;
  int down_rows;            // rows per workgroup of the prefetching down+combine
  // shared expert computed on a side stream: its per-token output fp32
  // [B][d]; the down+combine launch then leaves the shared entry out and
  // adds y_shared in the combine (null: the shared entry is one of its own)
  const float* y_shared;
  // gate/up on the matrix shape: the K-slice partial sums of tiles cut in
  // two (up_part, null: none are cut) and one arrival counter per such tile
  // (up_counter, zero on entry and left at zero)
  float* up_part;
  uint32_t* up_counter;
  // routing inside the gate/up launch with one selection per token (B >= 2):
  // workgroup t < B selects token t and stores id + 1 of each of its slots
  // to ready [B][k] (zeroed by the router launch); every workgroup waits for
  // all of them.  A wait that outlasts spin_limit polls sets *status.
  int32_t* ready;
  uint32_t* status;
  int spin_limit;
  // router rows inside the gate/up launch (B <= 2, vector shape): the first
  // router_wgs workgroups each score kRouterRowsInUp rows of Wr [E][d] (+
  // rbias [B][rbias_ld]) with the router launch's arithmetic and store each
  // logit's order key (never zero) to every copy of lkeys [kKeyCopies]
  // [kKeyStride] (a copy: [B][E]) with device-coherent stores; the other
  // workgroups poll the keys they need in their copy.  lkeys is zero on
  // entry, and the down + combine launch zeroes it again.
  const void* Wr;
  const float* rbias;
  int rbias_ld;
  int router_wgs;
  uint32_t* lkeys;
};

// Y[t][n] = sum_c X[t][c] W[n][c] for t < M, n < N, over K; either stored
// (Y, y_bf16) or, in router mode, turned into logits + bias and then top-k
// weights and the routing plan by the last workgroup to finish.  S is the
// number of waves per workgroup, which split K among themselves.
struct SkinnyLaunch {
  int bf16;                 // element type of X and W
  const void* X;
  const void* W;
  int M, N, K;
  int variant;              // VAR_GEMV / VAR_SPLITK / VAR_MFMA (resolved)
  int S;                    // waves per workgroup (in-workgroup K split)
  // store mode
  void* Y;
  int y_bf16;
  const void* R;            // residual [M][N] of the element type, added to Y (nullable)
  // router mode (router != 0); finish = 0: logits only (no top-k, no plan)
  int router;
  int finish;
  const float* bias;
  int bias_ld;
  float* logits;            // [M][E] workspace (E = N - L router rows)
  float* logits_out;        // optional copy [M][E]
  uint32_t* done_counter;   // zero on entry
  int k;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* plan;
  // router workgroups are blockIdx < router_wgs; in the fused block the
  // remaining shared_tiles workgroups run the shared expert's gate/up (ex);
  // router_arrivals workgroups arrive on done_counter
  int router_wgs;
  int shared_tiles;
  int router_arrivals;
  ExpertLaunch ex;
  // MFMA shape: K in ks_n slices of ks_steps 32-steps; with ks_n > 1 fp32
  // partial sums [ks_n][M][N] in part, one arrival counter per 64-row group
  int ks_n, ks_steps;
  float* part;
  uint32_t* rg_counter;
  // router on the MFMA shape with its finish launch: every K slice stores
  // its partial sums and the finish launch adds them (defer = 1); with
  // plan_by_consumer the finish stores ids and weights only and the gate/up
  // launch builds the plan from the ids
  int defer;
  int plan_by_consumer;
  // latent input projection concatenated with the router (router mode):
  // rows E .. N-1 of the product (E = N - L) are Wlat [L][K]; their sums go
  // to latent_out [M][L] (no bias), in the element type or fp32
  const void* Wlat;
  int L;
  void* latent_out;
  int latent_bf16;
  // words the launch zeroes before the gate/up launch uses them (ready of the
  // gate/up launch's per-token selection), or null
  int32_t* clear;
  int clear_n;
};

// The whole block in one launch (fused kernel, small batch on the vector
// shape): the router product r (logits into r.logits, 16-wave workgroups of
// kBlockRouterRows rows), then in every workgroup the top-k and plan, the
// gate/up of the routed experts, and the down projection with the weighted
// combine (ex, with ex.down_rows rows per workgroup).  Workgroups meet at
// two grid-wide barriers (grid_arrive / grid_wait: a count word each, zero
// between calls, and a flag line per workgroup each); a wait that outlasts
// spin_limit polls sets *status.
constexpr int kBlockMaxGrid = 512;   // flag lines per barrier in the workspace
struct BlockLaunch {
  SkinnyLaunch r;
  ExpertLaunch ex;
  uint32_t* count;          // router barrier at [0], h barrier at [kFlagStride]
  uint32_t* flags_r;        // kBlockMaxGrid flag lines of 128 bytes
  uint32_t* flags_h;
  uint32_t* status;         // 0; 1 after a wait gave up (never expected)
  int router_tasks;         // ceil(E / kBlockRouterRows)
  int shared_tasks;         // shared-expert gate/up tasks of 2 pairs
  int spin_limit;
};

struct CombineLaunch {
  int out_bf16;
  int B, d, k, has_shared;
  const float* Yslot;
  const float* topk_w;
  void* out;
};

// Kernel ids of the profiling hook (same values as the public moe_kernel_t).
enum KernelId {
  K_ROUTE = 0, K_EXPERT_UP = 1, K_EXPERT_DOWN = 2, K_COMBINE = 3, K_SKINNY = 4, K_BLOCK = 5, K_STREAM = 6,
  K_NONE = -1
};

// Events armed for kernel `id` by moe_profile_events (abi.cpp), if any.
bool profile_events_for(int id, hipEvent_t* start, hipEvent_t* stop);

// Launch; when the profiling hook is armed for `id`, the dispatch itself
// records the start and stop events (hipExtLaunchKernel), so the measured
// interval is the kernel's own execution, as a kernel trace reports it.
template <typename F, typename... Args>
inline void launch(int id, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (id != K_NONE && profile_events_for(id, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

hipError_t launch_skinny(const SkinnyLaunch& a, hipStream_t st, char* desc, size_t desc_len);
hipError_t launch_expert_up(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len);
hipError_t launch_expert_down(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len);
hipError_t launch_expert_down_combine(const ExpertLaunch& a, hipStream_t st, char* desc, size_t desc_len);
hipError_t launch_combine(const CombineLaunch& a, hipStream_t st);
// The shared expert alone (a launch with k = 0: h rows and outputs are the
// B tokens): gate/up + SwiGLU into a.h, then the down projection into
// a.Yslot fp32 [B][d], with the same products as the block's launches.
hipError_t launch_shared_up(const ExpertLaunch& a, hipStream_t st);
hipError_t launch_shared_down(const ExpertLaunch& a, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// Read-only streaming yardstick (stream.hip): `workgroups` workgroups read
// bytes (a multiple of 16) of src; sink[w] = XOR of slice w's 32-bit words.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t st);
// Weight prefetch (stream.hip): cached reads of up to kMaxPrefetch ranges.
constexpr int kMaxPrefetch = 8;
struct PrefetchRanges {
  const void* ptr[kMaxPrefetch];
  size_t bytes[kMaxPrefetch];   // multiples of 16
  int n;
};
hipError_t launch_prefetch(const PrefetchRanges& r, uint32_t* sink, int workgroups, hipStream_t st);
// Fused block: the workgroups it would launch (0: the fused kernel cannot
// hold the whole grid resident, so it must not be used), and the launch.
int moe_block_fused_grid(const ExpertLaunch& ex, int bf16, int B);
hipError_t launch_moe_block_fused(BlockLaunch& f, hipStream_t st, char* desc, size_t desc_len);

// moe_block_noalloc: bytes of the library's device-resident scratch (one
// array per GPU, noalloc.hip), and the device address of the current
// device's copy (looked up once per device).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// Row blocks of the skinny kernel for a given variant (host-side geometry).
int skinny_rows_per_block(int variant, int router);
int skinny_default_splits(int variant, int bf16, int M, int N, int K, int router);
// K slices of the MFMA shape (also sizes the partial-sum workspace)
void skinny_mfma_slices(int M, int N, int K, int* ks_n, int* ks_steps);
void router_mfma_slices(int M, int N, int K, int* ks_n, int* ks_steps);
int shared_up_tiles_host(const ExpertLaunch& ex, int nw);

}  // namespace moe
