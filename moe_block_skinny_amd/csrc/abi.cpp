// abi.cpp -- the C ABI declared in include/moe_skinny.h: host-side argument
// validation (complete before any HIP call), batch-shaped kernel choice,
// workspace layout, tracing of the chosen path, and the launches.
//
// Sources: [WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §1
// (kernel shape by batch size), part 2 §1 (the choice of path must be
// traceable at run time), part 2 §2 (a stated scope, outside which the
// standard path is used), part 2 §3 (tests must reach the changed path:
// hence the forced-shape switch and the per-call trace).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "expert_core.hpp"
#include "internal.hpp"
#include "moe_skinny.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";
thread_local char g_variant[256] = "";
std::atomic<int> g_force{-1};  // -1: not yet read from the environment
std::atomic<int> g_sched{-1};  // block schedule; -1: not yet read from the environment
std::atomic<int> g_shared{-1}; // where the shared expert's gate/up runs; -1: not yet read

constexpr int kMaxI = kMaxInter;   // kMaxB, kMaxE, kMaxK, kMaxInter: route_core.hpp
constexpr int kMaxLatent = 8192;   // latent rows of moe_route_latent
static_assert(kNoallocScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
constexpr size_t kAlign = 256;

// Profiling hook: events recorded by the dispatch of one kernel.
struct ProfileHook {
  int kernel = -1;
  hipEvent_t start = nullptr, stop = nullptr;
} g_prof;

static_assert((int)K_ROUTE == (int)MOE_KERNEL_ROUTE && (int)K_EXPERT_UP == (int)MOE_KERNEL_EXPERT_UP &&
                  (int)K_EXPERT_DOWN == (int)MOE_KERNEL_EXPERT_DOWN && (int)K_COMBINE == (int)MOE_KERNEL_COMBINE &&
                  (int)K_SKINNY == (int)MOE_KERNEL_SKINNY && (int)K_BLOCK == (int)MOE_KERNEL_BLOCK &&
                  (int)K_STREAM == (int)MOE_KERNEL_STREAM,
              "kernel ids");

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

int forced() {
  int f = g_force.load();
  if (f < 0) {
    f = MOE_VARIANT_AUTO;
    const char* e = getenv("MOE_FORCE_VARIANT");
    if (e) {
      if (!strcmp(e, "gemv")) f = MOE_VARIANT_GEMV;
      else if (!strcmp(e, "splitk")) f = MOE_VARIANT_SPLITK;
      else if (!strcmp(e, "mfma")) f = MOE_VARIANT_MFMA;
      else if (!strcmp(e, "rows")) f = MOE_VARIANT_ROWS;
    }
    int expect = -1;
    g_force.compare_exchange_strong(expect, f);
    f = g_force.load();
  }
  return f;
}

int schedule() {
  int f = g_sched.load();
  if (f < 0) {
    f = MOE_SCHEDULE_AUTO;
    const char* e = getenv("MOE_BLOCK_SCHEDULE");
    if (e) {
      if (!strcmp(e, "launches")) f = MOE_SCHEDULE_LAUNCHES;
      else if (!strcmp(e, "fused")) f = MOE_SCHEDULE_FUSED;
      else if (!strcmp(e, "router_in_up")) f = MOE_SCHEDULE_ROUTER_IN_UP;
    }
    int expect = -1;
    g_sched.compare_exchange_strong(expect, f);
    f = g_sched.load();
  }
  return f;
}

int shared_schedule() {
  int f = g_shared.load();
  if (f < 0) {
    f = MOE_SHARED_AUTO;
    const char* e = getenv("MOE_SHARED_SCHEDULE");
    if (e) {
      if (!strcmp(e, "up")) f = MOE_SHARED_IN_UP;
      else if (!strcmp(e, "router")) f = MOE_SHARED_IN_ROUTER;
    }
    int expect = -1;
    g_shared.compare_exchange_strong(expect, f);
    f = g_shared.load();
  }
  return f;
}

bool trace_on() {
  static const int on = [] {
    const char* e = getenv("MOE_TRACE");
    return (e && *e && strcmp(e, "0")) ? 1 : 0;
  }();
  return on != 0;
}

void record(const char* op, int B, const char* desc) {
  snprintf(g_variant, sizeof g_variant, "%s B=%d %s", op, B, desc);
  if (trace_on()) fprintf(stderr, "[moe_skinny] %s\n", g_variant);
}

bool aligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) % 16) == 0; }
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---- kernel shape of the skinny product --------------------------------------

// Automatic shapes: the small-matrix (gemv) shape at B <= 2, split-K above
// (fp32, and the router up to B = 8, where the gate/up launch selects from
// its logits).  The dense bf16 product takes the rows shape at B = 2..8
// (K <= 8192) and the matrix shape above; measured at N = 3072, K = 7168:
// rows 9.1 / 9.6 / 11.1 us at B = 2 / 4 / 8 against gemv 9.6, split-K 11.4
// and the matrix shape 13.8; at B = 1 gemv (8.7 us) stays ahead of rows
// (8.9).  With a short K (the output projection, K = 3072: 6 waves per
// workgroup) rows loses at B = 2 (9.9 against gemv 9.4 us), ties split-K
// at B = 4 (10.7) and wins at B = 8 (14.2 against the matrix shape's 14.7).
constexpr int kDenseRowsMaxB = 8;
constexpr int kDenseRowsMinKAtB2 = 6144;
constexpr int kDenseSplitkMaxB = 4;   // beyond the rows shape's K (bf16, K % 32 == 0)
bool rows_ok(int bf16, int B, int K) { return bf16 && B <= kDenseRowsMaxB && K % 8 == 0 && K / 8 <= 1024; }

moe_status_t resolve_skinny(int bf16, int B, int K, int* variant, bool router = true) {
  const int f = forced();
  int v = f;
  // the rows shape is the dense product's only: other products choose as
  // under MOE_VARIANT_AUTO
  const bool auto_choice = f == MOE_VARIANT_AUTO || (f == MOE_VARIANT_ROWS && router);
  if (auto_choice) {
    const bool mfma_ok = bf16 && K % 32 == 0;
    const int splitk_max = (router || !mfma_ok) ? 8 : kDenseSplitkMaxB;
    if (!router && (B >= 3 || (B == 2 && K >= kDenseRowsMinKAtB2)) && rows_ok(bf16, B, K)) v = VAR_ROWS;
    else v = B <= 2 ? VAR_GEMV : (B <= splitk_max ? VAR_SPLITK : VAR_MFMA);
  }
  if (v == VAR_GEMV && B > 2) return fail(MOE_EUNSUPPORTED, "gemv shape supports B <= 2 (B=%d)", B);
  if (v == VAR_SPLITK && B > 8) return fail(MOE_EUNSUPPORTED, "splitk shape supports B <= 8 (B=%d)", B);
  if (v == VAR_MFMA && !bf16) return fail(MOE_EUNSUPPORTED, "mfma shape needs bf16 (fp32 supports B <= 8)");
  if (v == VAR_MFMA && K % 32) return fail(MOE_EUNSUPPORTED, "mfma shape needs K %% 32 == 0 (K=%d)", K);
  if (v == VAR_ROWS && !rows_ok(bf16, B, K))
    return fail(MOE_EUNSUPPORTED, "rows shape needs bf16, B <= 8 and K %% 8 == 0, K <= 8192 (B=%d, K=%d)", B, K);
  *variant = v;
  return MOE_OK;
}

// Workspace layout.  Every call's workspace starts with the same header of
// counter and flag words at fixed offsets, whatever the op and the sizes, and
// every call's data follows the header, so one zero-filled workspace large
// enough for the biggest call can serve calls of any op and size in turn:
// each call leaves its counters at zero, and no call's data ever lands on a
// counter.  The header holds the router's completion counter (word 0), one
// arrival counter per 64-row group of the MFMA product (words 32.., for
// N <= 63488), then the fused block's barrier lines (2 count lines, 2 x
// kBlockMaxGrid flag lines, a status line), then the logit keys of the
// router rows inside the gate/up launch (kKeyCopies copies of [B][E] words,
// B <= 2).
constexpr size_t kCounterBytes = 4096;
constexpr size_t kSyncOff = kCounterBytes;
constexpr size_t kSyncBytes = (size_t)(3 + 2 * kBlockMaxGrid) * kFlagStride * 4;
constexpr int kKeysMaxB = 2;
constexpr size_t kKeysOff = kSyncOff + kSyncBytes;
constexpr size_t kKeysBytes = (size_t)kKeyCopies * kKeyStride * 4;
static_assert(kKeysMaxB * kMaxE <= kKeyStride, "a copy of the keys holds B * E words");
constexpr size_t kHeaderBytes = (kKeysOff + kKeysBytes + kAlign - 1) / kAlign * kAlign;

// Skinny product / router: after the header, the router logits fp32 [B][N]
// (router only) and, where the MFMA shape may run with K slices (bf16), the
// fp32 partial sums of its slices [slices][B][N].
struct SkinnyWs {
  size_t logits, done, part, rg, total;
};

SkinnyWs skinny_ws(int B, int N, int K, int bf16, bool router) {
  SkinnyWs w;
  w.done = 0;
  w.rg = 32 * 4;
  size_t o = kHeaderBytes;
  const size_t rg_end = w.rg + (size_t)((N + 63) / 64) * 4;
  if (rg_end > o) o = up(rg_end);
  w.logits = o;
  if (router) o = up(o + (size_t)B * N * 4);
  w.part = o;
  bool sliced = false;
  if (bf16 && K >= 32) {
    int ks = 1, steps = 0;
    if (router) {
      // the MFMA router (any B when forced) stores the partial sums of
      // every K slice, one slice included, for its finish launch
      router_mfma_slices(B, N, K, &ks, &steps);
      sliced = true;
    } else {
      skinny_mfma_slices(B, N, K, &ks, &steps);
      sliced = ks > 1;
    }
    if (sliced) o = up(o + (size_t)ks * B * N * 4);
  }
  w.total = (router || sliced) ? o : 0;   // a plain vector-shape product needs none
  return w;
}

// Experts: after the header, the SwiGLU intermediate h.
struct ExpertWs {
  size_t h, total;
  int hld;
};

ExpertWs expert_ws(int B, int k, int I, int Is) {
  ExpertWs w;
  w.hld = I > Is ? I : Is;
  w.h = kHeaderBytes;
  w.total = up(w.h + (size_t)(B * k + B) * w.hld * 4);
  return w;
}

// Block: the router's layout at offset 0 (its counters are the header's),
// the fused barrier lines in the header, then h, ids, weights and plan.
struct BlockWs {
  SkinnyWs route;
  size_t route_off, ffn_h, ids, w, plan, ready, sync, up_part, ht, side_h, side_y, total;
  int hld;
};

BlockWs block_ws(int bf16, int B, int d, int E, int k, int I, int Is) {
  BlockWs b;
  b.route = skinny_ws(B, E, d, bf16, true);
  b.route_off = 0;
  b.sync = kSyncOff;
  b.hld = I > Is ? I : Is;
  size_t o = up(b.route.total);
  b.ffn_h = o;
  o = up(o + (size_t)(B * k + B) * b.hld * 4);
  b.ids = o;
  o = up(o + (size_t)B * k * 4);
  b.w = o;
  o = up(o + (size_t)B * k * 4);
  b.plan = o;
  o = up(o + (size_t)moe_plan_words(B, k, E) * 4);
  // the per-token selection's ready words (B*k <= 64 when used)
  b.ready = o;
  o = up(o + (size_t)B * k * 4);
  // the gate/up launch's K-slice partial sums (matrix shape, B > 8): at most
  // one task per workgroup of its grid (512) when tiles are cut, so at most
  // 256 cut tiles of 2 slices x 4 token tiles x 4 KB
  b.up_part = 0;
  if (bf16 && B > 8) {
    b.up_part = o;
    o = up(o + (size_t)256 * 2 * 4 * 4096);
  }
  // the tiled copy of h read by the matrix-shape down (bf16): two planes
  b.ht = 0;
  if (bf16) {
    b.ht = o;
    o = up(o + (size_t)2 * ht_rows(B, k, E) * b.hld * 2);
  }
  // the shared expert on a side stream (moe_block_streams): its h (B rows)
  // and its outputs fp32 [B][d]
  b.side_h = o;
  o = up(o + (size_t)B * b.hld * 4);
  b.side_y = o;
  o = up(o + (size_t)B * d * 4);
  b.total = o;
  return b;
}

// ---- validation -----------------------------------------------------------

moe_status_t check_dtype(int dt) {
  if (dt != MOE_DT_F32 && dt != MOE_DT_BF16) return fail(MOE_EINVAL, "unknown dtype %d", dt);
  return MOE_OK;
}

moe_status_t check_route_dims(int dt, int B, int d, int E, int k) {
  moe_status_t s = check_dtype(dt);
  if (s) return s;
  if (B <= 0 || d <= 0 || E <= 0 || k <= 0) return fail(MOE_EINVAL, "non-positive size");
  if (k > E) return fail(MOE_EINVAL, "k=%d > E=%d", k, E);
  if (B > kMaxB) return fail(MOE_EUNSUPPORTED, "B=%d outside the decode range 1..%d", B, kMaxB);
  if (E > kMaxE) return fail(MOE_EUNSUPPORTED, "E=%d > %d", E, kMaxE);
  if (k > kMaxK) return fail(MOE_EUNSUPPORTED, "k=%d > %d", k, kMaxK);
  if (dt == MOE_DT_BF16 && d % 32) return fail(MOE_EUNSUPPORTED, "d=%d not a multiple of 32", d);
  if (dt == MOE_DT_F32 && d % 4) return fail(MOE_EUNSUPPORTED, "d=%d not a multiple of 4", d);
  if (dt == MOE_DT_F32 && B > 8) return fail(MOE_EUNSUPPORTED, "fp32 supports B <= 8 (B=%d)", B);
  return MOE_OK;
}

moe_status_t check_inter(int dt, int I, const char* name) {
  if (I <= 0) return fail(MOE_EINVAL, "%s=%d", name, I);
  if (dt == MOE_DT_BF16 && (I % 32 || I > kMaxI))
    return fail(MOE_EUNSUPPORTED, "%s=%d must be a multiple of 32 up to %d", name, I, kMaxI);
  if (dt == MOE_DT_F32 && (I % 4 || I > 256))
    return fail(MOE_EUNSUPPORTED, "%s=%d must be a multiple of 4 up to 256 (fp32)", name, I);
  return MOE_OK;
}

moe_status_t expert_force(int dt, int B, int* force) {
  const int f = forced();
  if (f == MOE_VARIANT_MFMA && dt != MOE_DT_BF16)
    return fail(MOE_EUNSUPPORTED, "mfma shape needs bf16");
  if ((f == MOE_VARIANT_GEMV || f == MOE_VARIANT_SPLITK) && B > 8)
    return fail(MOE_EUNSUPPORTED, "vector expert shape supports up to 8 tokens per expert (B=%d)", B);
  *force = f == MOE_VARIANT_MFMA ? VAR_MFMA : ((f == MOE_VARIANT_AUTO || f == MOE_VARIANT_ROWS) ? VAR_AUTO : VAR_GEMV);
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// ---- launch helpers (arguments already validated) ---------------------------

// Router launch arguments (variant v already resolved).
SkinnyLaunch route_launch(int dt, int v, int B, int d, int E, int k, const void* X, const void* Wr,
                          const float* bias, int bias_ld, int32_t* ids, float* w, int32_t* plan,
                          float* logits_out, char* ws, int finish) {
  const int bf16 = dt == MOE_DT_BF16;
  const SkinnyWs L = skinny_ws(B, E, d, bf16, true);
  SkinnyLaunch a = {};
  a.bf16 = bf16;
  a.X = X;
  a.W = Wr;
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.rg_counter = reinterpret_cast<uint32_t*>(ws + L.rg);
  a.M = B;
  a.N = E;
  a.K = d;
  a.variant = v;
  a.S = skinny_default_splits(v, bf16, B, E, d, 1);
  a.router = 1;
  a.finish = finish;
  a.bias = bias;
  a.bias_ld = bias_ld;
  a.logits = reinterpret_cast<float*>(ws + L.logits);
  a.logits_out = logits_out;
  a.done_counter = reinterpret_cast<uint32_t*>(ws + L.done);
  a.k = k;
  a.topk_ids = ids;
  a.topk_w = w;
  a.plan = plan;
  return a;
}

moe_status_t run_route(int dt, int B, int d, int E, int k, const void* X, const void* Wr,
                       const float* bias, int bias_ld, int32_t* ids, float* w, int32_t* plan,
                       float* logits_out, char* ws, hipStream_t st, char* desc, size_t dl,
                       const ExpertLaunch* shared = nullptr, int finish = 1, const float** logits = nullptr,
                       int plan_by_consumer = 0, int32_t* clear = nullptr, int clear_n = 0) {
  int v;
  moe_status_t s = resolve_skinny(dt == MOE_DT_BF16, B, d, &v);
  if (s) return s;
  SkinnyLaunch a = route_launch(dt, v, B, d, E, k, X, Wr, bias, bias_ld, ids, w, plan, logits_out, ws, finish);
  a.plan_by_consumer = plan_by_consumer && v == VAR_MFMA;
  a.clear = clear;
  a.clear_n = clear_n;
  if (shared) a.ex = *shared;
  if (logits) *logits = a.logits;
  return hip_status(launch_skinny(a, st, desc, dl), "moe_route launch");
}

ExpertLaunch expert_launch(int dt, int B, int d, int E, int k, int I, const void* X, const int32_t* plan,
                           const void* W13, const void* W2, int Is, const void* Ws13, const void* Ws2,
                           char* ws, int force) {
  const ExpertWs L = expert_ws(B, k, I, Ws13 ? Is : 0);
  ExpertLaunch a = {};
  a.bf16 = dt == MOE_DT_BF16;
  a.B = B;
  a.d = d;
  a.E = E;
  a.k = k;
  a.I = I;
  a.Is = Ws13 ? Is : 0;
  a.X = X;
  a.plan = plan;
  a.W13 = W13;
  a.W2 = W2;
  a.Ws13 = Ws13;
  a.Ws2 = Ws2;
  a.h = ws ? reinterpret_cast<float*>(ws + L.h) : nullptr;
  a.hld = L.hld;
  a.force = force;
  return a;
}

moe_status_t run_ffn(int dt, int B, int d, int E, int k, int I, const void* X, const int32_t* plan,
                     const void* W13, const void* W2, int Is, const void* Ws13, const void* Ws2,
                     float* Yslot, char* ws, int force, hipStream_t st, char* desc, size_t dl) {
  ExpertLaunch a = expert_launch(dt, B, d, E, k, I, X, plan, W13, W2, Is, Ws13, Ws2, ws, force);
  a.Yslot = Yslot;
  char d1[128] = "", d2[128] = "";
  moe_status_t s;
  {
    s = hip_status(launch_expert_up(a, st, d1, sizeof d1), "expert gate/up launch");
  }
  if (s) return s;
  {
    s = hip_status(launch_expert_down(a, st, d2, sizeof d2), "expert down launch");
  }
  if (desc) snprintf(desc, dl, "%s; %s", d1, d2);
  return s;
}

}  // namespace

bool moe::profile_events_for(int id, hipEvent_t* start, hipEvent_t* stop) {
  if (g_prof.kernel != id) return false;
  *start = g_prof.start;
  *stop = g_prof.stop;
  return true;
}

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported by the specialised decode path";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

moe_status_t moe_profile_events(int kernel, void* start_event, void* stop_event) {
  g_err[0] = 0;
  if (!start_event && !stop_event) {
    g_prof.kernel = -1;
    g_prof.start = g_prof.stop = nullptr;
    return MOE_OK;
  }
  if (kernel < MOE_KERNEL_ROUTE || kernel > MOE_KERNEL_STREAM) return fail(MOE_EINVAL, "unknown kernel %d", kernel);
  if (!start_event || !stop_event) return fail(MOE_EINVAL, "both events or neither");
  g_prof.kernel = kernel;
  g_prof.start = reinterpret_cast<hipEvent_t>(start_event);
  g_prof.stop = reinterpret_cast<hipEvent_t>(stop_event);
  return MOE_OK;
}
const char* moe_last_variant(void) { return g_variant; }

int moe_set_variant(int variant) {
  const int prev = forced();
  if (variant < MOE_VARIANT_AUTO || variant > MOE_VARIANT_ROWS) return prev;
  g_force.store(variant);
  return prev;
}

int moe_set_shared_schedule(int sched) {
  const int prev = shared_schedule();
  if (sched < MOE_SHARED_AUTO || sched > MOE_SHARED_IN_ROUTER) return prev;
  g_shared.store(sched);
  return prev;
}

int moe_set_block_schedule(int sched) {
  const int prev = schedule();
  if (sched < MOE_SCHEDULE_AUTO || sched > MOE_SCHEDULE_ROUTER_IN_UP) return prev;
  g_sched.store(sched);
  return prev;
}

int moe_plan_words(int B, int k, int E) {
  const int maxa = B * k < E ? B * k : E;
  return 2 + 2 * maxa + B * k;
}

size_t moe_workspace_bytes(int op, int dtype, int B, int d, int E, int k, int I, int Is, int N, int K) {
  const int bf16 = dtype == MOE_DT_BF16;
  if (B <= 0) return 0;
  switch (op) {
    case MOE_OP_SKINNY_GEMM:
      if (N <= 0 || K <= 0) return 0;
      return skinny_ws(B, N, K, bf16, false).total;
    case MOE_OP_ROUTE:
      if (E <= 0 || d <= 0) return 0;
      return skinny_ws(B, E, d, bf16, true).total;
    case MOE_OP_EXPERT_FFN:
      if (k <= 0) return 0;
      return expert_ws(B, k, I, Is).total;
    case MOE_OP_BLOCK:
      if (E <= 0 || d <= 0 || k <= 0) return 0;
      return block_ws(bf16, B, d, E, k, I, Is).total;
    case MOE_OP_ROUTE_LATENT:   // N = L, the latent rows
      if (E <= 0 || d <= 0 || N <= 0) return 0;
      return skinny_ws(B, E + N, d, bf16, true).total;
  }
  return 0;
}

size_t moe_workspace_status_offset(void) {
  return kSyncOff + (size_t)(2 + 2 * kBlockMaxGrid) * kFlagStride * 4;
}

moe_status_t moe_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  g_err[0] = 0;
  if (!aligned(src) || !aligned(sink)) return fail(MOE_EINVAL, "src or sink null or misaligned");
  if (bytes == 0 || bytes % 16) return fail(MOE_EINVAL, "bytes=%zu not a positive multiple of 16", bytes);
  if (workgroups < 1 || workgroups > 65536) return fail(MOE_EINVAL, "workgroups=%d outside 1..65536", workgroups);
  return hip_status(launch_stream_read(src, bytes, sink, workgroups, reinterpret_cast<hipStream_t>(stream)),
                    "stream read launch");
}

moe_status_t moe_prefetch(int n, const void* const* ptrs, const size_t* bytes, uint32_t* sink, int workgroups,
                          void* stream) {
  g_err[0] = 0;
  if (n < 1 || n > kMaxPrefetch) return fail(MOE_EINVAL, "n=%d outside 1..%d", n, kMaxPrefetch);
  if (!ptrs || !bytes) return fail(MOE_EINVAL, "ptrs or bytes null");
  if (!aligned(sink)) return fail(MOE_EINVAL, "sink null or misaligned");
  if (workgroups < 1 || workgroups > 65536) return fail(MOE_EINVAL, "workgroups=%d outside 1..65536", workgroups);
  PrefetchRanges r = {};
  r.n = n;
  for (int i = 0; i < n; ++i) {
    if (!aligned(ptrs[i])) return fail(MOE_EINVAL, "range %d null or misaligned", i);
    if (bytes[i] == 0 || bytes[i] % 16) return fail(MOE_EINVAL, "range %d: %zu bytes, not a positive multiple of 16", i, bytes[i]);
    r.ptr[i] = ptrs[i];
    r.bytes[i] = bytes[i];
  }
  return hip_status(launch_prefetch(r, sink, workgroups, reinterpret_cast<hipStream_t>(stream)), "prefetch launch");
}

moe_status_t moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  return hip_status(launch_fill_zero(ws, ws_bytes, reinterpret_cast<hipStream_t>(stream)),
                    "workspace fill");
}

}  // extern "C"

namespace {

// skinny_gemm and skinny_gemm_residual: the product, plus R when non-null.
moe_status_t run_skinny_gemm(const char* op, int dtype, int B, int N, int K, const void* X, const void* W,
                             const void* R, void* Y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status_t s = check_dtype(dtype);
  if (s) return s;
  if (y_dtype != dtype && y_dtype != MOE_DT_F32) return fail(MOE_EINVAL, "y_dtype %d", y_dtype);
  if (B <= 0 || N <= 0 || K <= 0) return fail(MOE_EINVAL, "non-positive size");
  if (!aligned(X) || !aligned(W) || !aligned(Y)) return fail(MOE_EINVAL, "X, W or Y null or not 16-byte aligned");
  if (B > kMaxB) return fail(MOE_EUNSUPPORTED, "B=%d outside 1..%d", B, kMaxB);
  if (K % (dtype == MOE_DT_BF16 ? 8 : 4)) return fail(MOE_EUNSUPPORTED, "K=%d not a multiple of the vector width", K);
  const int bf16 = dtype == MOE_DT_BF16;
  int v;
  s = resolve_skinny(bf16, B, K, &v, false);
  if (s) return s;
  const SkinnyWs L = skinny_ws(B, N, K, bf16, false);
  if (L.total && !aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  if (ws_bytes < L.total) return fail(MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  SkinnyLaunch a = {};
  a.bf16 = bf16;
  a.X = X;
  a.W = W;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + L.part);
  a.rg_counter = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.rg);
  a.M = B;
  a.N = N;
  a.K = K;
  a.variant = v;
  a.S = skinny_default_splits(v, bf16, B, N, K, 0);
  a.Y = Y;
  a.y_bf16 = y_dtype == MOE_DT_BF16;
  a.R = R;
  char desc[160];
  {
    s = hip_status(launch_skinny(a, reinterpret_cast<hipStream_t>(stream), desc, sizeof desc),
                   "skinny_gemm launch");
  }
  if (!s) record(op, B, desc);
  return s;
}

}  // namespace

extern "C" {

moe_status_t skinny_gemm(int dtype, int B, int N, int K, const void* X, const void* W, void* Y,
                         int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  return run_skinny_gemm("skinny_gemm", dtype, B, N, K, X, W, nullptr, Y, y_dtype, ws, ws_bytes, stream);
}

moe_status_t skinny_gemm_residual(int dtype, int B, int N, int K, const void* X, const void* W, const void* R,
                                  void* Y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!aligned(R)) return fail(MOE_EINVAL, "R null or not 16-byte aligned");
  return run_skinny_gemm("skinny_gemm_residual", dtype, B, N, K, X, W, R, Y, y_dtype, ws, ws_bytes, stream);
}

moe_status_t moe_route(int dtype, int B, int d, int E, int k, const void* X, const void* Wr,
                       const float* bias, int bias_ld, int32_t* topk_ids, float* topk_w,
                       int32_t* plan, float* logits_out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status_t s = check_route_dims(dtype, B, d, E, k);
  if (s) return s;
  if (!aligned(X) || !aligned(Wr)) return fail(MOE_EINVAL, "X or Wr null or misaligned");
  if (!aligned(topk_ids) || !aligned(topk_w) || !aligned(plan))
    return fail(MOE_EINVAL, "topk_ids, topk_w or plan null or misaligned");
  if (bias && !aligned(bias)) return fail(MOE_EINVAL, "bias misaligned");
  if (bias && bias_ld != 0 && bias_ld != E) return fail(MOE_EINVAL, "bias_ld must be 0 or E");
  if (logits_out && !aligned(logits_out)) return fail(MOE_EINVAL, "logits_out misaligned");
  const int bf16 = dtype == MOE_DT_BF16;
  int v;
  s = resolve_skinny(bf16, B, d, &v);
  if (s) return s;
  const size_t need = skinny_ws(B, E, d, bf16, true).total;
  if (!aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  char desc[160];
  s = run_route(dtype, B, d, E, k, X, Wr, bias, bias_ld, topk_ids, topk_w, plan, logits_out,
                static_cast<char*>(ws), reinterpret_cast<hipStream_t>(stream), desc, sizeof desc);
  if (!s) record("moe_route", B, desc);
  return s;
}

moe_status_t moe_route_latent(int dtype, int B, int d, int E, int k, int L, const void* X, const void* Wr,
                              const void* Wl, const float* bias, int bias_ld, int32_t* topk_ids, float* topk_w,
                              int32_t* plan, void* latent_out, int latent_dtype, float* logits_out, void* ws,
                              size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status_t s = check_route_dims(dtype, B, d, E, k);
  if (s) return s;
  if (L <= 0) return fail(MOE_EINVAL, "L=%d", L);
  if (L % 16 || L > kMaxLatent) return fail(MOE_EUNSUPPORTED, "L=%d must be a multiple of 16 up to %d", L, kMaxLatent);
  if (E % 4) return fail(MOE_EUNSUPPORTED, "E=%d must be a multiple of 4 with a latent projection", E);
  if (latent_dtype != dtype && latent_dtype != MOE_DT_F32) return fail(MOE_EINVAL, "latent_dtype %d", latent_dtype);
  if (!aligned(X) || !aligned(Wr) || !aligned(Wl) || !aligned(latent_out))
    return fail(MOE_EINVAL, "X, Wr, Wl or latent_out null or misaligned");
  if (!aligned(topk_ids) || !aligned(topk_w) || !aligned(plan))
    return fail(MOE_EINVAL, "topk_ids, topk_w or plan null or misaligned");
  if (bias && !aligned(bias)) return fail(MOE_EINVAL, "bias misaligned");
  if (bias && bias_ld != 0 && bias_ld != E) return fail(MOE_EINVAL, "bias_ld must be 0 or E");
  if (logits_out && !aligned(logits_out)) return fail(MOE_EINVAL, "logits_out misaligned");
  const int bf16 = dtype == MOE_DT_BF16;
  int v;
  if ((s = resolve_skinny(bf16, B, d, &v))) return s;
  const size_t need = skinny_ws(B, E + L, d, bf16, true).total;
  if (!aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  SkinnyLaunch a = route_launch(dtype, v, B, d, E + L, k, X, Wr, bias, bias_ld, topk_ids, topk_w, plan, logits_out,
                                static_cast<char*>(ws), 1);
  a.Wlat = Wl;
  a.L = L;
  a.latent_out = latent_out;
  a.latent_bf16 = latent_dtype == MOE_DT_BF16;
  char desc[200];
  s = hip_status(launch_skinny(a, reinterpret_cast<hipStream_t>(stream), desc, sizeof desc), "moe_route_latent launch");
  if (!s) record("moe_route_latent", B, desc);
  return s;
}

moe_status_t moe_expert_ffn(int dtype, int B, int d, int E, int k, int I, const void* X,
                            const int32_t* plan, const void* W13, const void* W2, int Is,
                            const void* Ws13, const void* Ws2, float* Yslot, void* ws,
                            size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status_t s = check_route_dims(dtype, B, d, E, k);
  if (s) return s;
  if ((s = check_inter(dtype, I, "I"))) return s;
  if (Ws13 && (s = check_inter(dtype, Is, "Is"))) return s;
  if (!aligned(X) || !aligned(plan) || !aligned(W13) || !aligned(W2) || !aligned(Yslot))
    return fail(MOE_EINVAL, "X, plan, W13, W2 or Yslot null or misaligned");
  if (Ws13 && (!aligned(Ws13) || !aligned(Ws2))) return fail(MOE_EINVAL, "Ws13 or Ws2 null or misaligned");
  int force;
  if ((s = expert_force(dtype, B, &force))) return s;
  const size_t need = expert_ws(B, k, I, Ws13 ? Is : 0).total;
  if (!aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  char desc[300];
  s = run_ffn(dtype, B, d, E, k, I, X, plan, W13, W2, Is, Ws13, Ws2, Yslot, static_cast<char*>(ws),
              force, reinterpret_cast<hipStream_t>(stream), desc, sizeof desc);
  if (!s) record("moe_expert_ffn", B, desc);
  return s;
}

moe_status_t moe_combine(int dtype, int B, int d, int k, const float* Yslot, const float* topk_w,
                         int has_shared, void* out, void* stream) {
  g_err[0] = 0;
  moe_status_t s = check_dtype(dtype);
  if (s) return s;
  if (B <= 0 || d <= 0 || k <= 0) return fail(MOE_EINVAL, "non-positive size");
  if (B > kMaxB) return fail(MOE_EUNSUPPORTED, "B=%d outside 1..%d", B, kMaxB);
  if (k > kMaxK) return fail(MOE_EUNSUPPORTED, "k=%d > %d", k, kMaxK);
  if (!aligned(Yslot) || !aligned(topk_w) || !aligned(out)) return fail(MOE_EINVAL, "Yslot, topk_w or out null or misaligned");
  CombineLaunch a = {};
  a.out_bf16 = dtype == MOE_DT_BF16;
  a.B = B;
  a.d = d;
  a.k = k;
  a.has_shared = has_shared ? 1 : 0;
  a.Yslot = Yslot;
  a.topk_w = topk_w;
  a.out = out;
  {
    s = hip_status(launch_combine(a, reinterpret_cast<hipStream_t>(stream)), "moe_combine launch");
  }
  if (!s) record("moe_combine", B, "elementwise");
  return s;
}

}  // extern "C"

namespace {

// Arguments of moe_block and of its allocation-free variant.
struct BlockArgs {
  int dtype, B, d, E, k, I, Is;
  const void *X, *Wr;
  const float* bias;
  int bias_ld;
  const void *W13, *W2, *Ws13, *Ws2;
  void* out;
  int32_t* topk_ids;
  float* topk_w;
};

// Every check of the block's arguments but the workspace's, on the host:
// the kernel shapes and the workspace layout the launch will use.
moe_status_t block_check(const BlockArgs& a, int* v, int* force, BlockWs* L) {
  moe_status_t s = check_route_dims(a.dtype, a.B, a.d, a.E, a.k);
  if (s) return s;
  if ((s = check_inter(a.dtype, a.I, "I"))) return s;
  if (a.Ws13 && (s = check_inter(a.dtype, a.Is, "Is"))) return s;
  if (!aligned(a.X) || !aligned(a.Wr) || !aligned(a.W13) || !aligned(a.W2) || !aligned(a.out))
    return fail(MOE_EINVAL, "X, Wr, W13, W2 or out null or misaligned");
  if (a.Ws13 && (!aligned(a.Ws13) || !aligned(a.Ws2))) return fail(MOE_EINVAL, "Ws13 or Ws2 null or misaligned");
  if (a.bias && !aligned(a.bias)) return fail(MOE_EINVAL, "bias misaligned");
  if (a.bias && a.bias_ld != 0 && a.bias_ld != a.E) return fail(MOE_EINVAL, "bias_ld must be 0 or E");
  if ((a.topk_ids && !aligned(a.topk_ids)) || (a.topk_w && !aligned(a.topk_w)))
    return fail(MOE_EINVAL, "topk_ids or topk_w misaligned");
  const int bf16 = a.dtype == MOE_DT_BF16;
  if ((s = resolve_skinny(bf16, a.B, a.d, v))) return s;
  if ((s = expert_force(a.dtype, a.B, force))) return s;
  *L = block_ws(bf16, a.B, a.d, a.E, a.k, a.I, a.Ws13 ? a.Is : 0);
  return MOE_OK;
}

// The block's launches on workspace w (layout L), arguments already checked.
moe_status_t block_run(const BlockArgs& A, int v, int force, const BlockWs& L, char* w, hipStream_t st,
                       hipStream_t side = nullptr, hipEvent_t fork = nullptr, hipEvent_t join = nullptr) {
  const int dtype = A.dtype, B = A.B, d = A.d, E = A.E, k = A.k, I = A.I, Is = A.Is;
  const void *X = A.X, *Wr = A.Wr, *W13 = A.W13, *W2 = A.W2, *Ws13 = A.Ws13, *Ws2 = A.Ws2;
  const float* bias = A.bias;
  const int bias_ld = A.bias_ld;
  void* out = A.out;
  int32_t* topk_ids = A.topk_ids;
  float* topk_w = A.topk_w;
  const int bf16 = dtype == MOE_DT_BF16;
  moe_status_t s;
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(w + L.ids);
  float* tw = topk_w ? topk_w : reinterpret_cast<float*>(w + L.w);
  int32_t* plan = reinterpret_cast<int32_t*>(w + L.plan);
  ExpertLaunch ex = expert_launch(dtype, B, d, E, k, I, X, plan, W13, W2, Is, Ws13, Ws2, nullptr, force);
  ex.h = reinterpret_cast<float*>(w + L.ffn_h);
  ex.topk_w = tw;
  ex.out = out;
  ex.out_bf16 = bf16;
  if (L.up_part) {
    ex.up_part = reinterpret_cast<float*>(w + L.up_part);
    ex.up_counter = reinterpret_cast<uint32_t*>(w + 32 * 4);   // the header's arrival words
  }
  // Two schedules.  Small batch on the vector shape (B*k <= 64): the router
  // launch only scores; the gate/up launch selects the top-k and builds the
  // plan in every workgroup (no cross-workgroup handshake) and runs the
  // shared expert's gate/up first.  Otherwise the router's last workgroup
  // selects and plans, and the shared expert's gate/up runs inside the
  // router launch when both take the same kernel family (the vector router
  // kernel carries only the vector gate/up, the MFMA one only the MFMA one).
  const int paths = expert_paths(bf16, force, B);
  if (paths != kPathValu) {
    ex.ht_hi = reinterpret_cast<uint16_t*>(w + L.ht);
    ex.ht_lo = ex.ht_hi + (size_t)ht_rows(B, k, E) * L.hld;
  }
  const bool route_in_up = paths == kPathValu && v != VAR_MFMA && B * k <= 64;
  const int sched = schedule();
  // AUTO takes the three launches: on MI355X each grid-wide barrier of the
  // fused kernel (atomic arrival, flag broadcast, acquire) costs more than
  // a kernel boundary, so the fused launch is only selected on request.
  const bool fused = route_in_up && sched == MOE_SCHEDULE_FUSED && moe_block_fused_grid(ex, bf16, B) > 0;
  if (sched == MOE_SCHEDULE_FUSED && !fused)
    return fail(MOE_EUNSUPPORTED, "the fused block kernel does not cover these sizes (B*k <= 64, short expert rows)");
  char d1[200] = "", d2[128] = "", d3[128] = "";
  if (fused) {
    // The whole block in one launch (fused.hip)
    BlockLaunch f = {};
    f.r = route_launch(dtype, v, B, d, E, k, X, Wr, bias, bias_ld, ids, tw, plan, nullptr, w + L.route_off, 0);
    f.ex = ex;
    f.ex.skip_shared = 0;
    f.ex.logits = f.r.logits;
    f.ex.ids_out = ids;
    f.ex.w_out = tw;
    f.ex.plan_out = plan;
    uint32_t* sync = reinterpret_cast<uint32_t*>(w + L.sync);
    f.count = sync;
    f.flags_r = sync + 2 * kFlagStride;
    f.flags_h = f.flags_r + (size_t)kBlockMaxGrid * kFlagStride;
    f.status = f.flags_h + (size_t)kBlockMaxGrid * kFlagStride;
    if ((s = hip_status(launch_moe_block_fused(f, st, d1, sizeof d1), "fused block launch"))) return s;
    record("moe_block", B, d1);
    return MOE_OK;
  }
  if (side && (!route_in_up || !Ws13 || fused))
    return fail(MOE_EUNSUPPORTED, "the shared expert runs on a side stream only in the small-batch schedule "
                                  "(B*k <= 64, vector shape) with a shared expert");
  char d0[64] = "";
  if (side) {
    // the shared expert alone on the side stream, overlapping routing and
    // the routed gate/up: a launch with k = 0, so h rows and outputs are the
    // B tokens (same products as in the block's own launches)
    ExpertLaunch exs = ex;
    exs.k = 0;
    exs.h = reinterpret_cast<float*>(w + L.side_h);
    exs.Yslot = reinterpret_cast<float*>(w + L.side_y);
    exs.ht_hi = exs.ht_lo = nullptr;
    if ((s = hip_status(hipEventRecord(fork, st), "fork event"))) return s;
    if ((s = hip_status(hipStreamWaitEvent(side, fork, 0), "side stream wait"))) return s;
    if ((s = hip_status(launch_shared_up(exs, side), "shared gate/up launch"))) return s;
    if ((s = hip_status(launch_shared_down(exs, side), "shared down launch"))) return s;
    if ((s = hip_status(hipEventRecord(join, side), "join event"))) return s;
    snprintf(d0, sizeof d0, "shared on side stream; ");
  }
  if (route_in_up) {
    // the shared expert's gate/up: in the gate/up launch (its tiles first,
    // streaming while the other workgroups select), in the router launch
    // (one pass over x), or on the side stream
    const int ssched = shared_schedule();
    const bool in_router = Ws13 && !side && ssched == MOE_SHARED_IN_ROUTER;
    // AUTO takes it where it applies: 22.6 -> 20.8 us at batch 1
    const bool router_in_up = (sched == MOE_SCHEDULE_ROUTER_IN_UP || sched == MOE_SCHEDULE_AUTO) && B <= kKeysMaxB &&
                              !in_router && !side;
    ex.skip_shared = (in_router || side) ? 1 : 0;
    ex.ids_out = ids;
    ex.w_out = tw;
    ex.plan_out = plan;
    ex.status = reinterpret_cast<uint32_t*>(w + moe_workspace_status_offset());
    ex.spin_limit = 1 << 20;   // about a second of polling
    if (router_in_up) {
      // the router rows in the gate/up launch itself (two launches): its
      // first workgroups score them and store the logits' keys in the
      // header, every gate/up workgroup waits for them and selects both
      // tokens itself; the down launch zeroes the keys again
      ex.Wr = Wr;
      ex.rbias = bias;
      ex.rbias_ld = bias_ld;
      ex.router_wgs = (E + kRouterRowsInUp - 1) / kRouterRowsInUp;
      ex.lkeys = reinterpret_cast<uint32_t*>(w + kKeysOff);
      snprintf(d1, sizeof d1, "rows in the gate/up launch, %d workgroups", ex.router_wgs);
    } else {
      // from batch 2 each token is selected once, by one gate/up workgroup,
      // and the others wait for it (the router launch clears the words);
      // at batch 1 every workgroup selects the one token itself (no wait)
      if (B >= 2) ex.ready = reinterpret_cast<int32_t*>(w + L.ready);
      if ((s = run_route(dtype, B, d, E, k, X, Wr, bias, bias_ld, ids, tw, plan, nullptr, w + L.route_off, st, d1,
                         sizeof d1, in_router ? &ex : nullptr, 0, &ex.logits, 0, ex.ready, ex.ready ? B * k : 0)))
        return s;
    }
  } else {
    // the vector router launch carries the shared expert's vector gate/up;
    // otherwise it is a task of the gate/up launch
    ex.skip_shared = Ws13 && paths == kPathValu && v != VAR_MFMA;
    // after the MFMA router the finish launch stores ids and weights only,
    // and every gate/up workgroup builds the plan from the ids (the gate/up
    // kernel then has the matrix shape, whose LDS holds the plan scratch)
    const bool consumer_plan = v == VAR_MFMA && paths != kPathValu;
    if (consumer_plan) {
      ex.ids_in = ids;
      ex.plan_out = plan;
    }
    if ((s = run_route(dtype, B, d, E, k, X, Wr, bias, bias_ld, ids, tw, plan, nullptr, w + L.route_off,
                       st, d1, sizeof d1, ex.skip_shared ? &ex : nullptr, 1, nullptr, consumer_plan ? 1 : 0)))
      return s;
  }
  {
    if ((s = hip_status(launch_expert_up(ex, st, d2, sizeof d2), "expert gate/up launch"))) return s;
  }
  {
    ExpertLaunch exd = ex;
    exd.ids_in = nullptr;   // the down launch reads the plan the gate/up launch stored
    if (side) {
      exd.y_shared = reinterpret_cast<const float*>(w + L.side_y);
      if ((s = hip_status(hipStreamWaitEvent(st, join, 0), "join wait"))) return s;
    }
    if ((s = hip_status(launch_expert_down_combine(exd, st, d3, sizeof d3), "expert down+combine launch")))
      return s;
  }
  char desc[480];
  snprintf(desc, sizeof desc, "%sroute[%s] %s; %s", d0, d1, d2, d3);
  record("moe_block", B, desc);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_block(int dtype, int B, int d, int E, int k, int I, int Is, const void* X,
                       const void* Wr, const float* bias, int bias_ld, const void* W13,
                       const void* W2, const void* Ws13, const void* Ws2, void* out,
                       int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  const BlockArgs a = {dtype, B, d, E, k, I, Is, X, Wr, bias, bias_ld, W13, W2, Ws13, Ws2, out, topk_ids, topk_w};
  int v, force;
  BlockWs L;
  moe_status_t s = block_check(a, &v, &force, &L);
  if (s) return s;
  if (!aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  if (ws_bytes < L.total) return fail(MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  return block_run(a, v, force, L, static_cast<char*>(ws), reinterpret_cast<hipStream_t>(stream));
}

moe_status_t moe_block_streams(int dtype, int B, int d, int E, int k, int I, int Is, const void* X,
                               const void* Wr, const float* bias, int bias_ld, const void* W13,
                               const void* W2, const void* Ws13, const void* Ws2, void* out,
                               int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream,
                               void* side_stream, void* fork_event, void* join_event) {
  g_err[0] = 0;
  const BlockArgs a = {dtype, B, d, E, k, I, Is, X, Wr, bias, bias_ld, W13, W2, Ws13, Ws2, out, topk_ids, topk_w};
  int v, force;
  BlockWs L;
  moe_status_t s = block_check(a, &v, &force, &L);
  if (s) return s;
  if (!side_stream || !fork_event || !join_event)
    return fail(MOE_EINVAL, "side_stream, fork_event and join_event are required");
  if (side_stream == stream) return fail(MOE_EINVAL, "side_stream must differ from stream");
  if (!aligned(ws)) return fail(MOE_EINVAL, "ws null or misaligned");
  if (ws_bytes < L.total) return fail(MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  const int bf16 = dtype == MOE_DT_BF16;
  const bool small = expert_paths(bf16, force, B) == kPathValu && v != VAR_MFMA && B * k <= 64;
  if (!small || !Ws13 || schedule() == MOE_SCHEDULE_FUSED)
    return fail(MOE_EUNSUPPORTED, "the shared expert runs on a side stream only in the three-launch small-batch "
                                  "schedule (B*k <= 64, vector shape) with a shared expert");
  return block_run(a, v, force, L, static_cast<char*>(ws), reinterpret_cast<hipStream_t>(stream),
                   reinterpret_cast<hipStream_t>(side_stream), reinterpret_cast<hipEvent_t>(fork_event),
                   reinterpret_cast<hipEvent_t>(join_event));
}

moe_status_t moe_block_noalloc(int dtype, int B, int d, int E, int k, int I, int Is, const void* X,
                               const void* Wr, const float* bias, int bias_ld, const void* W13,
                               const void* W2, const void* Ws13, const void* Ws2, void* out,
                               int32_t* topk_ids, float* topk_w, void* stream) {
  g_err[0] = 0;
  const BlockArgs a = {dtype, B, d, E, k, I, Is, X, Wr, bias, bias_ld, W13, W2, Ws13, Ws2, out, topk_ids, topk_w};
  int v, force;
  BlockWs L;
  moe_status_t s = block_check(a, &v, &force, &L);
  if (s) return s;
  if (L.total > kNoallocScratchBytes)
    return fail(MOE_EUNSUPPORTED, "these sizes need %zu bytes of workspace, above the %zu bytes of the "
                "library's scratch (use moe_block with a workspace)", L.total, (size_t)kNoallocScratchBytes);
  // the device address of this GPU's scratch array (looked up once per device)
  char* w = nullptr;
  if ((s = hip_status(noalloc_scratch(reinterpret_cast<void**>(&w)), "scratch address"))) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the scratch keeps the last call's contents: the header words every
  // launch expects at zero are cleared first (a kernel, so the call may be
  // captured in a graph)
  if ((s = hip_status(launch_fill_zero(w, kHeaderBytes, st), "scratch header"))) return s;
  return block_run(a, v, force, L, w, st);
}

}  // extern "C"
