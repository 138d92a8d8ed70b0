/*
 * moe_skinny.h -- C ABI of the MI355X (gfx950) decode-step MoE block.
 *
 * The block is the mixture-of-experts layer of a large MoE transformer at
 * decode time (batch 1-64), on one GPU's tensor-parallel weight shard:
 * router scoring and top-k selection, the token->expert plan, skinny
 * gate/up/down expert products with SwiGLU, a shared expert and the weighted
 * combine; plus the dense skinny product used for the attention input
 * projection.
 *
 * Sources (web pages on the Kimi K3 specialised decode path):
 *   [WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能" (Chinese translation
 *     of the vLLM write-up): part 1 §1 (batch-shaped kernels: a small-matrix
 *     kernel at batch 1-2, split-K above), part 1 §3 (router scores and the
 *     latent projection per rank, routed experts, a shared expert on its own
 *     stream), part 1 §4 (small-batch decode is bound by weight reads),
 *     part 2 §1 (the switch into and out of the specialised path must be
 *     traceable at run time), part 2 §2 (scope: decode batch up to 64 on the
 *     tested parallel settings; other work stays on the standard path),
 *     part 2 §3 (tests must exercise the changed path).
 *   [AREX] "vLLM 宣布 Kimi K3 在 GB300 NVL72 上实现 batch 1 解码 842
 *     tokens/s": sections "每层从 23 个内核减到 13 个" (the same four changes)
 *     and "DeepSeek-V4.1-Flash 跟进同一模式" (opt-in path, prefill and mixed
 *     batches fall back to the default implementation).
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller, 16-byte
 *     aligned, contiguous, row-major.  The library never allocates, frees or
 *     synchronises; it enqueues on `stream` (a hipStream_t, NULL = default
 *     stream) and returns.  Buffers must stay alive until the stream has run
 *     the work.
 *   - dtype: MOE_DT_BF16 (bf16 storage) or MOE_DT_F32.  Activations and
 *     weights share the dtype; all accumulation is fp32.
 *   - Weight layouts ([out][in], the in-dimension contiguous):
 *       Wr   [E][d]          router
 *       W13  [E][2I][d]      per expert: gate rows 0..I-1, then up rows I..2I-1
 *       W2   [E][d][I]       per expert down projection
 *       Ws13 [2Is][d], Ws2 [d][Is]   shared expert (same split)
 *       W    [N][K]          dense skinny product
 *   - Workspace: `ws` is caller-owned device memory of at least
 *     moe_workspace_bytes(...) bytes.  It holds the router logits, the
 *     SwiGLU intermediate, per-slot expert outputs and a completion counter.
 *     It must
 *     be zero-filled once before its first use (moe_workspace_init); every
 *     call leaves its counter words at zero again.  The counter words sit in
 *     a header at the start of the workspace, at offsets that depend neither
 *     on the op nor on the sizes (for N <= 63488), and every call's data
 *     follows that header, so one workspace large enough for the biggest
 *     call may serve calls of any op and size in turn.  Two calls that run
 *     concurrently must not share a workspace.
 *   - Errors: every call validates all arguments on the host BEFORE any HIP
 *     call and returns MOE_EINVAL (null or misaligned pointer, bad dimension,
 *     k > E, unknown dtype), MOE_EUNSUPPORTED (outside the specialised
 *     path's scope: B outside 1..64, E > 512, k > 16, sizes not multiples of
 *     the vector width, ...; the caller should use its standard path),
 *     MOE_EWORKSPACE (ws too small) or MOE_EHIP (a launch failed).  Nothing
 *     is enqueued unless MOE_OK is returned; no call ever silently switches
 *     to another path.  moe_last_error() gives the detail.
 *   - Kernel shape follows the batch (WRITEUP part 1 §1): "gemv" at B <= 2,
 *     "splitk" at B <= 8, "mfma" above; the dense bf16 products (skinny_gemm,
 *     skinny_gemm_residual) take "rows" at B = 3..8 (and at B = 2 when
 *     K >= 6144) where K <= 8192.  moe_set_variant() (or the
 *     MOE_FORCE_VARIANT environment variable: gemv, splitk, mfma, rows) forces one
 *     shape wherever it supports the sizes, and fails the call with
 *     MOE_EUNSUPPORTED where it does not.  MOE_TRACE=1 prints the chosen
 *     shape of every call to stderr; moe_last_variant() returns it
 *     (thread-local).
 */
#ifndef MOE_SKINNY_H
#define MOE_SKINNY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status_t;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_VARIANT_AUTO = 0,
  MOE_VARIANT_GEMV = 1,
  MOE_VARIANT_SPLITK = 2,
  MOE_VARIANT_MFMA = 3,
  MOE_VARIANT_ROWS = 4  /* dense product only (bf16, B <= 8, K <= 8192): each
                           workgroup owns 12 weight rows over all of K; other
                           products choose as under MOE_VARIANT_AUTO */
} moe_variant_t;

typedef enum {
  MOE_OP_SKINNY_GEMM = 0,
  MOE_OP_ROUTE = 1,
  MOE_OP_EXPERT_FFN = 2,
  MOE_OP_BLOCK = 3,
  MOE_OP_ROUTE_LATENT = 4
} moe_op_t;

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text for a status code (any int: "unknown status" outside
 * moe_status_t). */
const char* moe_status_str(int s);

/* Detail of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Kernel shape chosen by the last successful call on this thread. */
const char* moe_last_variant(void);

/* Force a kernel shape for every later call in the process
 * (MOE_VARIANT_AUTO restores the batch-based choice).  Returns the previous
 * setting. */
int moe_set_variant(int variant);

/* Schedule of moe_block: MOE_SCHEDULE_AUTO (MOE_SCHEDULE_ROUTER_IN_UP where
 * it applies, else three launches: on MI355X the fused launch's two
 * grid-wide barriers cost more than the kernel boundaries they replace),
 * MOE_SCHEDULE_LAUNCHES (three launches), MOE_SCHEDULE_FUSED (one launch;
 * MOE_EUNSUPPORTED outside its scope) or MOE_SCHEDULE_ROUTER_IN_UP (at
 * B <= 2 in the small-batch schedule with the shared expert's gate/up in the
 * gate/up launch, two launches: the router rows run in the gate/up launch,
 * whose other workgroups wait for the logits; elsewhere three launches).  Also set by
 * the MOE_BLOCK_SCHEDULE environment variable (auto, launches, fused,
 * router_in_up).  All schedules give identical bits.  Returns the previous
 * setting. */
typedef enum {
  MOE_SCHEDULE_AUTO = 0,
  MOE_SCHEDULE_LAUNCHES = 1,
  MOE_SCHEDULE_FUSED = 2,
  MOE_SCHEDULE_ROUTER_IN_UP = 3
} moe_schedule_t;
int moe_set_block_schedule(int schedule);

/* Where moe_block runs the shared expert's gate/up in the small-batch
 * schedule (B*k <= 64, vector shape; WRITEUP part 1 §3: the shared expert
 * overlaps routing): MOE_SHARED_IN_UP (its tiles first in the gate/up
 * launch, streaming while the other workgroups select the top-k) or
 * MOE_SHARED_IN_ROUTER (in the router launch: one pass over x for the router
 * rows and the shared gate/up rows).  MOE_SHARED_AUTO takes the one measured
 * faster on MI355X (currently MOE_SHARED_IN_UP).  Also set by the
 * MOE_SHARED_SCHEDULE environment variable (up, router).  All placements
 * give identical bits.  Returns the previous setting. */
typedef enum { MOE_SHARED_AUTO = 0, MOE_SHARED_IN_UP = 1, MOE_SHARED_IN_ROUTER = 2 } moe_shared_schedule_t;
int moe_set_shared_schedule(int schedule);

/* int32 words of a routing plan for B tokens, top-k of E experts:
 * 2 + 2*min(E, B*k) + B*k.  Layout, with maxa = min(E, B*k):
 *   plan[0]                    n, the number of distinct experts selected
 *   plan[1 .. 1+maxa)          those experts in ascending id (unused: -1)
 *   plan[1+maxa .. 2+2*maxa)   slot offsets per listed expert, n+1 used
 *                              (unused entries: B*k)
 *   plan[2+2*maxa .. +B*k)     slots s = t*k + j (token t's j-th choice),
 *                              grouped by expert, tokens ascending. */
int moe_plan_words(int B, int k, int E);

/* Bytes of workspace a call needs.  op: moe_op_t.  Unused sizes may be 0:
 *   MOE_OP_SKINNY_GEMM: dtype, B, N, K
 *   MOE_OP_ROUTE:       dtype, B, d, E, k
 *   MOE_OP_EXPERT_FFN:  dtype, B, d, E, k, I, Is
 *   MOE_OP_BLOCK:       dtype, B, d, E, k, I, Is
 *   MOE_OP_ROUTE_LATENT: dtype, B, d, E, k, and N = L (the latent rows) */
size_t moe_workspace_bytes(int op, int dtype, int B, int d, int E, int k, int I, int Is, int N,
                           int K);

/* Kernels, for moe_profile_events. */
typedef enum {
  MOE_KERNEL_ROUTE = 0,        /* router logits + top-k + plan */
  MOE_KERNEL_EXPERT_UP = 1,    /* expert gate/up + SwiGLU */
  MOE_KERNEL_EXPERT_DOWN = 2,  /* expert down projection */
  MOE_KERNEL_COMBINE = 3,      /* weighted combine */
  MOE_KERNEL_SKINNY = 4,       /* dense skinny product */
  MOE_KERNEL_BLOCK = 5,        /* the whole block in one launch (moe_block) */
  MOE_KERNEL_STREAM = 6        /* the read-only streaming yardstick (moe_stream_read) */
} moe_kernel_t;

/* Profiling hook (for timing one kernel with HIP events on the stream it is
 * launched on): while armed, every launch of `kernel` is dispatched with
 * hipExtLaunchKernel so that the dispatch itself records start_event when
 * the kernel starts and stop_event when it ends.  Both NULL disarms.
 * Process-wide; not for concurrent use.
 * start_event / stop_event are hipEvent_t handles owned by the caller.
 * Returns MOE_EINVAL for an unknown kernel or only one NULL event. */
moe_status_t moe_profile_events(int kernel, void* start_event, void* stop_event);

/* Byte offset in ws of the status word of moe_block's in-launch waits (a
 * uint32, inside the workspace header, the same for every op and size).  It
 * reads 0 unless a wait gave up (the call's outputs are then invalid): a
 * grid-wide barrier of the fused schedule, or, from B = 2 in the small-batch
 * schedule, a gate/up workgroup's wait for the tokens' ids.  No call clears
 * it; moe_workspace_init does.  The fused launch is cooperative (the runtime
 * refuses it when the grid cannot be resident at once), and the gate/up
 * workgroups wait only for workgroups of lower index, dispatched before
 * them, so the word is not expected to move. */
size_t moe_workspace_status_offset(void);

/* Measurement yardstick, not part of the block (WRITEUP part 1 §4: small-
 * batch decode is bound by reading weights): reads `bytes` of src (device
 * memory, 16-byte aligned, bytes a positive multiple of 16) with 128-bit
 * nontemporal loads -- each wave instruction one contiguous 1 KB, the access
 * of the weight streams -- in `workgroups` workgroups of 256 threads, each
 * over one contiguous slice, and stores the XOR of slice w's 32-bit words to
 * sink[w] (uint32 [workgroups], device memory), so the XOR of all of sink
 * equals the XOR of every word of src.  Its rate is the measured read
 * ceiling the kernels are compared with.  1 <= workgroups <= 65536;
 * MOE_EINVAL otherwise. */
moe_status_t moe_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream);

/* Weight prefetch (WRITEUP part 1 §4: weights that are about to be used are
 * read into the cache by a kernel on a side stream while the running work
 * uses little memory bandwidth).  Reads n (1..8) ranges of device memory --
 * ptrs[i] 16-byte aligned, bytes[i] a positive multiple of 16; ptrs and
 * bytes are HOST arrays -- with cached 128-bit loads, so the lines stay in
 * L2 and the Infinity Cache for the next kernels that read them, in
 * `workgroups` workgroups (1..65536) of 256 threads, each over one slice
 * of every range, and stores the XOR of the words it read to sink[w] (uint32
 * [workgroups], device memory): the XOR of all of sink is the XOR of every
 * word of the ranges.  Enqueued on `stream` (typically a second stream,
 * default priority, ordered against the block's stream by the caller's
 * events).  MOE_EINVAL on a bad argument. */
moe_status_t moe_prefetch(int n, const void* const* ptrs, const size_t* bytes, uint32_t* sink, int workgroups,
                          void* stream);

/* Zero-fill a workspace (with a kernel, so it may be captured in a graph). */
moe_status_t moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Dense skinny product Y[b][n] = sum_c X[b][c] * W[n][c]   (WRITEUP part 1
 * §1, the attention input projection at decode batch: small-matrix kernel at
 * batch 1-2, split-K at larger batch; here the rows shape takes the split-K
 * role for bf16: 12 weight rows per workgroup over all of K, no partial sums
 * outside the workgroup).
 *   X [B][K] dtype, W [N][K] dtype, Y [B][N] of y_dtype (dtype or
 *   MOE_DT_F32).  1 <= B <= 64; K a multiple of 8 (bf16) or 4 (fp32), and of
 *   32 for the mfma shape (bf16 only).  Output rounded to nearest-even when
 *   y_dtype is bf16.  Workspace: moe_workspace_bytes(MOE_OP_SKINNY_GEMM,
 *   ...) bytes, zero-filled once (0 for fp32; for bf16 the mfma shape keeps
 *   fp32 partial sums of its K slices there); ws may be NULL when 0. */
moe_status_t skinny_gemm(int dtype, int B, int N, int K, const void* X, const void* W, void* Y,
                         int y_dtype, void* ws, size_t ws_bytes, void* stream);

/* Attention output projection with the residual added (WRITEUP part 1 §2:
 * the output projection fused with its all-reduce and the following
 * residual; on one GPU the all-reduce is absent):
 *   Y[b][n] = sum_c X[b][c] * W[n][c] + R[b][n], accumulated in fp32, the
 *   residual added once after the sum, then rounded to y_dtype.
 *   R [B][N] of dtype, caller-owned device memory, 16-byte aligned; Y may be
 *   R itself (an in-place residual update: each element is read and
 *   written by the same thread) but must not otherwise overlap it.  Every
 *   other argument, the kernel shapes, the workspace and the errors are
 *   those of skinny_gemm; a null R is MOE_EINVAL. */
moe_status_t skinny_gemm_residual(int dtype, int B, int N, int K, const void* X, const void* W, const void* R,
                                  void* Y, int y_dtype, void* ws, size_t ws_bytes, void* stream);

/* Router (WRITEUP part 1 §3; selection and weights are the standard top-k
 * softmax the block's workload definitions name):
 *   logits[t][e] = sum_c X[t][c] * Wr[e][c] + bias(t, e), accumulated in fp32;
 *   the k experts with the largest fp32 logits (on an exact tie the lower
 *   expert index wins), in ascending expert id, with weights
 *   w_j = exp(l_j - max) / sum_{i in top-k} exp(l_i - max)
 *   (= softmax over all E renormalised over the top-k; no extra scale);
 *   and the routing plan (moe_plan_words layout).
 *   X [B][d], Wr [E][d]; bias: NULL, [E] (bias_ld = 0, added to every token)
 *   or [B][E] (bias_ld = E), fp32.  Outputs: topk_ids int32 [B][k],
 *   topk_w fp32 [B][k], plan int32 [moe_plan_words(B, k, E)], and, when
 *   logits_out is not NULL, the fp32 logits [B][E].
 *   Scope: 1 <= B <= 64, 1 <= k <= min(E, 16), E <= 512, d a multiple of 32
 *   (bf16) or 4 (fp32, B <= 8).  Inputs must be finite. */
moe_status_t moe_route(int dtype, int B, int d, int E, int k, const void* X, const void* Wr,
                       const float* bias, int bias_ld, int32_t* topk_ids, float* topk_w,
                       int32_t* plan, float* logits_out, void* ws, size_t ws_bytes, void* stream);

/* Router with the latent input projection in the same product (WRITEUP
 * part 1 §3: the router scores and the latent input projection both take
 * the token's hidden state and are computed as one matrix product, so x is
 * read once and both weight matrices stream in one launch):
 *   everything moe_route computes and returns, and
 *   latent_out[t][j] = sum_c X[t][c] * Wl[j][c]   (no bias), accumulated in
 *   fp32, stored as latent_dtype (dtype or MOE_DT_F32; bf16: round to
 *   nearest-even).
 *   Wl [L][d] of dtype; latent_out [B][L].  The product runs over the E + L
 *   rows [Wr; Wl] with moe_route's kernel shapes; selection, weights and
 *   plan use the E router rows only.  Scope: that of moe_route, plus L a
 *   multiple of 16 up to 8192 and E a multiple of 4.  Workspace:
 *   moe_workspace_bytes(MOE_OP_ROUTE_LATENT, dtype, B, d, E, k, 0, 0, L, 0). */
moe_status_t moe_route_latent(int dtype, int B, int d, int E, int k, int L, const void* X, const void* Wr,
                              const void* Wl, const float* bias, int bias_ld, int32_t* topk_ids, float* topk_w,
                              int32_t* plan, void* latent_out, int latent_dtype, float* logits_out, void* ws,
                              size_t ws_bytes, void* stream);

/* Routed and shared experts (WRITEUP part 1 §3; SwiGLU expert FFN):
 *   for every slot s = t*k + j of the plan, with e its expert:
 *     h = silu(X[t] . W13[e][0:I]^T) * (X[t] . W13[e][I:2I]^T),
 *     silu(z) = z / (1 + exp(-z)),  h kept in fp32,
 *     Yslot[t][j] = h . W2[e]^T                          (fp32 [d])
 *   and, when Ws13 is not NULL, the shared expert for every token t:
 *     Yslot[t][k] = the same FFN with Ws13 / Ws2 (Is).   Without a shared
 *   expert Yslot[t][k] is left untouched.
 *   Each selected expert's weights are read once however many tokens chose
 *   it; unselected experts are never read.  plan comes from moe_route (it
 *   must be complete before this call runs: same stream or synchronised).
 *   Yslot fp32 [B][k+1][d].  Scope as moe_route, plus I (and Is) multiples
 *   of 32 up to 256 (bf16; fp32: multiples of 4 up to 256, B <= 8). */
moe_status_t moe_expert_ffn(int dtype, int B, int d, int E, int k, int I, const void* X,
                            const int32_t* plan, const void* W13, const void* W2, int Is,
                            const void* Ws13, const void* Ws2, float* Yslot, void* ws,
                            size_t ws_bytes, void* stream);

/* Weighted combine (WRITEUP part 1 §3: each token's output is the sum of its
 * routed experts' outputs and the shared expert's, which runs for every
 * token; the routed outputs are weighted by the gate weights of moe_route, as
 * the block's workload definitions state -- softmax over the router logits,
 * renormalised over the top-k, no extra scale):
 *   out[t] = sum_{j ascending} topk_w[t][j] * Yslot[t][j] + (has_shared ?
 *   Yslot[t][k] : 0), accumulated in fp32 in that order, stored as dtype
 *   (bf16: round to nearest-even).  Yslot fp32 [B][k+1][d], topk_w fp32
 *   [B][k], out [B][d].  No workspace. */
moe_status_t moe_combine(int dtype, int B, int d, int k, const float* Yslot, const float* topk_w,
                         int has_shared, void* out, void* stream);

/* The whole block, every intermediate in ws (WRITEUP part 1 §3: router
 * scores, then the routed experts, and a shared expert for every token, its
 * output added to the routed ones; AREX "每层从 23 个内核减到 13 个": the
 * block's stages in fewer kernels; the arithmetic is that of moe_route,
 * moe_expert_ffn and moe_combine above).
 * Small batch on the vector shape with short expert rows (B*k <= 64, I and
 * Is at most 16 vector chunks -- 128 bf16, 64 fp32), on request ONE launch
 * (schedule "fused"): one 16-wave workgroup per compute unit, all resident,
 * runs router scoring (and the shared expert's gate/up), waits at a
 * grid-wide barrier, selects the top-k and builds the plan in every
 * workgroup, runs the routed gate/up, waits at a second barrier, then the
 * down projection with the weighted combine.  The barrier words live in ws
 * (count words return to zero after every call).  Used only when the
 * device reports room for one workgroup per compute unit.
 * By default at B <= 2 (B*k <= 64, vector shape, the shared expert's
 * gate/up not placed in the router launch), TWO launches (schedule
 * "router_in_up"): the gate/up launch's first workgroups score the router
 * rows, with the router launch's split of K, and store each logit's order
 * key in ws (16 copies); the others run the shared expert's tiles, poll the
 * keys (bounded; a wait that gives up sets the status word), select every
 * token's top-k and build the plan, then run the routed gate/up; the down +
 * combine launch (3. below) zeroes the keys again.
 * Otherwise, and outside that scope, three launches (schedule
 * "launches"); with B*k <= 64:
 *   1. router scoring only (logits + bias to ws; from B = 2 it also
 *      clears the words step 2 publishes ids in);
 *   2. gate/up + SwiGLU: at B = 1 every workgroup selects the token's top-k
 *      and builds the plan itself; from B = 2 workgroup t selects token t
 *      once, stores its topk_ids / topk_w and publishes its ids in ws, and
 *      every workgroup waits for all tokens' ids (bounded polling; a wait
 *      that gives up sets the status word) and builds the plan; the shared
 *      expert's tiles, which need no routing, go first; one workgroup stores
 *      the plan;
 *   3. down projection of every expert fused with the weighted combine: the
 *      per-slot outputs never leave the chip.
 * Otherwise, on the vector-ALU shape: 1. router scoring + top-k + plan
 * (the last workgroup to finish selects), with the shared expert's gate/up
 * in the same launch; 2. routed gate/up + SwiGLU; 3. as above.  On the
 * matrix-core shape (bf16, B > 8): 1. router products over K slices; 2. a
 * finish launch that adds the slices and the bias and stores topk_ids and
 * topk_w; 3. gate/up + SwiGLU, every workgroup building the plan from the
 * ids, the shared expert one more entry, the heaviest token tiles cut in two
 * K halves; 4. down + combine, reading h from a tiled copy in ws (in the
 * down's K order: see the tiled copy's layout).
 * Same scope and results as moe_route, moe_expert_ffn and moe_combine in
 * sequence (bit for bit with the vector-ALU shapes; with the matrix-core
 * shape the gate/up's K splits and the down's K order differ, within fp32
 * rounding).  topk_ids /
 * topk_w are optional outputs (NULL: kept in ws). */
moe_status_t moe_block(int dtype, int B, int d, int E, int k, int I, int Is, const void* X,
                       const void* Wr, const float* bias, int bias_ld, const void* W13,
                       const void* W2, const void* Ws13, const void* Ws2, void* out,
                       int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                       void* stream);

/* moe_block with the shared expert on a second stream (WRITEUP part 1 §3:
 * the shared expert runs on its own stream, overlapping routing and the
 * routed experts).  Same arguments, scope checks, workspace and results (bit
 * for bit) as moe_block, plus side_stream (a hipStream_t other than stream,
 * default priority) and two caller-owned hipEvent_t: fork_event is recorded
 * on stream and waited for by side_stream, which then runs the shared
 * expert's gate/up and down; join_event is recorded on side_stream and
 * waited for by stream before the down + combine launch, which adds the
 * shared expert's output.  The router and routed gate/up launches on stream
 * overlap the side stream's work.  Applies to the small-batch three-launch
 * schedule (B*k <= 64, vector shape) with a shared expert; MOE_EUNSUPPORTED
 * otherwise.  Both streams' work must be complete before ws is reused. */
moe_status_t moe_block_streams(int dtype, int B, int d, int E, int k, int I, int Is, const void* X,
                               const void* Wr, const float* bias, int bias_ld, const void* W13,
                               const void* W2, const void* Ws13, const void* Ws2, void* out,
                               int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream,
                               void* side_stream, void* fork_event, void* join_event);

/* moe_block without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus ws, ws_bytes),
 * scope, kernels and results as moe_block, bit for bit.  The workspace is a
 * library-owned device array of MOE_NOALLOC_SCRATCH_BYTES per GPU (held
 * until the process ends); sizes whose moe_workspace_bytes(MOE_OP_BLOCK, ...)
 * exceed it return MOE_EUNSUPPORTED (every B, E, k, I, Is moe_block accepts
 * fits up to d = 16384).
 * The call allocates nothing; before the block it clears the scratch's
 * counter words with a small kernel on `stream`.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status_t moe_block_noalloc(int dtype, int B, int d, int E, int k, int I, int Is, const void* X,
                               const void* Wr, const float* bias, int bias_ld, const void* W13,
                               const void* W2, const void* Ws13, const void* Ws2, void* out,
                               int32_t* topk_ids, float* topk_w, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SKINNY_H */
