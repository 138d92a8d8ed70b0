// expert_core.hpp -- device code of one expert task: gate/up + SwiGLU over a
// tile of (gate row i, up row I+i) pairs, and the down projection of a tile
// of 16 output rows.  Used by the expert kernels and, for the shared expert,
// by the router kernel of the fused block.
//
// Expert e computes h = silu(x . Wg^T) * (x . Wu^T), y = h . W2^T, with
// silu(z) = z / (1 + exp(-z)); W13[e] is [2I][d] (gate rows, then up rows),
// W2[e] is [d][I] (see expert.hip for the page citations).
//
// Shape by the expert's token count m:
//   m <= 8 : vector ALU.  Gate/up: one wave per pair over the whole of d, so
//            SwiGLU happens in registers.  Down: L lanes per W2 row (L*VEC >=
//            I), 64/L rows per load instruction.
//   m > 8  : MFMA 16x16x32 bf16.  Gate/up: 64 weight rows (32 gate/up
//            pairs) per task over all of d, the entry's token rows gathered
//            into LDS and shared by the four waves (mfma_core.hpp).
//            Down: 16 W2 rows per wave over all of I; h (fp32) enters as a
//            bf16 hi/lo pair so it keeps ~16 mantissa bits.
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "mfma_core.hpp"
#include "route_core.hpp"
#include "skinny_core.hpp"

namespace moe {

constexpr int kMaxPlanWords = 2 + 2 * 512 + 64 * 16;
constexpr int kDownTokGroup = 4; // tokens whose h the vector down requests together
constexpr int kUpPairsMfma = 32;  // gate/up pairs per MFMA up task (64 weight rows)
constexpr int kUpMfmaChunks = 2;  // chunks in flight per wave (two workgroups per CU)

// Routing plan staged in LDS (see moe_plan_words for the layout).
struct PlanView {
  int n, maxa;
  const int32_t* active;
  const int32_t* offs;
  const int32_t* slots;
};

// View of a plan held in LDS.
__device__ __forceinline__ PlanView plan_view(const ExpertLaunch& a, const int32_t* s_plan) {
  const int nslot = a.B * a.k;
  const int maxa = nslot < a.E ? nslot : a.E;
  PlanView p;
  p.maxa = maxa;
  p.n = s_plan[0];
  p.active = s_plan + 1;
  p.offs = s_plan + 1 + maxa;
  p.slots = s_plan + 2 + 2 * maxa;
  return p;
}

// Copy n words from global memory to LDS with the whole workgroup: the
// first 8 per thread are all requested before any is stored, so they cost
// one memory round trip (a plain loop waits for each load before the next,
// one round trip per word per thread).
__device__ __forceinline__ void stage_words(int32_t* dst, const int32_t* src, int n) {
  constexpr int R = 8;
  const int nt = (int)blockDim.x;
  int32_t r[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int i = threadIdx.x + q * nt;
    r[q] = i < n ? src[i] : 0;   // lanes past n request nothing
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int i = threadIdx.x + q * nt;
    if (i < n) dst[i] = r[q];
  }
  for (int i = threadIdx.x + R * nt; i < n; i += nt) dst[i] = src[i];
}

// Copy the plan into LDS with the whole workgroup (one coalesced pass) and
// return a view of it.  Ends with a barrier.
__device__ __forceinline__ PlanView stage_plan(const ExpertLaunch& a, int32_t* s_plan) {
  const int nslot = a.B * a.k;
  const int maxa = nslot < a.E ? nslot : a.E;
  const int words = 2 + 2 * maxa + nslot;
  stage_words(s_plan, a.plan, words);
  __syncthreads();
  return plan_view(a, s_plan);
}

// The plan built in this workgroup's LDS from the ids [B][k] stored by the
// router's finish launch (an earlier launch); the last workgroup of the grid
// also stores it (plan_out) for the down launch.  scratch: LDS free until
// the call returns, at least kPlanFromIdsBytes.  Ends with a barrier.
constexpr int kPlanFromIdsBytes = kMaxB * kMaxK * 4 + (int)sizeof(PlanScratch);
__device__ __forceinline__ PlanView plan_from_ids(const ExpertLaunch& a, int32_t* s_plan, unsigned char* scratch) {
  const int nslot = a.B * a.k;
  int32_t* s_ids = reinterpret_cast<int32_t*>(scratch);
  PlanScratch& ps = *reinterpret_cast<PlanScratch*>(scratch + kMaxB * kMaxK * 4);
  stage_words(s_ids, a.ids_in, nslot);
  __syncthreads();
  const bool writer = blockIdx.x == gridDim.x - 1;
  plan_block(s_ids, nslot, a.k, a.E, s_plan, writer ? a.plan_out : nullptr, ps);
  __syncthreads();
  return plan_view(a, s_plan);
}

// ---- router rows inside the gate/up launch (B <= 2) ------------------------

// The router launch's workgroups have 16 waves; its logits' bits depend on
// that split of K alone (not on rows or tokens per workgroup), so the gate/up
// launch's 4-wave router workgroups play 16 waves.
constexpr int kRouterPlayedWaves = 16;

// Router workgroup r of the gate/up launch: rows r * kRouterRowsInUp .. of
// x . Wr^T (+ bias), each logit's order key (ord_key; a NaN's kept nonzero)
// stored device-coherent to every copy of lkeys for the gate/up workgroups
// (hundreds of workgroups polling one copy queue at the lines' memory
// channel, and the stores behind them: one copy cost ~1 us at batch 1).
// s_rr: kRouterPlayedWaves * kRouterRowsInUp * 2 floats.
template <typename T, int NR>
__device__ __forceinline__ void router_rows_in_up(const ExpertLaunch& a, int r, float* s_rr) {
  const RowsSrc src = {a.X, a.Wr, a.B, a.E, a.d};
  auto fin = [&](int t, int n, float v) {
    if (a.rbias) v += a.rbias[(size_t)t * a.rbias_ld + n];
    uint32_t key = ord_key(v);
    if (key == 0u) key = ord_key(__builtin_nanf(""));
#pragma unroll
    for (int c = 0; c < kKeyCopies; ++c)
      __hip_atomic_store(a.lkeys + c * kKeyStride + t * a.E + n, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const int n0 = r * kRouterRowsInUp;
  if (a.B <= 1) valu_rows_as<T, kRouterRowsInUp, 1, 1, kRouterPlayedWaves, NR>(src, n0, s_rr, fin);
  else valu_rows_as<T, kRouterRowsInUp, 2, 1, kRouterPlayedWaves, NR>(src, n0, s_rr, fin);
}

// Token t's logits as topk_wave takes them, from the keys the router
// workgroups of this launch store: the wave polls its experts' keys in the
// workgroup's copy until none is zero.  After spin_limit polls it gives up,
// sets *status and takes the keys as they are.
__device__ __forceinline__ void wait_logit_keys(const ExpertLaunch& a, int t, float (&lv)[kNI]) {
  const int lane = threadIdx.x & 63;
  const uint32_t* kp = a.lkeys + (blockIdx.x % kKeyCopies) * kKeyStride + t * a.E;
  uint32_t key[kNI];
  for (int n = 0;; ++n) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int e = lane + 64 * i;
      key[i] = e < a.E ? __hip_atomic_load(kp + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1u;
      all = all && key[i] != 0u;
    }
    if (__ballot(!all) == 0ull) break;
    if (n >= a.spin_limit) {
      if (lane == 0) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < kNI; ++i) lv[i] = key_value(key[i]);
}

// Routing inside the gate/up launch (B*k <= 64): the workgroup selects the
// top-k of all B tokens from the router's logits [B][E] (bias included), or
// from their keys when the router rows run in this launch, and builds the
// plan in LDS -- the same functions, hence the same bits, as the
// router's finishing workgroup.  s_tk: one TopkScratch per selecting wave
// (at most kTopkWaves).  The last workgroup of the grid also stores
// ids, weights and plan for the down launch and the caller.  Ends with a
// barrier.  SAME_LAUNCH: the logits were stored in this launch (fused block).
// QB: tokens a wave requests logits for before selecting (one memory round
// trip per QB tokens); the gate/up launch selects here only at batch 1 and
// takes QB = 1, which also keeps one copy of the selection code.
template <bool SAME_LAUNCH, int QB = 2>
__device__ __forceinline__ PlanView route_here(const ExpertLaunch& a, int32_t* s_plan, TopkScratch* s_tk,
                                               int32_t* s_ids, float* s_w) {
  const int nw = (blockDim.x >> 6) < kTopkWaves ? (blockDim.x >> 6) : kTopkWaves;
  const int wave = threadIdx.x >> 6;
  const bool writer = blockIdx.x == gridDim.x - 1;
  const int B = a.B, E = a.E, k = a.k;
  for (int t0 = wave; wave < nw && t0 < B; t0 += nw * QB) {
    float lv[QB][kNI];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int t = t0 + nw * q;
      if (a.lkeys) wait_logit_keys(a, t < B ? t : B - 1, lv[q]);
      else load_logit_row<SAME_LAUNCH>(a.logits, t < B ? t : B - 1, E, lv[q]);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int t = t0 + nw * q;
      if (t < B)
        topk_wave(lv[q], E, k, s_tk[wave], s_ids + t * k, s_w + t * k, writer ? a.ids_out + (size_t)t * k : nullptr,
                  writer ? a.w_out + (size_t)t * k : nullptr);
    }
  }
  __syncthreads();
  if (wave == 0) {
    if (B == 1) plan_one_token(s_ids, k, s_plan, writer ? a.plan_out : nullptr);
    else plan_wave(s_ids, B * k, E, reinterpret_cast<int*>(s_tk), s_plan, writer ? a.plan_out : nullptr);
  }
  __syncthreads();
  return plan_view(a, s_plan);
}

// Routing inside the gate/up launch with one selection per token (B >= 2,
// B*k <= 64): workgroup t < B selects token t's top-k with one wave (the
// same function as route_here, hence the same bits), stores its ids and
// weights for the down launch and the caller, and id + 1 of each slot to
// a.ready with device-coherent stores (the router launch zeroed the words).
// Selecting all B tokens in every workgroup made the routing ALU-bound at
// batch 8 (1024 workgroups x 8 selections: 8-17 us before the first routed
// weight request).
__device__ __forceinline__ void select_own_token(const ExpertLaunch& a, TopkScratch* s_tk, int32_t* s_ids,
                                                 float* s_w) {
  const int t = blockIdx.x, lane = threadIdx.x & 63;
  if (t >= a.B || (threadIdx.x >> 6) != 0) return;
  float lv[kNI];
  load_logit_row<false>(a.logits, t, a.E, lv);
  topk_wave(lv, a.E, a.k, s_tk[0], s_ids, s_w, nullptr, nullptr);
  wave_lds_sync();
  if (lane < a.k) {
    const int s = t * a.k + lane, e = s_ids[lane];
    a.ids_out[s] = e;
    a.w_out[s] = s_w[lane];
    __hip_atomic_store(a.ready + s, e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Every workgroup: wave 0 polls the B*k ready words (one device-coherent
// load per lane) until none is zero, takes the ids from them (each word
// carries its own id, so nothing else needs ordering) and builds the plan
// in LDS -- the last workgroup also stores it for the down launch.  A
// workgroup waits only for workgroups of lower index, which were dispatched
// before it.  After spin_limit polls it gives up, sets *status and plans
// with the ids it has (clamped into range).  Ends with a barrier.
__device__ __forceinline__ PlanView wait_token_plan(const ExpertLaunch& a, int32_t* s_plan, TopkScratch* s_tk,
                                                    int32_t* s_ids) {
  const int lane = threadIdx.x & 63;
  const int ns = a.B * a.k;
  if ((threadIdx.x >> 6) == 0) {
    int v = 1;
    for (int n = 0;; ++n) {
      v = lane < ns ? ld_coherent_i32(a.ready + lane) : 1;
      if (__ballot(v == 0) == 0ull) break;
      if (n >= a.spin_limit) {
        if (lane == 0) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const int e = v - 1;
    if (lane < ns) s_ids[lane] = (e >= 0 && e < a.E) ? e : 0;
    wave_lds_sync();
    plan_wave(s_ids, ns, a.E, reinterpret_cast<int*>(s_tk), s_plan,
              blockIdx.x == gridDim.x - 1 ? a.plan_out : nullptr);
  }
  __syncthreads();
  return plan_view(a, s_plan);
}

// Entry e_idx of the plan: a routed expert (e_idx < n) or the shared one.
struct ExpertView {
  int m;              // tokens
  int I;              // intermediate size
  const void* W13;    // [2I][d]
  const void* W2;     // [d][I]
  int slot0;          // first plan slot (routed) or -1 (shared)
  int hbase;          // first row of its tiles in the tiled copy of h
};

// Tiled copy of h: the shared expert's tiles from row 0, routed entry e's
// from row roundup(B, 16) + offs[e] + 16 e.  Entry e needs 16 ceil(m_e/16)
// <= m_e + 15 rows, so the ranges do not overlap, and all entries fit in
// roundup(B, 16) + B k + 16 min(E, B k) rows.
__host__ __device__ __forceinline__ int ht_rows(int B, int k, int E) {
  return ((B + 15) & ~15) + B * k + 16 * (E < B * k ? E : B * k);
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
    v.hbase = ((a.B + 15) & ~15) + p.offs[e_idx] + 16 * e_idx;
  } else {
    v.m = a.B;
    v.I = a.Is;
    v.W13 = a.Ws13;
    v.W2 = a.Ws2;
    v.slot0 = -1;
    v.hbase = 0;
  }
  return v;
}

// The shared expert alone (no plan needed).
__device__ __forceinline__ ExpertView shared_view(const ExpertLaunch& a) {
  ExpertView v;
  v.m = a.B;
  v.I = a.Is;
  v.W13 = a.Ws13;
  v.W2 = a.Ws2;
  v.slot0 = -1;
  v.hbase = 0;
  return v;
}

// Token index and slot row (row of h / of the per-slot outputs) of the i-th
// token of an entry: routed slot s = t*k + j sits at row s, shared token t
// at row B*k + t.
__device__ __forceinline__ void token_of(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v,
                                         int i, int& tok, int& srow) {
  if (v.slot0 >= 0) {
    const int s = slots[v.slot0 + i];
    tok = s / a.k;
    srow = s;
  } else {
    tok = i;
    srow = a.B * a.k + i;
  }
}

// The SwiGLU output h of the slot rows (B*k routed slots, then B shared
// tokens; row stride hld).  For fp32 weights h is fp32 [rows][hld].  For
// bf16 weights every value v is kept as the pair hi = bf16(v), lo =
// bf16(v - hi) (about 16 significant bits, the bf16 operand pair the down
// products consume), in two planes of [rows][hld] bf16: hi at a.h, lo right
// after it -- the same bytes as fp32, split once by the producer instead of
// by every down workgroup.  Stored device-coherent (the fused block reads h
// across workgroups of one launch).
__device__ __forceinline__ int h_rows(const ExpertLaunch& a) { return a.B * a.k + a.B; }
__device__ __forceinline__ uint16_t* h_hi(const ExpertLaunch& a) { return reinterpret_cast<uint16_t*>(a.h); }
__device__ __forceinline__ uint16_t* h_lo(const ExpertLaunch& a) {
  return reinterpret_cast<uint16_t*>(a.h) + (size_t)h_rows(a) * a.hld;
}

// K order of the matrix-shape down (the same for its W2 operands and the
// tiled copy of h, so the products are unchanged): column i of a pair of K
// steps (i < I rounded down to 64) sits in step 2 (i / 64) + (i / 8) % 2,
// lane group (i / 16) % 4 -- so that one load of 8 W2 rows x 128 bytes (full
// lines) and a DPP row shift give every lane its operand (load_w2_operands);
// an odd last step keeps the plain order: step i / 32, group (i / 8) % 4.
__device__ __forceinline__ void down_k_slot(int i, int I, int& j, int& kq) {
  if (i < (I & ~63)) {
    j = ((i >> 6) << 1) | ((i >> 3) & 1);
    kq = (i >> 4) & 3;
  } else {
    j = i >> 5;
    kq = (i >> 3) & 3;
  }
}

// Element (token t of entry v, column i) of the tiled copy: within a tile,
// K step j, lane kq * 16 + row (down_k_slot; row = t % 16) holds the 8
// values the matrix operand takes from that lane.  hld is a multiple of 32
// for bf16 weights.
__device__ __forceinline__ size_t ht_index(const ExpertLaunch& a, const ExpertView& v, int t, int i) {
  int j, kq;
  down_k_slot(i, v.I, j, kq);
  return (size_t)(v.hbase + (t & ~15)) * a.hld + (size_t)(((j * 64 + kq * 16 + (t & 15)) << 3) + (i & 7));
}

// MFMA A operands of W2 rows r0 .. r0+15 (rows from r_end on re-read row
// r_end - 1 and are not stored) for the J = I / 32 K steps, in the order of
// down_k_slot.  Per pair of steps one instruction loads rows 0-7 (lane l: row
// l % 8, columns 8 (l / 8) .. +7 of the pair's 64) and one rows 8-15, each 8
// full 128-byte lines; lane l = R + 16 g then holds row R's columns 16 g ..
// +7 (R < 8: first step) or 16 g + 8 .. +7 (R >= 8: second step), and takes
// the other step's from lane l +- 8 (a DPP row shift), as the gate/up's
// operands do.  (16 rows x 64 bytes per instruction -- half lines -- streamed
// at ~5.5 TB/s where full lines reach ~6.9.)  An odd last step is loaded as
// 16 rows x 64 bytes in the plain order.
constexpr int kDownJM = kMaxInter / 32;
__device__ __forceinline__ void load_w2_operands(const bf16_t* W2, int I, int r0, int r_end, int J,
                                                 u32x4 (&wv)[kDownJM]) {
  const int lane = threadIdx.x & 63;
  const int P = J >> 1;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 va[kDownJM / 2], vb[kDownJM / 2];
  if (P > 0) {
    const int rl = r0 + (lane & 7), rh = r0 + 8 + (lane & 7);
    const bf16_t* pl = W2 + (size_t)(rl < r_end ? rl : r_end - 1) * I + (lane >> 3) * 8;
    const bf16_t* ph = W2 + (size_t)(rh < r_end ? rh : r_end - 1) * I + (lane >> 3) * 8;
#pragma unroll
    for (int p = 0; p < kDownJM / 2; ++p) {
      const int pc = p < P ? p : P - 1;
      va[p] = ld128_stream(pl + (size_t)pc * 64);
      vb[p] = ld128_stream(ph + (size_t)pc * 64);
    }
  } else {
#pragma unroll
    for (int p = 0; p < kDownJM / 2; ++p) va[p] = vb[p] = zero;
  }
  u32x4 vt = zero;
  if (J & 1) {
    const int r = r0 + (lane & 15);
    vt = ld128_stream(W2 + (size_t)(r < r_end ? r : r_end - 1) * I + (size_t)(J - 1) * 32 + (lane >> 4) * 8);
  }
  const bool low = (lane & 15) < 8;
#pragma unroll
  for (int p = 0; p < kDownJM / 2; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b_up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)vb[p][e], 0x118, 0xf, 0xf, false);  // row_shr:8
      const uint32_t a_dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)va[p][e], 0x108, 0xf, 0xf, false);  // row_shl:8
      wv[2 * p][e] = low ? va[p][e] : b_up;
      wv[2 * p + 1][e] = low ? a_dn : vb[p][e];
    }
  if (J & 1) {
#pragma unroll
    for (int j = 0; j < kDownJM; ++j)
      if (j == J - 1) wv[j] = vt;
  }
}

// h of token t (slot row sr) of entry v, column i: to the slot rows, or,
// when the launch has the tiled copy (its down reads h only from there,
// every entry on the matrix shape), to the tiled copy alone.
template <typename T>
__device__ __forceinline__ void h_store(const ExpertLaunch& a, const ExpertView& ev, int t, int sr, int i, float v) {
  const size_t o = (size_t)sr * a.hld + i;
  if constexpr (sizeof(T) == 2) {
    const bf16_t hi = f32_to_bf16(v);
    const bf16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
    if (a.ht_hi) {
      const size_t q = ht_index(a, ev, t, i);
      st_coherent16b(a.ht_hi + q, hi);
      st_coherent16b(a.ht_lo + q, lo);
      return;
    }
    st_coherent16b(h_hi(a) + o, hi);
    st_coherent16b(h_lo(a) + o, lo);
  } else {
    st_coherent(a.h + o, v);
  }
}

// Values i .. i+3 (i a multiple of 4) of token t (slot row sr) of entry ev.
template <typename T>
__device__ __forceinline__ void h_store4(const ExpertLaunch& a, const ExpertView& ev, int t, int sr, int i, f32x4 v) {
  const size_t o = (size_t)sr * a.hld + i;
  if constexpr (sizeof(T) == 2) {
    uint32_t h0, l0, h1, l1;
    split_bf16x2(v[0], v[1], h0, l0);
    split_bf16x2(v[2], v[3], h1, l1);
    if (a.ht_hi) {
      const uint32_t q = (uint32_t)(ht_index(a, ev, t, i) * 2);
      st_coherent8(coherent_rsrc(a.ht_hi), q, u32x2{h0, h1});
      st_coherent8(coherent_rsrc(a.ht_lo), q, u32x2{l0, l1});
      return;
    }
    const coherent_rsrc_t r = coherent_rsrc(a.h);
    st_coherent8(r, (uint32_t)(o * 2), u32x2{h0, h1});
    st_coherent8(r, (uint32_t)(((size_t)h_rows(a) * a.hld + o) * 2), u32x2{l0, l1});
  } else {
    st_coherent4(coherent_rsrc(a.h), (uint32_t)(o * 4), __builtin_bit_cast(u32x4, v));
  }
}

// Kernel shape per entry.  PATHS is fixed per kernel instantiation: 1 = the
// vector shape only (fp32, B <= 8 or forced), 2 = MFMA only (forced), 3 =
// either, by token count (m > 8: MFMA).  Keeping unused shapes out of an
// instantiation keeps its register count, hence its occupancy, down.
constexpr int kPathValu = 1, kPathMfma = 2, kPathBoth = 3;

template <int PATHS>
__device__ __forceinline__ bool use_mfma(int m) {
  if constexpr (PATHS == kPathValu) return false;
  else if constexpr (PATHS == kPathMfma) return true;
  else return m > 8;
}

// Host and device agree on the path set of a launch.
__host__ __device__ __forceinline__ int expert_paths(int bf16, int force, int B) {
  if (!bf16) return kPathValu;
  if (force == VAR_MFMA) return kPathMfma;
  if (force == VAR_GEMV || B <= 8) return kPathValu;
  return kPathBoth;
}

// ---- gate/up + SwiGLU ------------------------------------------------------

// Pair i (gate row i, up row I+i) of entry v: this wave takes the `half`-th
// of NH slices of d; h[srow][i] = silu(g) * u for the entry's tokens.  With
// NH = 2 the two waves of a pair meet in s_part ([pair slots][2][8] floats,
// pair slot ps; the stride is fixed so that pairs of entries with different
// token counts can share a workgroup) and the whole workgroup passes one
// barrier; with NH = 1 a wave works alone.  Waves whose pair is past I still
// reach the barrier.
constexpr int kPartStride = 8;
// U1: chunks per lane in flight at one token (7, all of a 7168-wide half row
// at once, measured slower at batch 1 than 4).  The number in flight does not
// change any lane's order of accumulation.
template <typename T, int MB, int NH, int U1>
__device__ __forceinline__ void up_valu(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v, int i,
                                        int half, int ps, float* s_part) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int U = MB <= 1 ? U1 : (MB <= 2 ? 4 : (MB <= 4 ? 2 : 1));
  const int lane = threadIdx.x & 63;
  const bool live = i < v.I;
  const T* W13 = reinterpret_cast<const T*>(v.W13);
  const T* X = reinterpret_cast<const T*>(a.X);
  const int ic = live ? i : 0;
  const T* wr[2] = {W13 + (size_t)ic * a.d, W13 + (size_t)(v.I + ic) * a.d};
  const T* xr[MB];
  int srow[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) {
    int tok = 0, sr = 0;
    if (t < v.m) token_of(a, slots, v, t, tok, sr);
    xr[t] = X + (size_t)tok * a.d;
    srow[t] = sr;
  }
  const int C = a.d / VEC;
  float acc[2][MB];
  if (live) {
    valu_dot<T, 2, MB, U>(wr, xr, v.m, half * C / NH, (half + 1) * C / NH, acc);
  } else {
#pragma unroll
    for (int t = 0; t < MB; ++t) acc[0][t] = acc[1][t] = 0.f;
  }
  if constexpr (NH == 2) {
    if (half == 1 && lane == 0) {
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        s_part[(ps * 2 + 0) * kPartStride + t] = acc[0][t];
        s_part[(ps * 2 + 1) * kPartStride + t] = acc[1][t];
      }
    }
    __syncthreads();
    if (half == 1 || !live) return;
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      acc[0][t] += s_part[(ps * 2 + 0) * kPartStride + t];
      acc[1][t] += s_part[(ps * 2 + 1) * kPartStride + t];
    }
  }
  if (live && lane < v.m) {
    const float g = pick_lane<MB>(acc[0], lane), u = pick_lane<MB>(acc[1], lane);
    int sr = 0;
#pragma unroll
    for (int t = 0; t < MB; ++t)
      if (t == lane) sr = srow[t];
    h_store<T>(a, v, lane, sr, i, silu(g) * u);
  }
}

template <typename T, int NH, int U1 = 8 / NH>
__device__ __forceinline__ void up_valu_dispatch(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v,
                                                 int i, int half, int ps, float* s_part) {
  if (v.m <= 1) up_valu<T, 1, NH, U1>(a, slots, v, i, half, ps, s_part);
  else if (v.m <= 2) up_valu<T, 2, NH, U1>(a, slots, v, i, half, ps, s_part);
  else if (v.m <= 4) up_valu<T, 4, NH, U1>(a, slots, v, i, half, ps, s_part);
  else up_valu<T, 8, NH, U1>(a, slots, v, i, half, ps, s_part);
}

// Pairs p0 .. p0+31 of entry v (m > 8 tokens) over all of d with the four
// waves of the workgroup (mfma_rows): wave w's A rows 0-7 are the gate rows
// of pairs p0+8w .. p0+8w+7, rows 8-15 the up rows of the same pairs, so
// after the product lane l < 32 holds gate sums of pairs p0 + 8w + 4(l/16)
// + q (q = 0..3) for token nt*16 + l%16 and lane l + 32 the matching up
// sums; SwiGLU pairs them across the two lane halves.  The entry's token
// rows are gathered into LDS (s_x).
// K range of an MFMA gate/up task: all of d, or one of `split` slices of it
// whose fp32 sums go to `part` (this tile's block: split x 4 waves x NT x 64
// lanes of f32x4); the tile's last slice to arrive on `counter` adds the
// slices in slice order and applies SwiGLU.
struct UpSlice {
  int s0, s1, slice, split;
  float* part;
  uint32_t* counter;
};

template <int NT>
__device__ __forceinline__ void up_mfma(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v, int p0,
                                        unsigned char* s_x, const UpSlice& sl) {
  constexpr int PPT = MfmaX<NT>::kPerThread;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // rows 0-7 of the wave: gate rows of its 8 pairs; rows 8-15: their up rows
  const int pair = p0 + 8 * wave + mfma_row_a();
  const bool wok = pair < v.I;
  const bf16_t* W13 = reinterpret_cast<const bf16_t*>(v.W13);
  const bf16_t* wa = W13 + (size_t)(wok ? pair : 0) * a.d + mfma_col_off();
  const bf16_t* wb = W13 + (size_t)(v.I + (wok ? pair : 0)) * a.d + mfma_col_off();
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  const bf16_t* xrow[PPT];
  bool xok[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int t = mfma_piece_token<NT>(i);
    int tok = 0, sr = 0;
    xok[i] = t < v.m;
    if (xok[i]) token_of(a, slots, v, t, tok, sr);
    xrow[i] = X + (size_t)tok * a.d;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_rows_db<NT, kUpMfmaChunks / 2, true>(wa, wok, wb, wok, xrow, xok, sl.s0, sl.s1, s_x, acc);
  if (sl.split > 1) {
    // one K slice: store its sums (device-coherent: the tile's last slice,
    // another workgroup of this launch, reads them) and arrive
    const coherent_rsrc_t prs = coherent_rsrc(sl.part);
    auto off = [&](int q, int nt) { return (uint32_t)((((q * kMfmaWaves + wave) * NT + nt) * 64 + lane) * 16); };
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) st_coherent4(prs, off(sl.slice, nt), __builtin_bit_cast(u32x4, acc[nt]));
    __shared__ int s_last;
    if (!arrive_last(sl.counter, (uint32_t)sl.split, &s_last)) return;
    constexpr int kMaxSplit = 2;
    u32x4 pv[kMaxSplit][NT];
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pv[q][nt] = ld_coherent4(prs, off(q < sl.split ? q : 0, nt));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] = __builtin_bit_cast(f32x4, pv[0][nt]);
#pragma unroll
      for (int q = 1; q < kMaxSplit; ++q)
        if (q < sl.split) acc[nt] += __builtin_bit_cast(f32x4, pv[q][nt]);
    }
  }
  // lane l < 32: pairs i .. i+3 (i = p0 + 8w + 4(l/16), a multiple of 4,
  // I a multiple of 32) of token nt*16 + l%16: one 16-byte store of h
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 hv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float u = __shfl_xor(acc[nt][q], 32);
      hv[q] = silu(acc[nt][q]) * u;
    }
    const int i = p0 + 8 * wave + 4 * (lane >> 4);
    const int t = nt * 16 + (lane & 15);
    if (lane < 32 && i < v.I && t < v.m) {
      int tok, sr;
      token_of(a, slots, v, t, tok, sr);
      h_store4<bf16_t>(a, v, t, sr, i, hv);
    }
  }
}

template <typename T>
__device__ __forceinline__ void up_mfma_dispatch(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v,
                                                 int p0, unsigned char* s_x, const UpSlice& sl) {
  if constexpr (sizeof(T) == 2) {
    const int nt = (v.m + 15) / 16;
    if (nt <= 1) up_mfma<1>(a, slots, v, p0, s_x, sl);
    else if (nt == 2) up_mfma<2>(a, slots, v, p0, s_x, sl);
    else if (nt == 3) up_mfma<3>(a, slots, v, p0, s_x, sl);
    else up_mfma<4>(a, slots, v, p0, s_x, sl);
  }
}

// Shared-expert gate/up tile `tile` with the whole workgroup (nw waves) on
// the vector shape: nw/2 pairs, each split over two waves into the same two
// halves of d as the gate/up kernel (so both give identical bits).  s_red:
// the caller's LDS scratch (nw/2 pair slots of 2 x kPartStride floats).
template <typename T>
__device__ __forceinline__ void shared_up_task(const ExpertLaunch& a, int tile, float* s_red) {
  const ExpertView v = shared_view(a);
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
  const int pp = nw >> 1;
  up_valu_dispatch<T, 2>(a, nullptr, v, tile * pp + wave % pp, wave / pp, wave % pp, s_red);
}

// ---- weighted combine ---------------------------------------------------------

// out[t][r] = sum_j w[t][j] * y[t*k+j][r] (j ascending), then + y[B*k+t][r]
// for the shared expert: fp32 fused multiply-adds in this order.
template <typename LoadY>
__device__ __forceinline__ float combine_one(const float* w_t, int k, int has_shared, LoadY y) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) acc = __builtin_fmaf(w_t[j], y(j), acc);
  if (has_shared) acc += y(k);
  return acc;
}

// ---- down projection ---------------------------------------------------------

// Destination of the per-slot outputs of one row tile: either the global
// Yslot [B][k+1][d] or an LDS tile [B*k + B][rt].
struct YSink {
  float* base;
  int lds;       // 1: LDS tile, rows of rt floats; 0: global Yslot
  int r0;        // first row of the tile (LDS)
  int rt;        // rows per LDS tile
  __device__ __forceinline__ float* at(const ExpertLaunch& a, int srow, int row) const {
    if (lds) return base + srow * rt + (row - r0);
    int t, j;
    if (srow < a.B * a.k) { t = srow / a.k; j = srow % a.k; }
    else { t = srow - a.B * a.k; j = a.k; }
    return base + ((size_t)t * (a.k + 1) + j) * a.d + row;
  }
};

// Rows r0..r0+ROWS-1 of entry v with one wave: L lanes per W2 row
// (L*VEC >= I), P = 64/L rows per load instruction, R = ROWS/P rows per lane.
template <typename T, int L, int ROWS>
__device__ __forceinline__ void down_valu(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v, int r0,
                          const YSink& sink) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int P = 64 / L;
  constexpr int R = ROWS / P;
  const int lane = threadIdx.x & 63;
  const int c = lane % L, g = lane / L;
  const bool cok = c * VEC < v.I;
  const int rbase = r0 + g;
  const T* W2 = reinterpret_cast<const T*>(v.W2);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = rbase + P * r;
    wv[r] = (cok && row < a.d) ? ld128_stream(W2 + (size_t)row * v.I + (size_t)c * VEC) : zero;
  }
  if constexpr (sizeof(T) == 2) {
    // h of kDownTokGroup tokens requested before any is used (one memory
    // round trip per group, not per token); a token past m re-reads the last
    const size_t co = (size_t)(cok ? c * VEC : 0);
    for (int t0 = 0; t0 < v.m; t0 += kDownTokGroup) {
      u32x4 h4[kDownTokGroup], l4[kDownTokGroup];
      int srs[kDownTokGroup];
#pragma unroll
      for (int q = 0; q < kDownTokGroup; ++q) {
        const int t = t0 + q < v.m ? t0 + q : v.m - 1;
        int tok;
        token_of(a, slots, v, t, tok, srs[q]);
        const size_t ho = (size_t)srs[q] * a.hld + co;
        h4[q] = cok ? *reinterpret_cast<const u32x4*>(h_hi(a) + ho) : zero;
        l4[q] = cok ? *reinterpret_cast<const u32x4*>(h_lo(a) + ho) : zero;
      }
#pragma unroll
      for (int q = 0; q < kDownTokGroup; ++q) {
        if (t0 + q >= v.m) break;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = group_sum<L>(dot_chunk_hilo(wv[r], h4[q], l4[q]));
        if (c == 0) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int row = rbase + P * r;
            if (row < a.d) *sink.at(a, srs[q], row) = acc[r];
          }
        }
      }
    }
  } else {
    for (int t = 0; t < v.m; ++t) {
      int tok, sr;
      token_of(a, slots, v, t, tok, sr);
      const size_t ho = (size_t)sr * a.hld + (size_t)(cok ? c * VEC : 0);
      float xs[VEC], acc[R];
#pragma unroll
      for (int e = 0; e < VEC; ++e) xs[e] = cok ? a.h[ho + e] : 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = group_sum<L>(dot_chunk_f32x(wv[r], xs, 0.f, T()));
      if (c == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = rbase + P * r;
          if (row < a.d) *sink.at(a, sr, row) = acc[r];
        }
      }
    }
  }
}

// Values every lane of the wave holds alike, moved to scalar registers so the
// compiler sees uniform control flow (and does not wait for every load in
// flight where lanes could have diverged).
// (Integers only: a pointer passed through readfirstlane would lose its
// global address space and turn its loads into flat ones.)
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ ExpertView wave_uniform(ExpertView v) {
  v.m = wave_uniform(v.m);
  v.I = wave_uniform(v.I);
  v.slot0 = wave_uniform(v.slot0);
  return v;
}

// Rows r0 .. r0 + rows - 1 (rows a multiple of 4, at most ROWS) of the
// entries this wave is given, vector shape with L = 16 lanes per W2 row
// (I <= 16 * VEC).  Entry order: s_order lists the entries by falling token
// count and the waves take them in snake order (w, 2nw-1-w, 2nw+w, ...), so
// the waves' token totals come out close.  The W2 rows of the wave's next
// entry are requested before the current entry's products (two register
// buffers used in turn, so no copy waits on a load), so a wave always has
// one entry in flight.  Every load is issued unconditionally from a clamped
// address -- past the last entry, and for row slots past `rows`, from rows
// this wave reads anyway -- so the compiler never has to wait for all loads
// at a branch.  h is read from LDS (s_h: bf16 hi/lo word rows for bf16
// weights, fp32 rows otherwise), so waiting for it never waits for the
// prefetch.  Same products in the same order as down_valu<T, 16, *>, hence
// the same bits.
template <typename T, int ROWS>
__device__ __forceinline__ void down_valu_pipe(const ExpertLaunch& a, const PlanView& p, int ne, const int* s_order,
                                               int r0, int rows, const YSink& sink, const void* s_h) {
  constexpr int L = 16;
  constexpr int VEC = Elem<T>::VEC;
  constexpr int P = 64 / L;
  constexpr int R = ROWS / P;
  const int lane = threadIdx.x & 63;
  const int nw = wave_uniform(blockDim.x >> 6), w = wave_uniform(threadIdx.x >> 6);
  const int c = lane % L, g = lane / L;
  const int rbase = r0 + g;
  const int rn = rows / P;   // row slots in use (uniform)
  const int hw = a.hld / 2;  // words per bf16 hi (or lo) row
  const int nrows = a.B * a.k + a.B;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  ne = wave_uniform(ne);
  auto pos = [&](int j) { return j * nw + ((j & 1) ? nw - 1 - w : w); };
  if (pos(0) >= ne) return;
  auto load = [&](const ExpertView& v, u32x4(&wv)[R]) {
    const char* W2 = reinterpret_cast<const char*>(v.W2);
    const int cc = (c * VEC < v.I ? c * VEC : 0) * (int)sizeof(T);
    const int ld = v.I * (int)sizeof(T);   // bytes per W2 row
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int row = rbase + P * (r < rn ? r : 0);
      row = row < a.d ? row : a.d - 1;
      wv[r] = ld128_stream(W2 + (unsigned)(row * ld + cc));
    }
  };
  auto products = [&](const ExpertView& v, const u32x4(&wv)[R]) {
    const bool cok = c * VEC < v.I;
    for (int t = 0; t < v.m; ++t) {
      int tok, sr;
      token_of(a, p.slots, v, t, tok, sr);
      float acc[R];
      if constexpr (sizeof(T) == 2) {
        const uint32_t* hh = static_cast<const uint32_t*>(s_h) + (size_t)sr * hw + (cok ? c * 4 : 0);
        const uint32_t* hl = hh + (size_t)nrows * hw;
        const u32x4 h4 = cok ? *reinterpret_cast<const u32x4*>(hh) : zero;
        const u32x4 l4 = cok ? *reinterpret_cast<const u32x4*>(hl) : zero;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = rbase + P * r;
          acc[r] = group_sum<L>(dot_chunk_hilo((cok && row < a.d) ? wv[r] : zero, h4, l4));
        }
      } else {
        const float* hp = static_cast<const float*>(s_h) + (size_t)sr * a.hld + (cok ? c * VEC : 0);
        float xs[VEC];
#pragma unroll
        for (int q = 0; q < VEC; ++q) xs[q] = cok ? hp[q] : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = rbase + P * r;
          acc[r] = group_sum<L>(dot_chunk_f32x((cok && row < a.d) ? wv[r] : zero, xs, 0.f, T()));
        }
      }
      if (c == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = rbase + P * r;
          if (r < rn && row < a.d) *sink.at(a, sr, row) = acc[r];
        }
      }
    }
  };
  auto view = [&](int j) { return wave_uniform(expert_view<T>(a, p, s_order[pos(j)])); };
  ExpertView v = view(0);
  u32x4 b0[R], b1[R];
  if (pos(1) >= ne) {
    // one entry: nothing to prefetch (re-requesting its rows as the "next"
    // entry doubled the loads a compute unit had to take in at batch 1)
    load(v, b0);
    products(v, b0);
    return;
  }
  load(v, b0);
  for (int j = 0;;) {
    // past the last entry the "next" loads re-read this entry's rows (cached)
    bool more = pos(j + 1) < ne;
    ExpertView vn = more ? view(j + 1) : v;
    load(vn, b1);
    products(v, b0);
    if (!more) break;
    v = vn;
    ++j;
    more = pos(j + 1) < ne;
    vn = more ? view(j + 1) : v;
    load(vn, b0);
    products(v, b1);
    if (!more) break;
    v = vn;
    ++j;
  }
}

// Entries of the plan (routed, then the shared one) ordered by falling token
// count, ties by entry index, into s_order -- one wave.  Each entry's count
// sits in a register (KC registers of 64 entries); for every count that
// occurs, from the largest down, one ballot per 64 entries places its
// entries.  (Ranking each entry against every other one through LDS took
// ~3 us at 51 entries and grows with the square of the count.)
template <int KC>
__device__ __forceinline__ void order_by_count(const ExpertLaunch& a, const PlanView& p, int ne, int* s_order) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int m[KC];
  uint64_t present = 0ull;   // bit c-1: some entry has c tokens (1 <= c <= B <= 64)
#pragma unroll
  for (int q = 0; q < KC; ++q) {
    const int i = q * 64 + lane;
    m[q] = i < ne ? (i < p.n ? p.offs[i + 1] - p.offs[i] : a.B) : 0;
    if (m[q] > 0) present |= 1ull << (m[q] - 1);
  }
  present = ((uint64_t)wave_or_u32((uint32_t)(present >> 32)) << 32) | wave_or_u32((uint32_t)present);
  int pos = 0;
  while (present) {
    const int c = 64 - __builtin_clzll(present);   // the largest count left
    present &= ~(1ull << (c - 1));
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      if (q * 64 >= ne) break;
      const uint64_t bm = __ballot(m[q] == c);
      if (m[q] == c) s_order[pos + __popcll(bm & below)] = q * 64 + lane;
      pos += __popcll(bm);
    }
  }
}

__device__ __forceinline__ void order_entries(const ExpertLaunch& a, const PlanView& p, int ne, int* s_order) {
  if (ne <= 64) order_by_count<1>(a, p, ne, s_order);
  else if (ne <= 256) order_by_count<4>(a, p, ne, s_order);
  else order_by_count<(kMaxB * kMaxK + kMaxB + 63) / 64>(a, p, ne, s_order);   // entries <= B k + 1
}

// Entries ordered by falling number of 16-token tiles (4 classes at B <= 64),
// ties by entry index, into s_order -- one wave, with ballots: no loop over
// the other entries per entry (the ranking above took ~3 us at 51 entries).
__device__ __forceinline__ void order_entries_by_tiles(const ExpertLaunch& a, const PlanView& p, int ne,
                                                       int* s_order) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto tiles_of = [&](int i) {
    const int m = i < p.n ? p.offs[i + 1] - p.offs[i] : a.B;
    const int t = (m + 15) >> 4;
    return t < 1 ? 1 : (t > 4 ? 4 : t);
  };
  // entries per class (1..4 tiles)
  int cnt[5] = {0, 0, 0, 0, 0};
  for (int i0 = 0; i0 < ne; i0 += 64) {
    const int i = i0 + lane;
    const int t = i < ne ? tiles_of(i) : 0;
#pragma unroll
    for (int c = 1; c <= 4; ++c) cnt[c] += __popcll(__ballot(t == c));
  }
  // first position of each class: 4-tile entries first
  int start[5];
  start[4] = 0;
  start[3] = cnt[4];
  start[2] = start[3] + cnt[3];
  start[1] = start[2] + cnt[2];
  int seen[5] = {0, 0, 0, 0, 0};
  for (int i0 = 0; i0 < ne; i0 += 64) {
    const int i = i0 + lane;
    const int t = i < ne ? tiles_of(i) : 0;
    int pos = 0;
#pragma unroll
    for (int c = 1; c <= 4; ++c) {
      const uint64_t m = __ballot(t == c);
      if (t == c) pos = start[c] + seen[c] + __popcll(m & below);
      seen[c] += __popcll(m);
    }
    if (i < ne) s_order[pos] = i;
  }
}

template <int NT>
__device__ __forceinline__ void down_mfma(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v, int r0,
                          const YSink& sink, int r_end) {
  constexpr int JM = kMaxInter / 32;   // K steps of the longest row
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const bf16_t* W2 = reinterpret_cast<const bf16_t*>(v.W2);
  // rows from r_end on (past d, or another workgroup's tile) re-read the
  // last row of the range (cached) and are not stored
  const int J = wave_uniform(v.I / 32);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int JH = JM / 2;
  // h of one token tile in two halves of K: 32 registers of h at a time keep
  // the wave within its register budget.  h comes from the tiled copy, where
  // a K step of a tile is 1 KB in lane order (one fully used cache line per
  // four lanes; from the slot rows, each lane of a quad hit a different
  // line, and at batch 64 the h reads took longer than the weight stream).
  // Only the lanes of real tokens load; the others neither load nor zero
  // their registers (the products take zero for them): writing a register
  // that a load might still own makes the compiler wait for every load in
  // flight.
  auto load_half = [&](bool ok, const uint16_t* hh, const uint16_t* hl, int half, u32x4 (&hv)[JH], u32x4 (&lv)[JH]) {
    if (ok) {
#pragma unroll
      for (int jj = 0; jj < JH; ++jj) {
        const int j = half * JH + jj;
        const size_t off = (size_t)(j < J ? j : J - 1) * 512;
        hv[jj] = *reinterpret_cast<const u32x4*>(hh + off);
        lv[jj] = *reinterpret_cast<const u32x4*>(hl + off);
      }
    }
  };
  auto mul_half = [&](bool ok, int half, const u32x4 (&wv)[JM], const u32x4 (&hv)[JH], const u32x4 (&lv)[JH],
                      f32x4& acc) {
#pragma unroll
    for (int jj = 0; jj < JH; ++jj) {
      const int j = half * JH + jj;
      if (j < J) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[j]),
                                                      __builtin_bit_cast(bf16x8, ok ? hv[jj] : zero), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[j]),
                                                      __builtin_bit_cast(bf16x8, ok ? lv[jj] : zero), acc, 0, 0, 0);
      }
    }
  };
  auto store = [&](bool ok, int sr, const f32x4& acc) {
    if (ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * kq + i;
        if (r < r_end) *sink.at(a, sr, r) = acc[i];
      }
    }
  };
  // token tile 0: the first half of its h is requested before the weights
  // (all K steps of the wave's 16 rows at once, steps past J re-reading the
  // last one), so waiting for the weights never delays the request for h
  int tok0 = 0, sr0 = 0;
  const bool ok0 = row < v.m;
  if (ok0) token_of(a, slots, v, row, tok0, sr0);
  const size_t tb0 = (size_t)v.hbase * a.hld + lane * 8;   // tile 0, this lane's 16 bytes
  const uint16_t* hh0 = a.ht_hi + tb0;
  const uint16_t* hl0 = a.ht_lo + tb0;
  u32x4 wv[JM];
  {
    u32x4 hv[JH], lv[JH];
    load_half(ok0, hh0, hl0, 0, hv, lv);
    load_w2_operands(W2, v.I, r0, r_end, J, wv);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mul_half(ok0, 0, wv, hv, lv, acc);
    if (JH < J) {
      load_half(ok0, hh0, hl0, 1, hv, lv);
      mul_half(ok0, 1, wv, hv, lv, acc);
    }
    store(ok0, sr0, acc);
  }
  // the other token tiles, one at a time
#pragma unroll 1
  for (int nt = 1; nt < NT; ++nt) {
    const int ti = nt * 16 + row;
    int tok = 0, sr = 0;
    const bool ok = ti < v.m;
    if (ok) token_of(a, slots, v, ti, tok, sr);
    const size_t tb = (size_t)(v.hbase + nt * 16) * a.hld + lane * 8;
    const uint16_t* hh = a.ht_hi + tb;
    const uint16_t* hl = a.ht_lo + tb;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half * JH >= J) break;
      u32x4 hv[JH], lv[JH];
      load_half(ok, hh, hl, half, hv, lv);
      mul_half(ok, half, wv, hv, lv, acc);
    }
    store(ok, sr, acc);
  }
}

// Rows r0 .. r0+31 of entry v with one wave (matrix shape, the two 16-row
// halves of a 17..32-row tile): the wave holds the W2 rows of both halves
// (64 registers, all K steps) and a token tile's h in full K (hi and lo
// planes, 64 registers), so each tile of h crosses from L2 once for the 32
// rows and in one memory round trip; the next tile's h is requested before
// the products of the current one (a second 64-register buffer).  Needs the
// 256-register budget of two waves per SIMD.  Rows from r_end on re-read the
// last row of the range and are not stored.  Each output is the same chain
// of products as in down_mfma, hence the same bits.
template <int NT>
__device__ __forceinline__ void down_mfma_duo(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v,
                                              int r0, const YSink& sink, int r_end) {
  constexpr int JM = kMaxInter / 32;
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const bf16_t* W2 = reinterpret_cast<const bf16_t*>(v.W2);
  const int J = wave_uniform(v.I / 32);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load_h = [&](int nt, u32x4 (&hv)[JM], u32x4 (&lv)[JM]) {
    if (nt * 16 + row < v.m) {
      const size_t tb = (size_t)(v.hbase + nt * 16) * a.hld + lane * 8;
#pragma unroll
      for (int j = 0; j < JM; ++j) {
        const size_t off = tb + (size_t)(j < J ? j : J - 1) * 512;
        hv[j] = *reinterpret_cast<const u32x4*>(a.ht_hi + off);
        lv[j] = *reinterpret_cast<const u32x4*>(a.ht_lo + off);
      }
    }
  };
  auto tile = [&](int nt, const u32x4 (&wva)[JM], const u32x4 (&wvb)[JM], const u32x4 (&hv)[JM],
                  const u32x4 (&lv)[JM]) {
    const bool ok = nt * 16 + row < v.m;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      if (j < J) {
        const bf16x8 h = __builtin_bit_cast(bf16x8, ok ? hv[j] : zero);
        const bf16x8 l = __builtin_bit_cast(bf16x8, ok ? lv[j] : zero);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wva[j]), h, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wvb[j]), h, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wva[j]), l, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wvb[j]), l, acc1, 0, 0, 0);
      }
    }
    if (ok) {
      int tok, sr;
      token_of(a, slots, v, nt * 16 + row, tok, sr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * kq + i;
        if (r < r_end) *sink.at(a, sr, r) = acc0[i];
        if (r + 16 < r_end) *sink.at(a, sr, r + 16) = acc1[i];
      }
    }
  };
  u32x4 hA[JM], lA[JM], hB[JM], lB[JM];
  load_h(0, hA, lA);
  u32x4 wva[JM], wvb[JM];
  load_w2_operands(W2, v.I, r0, r_end, J, wva);
  load_w2_operands(W2, v.I, r0 + 16, r_end, J, wvb);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt % 2 == 0) {
      if (nt + 1 < NT) load_h(nt + 1, hB, lB);
      tile(nt, wva, wvb, hA, lA);
    } else {
      if (nt + 1 < NT) load_h(nt + 1, hA, lA);
      tile(nt, wva, wvb, hB, lB);
    }
  }
}

// ---- down projection as (entry, 64-row tile) tasks ------------------------

// LDS image of one entry's h for the MFMA down: the token rows of the hi
// plane (rows 0..63), then of the lo plane (rows 64..127), I bf16 each;
// rows padded by 16 bytes so the 16 lanes reading one B operand (16 token
// rows) spread over the LDS banks.
constexpr int kHRowBytes = kMaxInter * 2 + 16;
constexpr int kHLdsBytes = 2 * kMaxB * kHRowBytes;

// Copy h of entry v's tokens (bf16 planes) into s_h with the whole workgroup.
__device__ __forceinline__ void stage_h_entry(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v,
                                              unsigned char* s_h) {
  const int per_row = v.I / 8;   // 16-byte pieces per plane row
  const int n = v.m * 2 * per_row;
  for (int pc = threadIdx.x; pc < n; pc += blockDim.x) {
    const int t = pc / (2 * per_row), rem = pc % (2 * per_row);
    const int plane = rem / per_row, q = rem % per_row;
    int tok, sr;
    token_of(a, slots, v, t, tok, sr);
    const uint16_t* src = (plane ? h_lo(a) : h_hi(a)) + (size_t)sr * a.hld + q * 8;
    *reinterpret_cast<u32x4*>(s_h + (plane * kMaxB + t) * kHRowBytes + q * 16) = *reinterpret_cast<const u32x4*>(src);
  }
}

// Rows r0 .. r0+15 of entry v (m > 8) with one wave: the W2 rows (all K
// steps, wv) were requested before h was staged; h from s_h.  Same products
// in the same order as down_mfma, hence the same bits.  The per-slot outputs
// (4 consecutive rows per lane) go to the global Yslot.
template <int NT>
__device__ __forceinline__ void down_mfma_lds(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v, int r0,
                                              const u32x4 (&wv)[kMaxInter / 32], const unsigned char* s_h) {
  constexpr int JM = kMaxInter / 32;
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const int J = wave_uniform(v.I / 32);
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = nt * 16 + row;
    const bool ok = t < v.m;
    const unsigned char* hh = s_h + (size_t)(ok ? t : 0) * kHRowBytes;
    const unsigned char* hl = hh + (size_t)kMaxB * kHRowBytes;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      if (j < J) {
        // the K order of the W2 operands (down_k_slot): step j of a pair
        // takes columns 64 (j / 2) + 16 kq + 8 (j % 2) .. +7
        const int off = j < (J & ~1) ? (j >> 1) * 128 + kq * 32 + (j & 1) * 16 : j * 64 + kq * 16;
        const u32x4 hv = ok ? *reinterpret_cast<const u32x4*>(hh + off) : zero;
        const u32x4 lv = ok ? *reinterpret_cast<const u32x4*>(hl + off) : zero;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[j]),
                                                      __builtin_bit_cast(bf16x8, hv), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[j]),
                                                      __builtin_bit_cast(bf16x8, lv), acc, 0, 0, 0);
      }
    }
    if (ok) {
      int tok, sr;
      token_of(a, slots, v, t, tok, sr);
      const YSink sink = {a.Yslot, 0, 0, 0};
      const int r = r0 + 4 * kq;
      float* dst = sink.at(a, sr, r);
      if (r + 3 < a.d && (a.d & 3) == 0) {
        *reinterpret_cast<f32x4*>(dst) = acc;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r + i < a.d) dst[i] = acc[i];
      }
    }
  }
}

// Rows r0..r0+ROWS-1 of entry v with one wave (the MFMA shape covers 16).
template <typename T, int PATHS, int ROWS = 16>
__device__ __forceinline__ void down_dispatch(const ExpertLaunch& a, const int32_t* slots, const ExpertView& v,
                                              int r0, const YSink& sink, int r_end = -1) {
  static_assert(ROWS == 16 || PATHS == kPathValu, "the MFMA down shape covers 16 rows");
  if (r_end < 0) r_end = a.d;
  if (use_mfma<PATHS>(v.m)) {
    if constexpr (sizeof(T) == 2) {
      const int nt = (v.m + 15) / 16;
      if (nt <= 1) down_mfma<1>(a, slots, v, r0, sink, r_end);
      else if (nt == 2) down_mfma<2>(a, slots, v, r0, sink, r_end);
      else if (nt == 3) down_mfma<3>(a, slots, v, r0, sink, r_end);
      else down_mfma<4>(a, slots, v, r0, sink, r_end);
    }
  } else {
    constexpr int VEC = Elem<T>::VEC;
    const int chunks = v.I / VEC;
    if constexpr (ROWS > 16) {
      down_valu<T, 16, ROWS>(a, slots, v, r0, sink);  // host guarantees I <= 16 * VEC
    } else {
      if (chunks <= 16) down_valu<T, 16, ROWS>(a, slots, v, r0, sink);
      else if (chunks <= 32 || sizeof(T) == 2) down_valu<T, 32, ROWS>(a, slots, v, r0, sink);
      else if constexpr (sizeof(T) == 4) down_valu<T, 64, ROWS>(a, slots, v, r0, sink);
    }
  }
}

}  // namespace moe
