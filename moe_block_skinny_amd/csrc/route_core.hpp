// route_core.hpp -- top-k selection with softmax weights (one token per
// wave) and the routing plan of up to 64 slots (one wave).  Used by the
// router kernel's finishing workgroup and, in the fused block at small
// batch, by every workgroup of the gate/up kernel.
//
// Source: "vLLM 如何用智能体辅助优化 Kimi K3 解码性能", part 1 §3 (MoE
// scheduling): a router picks the routed experts of each token.  The
// selection rule: the k largest logits, equal logits ordered by lower expert
// index; weights = softmax over the selected logits; ids are returned in
// ascending expert order.
//
// Selection without k serial rounds: lane l holds experts l, l+64, ...
// (1) T = the k-th largest of the 64 lane maxima, rounded down to its top
// 16 bits, found bit by bit with ballots (two bits per step); at least k
// logits reach T, so every top-k logit does too.  (2) The logits >= T (k of
// them plus a few, in the usual case) are compacted into LDS by ballots.
// (3) Each candidate is ranked against the others by (logit, lower index);
// ranks 0..k-1 win.  Ties of logits only enlarge the candidate set.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMaxE = 512;
constexpr int kMaxK = 16;
constexpr int kMaxB = 64;
constexpr int kNI = kMaxE / 64;   // logits per lane
constexpr int kMaxInter = 256;    // expert intermediate size (bf16; fp32: 256 as well)

constexpr int kTopkWaves = 8;     // waves of a workgroup that select (each holds a TopkScratch)

// LDS scratch of one wave for topk_wave.
struct TopkScratch {
  uint64_t cand[kMaxE];
  uint64_t win[kMaxK];
};

// Order this wave's LDS writes before its later LDS reads by other lanes
// (the DS unit serves one wave's instructions in order; the wait and the
// memory clobber keep the hardware and the compiler from running ahead).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Composite key (ord_key(logit) << 32 | ~expert): larger <=> larger logit,
// then lower expert index.
__device__ __forceinline__ int sel_expert(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }
__device__ __forceinline__ float sel_value(uint64_t c) { return key_value((uint32_t)(c >> 32)); }

// Top-k of one token with the whole wave.  lv[i] is the logit of expert
// lane + 64 i (ignored at or past E).  Writes the k ids in ascending order
// and their weights exp(l - l_max) / sum over the selection to ids / w, and
// also to ids2 / w2 when those are non-null (device-coherent stores).
// Requires 1 <= k <= min(E, 16).
__device__ __forceinline__ void topk_wave(const float (&lv)[kNI], int E, int k, TopkScratch& sc, int32_t* ids,
                                          float* w, int32_t* ids2, float* w2) {
  const int lane = threadIdx.x & 63;
  uint32_t key[kNI];
  uint32_t lmax = 0u;
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ord_key(lv[i]) : 0u;
    lmax = key[i] > lmax ? key[i] : lmax;
  }
  // (1) the largest T = p << 16 with at least k lane maxima >= T (16-bit
  // prefixes: fewer steps, a few more candidates); T > 0 because at least
  // min(E, 64) >= k lanes hold an expert and every finite logit's key has a
  // nonzero top half
  uint32_t T = 0u;
#pragma unroll
  for (int b = 30; b >= 16; b -= 2) {
    const uint32_t t1 = T | (1u << b), t2 = T | (2u << b), t3 = T | (3u << b);
    const int c1 = __popcll(__ballot(lmax >= t1));
    const int c2 = __popcll(__ballot(lmax >= t2));
    const int c3 = __popcll(__ballot(lmax >= t3));
    T = c3 >= k ? t3 : (c2 >= k ? t2 : (c1 >= k ? t1 : T));
  }
  // (2) compact the candidates (key >= T) into LDS: per slot i a ballot,
  // each lane's place = candidates of earlier slots + lower lanes
  int C = 0;
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    const bool c = key[i] >= T;
    const uint64_t m = __ballot(c);
    if (c) {
      const int at = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      sc.cand[at] = ((uint64_t)key[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * i));
    }
    C += __popcll(m);
  }
  wave_lds_sync();
  // (3) rank each candidate among the candidates; ranks 0..k-1 win
  if (C <= 16) {
    // lane 16 q + j compares candidate j with candidates q, q+4, q+8, q+12;
    // a row sum gives each one's rank
    const int j = lane & 15, q = lane >> 4;
    const uint64_t cj = j < C ? sc.cand[j] : 0ull;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int i = q + 4 * r4;
      const uint64_t ci = i < C ? sc.cand[i] : ~0ull;
      const int rank = (int)group_sum<16>(cj > ci ? 1.f : 0.f);
      if (j == 0 && i < C && rank < k) sc.win[rank] = ci;
    }
  } else {
    for (int base = 0; base < C; base += 64) {
      const int idx = base + lane;
      const uint64_t my = idx < C ? sc.cand[idx] : 0ull;
      int r = 0;
      for (int jj = 0; jj < C; ++jj) r += sc.cand[jj] > my ? 1 : 0;
      if (idx < C && r < k) sc.win[r] = my;
    }
  }
  wave_lds_sync();
  // winners, largest first: lane j < k takes the j-th; its place in
  // ascending-id order counts the winners with a lower id
  uint64_t wv[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) wv[i] = sc.win[i];
  const uint64_t cw = lane < k ? sc.win[lane] : 0ull;
  const int e = lane < k ? sel_expert(cw) : 0x7fffffff;
  int pos = 0;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) pos += (i < k && sel_expert(wv[i]) < e) ? 1 : 0;
  const float m = sel_value(wv[0]);
  const float ex = lane < k ? expf(sel_value(cw) - m) : 0.f;
  const float z = group_sum<16>(ex);   // k <= 16: lanes 0..15 hold the sum
  if (lane < k) {
    const float wt = ex / z;
    ids[pos] = e;
    w[pos] = wt;
    if (ids2) {   // read by other workgroups of the launch in the split finish
      __hip_atomic_store(ids2 + pos, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(w2 + pos, wt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Load the logits of token t (row t of [M][E]) as topk_wave expects them:
// device-coherent loads when other workgroups of the same launch stored them
// (SAME_LAUNCH), plain loads when an earlier launch did.
template <bool SAME_LAUNCH>
__device__ __forceinline__ void load_logit_row(const float* logits, int t, int E, float (&lv)[kNI]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    const int e = lane + 64 * i;
    const float* p = logits + (size_t)t * E + (e < E ? e : E - 1);
    lv[i] = SAME_LAUNCH ? ld_coherent(p) : *p;
  }
}

// Routing plan (layout of moe_plan_words: n, active[maxa], offs[maxa + 1],
// slots[nslot]) of nslot <= 64 slots with one wave; slot s = t*k + j chose
// expert ids[s].  Active experts ascend; each expert's slots ascend (by
// token).  Writes P and, when non-null, P2.  sc: 128 ints of LDS.
__device__ __forceinline__ void plan_wave(const int32_t* ids, int nslot, int E, int* sc, int32_t* P, int32_t* P2) {
  const int lane = threadIdx.x & 63;
  const int maxa = nslot < E ? nslot : E;
  const bool in = lane < nslot;
  const int e = in ? ids[lane] : 0x7fffffff;
  const int key = in ? e * 64 + lane : 0x7fffffff;   // unique: lane < 64
  int* s_key = sc;
  int* s_sorted = sc + 64;
  s_key[lane] = key;
  wave_lds_sync();
  int pos = 0;   // lanes past nslot hold INT_MAX: never below a slot key
  const int jn = (nslot + 7) & ~7;
  for (int j0 = 0; j0 < jn; j0 += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) pos += s_key[j0 + j] < key ? 1 : 0;
  }
  if (in) {
    s_sorted[pos] = e;
    P[2 + 2 * maxa + pos] = lane;
    if (P2) P2[2 + 2 * maxa + pos] = lane;
  }
  wave_lds_sync();
  const int ep = in ? s_sorted[lane] : -1;
  const int eprev = (in && lane > 0) ? s_sorted[lane - 1] : -1;
  const int first = (in && ep != eprev) ? 1 : 0;
  const int incl = wave_incl_scan(first);
  const int n = __builtin_amdgcn_readlane(incl, 63);
  for (int q = 0; q < 2; ++q) {
    int32_t* D = q ? P2 : P;
    if (!D) continue;
    if (first) {
      D[1 + incl - 1] = ep;
      D[1 + maxa + incl - 1] = lane;
    }
    for (int i = n + lane; i < maxa; i += 64) D[1 + i] = -1;
    for (int i = n + lane; i <= maxa; i += 64) D[1 + maxa + i] = nslot;
    if (lane == 0) D[0] = n;
  }
}

// The plan of one token (B = 1, nslot = k <= E, ids ascending and distinct,
// as topk_wave leaves them): n = k, active = ids, offs = 0..k, slots =
// 0..k-1 -- what plan_wave computes for it, without the sort.  One wave;
// writes P and, when non-null, P2.
__device__ __forceinline__ void plan_one_token(const int32_t* ids, int k, int32_t* P, int32_t* P2) {
  const int lane = threadIdx.x & 63;
  for (int q = 0; q < 2; ++q) {
    int32_t* D = q ? P2 : P;
    if (!D) continue;
    if (lane < k) {
      D[1 + lane] = ids[lane];
      D[1 + k + lane] = lane;
      D[2 + 2 * k + lane] = lane;
    }
    if (lane == 0) {
      D[0] = k;
      D[1 + 2 * k] = k;
    }
  }
}

// LDS scratch of plan_block.
struct PlanScratch {
  unsigned long long mask[kMaxE];   // bit t: token t chose expert e
  int cnt[kMaxE];                   // first plan slot of expert e
  int act[kMaxE];                   // rank of expert e among the active ones
  int incl[kMaxE];
  int wtot[kMaxE / 64];
  int n;
  int sc[128];                      // plan_wave's scratch
};

// The routing plan of nslot = B*k slots (slot s = t*k + j chose expert
// ids[s], ids in LDS) with the whole workgroup, into P and, when non-null,
// P2 (same layout as plan_wave; either may be LDS or global memory).  Up to
// 64 slots one wave sorts them (plan_wave); beyond, per-expert token masks
// and a scan over experts.  Ends after the last write, without a barrier.
__device__ __forceinline__ void plan_block(const int32_t* ids, int nslot, int k, int E, int32_t* P, int32_t* P2,
                                           PlanScratch& ps) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (nslot <= 64) {
    if (wave == 0) plan_wave(ids, nslot, E, ps.sc, P, P2);
    return;
  }
  for (int e = tid; e < E; e += blockDim.x) ps.mask[e] = 0ull;
  __syncthreads();
  // bit t of mask[e] is set when token t selected expert e (B <= 64)
  for (int s = tid; s < nslot; s += blockDim.x) atomicOr(&ps.mask[ids[s]], 1ull << (s / k));
  __syncthreads();
  // exclusive prefix sums over experts of slot counts and of "is active",
  // packed in one int (counts <= 1024 in the low half, actives <= 512 in
  // the high half): a DPP scan per 64-expert group (waves take groups in
  // turn, so any workgroup size works), group totals through LDS.
  const int nwv = (E + 63) >> 6, nw = blockDim.x >> 6;
  for (int grp = wave; grp < nwv; grp += nw) {
    const int e = grp * 64 + lane;
    const int c = e < E ? __popcll(ps.mask[e]) : 0;
    const int packed = c | ((c > 0 ? 1 : 0) << 16);
    const int incl = wave_incl_scan(packed);
    ps.incl[e] = incl - packed;   // exclusive within the group
    if (lane == 63) ps.wtot[grp] = incl;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int grp = e >> 6;
    int base = 0;
    for (int g = 0; g < grp; ++g) base += ps.wtot[g];
    const int ex = base + ps.incl[e];
    ps.cnt[e] = ex & 0xffff;
    ps.act[e] = ex >> 16;
  }
  if (tid == 0) {
    int tot = 0;
    for (int g = 0; g < nwv; ++g) tot += ps.wtot[g];
    ps.n = tot >> 16;
  }
  __syncthreads();
  const int n = ps.n;
  const int maxa = nslot < E ? nslot : E;
  for (int q = 0; q < 2; ++q) {
    int32_t* D = q ? P2 : P;
    if (!D) continue;
    int32_t* active = D + 1;
    int32_t* offs = D + 1 + maxa;
    int32_t* slots = D + 2 + 2 * maxa;
    if (tid == 0) D[0] = n;
    for (int e = tid; e < E; e += blockDim.x)
      if (ps.mask[e]) {
        active[ps.act[e]] = e;
        offs[ps.act[e]] = ps.cnt[e];
      }
    for (int i = n + tid; i < maxa; i += blockDim.x) active[i] = -1;
    for (int i = n + tid; i <= maxa; i += blockDim.x) offs[i] = nslot;
    for (int s = tid; s < nslot; s += blockDim.x) {
      const int e = ids[s], t = s / k;
      const unsigned long long below = (t == 0) ? 0ull : (ps.mask[e] & ((1ull << t) - 1ull));
      slots[ps.cnt[e] + __popcll(below)] = s;
    }
  }
}

}  // namespace moe
