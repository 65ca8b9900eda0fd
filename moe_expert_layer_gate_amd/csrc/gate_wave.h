// Wave-level top-k softmax of one router row (shared by the gate kernel and
// the single-block routing kernel).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// section 快速选择专家: one fused router op replaces top-k followed by softmax.
// [P2] "LongCat-Flash inference on Atlas A3 clusters", MoE模块 / Router: sort
// the router output and keep the top-k experts.
//
// Selection compares the fp32 logits exactly, key (logit desc, id asc); the
// weights are the softmax over the k selected logits (equal to the full
// softmax renormalised over the top-k). Requires 1 <= k <= min(E, 64).
//
// Each lane holds VPL logits (expert e = lane + 64 * i) as order-preserving
// unsigned keys. The k-th largest key is found one bit at a time from the
// top: a bit stays set when at least k keys reach the candidate, counted with
// one ballot per register (no cross-lane shuffles). Keys above that threshold
// win, and so do the lowest-id keys equal to it until k are taken. Winners
// are compacted into a 64-entry LDS slot array in id order; lane j < k then
// ranks winner j against all k (broadcast reads) and stores (id, weight) at
// its rank, so row r of the output lists the experts best first.
#pragma once
#include "common.h"

namespace moe {

// Monotone map from finite floats to uint32 (-0 ranks with +0). Key 0 is
// below every finite float's key and marks an absent entry.
MOE_DEV uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

MOE_DEV float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// This lane's keys of one router row: expert e = lane + 64 * i.
template <int VPL>
MOE_DEV void load_row_keys(const float* __restrict__ row, int E,
                           uint32_t (&key)[VPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_key(row[e]) : 0u;
  }
}

// Top-k + softmax of a row whose keys are already in registers.
// slot: this wave's 64 (key, id) pairs in LDS.
template <int VPL>
MOE_DEV void topk_softmax_keys(const uint32_t (&key)[VPL], int k,
                               int32_t* __restrict__ ids,
                               float* __restrict__ wout, uint2* slot) {
  const int lane = threadIdx.x & 63;
  // the k-th largest key
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) cnt += popc64(ballot(key[i] >= cand));
    if (cnt >= k) thr = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) n_gt += popc64(ballot(key[i] > thr));
  const int need_eq = k - n_gt;  // >= 1 ties at the threshold are taken
  const uint64_t lt = lanemask_lt();
  int eq_before = 0, win_before = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const bool eq = key[i] == thr;
    const uint64_t meq = ballot(eq);
    const bool win = key[i] > thr ||
                     (eq && eq_before + popc64(meq & lt) < need_eq);
    const uint64_t mw = ballot(win);
    if (win)
      slot[win_before + popc64(mw & lt)] =
          make_uint2(key[i], (uint32_t)(lane + 64 * i));
    eq_before += popc64(meq);
    win_before += popc64(mw);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  uint2 mine = make_uint2(0u, 0u);
  if (lane < k) mine = slot[lane];
  // rank among the winners; the best key sets the softmax shift
  int rank = 0;
  uint32_t kmax = 0;
  for (int j = 0; j < k; ++j) {
    const uint2 o = slot[j];
    kmax = max(kmax, o.x);
    rank += (o.x > mine.x || (o.x == mine.x && o.y < mine.y)) ? 1 : 0;
  }
  const float vmax = key_value(kmax);
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += expf(key_value(slot[j].x) - vmax);
  if (lane < k) {
    ids[rank] = (int32_t)mine.y;
    wout[rank] = expf(key_value(mine.x) - vmax) / sum;
  }
  // the slots are reused by this wave's next row
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// slot: this wave's 64 (key, id) pairs in LDS.
template <int VPL>
MOE_DEV void topk_softmax_wave(const float* __restrict__ row, int E, int k,
                               int32_t* __restrict__ ids,
                               float* __restrict__ wout, uint2* slot) {
  uint32_t key[VPL];
  load_row_keys<VPL>(row, E, key);
  topk_softmax_keys<VPL>(key, k, ids, wout, slot);
}

}  // namespace moe
