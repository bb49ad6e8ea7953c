// Router building blocks shared by the router kernels and the fused decode
// layer launches: the float32 logit GEMV of one expert row (a 256-thread
// block) and the top-k of one token's logits (one wave).
//
// "Strata-DSV4.1", §How it works (the router runs on the GPU with the dense
// half); §DeepSeek-V4.1-Flash (384 experts, top-6).  Selection is by logit
// (softmax is monotone), an exact tie going to the lower expert index; the
// weights are exp(L_j - L_max) / sum over the selected experts, which equals
// the full softmax renormalised over them.
#pragma once

#include "common.h"

#include <type_traits>

namespace bm {

// One block per expert row: thread i reads the float4 slices 4i + 1024j of the
// row and its slices of every token's activations (all of them issued before
// the arithmetic; NT >= T token slots, those past T re-read token T-1 and are
// dropped), the block sums through LDS.
template <bool XBF16, int NT>
BM_DEVICE void router_gemv_block(const void *__restrict__ x, int T, int D, int E, const float *__restrict__ wr,
                                 const float *__restrict__ bias, float *__restrict__ logits, int e) {
  constexpr int MAXJ = 4;  // D <= 4096
  __shared__ float part[4][NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *row = wr + int64_t(e) * D;
  float4 w[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = 4 * tid + 1024 * j;
    w[j] = c < D ? *reinterpret_cast<const float4 *>(row + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // raw activation slices: 4 bf16 (uint2) or 4 float32 (float4) per slot
  typename std::conditional<XBF16, uint2, float4>::type xv[NT][MAXJ];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t tt = min(t, T - 1);
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int c = 4 * tid + 1024 * j;
      if constexpr (XBF16)
        xv[t][j] = c < D ? *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + tt * D + c)
                         : make_uint2(0u, 0u);
      else
        xv[t][j] = c < D ? *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + tt * D + c)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      float4 v;
      if constexpr (XBF16) v = make_float4(bf16_lo(xv[t][j].x), bf16_hi(xv[t][j].x), bf16_lo(xv[t][j].y), bf16_hi(xv[t][j].y));
      else v = xv[t][j];
      acc = __builtin_fmaf(w[j].x, v.x, acc);
      acc = __builtin_fmaf(w[j].y, v.y, acc);
      acc = __builtin_fmaf(w[j].z, v.z, acc);
      acc = __builtin_fmaf(w[j].w, v.w, acc);
    }
    const float s = wave_sum(acc);
    if (lane == 0) part[wave][t] = s;
  }
  __syncthreads();
  if (tid < T) {
    const float s = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
    logits[int64_t(tid) * E + e] = s + (bias ? bias[e] : 0.f);
  }
}

// Order-preserving key of a float32 logit: larger value -> larger key, +0 and
// -0 alike; NaN and absent entries get key 0, below every number.
BM_DEVICE uint32_t logit_key(float v) {
  if (v != v) return 0u;
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
BM_DEVICE float key_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Top-k of one token's logits by one wave; lane 0 writes ids and weights.
// Round j: every lane takes its largest remaining key and the lowest slot
// holding it, the wave-wide largest key M comes from a DPP reduction, and the
// selected expert is the lowest index e = lane + 64 slot among the lanes
// holding M (one ballot; an exact tie across lanes is settled in a short
// scalar loop), so an exact tie goes to the lower expert index.
template <int PER>  // logits per lane: E <= 64 PER
BM_DEVICE void topk_token(const float *L, int E, int k, int32_t *ids, float *wts, int lane) {
  // all PER loads issued before any use (slots past E read logit E - 1 and
  // are dropped), so their latencies overlap
  float lv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) lv[i] = L[min(lane + 64 * i, E - 1)];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = lane + 64 * i < E ? logit_key(lv[i]) : 0u;
  float sel_v[8];
  int sel_i[8];
  // unrolled to the largest k, so that every round writes its selection to a
  // fixed register (a run-time index would cost a select chain per round)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    uint32_t m = key[0];
    int s = 0;
#pragma unroll
    for (int i = 1; i < PER; ++i) {
      const bool gt = key[i] > m;  // strictly: the lowest slot keeps an equal key
      m = gt ? key[i] : m;
      s = gt ? i : s;
    }
    const uint32_t M = wave_max_u32(m);
    int bi = -1;  // only NaN logits left: no valid expert
    if (M != 0u) {
      uint64_t hit = __ballot(m == M);
      const int l = __builtin_ctzll(hit);
      bi = l + 64 * __builtin_amdgcn_readlane(s, l);
      hit &= hit - 1;
      while (hit) {  // several lanes hold M: the lowest expert index among them
        const int l2 = __builtin_ctzll(hit);
        bi = min(bi, l2 + 64 * __builtin_amdgcn_readlane(s, l2));
        hit &= hit - 1;
      }
      const int wl = bi & 63, wsl = bi >> 6;
#pragma unroll
      for (int i = 0; i < PER; ++i) key[i] = (lane == wl && i == wsl) ? 0u : key[i];
    }
    sel_v[j] = bi < 0 ? -INFINITY : key_logit(M);
    sel_i[j] = bi;
  }
  if (lane == 0) {
    float s = 0.f, ex[8];
    for (int j = 0; j < k; ++j) {
      ex[j] = sel_i[j] < 0 ? 0.f : __expf(sel_v[j] - sel_v[0]);
      s += ex[j];
    }
    const float inv = 1.0f / s;
    for (int j = 0; j < k; ++j) {
      ids[j] = sel_i[j];
      wts[j] = ex[j] * inv;
    }
  }
}

}  // namespace bm
