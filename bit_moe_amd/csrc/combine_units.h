// The weighted combine of one token's outputs, four consecutive columns per
// thread, shared by the combine launch and the combine + residual launch.
//
// Pages: "Strata-DSV4.1", §How it works (the routed experts' outputs weighted
// by the renormalised router probabilities, plus the shared expert's);
// "Feature Request: support DeepSeek V4.1 Flash with bounded SSD expert
// caching", §Runtime stack progress (one expert-reduction order).
//   out[t][c] = sum_{j = 0..k-1} w[t,j] y[t*k + j][c]  (+ ys[t][c]),
// j in order as float32 FMAs, the shared row added last, rounded once.  A
// slot with an id outside [0, E) or repeating an earlier slot's id adds
// nothing and is recorded in status (by the thread of column 0).
#pragma once
#include <type_traits>

#include "common.h"

namespace bm {

// K = top_k (1 .. 8, a template argument so that exactly K rows are loaded)
template <int K>
BM_DEVICE float4 combine4(const float *__restrict__ y, const float *__restrict__ ys, const int32_t *__restrict__ ids,
                          const float *__restrict__ wts, int t, int c, int D, int E, int64_t *status) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // every load is issued before any use, so their latencies overlap: the
  // pair rows (all in bounds; rows of skipped pairs are never used), the ids,
  // the weights and the shared expert's row
  float4 v[K];
  int idv[K];
  float wv[K];
  const int64_t tk = int64_t(t) * K;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    v[j] = *reinterpret_cast<const float4 *>(y + (tk + j) * D + c);
    idv[j] = ids[tk + j];
    wv[j] = wts[tk + j];
  }
  const float4 vs = ys ? *reinterpret_cast<const float4 *>(ys + int64_t(t) * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int e = idv[j];
    if (e < 0 || e >= E) {
      if (c == 0) record_fault(status, FAULT_BAD_EXPERT, tk + j);
      continue;
    }
    bool dup = false;  // served once, at its first slot
#pragma unroll
    for (int i = 0; i < j; ++i) dup = dup || idv[i] == e;
    if (dup) {
      if (c == 0) record_fault(status, FAULT_DUP_EXPERT, tk + j);
      continue;
    }
    const float w = wv[j];
    acc.x = __builtin_fmaf(w, v[j].x, acc.x);
    acc.y = __builtin_fmaf(w, v[j].y, acc.y);
    acc.z = __builtin_fmaf(w, v[j].z, acc.z);
    acc.w = __builtin_fmaf(w, v[j].w, acc.w);
  }
  if (ys) {
    acc.x += vs.x;
    acc.y += vs.y;
    acc.z += vs.z;
    acc.w += vs.w;
  }
  return acc;
}

// Store four combined columns as bf16 (RNE) or float32; returns the values as
// stored (the bf16 roundings, widened).
// Launch helper: calls body(std::integral_constant<int, k>()) for k in 1 .. 8.
template <typename F>
hipError_t with_top_k(int k, F body) {
  switch (k) {
    case 1: return body(std::integral_constant<int, 1>());
    case 2: return body(std::integral_constant<int, 2>());
    case 3: return body(std::integral_constant<int, 3>());
    case 4: return body(std::integral_constant<int, 4>());
    case 5: return body(std::integral_constant<int, 5>());
    case 6: return body(std::integral_constant<int, 6>());
    case 7: return body(std::integral_constant<int, 7>());
    case 8: return body(std::integral_constant<int, 8>());
    default: return hipErrorInvalidValue;
  }
}

BM_DEVICE float4 store_out4(void *out, int out_bf16, int t, int D, int c, float4 acc) {
  if (out_bf16) {
    const uint2 o = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + int64_t(t) * D + c) = o;
    return make_float4(bf16_lo(o.x), bf16_hi(o.x), bf16_lo(o.y), bf16_hi(o.y));
  }
  *reinterpret_cast<float4 *>(static_cast<float *>(out) + int64_t(t) * D + c) = acc;
  return acc;
}

}  // namespace bm
