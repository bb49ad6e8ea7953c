// Router: float32 logits, softmax, top-k and renormalisation.
//
// "Strata-DSV4.1", §How it works: the router runs with the dense half on the
// GPU and its result stays there; §DeepSeek-V4.1-Flash: 384 routed experts,
// top-6.  Selection is by logit (softmax is monotone), an exact tie going to
// the lower expert index; the weights are exp(L_j - L_max) / sum over the
// selected experts, which equals the full softmax renormalised over them.
//
// Kernels
//  router_gemv_kernel   T <= 8: one wave per expert row; every lane streams
//                       16-byte slices of the row (coalesced 1 KB per wave
//                       load) and keeps one partial sum per token.  HBM-bound
//                       on the 4 B/weight router matrix.
//  router_tile_kernel   T > 8: 64 tokens x 64 experts per 256-thread block,
//                       K staged through LDS in steps of 32, 4x4 outputs per
//                       thread.
//  topk_kernel          one wave per token: k rounds of a wave-wide
//                       (value, index) argmax over the E logits.
#include "common.h"
#include "internal.h"

namespace bm {

template <bool XBF16>
BM_DEVICE float4 load_x4(const void *x, int64_t idx) {
  if constexpr (XBF16) {
    const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + idx);
    return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
  } else {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + idx);
  }
}

template <bool XBF16>
__global__ void __launch_bounds__(256) router_gemv_kernel(const void *__restrict__ x, int T, int D, int E,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.f;
  const float *row = wr + int64_t(e) * D;
  for (int c = lane * 4; c < D; c += 256) {
    const float4 w = *reinterpret_cast<const float4 *>(row + c);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < T) {
        const float4 v = load_x4<XBF16>(x, int64_t(t) * D + c);
        acc[t] = __builtin_fmaf(w.x, v.x, acc[t]);
        acc[t] = __builtin_fmaf(w.y, v.y, acc[t]);
        acc[t] = __builtin_fmaf(w.z, v.z, acc[t]);
        acc[t] = __builtin_fmaf(w.w, v.w, acc[t]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t < T) {
      const float s = group_sum<64>(acc[t]);
      if (lane == 0) logits[int64_t(t) * E + e] = s + b;
    }
  }
}

template <bool XBF16>
__global__ void __launch_bounds__(256) router_tile_kernel(const void *__restrict__ x, int T, int D, int E,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits) {
  __shared__ float xs[32][65];
  __shared__ float ws[32][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < D; k0 += 32) {
    // 64 rows x 32 columns for each operand: 2048 values, 8 per thread
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = threadIdx.x + r * 256;  // 0..511 -> (row, quad)
      const int row = idx >> 3, q = (idx & 7) * 4;
      float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), wv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t0 + row < T) xv = load_x4<XBF16>(x, int64_t(t0 + row) * D + k0 + q);
      if (e0 + row < E) wv = *reinterpret_cast<const float4 *>(wr + int64_t(e0 + row) * D + k0 + q);
      xs[q + 0][row] = xv.x; xs[q + 1][row] = xv.y; xs[q + 2][row] = xv.z; xs[q + 3][row] = xv.w;
      ws[q + 0][row] = wv.x; ws[q + 1][row] = wv.y; ws[q + 2][row] = wv.z; ws[q + 3][row] = wv.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = xs[kk][ty * 4 + i];
        b[i] = ws[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[int64_t(t) * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
    }
  }
}

// (value, index) "better than": larger value, or equal value and lower index.
BM_DEVICE bool better(float v, int i, float v2, int i2) { return v > v2 || (v == v2 && i < i2); }

// Top-k of one token's logits by one wave; lane 0 writes ids and weights.
BM_DEVICE void topk_token(const float *L, int E, int k, int32_t *ids, float *wts, int lane) {
  constexpr int PER = 16;  // E <= 1024
  float v[PER];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? L[e] : -INFINITY;
  }
  float sel_v[8];
  int sel_i[8];
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi == 0x7FFFFFFF) bi = -1;  // only NaN logits left: no valid expert
    else if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    sel_v[j] = bv;
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

__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                   int32_t *__restrict__ ids, float *__restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token(logits + int64_t(t) * E, E, k, ids + int64_t(t) * k, wts + int64_t(t) * k, threadIdx.x & 63);
}

hipError_t launch_route(const void *x, bool xbf16, int T, int D, int E, int k, const float *wr,
                        const float *bias, float *logits, int32_t *ids, float *wts, hipStream_t stream) {
  if (T <= 8) {
    dim3 grid((E + 3) / 4);
    if (xbf16)
      BM_LAUNCH("router_gemv_kernel", router_gemv_kernel<true>, grid, dim3(256), 0, stream, x, T, D, E, wr, bias, logits);
    else
      BM_LAUNCH("router_gemv_kernel", router_gemv_kernel<false>, grid, dim3(256), 0, stream, x, T, D, E, wr, bias, logits);
  } else {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    if (xbf16)
      BM_LAUNCH("router_tile_kernel", router_tile_kernel<true>, grid, dim3(256), 0, stream, x, T, D, E, wr, bias, logits);
    else
      BM_LAUNCH("router_tile_kernel", router_tile_kernel<false>, grid, dim3(256), 0, stream, x, T, D, E, wr, bias, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  BM_LAUNCH("topk_kernel", topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, ids, wts);
  return hipGetLastError();
}

}  // namespace bm
