// Router: float32 logits, softmax, top-k and renormalisation.
//
// "Strata-DSV4.1", §How it works: the router runs with the dense half on the
// GPU and its result stays there; §DeepSeek-V4.1-Flash: 384 routed experts,
// top-6.  Selection is by logit (softmax is monotone), an exact tie going to
// the lower expert index; the weights are exp(L_j - L_max) / sum over the
// selected experts, which equals the full softmax renormalised over them.
//
// Kernels
//  router_gemv_kernel   T <= 8: one block per expert row; every thread loads
//                       its 16-byte slices of the row at once and keeps one
//                       partial sum per token.  HBM-bound on the 4 B/weight
//                       router matrix.
//  router_split_kernel  T > 8, bf16 x: the float32 router matrix as three bf16
//                       parts (stored in the MFMA operand order) hi = bf16(w), mid = bf16(w - hi), lo =
//                       bf16(w - hi - mid).  Both differences are exact in
//                       float32 and lo is exact in bf16 (w - hi - mid is a
//                       multiple of w's float32 ulp below 2^8 of them), so
//                       hi + mid + lo = w exactly.
//  router_mfma_kernel   T > 8, bf16 x: logits = sum over the three parts of
//                       x W_part^T on v_mfma_f32_16x16x32_bf16 (bf16 x bf16
//                       products are exact in float32): 32 tokens x 64
//                       experts per block, K split over its four waves, K
//                       steps of 32 with the next step's operands loaded
//                       ahead (each weight operand load is 1 KB of
//                       contiguous bytes and feeds two MFMAs).
//  router_tile_kernel   T > 8, float32 x: 64 tokens x 64 experts per
//                       256-thread block, K staged through LDS in steps of
//                       32, 4x4 outputs per thread.
//  topk_kernel          one wave per token: k rounds of a wave-wide
//                       maximum over order-preserving integer keys of the
//                       logits (DPP), ties resolved by ballot.
#include "common.h"
#include "internal.h"
#include "mfma_q2.h"
#include "router_units.h"

#include <type_traits>

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

template <bool XBF16, int NT>
__global__ void __launch_bounds__(256) router_gemv_kernel(const void *__restrict__ x, int T, int D, int E,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits) {
  router_gemv_block<XBF16, NT>(x, T, D, E, wr, bias, logits, blockIdx.x);
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

// Swizzled part layout: for part p, expert tile et (16 experts) and K step
// ks (32 columns) one 1 KB record holding, for MFMA lane l, the 8 columns
// 32 ks + 8 (l / 16) + 0..7 of expert 16 et + l % 16; records ordered
// (p, et, ks).  A wave's operand load of one (p, et, ks) is then 1 KB of
// contiguous bytes.
BM_HOST_DEVICE inline size_t split_index(int p, int e, int k, int n_et, int D) {
  const int et = e >> 4, ks = k >> 5, lane = (e & 15) + 16 * ((k & 31) >> 3);
  return (((size_t(p) * n_et + et) * (D / 32) + ks) * 64 + lane) * 8 + (k & 7);
}

// Thread per 4 consecutive weights of a row (n = E * D, D a multiple of 256).
__global__ void __launch_bounds__(256) router_split_kernel(const float *__restrict__ wr, int E, int D,
                                                           uint16_t *__restrict__ parts) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= int64_t(E) * D) return;
  const int e = int(i / D), k = int(i % D), n_et = (E + 15) / 16;
  const float4 v = *reinterpret_cast<const float4 *>(wr + i);
  const float w[4] = {v.x, v.y, v.z, v.w};
  uint16_t h[4], m[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = f32_to_bf16(w[j]);
    const float r1 = w[j] - bf16_to_f32(h[j]);
    m[j] = f32_to_bf16(r1);
    l[j] = f32_to_bf16(r1 - bf16_to_f32(m[j]));
  }
  const uint16_t *q[3] = {h, m, l};
#pragma unroll
  for (int p = 0; p < 3; ++p)
    *reinterpret_cast<uint2 *>(parts + split_index(p, e, k, n_et, D)) =
        make_uint2(q[p][0] | (uint32_t(q[p][1]) << 16), q[p][2] | (uint32_t(q[p][3]) << 16));
}

// Lane layout of v_mfma_f32_16x16x32_bf16: A lane l holds row l % 16 and k =
// 8 (l / 16) + 0..7, B lane l column l % 16 and the same k, the result lane l
// rows 4 (l / 16) + 0..3 of column l % 16.  A block computes 32 tokens x 64
// experts; its four waves take a quarter of K each (one step's loads in
// flight ahead of its MFMAs), and the partial sums are added in wave order
// through LDS.  Token rows past T read a clamped row, and neither they nor
// experts past E are written.
__global__ void __launch_bounds__(256) router_mfma_kernel(const uint16_t *__restrict__ x, int T, int D, int E,
                                                          const uint16_t *__restrict__ parts,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits) {
  constexpr int MT = 2;                      // 16-token tiles per block (each weight operand feeds MT MFMAs)
  __shared__ float red[4][MT][4][4][64];     // [wave][token tile][expert tile][row r][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16 * MT, e0 = blockIdx.y * 64;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int n_et = (E + 15) / 16, nks = D / 32, nq = nks / 4, ks0 = wave * nq;  // nq is even (D >= 256)
  const uint16_t *xa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xa[mt] = x + size_t(min(t0 + 16 * mt + r16, T - 1)) * D + kq;
  // records of (part 0, expert tile e0/16 + n, step 0), this lane's 8 values
  const uint16_t *wb = parts + (size_t(e0 >> 4) * nks * 64 + lane) * 8;
  const size_t tile_stride = size_t(nks) * 512, part_stride = size_t(n_et) * tile_stride;
  f32x4_t acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[mt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int ks, uint32_t (&a)[MT][4], uint32_t (&b)[4][3][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ld16(xa[mt] + 32 * ks, a[mt]);
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int p = 0; p < 3; ++p) ld16(wb + p * part_stride + n * tile_stride + size_t(ks) * 512, b[n][p]);
  };
  auto mma = [&](const uint32_t (&a)[MT][4], const uint32_t (&b)[4][3][4]) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][n] = mfma16(a[mt], b[n][p], acc[mt][n]);
  };
  // two register sets in turn, the loop unrolled by two so neither is copied
  // (a copy would wait for the load in flight)
  uint32_t A0[MT][4], B0[4][3][4], A1[MT][4], B1[4][3][4];
  load(ks0, A0, B0);
  for (int i = 0; i < nq; i += 2) {
    load(ks0 + i + 1, A1, B1);
    mma(A0, B0);
    if (i + 2 < nq) load(ks0 + i + 2, A0, B0);
    mma(A1, B1);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][mt][n][r][lane] = acc[mt][n][r];
  __syncthreads();
  // wave w finishes expert tile w of every token tile
  const int e = e0 + 16 * wave + r16;
  if (e >= E) return;
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * mt + 4 * (lane >> 4) + r;
      const float v = ((red[0][mt][wave][r][lane] + red[1][mt][wave][r][lane]) + red[2][mt][wave][r][lane]) +
                      red[3][mt][wave][r][lane];
      if (t < T) logits[int64_t(t) * E + e] = v + b;
    }
}

size_t router_split_bytes(int E, int D) { return size_t(3) * ((E + 63) / 64 * 64) * D * 2; }

// Router logits for T tokens (wsplit: router_split_bytes(E, D) of scratch for
// the swizzled bf16 parts, used for T > 8 with bf16 x).
static hipError_t launch_logits(const void *x, bool xbf16, int T, int D, int E, const float *wr, const float *bias,
                                float *logits, uint16_t *wsplit, hipStream_t stream);

hipError_t launch_route_logits(const void *x, bool xbf16, int T, int D, int E, const float *wr, const float *bias,
                               float *logits, hipStream_t stream) {
  if (T > 8) return hipErrorNotSupported;
  return launch_logits(x, xbf16, T, D, E, wr, bias, logits, nullptr, stream);
}

static hipError_t launch_logits(const void *x, bool xbf16, int T, int D, int E, const float *wr, const float *bias,
                                float *logits, uint16_t *wsplit, hipStream_t stream) {
  if (T <= 8) {
    // token slots per block: the smallest of 1, 2, 4, 8 that holds T
#define BM_ROUTER_GEMV(XB, NT)                                                                                   \
  BM_LAUNCH("router_gemv_kernel", (router_gemv_kernel<XB, NT>), dim3(E), dim3(256), 0, stream, x, T, D, E, wr, bias, \
            logits)
    if (xbf16) {
      if (T == 1) BM_ROUTER_GEMV(true, 1);
      else if (T == 2) BM_ROUTER_GEMV(true, 2);
      else if (T <= 4) BM_ROUTER_GEMV(true, 4);
      else BM_ROUTER_GEMV(true, 8);
    } else {
      if (T == 1) BM_ROUTER_GEMV(false, 1);
      else if (T == 2) BM_ROUTER_GEMV(false, 2);
      else if (T <= 4) BM_ROUTER_GEMV(false, 4);
      else BM_ROUTER_GEMV(false, 8);
    }
#undef BM_ROUTER_GEMV
  } else if (xbf16 && wsplit) {
    const int64_t n = int64_t(E) * D;  // a multiple of 256 (D is)
    BM_LAUNCH("router_split_kernel", router_split_kernel, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0, stream,
              wr, E, D, wsplit);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid((T + 31) / 32, (E + 63) / 64);
    BM_LAUNCH("router_mfma_kernel", router_mfma_kernel, grid, dim3(256), 0, stream,
              static_cast<const uint16_t *>(x), T, D, E, wsplit, bias, logits);
  } else {
    const dim3 grid((T + 63) / 64, (E + 63) / 64);
    if (xbf16)
      BM_LAUNCH("router_tile_kernel", router_tile_kernel<true>, grid, dim3(256), 0, stream, x, T, D, E, wr, bias,
                logits);
    else
      BM_LAUNCH("router_tile_kernel", router_tile_kernel<false>, grid, dim3(256), 0, stream, x, T, D, E, wr, bias,
                logits);
  }
  return hipGetLastError();
}

template <int PER>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                   int32_t *__restrict__ ids, float *__restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<PER>(logits + int64_t(t) * E, E, k, ids + int64_t(t) * k, wts + int64_t(t) * k, threadIdx.x & 63);
}

// ---- router variants ----------------------------------------------------------
// Scores s_e = softmax(L)_e or sqrt(softplus(L_e)); the selection is either
// the rows of a hash-routed layer's token table or the top-k of s + b (b a
// selection-only bias; tie -> lower index); the weights are the unbiased
// scores of the selected experts over their sum.  One wave per token.

// value held in slot `slot` of lane `src` (both wave-uniform)
template <int PER>
BM_DEVICE float slot_value(const float (&v)[PER], int src, int slot) {
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (i == slot) r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), src));
  return r;
}

BM_DEVICE float wave_max_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int PER>
BM_DEVICE void topk_variant_token(const float *L, int E, int k, int score, const float *sbias, const int32_t *hrow,
                                  int32_t *ids, float *wts, int64_t *status, int64_t pair0, int lane) {
  float sc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sc[i] = L[min(lane + 64 * i, E - 1)];  // every load issued before any use
#pragma unroll
  for (int i = 0; i < PER; ++i) sc[i] = lane + 64 * i < E ? sc[i] : -INFINITY;
  if (score == 0) {  // softmax over the E logits
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) m = fmaxf(m, sc[i]);
    m = wave_max_f(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      sc[i] = lane + 64 * i < E ? __expf(sc[i] - m) : 0.f;
      z += sc[i];
    }
    const float inv = 1.0f / wave_sum(z);
#pragma unroll
    for (int i = 0; i < PER; ++i) sc[i] *= inv;
  } else {  // sqrt(softplus(L)), softplus(v) = max(v, 0) + log1p(e^-|v|)
#pragma unroll
    for (int i = 0; i < PER; ++i)
      sc[i] = lane + 64 * i < E ? sqrtf(fmaxf(sc[i], 0.f) + log1pf(__expf(-fabsf(sc[i])))) : 0.f;
  }
  int sel[8];
  if (hrow) {
    for (int j = 0; j < k; ++j) sel[j] = hrow[j];
  } else {
    uint32_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      key[i] = e < E ? logit_key(sc[i] + (sbias ? sbias[e] : 0.f)) : 0u;
    }
    for (int j = 0; j < k; ++j) {
      uint32_t mk = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) mk = max(mk, key[i]);
      const uint32_t M = wave_max_u32(mk);
      int bi = -1;  // only NaN scores left: no valid expert
      if (M != 0u) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const uint64_t hit = __ballot(key[i] == M);
          if (hit) {
            const int l = __builtin_ctzll(hit);
            bi = l + 64 * i;
            if (lane == l) key[i] = 0u;
            break;
          }
        }
      }
      sel[j] = bi;
    }
  }
  // unbiased scores of the selection, renormalised
  // (a table row may name an expert outside [0, E) or repeat one: such slots
  // get weight 0 and are recorded; the top-k selection never does either)
  float g[8], gs = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = sel[j];
    const bool ok = e >= 0 && e < E;
    bool dup = false;
    for (int i = 0; i < j; ++i) dup = dup || (ok && sel[i] == e);
    g[j] = ok && !dup ? slot_value<PER>(sc, e & 63, e >> 6) : 0.f;
    gs += g[j];
    if (hrow && lane == 0) {
      if (!ok) record_fault(status, FAULT_BAD_EXPERT, pair0 + j);
      else if (dup) record_fault(status, FAULT_DUP_EXPERT, pair0 + j);
    }
  }
  if (lane == 0) {
    const float inv = gs > 0.f ? 1.0f / gs : 0.f;
    for (int j = 0; j < k; ++j) {
      ids[j] = sel[j];
      wts[j] = g[j] * inv;
    }
  }
}

template <int PER>
__global__ void __launch_bounds__(256) topk_variant_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                           int score, const float *__restrict__ sbias,
                                                           const int32_t *__restrict__ htab,
                                                           const int32_t *__restrict__ tok, int64_t vocab,
                                                           int32_t *__restrict__ ids, float *__restrict__ wts,
                                                           int64_t *status) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int32_t *hrow = nullptr;
  if (htab) {
    const int64_t id = tok[t];
    if (id < 0 || id >= vocab) {  // no table row: the token routes nowhere
      if (lane < k) {
        ids[int64_t(t) * k + lane] = -1;
        wts[int64_t(t) * k + lane] = 0.f;
      }
      if (lane == 0) record_fault(status, FAULT_BAD_TOKEN, t);
      return;
    }
    hrow = htab + id * k;
  }
  topk_variant_token<PER>(logits + int64_t(t) * E, E, k, score, sbias, hrow, ids + int64_t(t) * k,
                          wts + int64_t(t) * k, status, int64_t(t) * k, lane);
}

hipError_t launch_route_variant(const void *x, bool xbf16, int T, int D, int E, int k, const float *wr,
                                const float *logit_bias, int score, const float *select_bias,
                                const int32_t *hash_table, const int32_t *token_ids, int64_t vocab, float *logits,
                                int32_t *ids, float *wts, int64_t *status, uint16_t *wsplit,
                                hipStream_t stream) {
  hipError_t err = launch_logits(x, xbf16, T, D, E, wr, logit_bias, logits, wsplit, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((T + 3) / 4), block(T == 1 ? 64 : 256);
  if (E <= 6 * 64)
    BM_LAUNCH("topk_variant_kernel", topk_variant_kernel<6>, grid, block, 0, stream, logits, T, E, k, score,
              select_bias, hash_table, token_ids, vocab, ids, wts, status);
  else
    BM_LAUNCH("topk_variant_kernel", topk_variant_kernel<16>, grid, block, 0, stream, logits, T, E, k, score,
              select_bias, hash_table, token_ids, vocab, ids, wts, status);
  return hipGetLastError();
}

hipError_t launch_route(const void *x, bool xbf16, int T, int D, int E, int k, const float *wr,
                        const float *bias, float *logits, int32_t *ids, float *wts, uint16_t *wsplit,
                        hipStream_t stream) {
  hipError_t err = launch_logits(x, xbf16, T, D, E, wr, bias, logits, wsplit, stream);
  if (err != hipSuccess) return err;
  // blocks of 4 waves for T > 1; a single wave for one token
  const dim3 grid((T + 3) / 4), block(T == 1 ? 64 : 256);
  if (E <= 6 * 64)
    BM_LAUNCH("topk_kernel", topk_kernel<6>, grid, block, 0, stream, logits, T, E, k, ids, wts);
  else
    BM_LAUNCH("topk_kernel", topk_kernel<16>, grid, block, 0, stream, logits, T, E, k, ids, wts);
  return hipGetLastError();
}

}  // namespace bm
