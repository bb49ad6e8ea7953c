// Decode path: dequant-fused GEMV over the union of selected experts, the
// Q8_0 shared expert, and the fixed-order weighted combine.
//
// Pages: "Strata-DSV4.1", §How it works (expert tier, shared expert + routed
// sum) and §Latest (10-14) (a verify pass serves the union of its experts once
// per layer); "Feature Request: support DeepSeek V4.1 Flash with bounded SSD
// expert caching", §Runtime stack progress (a single expert-reduction order);
// "run the DeepSeek-V4-Flash-Vision tower on CUDA", commit notes (SwiGLU: the
// gate half is the SiLU operand).
//
// Kernels (one wave = 64 lanes; a "unit" is 64 weights of one row):
//  ffn_gateup_kernel  routed jobs: (union slot, chunk of rows); shared jobs:
//                     chunk of rows of the Q8_0 shared gate/up.  Every lane
//                     owns one unit per row and keeps its tokens' activations
//                     in registers; h = silu(Wg x) * (Wu x) is stored as a
//                     bf16 hi + lo pair (h - hi is exact in float32).
//  ffn_down_kernel    same shape over the down matrices, y = Wd h in float32
//                     per (token, slot) pair and per token for the shared one;
//                     the hi and lo parts of h are two bf16 operand streams.
//  combine_kernel     out[t] = sum_j w[t,j] y[t,j] + y_shared[t], j in order,
//                     rounded once.
//
// Q2 unit (quarter q of a super-block, h = q/2, p = q%2): the 16 code bytes
// 16 + 32h + 16p .. +15 hold sub-blocks 8h + 2s + p (s = 0..3) at bit 2s.  Codes
// are turned into bf16 pairs by one and-or with 0x43004300 (a bf16 0x43xx is
// 128 + xx for xx < 128): codes at shift 2s read 128 + 4^s q (s = 3 is
// pre-shifted to 16 q).  v_dot2_f32_bf16 against bf16 activation pairs gives
// sum (128 + F q) x, and the sub-block's sum of x removes the offset:
//   sum q x = (acc - 128 X) / F,   row += d*sc*(sum q x) - dmin*m*X.
// Bytes 0 and 2 of a code dword form one pair, bytes 1 and 3 (after >> 8) the
// other, so the activation pairs are stored in that order.
#include "common.h"
#include "internal.h"

#include <type_traits>

namespace bm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 __attribute__((aligned(4))) u32x4_a4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 __attribute__((aligned(4))) u32x2_a4;

constexpr int NTOK = 4;  // tokens held in registers per pass

// ---- activation operands ----------------------------------------------------

struct XQ2 {  // one bf16 "virtual token" for one Q2 unit
  uint32_t a[16], b[16];
  float sum[4], c[4];
};

BM_DEVICE float inv_f(int s) { return s == 0 ? 1.f : (s == 1 ? 0.25f : 0.0625f); }

BM_DEVICE void xq2_finish(XQ2 &X) {
#pragma unroll
  for (int s = 0; s < 4; ++s) X.c[s] = -128.f * inv_f(s) * X.sum[s];
}

BM_DEVICE void xq2_from_words(XQ2 &X, int s, const uint32_t (&d)[8]) {
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = d[2 * j], hi = d[2 * j + 1];
    X.a[4 * s + j] = (lo & 0xFFFFu) | (hi << 16);
    X.b[4 * s + j] = (lo >> 16) | (hi & 0xFFFF0000u);
    sum += (bf16_lo(lo) + bf16_hi(lo)) + (bf16_lo(hi) + bf16_hi(hi));
  }
  X.sum[s] = sum;
}

// bf16 activations: 16 contiguous values at row + c0 + 32 s
BM_DEVICE void load_xq2_bf16(const uint16_t *row, int c0, XQ2 &X) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 *p = reinterpret_cast<const uint4 *>(row + c0 + 32 * s);
    const uint4 v0 = p[0], v1 = p[1];
    const uint32_t d[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    xq2_from_words(X, s, d);
  }
  xq2_finish(X);
}

// float32 activations: split exactly enough into bf16 hi + bf16 lo parts
// (x - hi is exact in float32), two virtual tokens whose results are summed.
BM_DEVICE void load_xq2_f32(const float *row, int c0, XQ2 &Xh, XQ2 &Xl) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float4 *p = reinterpret_cast<const float4 *>(row + c0 + 32 * s);
    uint32_t dh[8], dl[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = p[q];
      const float f[4] = {v.x, v.y, v.z, v.w};
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = f32_to_bf16(f[i]);
        lb[i] = f32_to_bf16(f[i] - bf16_to_f32(uint16_t(hb[i])));
      }
      dh[2 * q] = hb[0] | (hb[1] << 16);
      dh[2 * q + 1] = hb[2] | (hb[3] << 16);
      dl[2 * q] = lb[0] | (lb[1] << 16);
      dl[2 * q + 1] = lb[2] | (lb[3] << 16);
    }
    xq2_from_words(Xh, s, dh);
    xq2_from_words(Xl, s, dl);
  }
  xq2_finish(Xh);
  xq2_finish(Xl);
}

struct XQ8 {  // one bf16 virtual token for one Q8_0 unit (two 32-weight blocks)
  uint32_t p[32];
  float c[2];
};

BM_DEVICE void load_xq8_bf16(const uint16_t *row, int c0, XQ8 &X) {
  const uint4 *p = reinterpret_cast<const uint4 *>(row + c0);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = p[4 * b + q];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        X.p[16 * b + 4 * q + i] = d[i];
        sum += bf16_lo(d[i]) + bf16_hi(d[i]);
      }
    }
    X.c[b] = -128.f * sum;
  }
}

BM_DEVICE void load_xq8_f32(const float *row, int c0, XQ8 &Xh, XQ8 &Xl) {
  const float4 *p = reinterpret_cast<const float4 *>(row + c0);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float sh = 0.f, sl = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = p[8 * b + q];
      const float f[4] = {v.x, v.y, v.z, v.w};
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = f32_to_bf16(f[i]);
        const float hf = bf16_to_f32(uint16_t(hb[i]));
        lb[i] = f32_to_bf16(f[i] - hf);
        sh += hf;
        sl += bf16_to_f32(uint16_t(lb[i]));
      }
      Xh.p[16 * b + 2 * q] = hb[0] | (hb[1] << 16);
      Xh.p[16 * b + 2 * q + 1] = hb[2] | (hb[3] << 16);
      Xl.p[16 * b + 2 * q] = lb[0] | (lb[1] << 16);
      Xl.p[16 * b + 2 * q + 1] = lb[2] | (lb[3] << 16);
    }
    Xh.c[b] = -128.f * sh;
    Xl.c[b] = -128.f * sl;
  }
}

// ---- one row unit against NV virtual tokens ----------------------------------

template <int NV>
BM_DEVICE void q2_unit_dot(const uint8_t *sb, int h, int p, const XQ2 *X, float *out) {
  const u32x4 q = *reinterpret_cast<const u32x4_a4 *>(sb + 16 + 32 * h + 16 * p);
  const u32x2 sc = *reinterpret_cast<const u32x2_a4 *>(sb + 8 * h);
  const uint32_t dd = *reinterpret_cast<const uint32_t *>(sb + 80);
  const float d = half_to_f32(dd & 0xFFFFu), dmin = half_to_f32(dd >> 16);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  const uint32_t sw0 = sc.x >> (8 * p), sw1 = sc.y >> (8 * p);
  float yd[NV], ym[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) yd[v] = ym[v] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t sbyte = ((s < 2 ? sw0 : sw1) >> (16 * (s & 1))) & 0xFFu;
    const float scf = float(sbyte & 15u), mf = float(sbyte >> 4);
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t A, B;
      if (s < 3) {
        const uint32_t m = 0x00030003u << (2 * s);
        A = (w[j] & m) | 0x43004300u;
        B = ((w[j] >> 8) & m) | 0x43004300u;
      } else {
        A = ((w[j] >> 2) & 0x00300030u) | 0x43004300u;
        B = ((w[j] >> 10) & 0x00300030u) | 0x43004300u;
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        acc[v] = dot2_bf16(A, X[v].a[4 * s + j], acc[v]);
        acc[v] = dot2_bf16(B, X[v].b[4 * s + j], acc[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float qx = __builtin_fmaf(acc[v], inv_f(s), X[v].c[s]);
      yd[v] = __builtin_fmaf(scf, qx, yd[v]);
      ym[v] = __builtin_fmaf(mf, X[v].sum[s], ym[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) out[v] += d * yd[v] - dmin * ym[v];
}

template <int NV>
BM_DEVICE void q8_unit_dot(const uint8_t *u68, const XQ8 *X, float *out) {
  const u32x4 *p4 = reinterpret_cast<const u32x4 *>(u68);
  uint32_t dw[17];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4_a4 *>(u68 + 16 * i);
    dw[4 * i] = v.x;
    dw[4 * i + 1] = v.y;
    dw[4 * i + 2] = v.z;
    dw[4 * i + 3] = v.w;
  }
  (void)p4;
  dw[16] = *reinterpret_cast<const uint32_t *>(u68 + 64);
  const float dA = half_to_f32(dw[0] & 0xFFFFu), dB = half_to_f32(dw[8] >> 16);
  uint32_t ux[17];
#pragma unroll
  for (int i = 0; i < 17; ++i) ux[i] = dw[i] ^ 0x80808080u;  // q + 128 as unsigned bytes
  float acc[2][NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[0][v] = acc[1][v] = 0.f;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const int byte0 = (b ? 36 : 2) + i;  // byte offset of q_i inside the 68-byte unit
      const int byte1 = byte0 + 1;
      const float f0 = float((ux[byte0 >> 2] >> (8 * (byte0 & 3))) & 0xFFu);
      const float f1 = float((ux[byte1 >> 2] >> (8 * (byte1 & 3))) & 0xFFu);
      const uint32_t pr = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[b][v] = dot2_bf16(pr, X[v].p[16 * b + i / 2], acc[b][v]);
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) out[v] += dA * (acc[0][v] + X[v].c[0]) + dB * (acc[1][v] + X[v].c[1]);
}

// ---- job bookkeeping -------------------------------------------------------


struct Job {
  int e;         // expert (-1: shared)
  int n;         // tokens (pairs) of the job
  int tok[64];   // token index
  int pair[64];  // pair index t*k + j (routed)
};

// Block prologue: find the expert of routed slot `slot` (ascending union of
// the valid ids) and its pairs, into LDS.  Returns false when the slot is past
// the union.  Needs T*k <= blockDim.x.
BM_DEVICE bool routed_job(const FfnArgs &a, int slot, Job &job, int *s_bits) {
  const int P = a.T * a.k;
  const int nwords = (a.E + 31) >> 5;
  for (int i = threadIdx.x; i < nwords; i += blockDim.x) s_bits[i] = 0;
  __syncthreads();
  if (threadIdx.x < P) {
    const int e = a.ids[threadIdx.x];
    if (e >= 0 && e < a.E) atomicOr(reinterpret_cast<unsigned *>(&s_bits[e >> 5]), 1u << (e & 31));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int e = -1, seen = 0;
    for (int wd = 0; wd < nwords && e < 0; ++wd) {
      const unsigned bits = unsigned(s_bits[wd]);
      const int c = __builtin_popcount(bits);
      if (seen + c > slot) {
        unsigned b = bits;
        for (int r = slot - seen; r > 0; --r) b &= b - 1;
        e = (wd << 5) + __builtin_ctz(b);
      }
      seen += c;
    }
    job.e = e;
    job.n = 0;
    if (e >= 0)
      for (int p = 0; p < P; ++p)
        if (a.ids[p] == e) {
          job.tok[job.n] = p / a.k;
          job.pair[job.n] = p;
          ++job.n;
        }
  }
  __syncthreads();
  return job.e >= 0;
}

BM_DEVICE void shared_job(const FfnArgs &a, Job &job) {
  if (threadIdx.x == 0) {
    job.e = -1;
    job.n = a.T;
  }
  for (int t = threadIdx.x; t < a.T; t += blockDim.x) job.tok[t] = t;
  __syncthreads();
}

BM_DEVICE int q2_c0(int n, int q, int K) { return (256 * n + 128 * (q >> 1) + 16 * (q & 1)) % K; }

// ---- gate/up ----------------------------------------------------------------

// Rows [r_begin, r_end) of one job for tokens t0 .. t0+nt-1 of the job.
// IS_Q8: shared expert (Q8_0) instead of a routed expert (Q2).
template <int NT, bool XF32, bool IS_Q8>
BM_DEVICE void gateup_rows(const FfnArgs &a, const Job &job, int t0, int nt, int r_begin, int r_end) {
  constexpr int NV = XF32 ? 2 * NT : NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.D, LPR = K / 64, RPI = 64 / LPR;
  const int jj = lane % LPR, rsub = lane / LPR;
  // the lane's columns do not depend on the row: K is a multiple of 128
  const int c0 = IS_Q8 ? jj * 64 : q2_c0(jj >> 2, jj & 3, K);
  typename std::conditional<IS_Q8, XQ8, XQ2>::type X[NV];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = job.tok[t0 + min(i, nt - 1)];
    if constexpr (IS_Q8) {
      if constexpr (XF32)
        load_xq8_f32(static_cast<const float *>(a.x) + size_t(t) * K, c0, X[2 * i], X[2 * i + 1]);
      else
        load_xq8_bf16(static_cast<const uint16_t *>(a.x) + size_t(t) * K, c0, X[i]);
    } else {
      if constexpr (XF32)
        load_xq2_f32(static_cast<const float *>(a.x) + size_t(t) * K, c0, X[2 * i], X[2 * i + 1]);
      else
        load_xq2_bf16(static_cast<const uint16_t *>(a.x) + size_t(t) * K, c0, X[i]);
    }
  }
  const size_t mat_bytes_q2 = size_t(a.F) * a.D / 256 * 84;
  for (int it = wave; it * RPI < r_end - r_begin; it += 4) {
    const int r = r_begin + it * RPI + rsub;
    const bool active = r < r_end;
    const int rr = active ? r : r_begin;
    float g[NV], u[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) g[v] = u[v] = 0.f;
    const int unit = rr * LPR + jj;
    if constexpr (IS_Q8) {
      q8_unit_dot<NV>(a.sg + size_t(unit) * 68, X, g);
      q8_unit_dot<NV>(a.su + size_t(unit) * 68, X, u);
    } else {
      const int n = unit >> 2, q = unit & 3;
      q2_unit_dot<NV>(a.wg + size_t(job.e) * mat_bytes_q2 + size_t(n) * 84, q >> 1, q & 1, X, g);
      q2_unit_dot<NV>(a.wu + size_t(job.e) * mat_bytes_q2 + size_t(n) * 84, q >> 1, q & 1, X, u);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float gs, us;
      if constexpr (XF32) {
        gs = g[2 * i] + g[2 * i + 1];
        us = u[2 * i] + u[2 * i + 1];
      } else {
        gs = g[i];
        us = u[i];
      }
      for (int o = LPR / 2; o > 0; o >>= 1) {  // sum over the LPR lanes of the row
        gs += __shfl_xor(gs, o);
        us += __shfl_xor(us, o);
      }
      if (active && jj == 0 && i < nt) {
        const float hf = silu(gs) * us;
        const uint16_t hv = f32_to_bf16(hf);
        const size_t o = IS_Q8 ? size_t(job.tok[t0 + i]) * a.F + r : size_t(job.pair[t0 + i]) * a.F + r;
        // h travels as bf16 hi + lo parts (16 significant bits): a single bf16
        // rounding of h would dominate the layer's output error
        (IS_Q8 ? a.hs : a.h)[o] = hv;
        (IS_Q8 ? a.hs_lo : a.h_lo)[o] = f32_to_bf16(hf - bf16_to_f32(hv));
      }
    }
  }
}

template <int NT, bool XF32>
__global__ void __launch_bounds__(256) ffn_gateup_kernel(FfnArgs a) {
  __shared__ int s_bits[32];
  __shared__ Job job;
  const int n_routed_blocks = a.u_max * a.chunks_gu;
  const bool shared = int(blockIdx.x) >= n_routed_blocks;
  int chunk;
  if (!shared) {
    if (!routed_job(a, blockIdx.x / a.chunks_gu, job, s_bits)) return;
    chunk = blockIdx.x % a.chunks_gu;
  } else {
    shared_job(a, job);
    chunk = blockIdx.x - n_routed_blocks;
  }
  const int r_begin = chunk * a.rows_gu, r_end = min(a.F, r_begin + a.rows_gu);
  for (int t0 = 0; t0 < job.n; t0 += NT) {
    const int nt = min(NT, job.n - t0);
    if (shared)
      gateup_rows<NT, XF32, true>(a, job, t0, nt, r_begin, r_end);
    else
      gateup_rows<NT, XF32, false>(a, job, t0, nt, r_begin, r_end);
  }
}

// ---- down -------------------------------------------------------------------

template <int NT, bool IS_Q8>
BM_DEVICE void down_rows(const FfnArgs &a, const Job &job, int t0, int nt, int r_begin, int r_end) {
  constexpr bool XF32 = true;  // h always arrives as hi + lo parts
  constexpr int NV = 2 * NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.F, LPR = K / 64, RPI = 64 / LPR;
  const int jj = lane % LPR, rsub = lane / LPR;
  const int c0 = IS_Q8 ? jj * 64 : q2_c0(jj >> 2, jj & 3, K);
  typename std::conditional<IS_Q8, XQ8, XQ2>::type X[NV];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const size_t row = IS_Q8 ? size_t(job.tok[t0 + min(i, nt - 1)]) : size_t(job.pair[t0 + min(i, nt - 1)]);
    const uint16_t *hi = (IS_Q8 ? a.hs : a.h) + row * K;
    const uint16_t *lo = (IS_Q8 ? a.hs_lo : a.h_lo) + row * K;
    if constexpr (IS_Q8) {
      load_xq8_bf16(hi, c0, X[XF32 ? 2 * i : i]);
      if constexpr (XF32) load_xq8_bf16(lo, c0, X[2 * i + 1]);
    } else {
      load_xq2_bf16(hi, c0, X[XF32 ? 2 * i : i]);
      if constexpr (XF32) load_xq2_bf16(lo, c0, X[2 * i + 1]);
    }
  }
  const size_t mat_bytes_q2 = size_t(a.F) * a.D / 256 * 84;
  for (int it = wave; it * RPI < r_end - r_begin; it += 4) {
    const int r = r_begin + it * RPI + rsub;
    const bool active = r < r_end;
    const int rr = active ? r : r_begin;
    float y[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) y[v] = 0.f;
    const int unit = rr * LPR + jj;
    if constexpr (IS_Q8) {
      q8_unit_dot<NV>(a.sd + size_t(unit) * 68, X, y);
    } else {
      const int n = unit >> 2, q = unit & 3;
      q2_unit_dot<NV>(a.wd + size_t(job.e) * mat_bytes_q2 + size_t(n) * 84, q >> 1, q & 1, X, y);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float ys = XF32 ? y[2 * i] + y[2 * i + 1] : y[i];
      for (int o = LPR / 2; o > 0; o >>= 1) ys += __shfl_xor(ys, o);
      if (active && jj == 0 && i < nt) {
        if constexpr (IS_Q8)
          a.ys[size_t(job.tok[t0 + i]) * a.D + r] = ys;
        else
          a.y[size_t(job.pair[t0 + i]) * a.D + r] = ys;
      }
    }
  }
}

template <int NT>
__global__ void __launch_bounds__(256) ffn_down_kernel(FfnArgs a) {
  __shared__ int s_bits[32];
  __shared__ Job job;
  const int n_routed_blocks = a.u_max * a.chunks_dn;
  const bool shared = int(blockIdx.x) >= n_routed_blocks;
  int chunk;
  if (!shared) {
    if (!routed_job(a, blockIdx.x / a.chunks_dn, job, s_bits)) return;
    chunk = blockIdx.x % a.chunks_dn;
  } else {
    shared_job(a, job);
    chunk = blockIdx.x - n_routed_blocks;
  }
  const int r_begin = chunk * a.rows_dn, r_end = min(a.D, r_begin + a.rows_dn);
  for (int t0 = 0; t0 < job.n; t0 += NT) {
    const int nt = min(NT, job.n - t0);
    if (shared)
      down_rows<NT, true>(a, job, t0, nt, r_begin, r_end);
    else
      down_rows<NT, false>(a, job, t0, nt, r_begin, r_end);
  }
}

// ---- combine ----------------------------------------------------------------
// y is indexed by pair; pairs whose id is out of range contribute nothing.

__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ y, const float *__restrict__ ys,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ wts, int T, int k, int D, int E,
                                                      void *out, int out_bf16, int64_t *status) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;  // one thread per 4 outputs
  const int64_t per_tok = D / 4;
  if (idx >= int64_t(T) * per_tok) return;
  const int t = int(idx / per_tok);
  const int c = int(idx % per_tok) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    if (e < 0 || e >= E) {
      if (c == 0) record_fault(status, 1, int64_t(t) * k + j);
      continue;
    }
    const float w = wts[t * k + j];
    const float4 v = *reinterpret_cast<const float4 *>(y + (int64_t(t) * k + j) * D + c);
    acc.x = __builtin_fmaf(w, v.x, acc.x);
    acc.y = __builtin_fmaf(w, v.y, acc.y);
    acc.z = __builtin_fmaf(w, v.z, acc.z);
    acc.w = __builtin_fmaf(w, v.w, acc.w);
  }
  if (ys) {
    const float4 v = *reinterpret_cast<const float4 *>(ys + int64_t(t) * D + c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (out_bf16) {
    uint2 o = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + int64_t(t) * D + c) = o;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(out) + int64_t(t) * D + c) = acc;
  }
}

// ---- launch -----------------------------------------------------------------

template <int NT_GU, int NT_DN>
static hipError_t launch_decode_nt(const FfnArgs &a, bool xf32, hipStream_t stream) {
  const int shared_gu = a.sg ? a.chunks_gu : 0;
  const int shared_dn = a.sd ? a.chunks_dn : 0;
  dim3 g1(a.u_max * a.chunks_gu + shared_gu), g2(a.u_max * a.chunks_dn + shared_dn);
  if (xf32)
    BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_kernel<NT_GU, true>), g1, dim3(256), 0, stream, a);
  else
    BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_kernel<NT_GU, false>), g1, dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  BM_LAUNCH("ffn_down_kernel", (ffn_down_kernel<NT_DN>), g2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_ffn(FfnArgs a, bool xf32, hipStream_t stream) {
  // rows per block: 16 row-iterations of a wave at 64/LPR rows each
  const int rpi_gu = 64 / (a.D / 64), rpi_dn = 64 / (a.F / 64);
  a.rows_gu = min(a.F, 16 * rpi_gu);
  a.rows_dn = min(a.D, 16 * rpi_dn);
  a.chunks_gu = (a.F + a.rows_gu - 1) / a.rows_gu;
  a.chunks_dn = (a.D + a.rows_dn - 1) / a.rows_dn;
  a.u_max = min(a.E, a.T * a.k);
  // tokens held in registers per pass (a job's tokens beyond that take more passes)
  hipError_t err;
  if (a.T == 1)
    err = launch_decode_nt<1, 1>(a, xf32, stream);
  else if (a.T == 2 || xf32)
    err = launch_decode_nt<2, 2>(a, xf32, stream);
  else
    err = launch_decode_nt<NTOK, 2>(a, xf32, stream);
  if (err != hipSuccess) return err;
  return launch_combine(a.y, a.sd ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        stream);
}

hipError_t launch_combine(const float *y, const float *ys, const int32_t *ids, const float *wts, int T, int k, int D,
                          int E, void *out, int out_bf16, int64_t *status, hipStream_t stream) {
  const int64_t n4 = int64_t(T) * (D / 4);
  BM_LAUNCH("combine_kernel", combine_kernel, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, stream, y, ys, ids, wts,
            T, k, D, E, out, out_bf16, status);
  return hipGetLastError();
}

}  // namespace bm
