// Decode GEMV building blocks shared by the decode kernels: activation
// operands of one Q2 / Q8_0 unit in registers, the unit loads and dot products,
// and the direct-to-LDS stage copies with their vmcnt waits.
//
// Q2 unit (quarter q of a super-block, h = q/2, p = q%2): the 16 code bytes
// 16 + 32h + 16p .. +15 hold sub-blocks 8h + 2s + p (s = 0..3) at bit 2s.  Codes
// become bf16 pairs with one and-or against 0x43004300 (a bf16 0x43xx is 128 +
// xx for xx < 128): codes at shift 2s read 128 + 4^s q (s = 3 is pre-shifted to
// 16 q).  v_dot2_f32_bf16 against bf16 activation pairs gives sum (128 + F q) x,
// and the sub-block sum of x removes the offset:
//   sum q x = (acc - 128 X) / F,   row += d*sc*(sum q x) - dmin*m*X.
// Bytes 0 and 2 of a code dword form one pair, bytes 1 and 3 (after >> 8) the
// other, so the activation pairs are stored in that order.
#pragma once

#include "common.h"

namespace bm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 __attribute__((aligned(4))) u32x4_a4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 __attribute__((aligned(4))) u32x2_a4;

constexpr uint32_t BF16_128x2 = 0x43004300u;  // two bf16 128.0
constexpr uint32_t BF16_ONEx2 = 0x3F803F80u;  // two bf16 1.0

BM_DEVICE float inv_f(int s) { return s == 0 ? 1.f : (s == 1 ? 0.25f : 0.0625f); }

// first column of Q2 unit (super-block n of the row, quarter q)
BM_DEVICE int q2_c0(int n, int q, int K) { return (256 * n + 128 * (q >> 1) + 16 * (q & 1)) % K; }

// ---- gate/up GEMV: activation operands in registers -----------------------------
// Every lane keeps its unit's operands (x pairs in code-byte order, sub-block
// sums) in registers for all the rows it visits; the weight bytes of up to
// DEPTH row iterations are loaded before any arithmetic.

struct XQ2 {  // one bf16 "virtual token" for one Q2 unit
  uint32_t a[16], b[16];
  float sum[4], c[4];
};



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
    sum = dot2_bf16(hi, BF16_ONEx2, dot2_bf16(lo, BF16_ONEx2, sum));
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
        sum = dot2_bf16(d[i], BF16_ONEx2, sum);
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

struct Q2Unit {  // raw bytes of one lane's quarter super-block
  u32x4 q;
  u32x2 sc;
  uint32_t dd;
};

BM_DEVICE Q2Unit q2_unit_load(const uint8_t *sb, int h, int p) {
  Q2Unit r;
  r.q = *reinterpret_cast<const u32x4_a4 *>(sb + 16 + 32 * h + 16 * p);
  r.sc = *reinterpret_cast<const u32x2_a4 *>(sb + 8 * h);
  r.dd = *reinterpret_cast<const uint32_t *>(sb + 80);
  return r;
}

template <int NV>
BM_DEVICE void q2_unit_dot(const Q2Unit &u, int p, const XQ2 *X, float *out) {
  const float d = half_to_f32(u.dd & 0xFFFFu), dmin = half_to_f32(u.dd >> 16);
  const uint32_t w[4] = {u.q.x, u.q.y, u.q.z, u.q.w};
  const uint32_t sw0 = u.sc.x >> (8 * p), sw1 = u.sc.y >> (8 * p);
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
        A = and_or(w[j], m, BF16_128x2);
        B = and_or(w[j] >> 8, m, BF16_128x2);
      } else {
        A = and_or(w[j] >> 2, 0x00300030u, BF16_128x2);
        B = and_or(w[j] >> 10, 0x00300030u, BF16_128x2);
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

struct Q8Unit {  // raw bytes of one lane's two Q8_0 blocks (68 bytes)
  uint32_t dw[17];
};

BM_DEVICE Q8Unit q8_unit_load(const uint8_t *u68) {
  Q8Unit r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4_a4 *>(u68 + 16 * i);
    r.dw[4 * i] = v.x;
    r.dw[4 * i + 1] = v.y;
    r.dw[4 * i + 2] = v.z;
    r.dw[4 * i + 3] = v.w;
  }
  r.dw[16] = *reinterpret_cast<const uint32_t *>(u68 + 64);
  return r;
}

template <int NV>
BM_DEVICE void q8_unit_dot(const Q8Unit &u, const XQ8 *X, float *out) {
  const float dA = half_to_f32(u.dw[0] & 0xFFFFu), dB = half_to_f32(u.dw[8] >> 16);
  uint32_t ux[17];
#pragma unroll
  for (int i = 0; i < 17; ++i) ux[i] = u.dw[i] ^ 0x80808080u;  // q + 128 as unsigned bytes
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


// copy one stage (STB bytes at src, 16-byte aligned) into LDS at slot
template <int STB, int NI>
BM_DEVICE void stream_issue(uint8_t *slot, const uint8_t *src) {
  const int lane = threadIdx.x & 63;
  const uint32_t base = lds_offset(slot);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if (i * 1024 + lane * 16 < STB) lds_dma16(src + i * 1024 + lane * 16, base + i * 1024);
}

template <int N>
BM_DEVICE void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most `ahead` stages of NI loads each are outstanding
template <int NI, int MAXA>
BM_DEVICE void stream_wait(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) {
      vm_wait<NI * MAXA>();
      return;
    }
    stream_wait<NI, MAXA - 1>(ahead);
  } else {
    vm_wait<0>();
  }
}


}  // namespace bm
