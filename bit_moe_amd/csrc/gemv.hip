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
//  ffn_stream_kernel  (T >= 2) either half over one-wave blocks that stream
//                     their chunk of rows through an LDS ring with coalesced
//                     direct-to-LDS loads (details at the kernel).
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

#include <algorithm>
#include <type_traits>

#include "combine_units.h"
#include "decode_job.h"
#include "gemv_units.h"
#include "router_units.h"

namespace bm {


constexpr int NTOK = 4;  // tokens per pass of a job

// ---- GEMV: weights and activation operands staged in LDS ---------------------
// A block owns one job (a routed expert of the union, or the shared expert)
// and a chunk of consecutive weight rows.  Its 256 threads copy the chunk's
// bytes (contiguous in HBM) into LDS with 16-byte direct-to-LDS loads, fully
// coalesced, while they build the activation operands of the job's tokens in
// LDS once for the whole block.  Each wave then computes rows from LDS: lane
// jj = lane % LPR owns unit jj (64 weights) of every row it visits, LPR lanes
// per row, RPI = 64 / LPR rows per wave iteration.


// Activation operands in LDS, groups of four dwords XL[(t * XG + g) * LPR + jj]
// for token t of the pass and lane slot jj; PARTS bf16 parts add up to the
// activations (1: bf16 x; 2: hi + lo of float32 x or of h) and multiply the
// same weight operand into the same accumulator.
//   Q2 unit: g = 8 part + s      a[part][4s .. 4s+3]  pairs of code bytes 0, 2
//            g = 8 part + 4 + s  b[part][4s .. 4s+3]  pairs of code bytes 1, 3
//            g = 8 PARTS         X_0 .. X_3 (sub-block sums over all parts)
//            g = 8 PARTS + 1     c_s = -128 X_s / F_s,  F_s = 1, 4, 16, 16
//   Q8_0 unit (two blocks): g = 8 part + i  pairs 4i .. 4i+3 in order;
//            g = 8 PARTS: (-128 * block-0 sum, -128 * block-1 sum)
template <int PARTS>
constexpr int xgroups() { return 8 * PARTS + 2; }

// 8 floats at p -> bf16 hi words and lo words (lo = v - hi, exact)
BM_DEVICE void split8(const float *p, uint32_t *dh, uint32_t *dl) {
  const float4 v0 = reinterpret_cast<const float4 *>(p)[0], v1 = reinterpret_cast<const float4 *>(p)[1];
  const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t h0 = f32_to_bf16(f[2 * q]), h1 = f32_to_bf16(f[2 * q + 1]);
    dh[q] = h0 | (h1 << 16);
    dl[q] = f32_to_bf16(f[2 * q] - bf16_to_f32(uint16_t(h0))) |
            (uint32_t(f32_to_bf16(f[2 * q + 1] - bf16_to_f32(uint16_t(h1)))) << 16);
  }
}

// n consecutive activations (n = 16 or 32) of part `part` as bf16 words: from
// a float32 row (split) or from bf16 rows hi / lo
template <bool SRC_F32>
BM_DEVICE void act_words(const void *hi, const void *lo, size_t off, int part, int n, uint32_t *d) {
  if constexpr (SRC_F32) {
    const float *p = static_cast<const float *>(hi) + off;
    uint32_t th[4], tl[4];
    for (int i = 0; i < n / 8; ++i) {
      split8(p + 8 * i, th, tl);
#pragma unroll
      for (int w = 0; w < 4; ++w) d[4 * i + w] = part ? tl[w] : th[w];
    }
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(part ? lo : hi) + off);
    for (int i = 0; i < n / 8; ++i) {
      const uint4 v = p[i];
      d[4 * i] = v.x;
      d[4 * i + 1] = v.y;
      d[4 * i + 2] = v.z;
      d[4 * i + 3] = v.w;
    }
  }
}

// Build the operands of NT tokens (activation row of token t: row_of(t)) for
// the LPR lane slots of a K-long row.  Caller synchronises.
template <bool IS_Q8, int PARTS, bool SRC_F32, typename RowOf>
BM_DEVICE void stage_x(uint4 *XL, const void *hi, const void *lo, int K, int NT, RowOf row_of) {
  constexpr int XG = xgroups<PARTS>();
  const int LPR = K / 64;
  const int pieces = IS_Q8 ? 2 : 4;  // Q8: two 32-weight blocks; Q2: four sub-block slots
  for (int idx = threadIdx.x; idx < NT * LPR * pieces; idx += blockDim.x) {
    const int pc = idx % pieces, jj = (idx / pieces) % LPR, t = idx / (pieces * LPR);
    const size_t row = size_t(row_of(t)) * K;
    uint4 *base = XL + size_t(t) * XG * LPR + jj;
    float sum = 0.f;
    if constexpr (IS_Q8) {
      const size_t off = row + jj * 64 + 32 * pc;
#pragma unroll
      for (int part = 0; part < PARTS; ++part) {
        uint32_t d[16];
        act_words<SRC_F32>(hi, lo, off, part, 32, d);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          base[(8 * part + 4 * pc + q) * LPR] = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
#pragma unroll
          for (int w = 0; w < 4; ++w) sum = dot2_bf16(d[4 * q + w], BF16_ONEx2, sum);
        }
      }
      reinterpret_cast<float *>(base + 8 * PARTS * LPR)[pc] = -128.f * sum;
    } else {
      const size_t off = row + q2_c0(jj >> 2, jj & 3, K) + 32 * pc;
#pragma unroll
      for (int part = 0; part < PARTS; ++part) {
        uint32_t d[8], A[4], B[4];
        act_words<SRC_F32>(hi, lo, off, part, 16, d);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w0 = d[2 * j], w1 = d[2 * j + 1];
          A[j] = (w0 & 0xFFFFu) | (w1 << 16);
          B[j] = (w0 >> 16) | (w1 & 0xFFFF0000u);
          sum = dot2_bf16(w1, BF16_ONEx2, dot2_bf16(w0, BF16_ONEx2, sum));
        }
        base[(8 * part + pc) * LPR] = make_uint4(A[0], A[1], A[2], A[3]);
        base[(8 * part + 4 + pc) * LPR] = make_uint4(B[0], B[1], B[2], B[3]);
      }
      reinterpret_cast<float *>(base + 8 * PARTS * LPR)[pc] = sum;
      reinterpret_cast<float *>(base + (8 * PARTS + 1) * LPR)[pc] = -128.f * inv_f(pc) * sum;
    }
  }
}

// Copy nbytes at src (4-byte aligned) into LDS at dst + (src & 15) with 16-byte
// direct-to-LDS loads (each wave fills 64 consecutive 16-byte slots); returns
// the byte offset src & 15.  The copy completes at s_waitcnt vmcnt(0).
BM_DEVICE int stage_bytes(uint8_t *dst, const uint8_t *src, int nbytes) {
  const int pad = int(reinterpret_cast<uintptr_t>(src) & 15u);
  const uint8_t *base = src - pad;
  const int n16 = (pad + nbytes + 15) >> 4;
  const int lane = threadIdx.x & 63, wave0 = threadIdx.x & ~63;
  for (int c0 = wave0; c0 < n16; c0 += blockDim.x) {
    if (c0 + lane < n16)
      lds_dma16(base + 16 * (c0 + lane), lds_offset(dst + 16 * c0));
  }
  return pad;
}

BM_DEVICE uint32_t lds32(const uint8_t *p, int off) { return *reinterpret_cast<const uint32_t *>(p + off); }

// Q2 units of NM matrices (LDS pointers at the units' super-blocks) against NT
// tokens; out[m][t] += the unit's partial dot product.
template <int NT, int PARTS, int NM>
BM_DEVICE void q2_dot(const uint8_t *const (&sb)[NM], int h, int p, const uint4 *X, int LPR, float (&out)[NM][NT]) {
  constexpr int XG = xgroups<PARTS>();
  uint32_t w[NM][4], sw[NM][2];
  float d[NM], dmin[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[m][i] = lds32(sb[m], 16 + 32 * h + 16 * p + 4 * i);
    sw[m][0] = lds32(sb[m], 8 * h) >> (8 * p);
    sw[m][1] = lds32(sb[m], 8 * h + 4) >> (8 * p);
    const uint32_t dd = lds32(sb[m], 80);
    d[m] = half_to_f32(dd & 0xFFFFu);
    dmin[m] = half_to_f32(dd >> 16);
  }
  float yd[NM][NT], ym[NM][NT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) yd[m][t] = ym[m][t] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 xa[NT][PARTS], xb[NT][PARTS];
    float xs[NT], xc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int part = 0; part < PARTS; ++part) {
        xa[t][part] = X[(t * XG + 8 * part + s) * LPR];
        xb[t][part] = X[(t * XG + 8 * part + 4 + s) * LPR];
      }
      xs[t] = reinterpret_cast<const float *>(X + (t * XG + 8 * PARTS) * LPR)[s];
      xc[t] = reinterpret_cast<const float *>(X + (t * XG + 8 * PARTS + 1) * LPR)[s];
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t sbyte = (sw[m][s >> 1] >> (16 * (s & 1))) & 0xFFu;
      const float scf = float(sbyte & 15u), mf = float(sbyte >> 4);
      uint32_t A[4], B[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (s < 3) {
          const uint32_t msk = 0x00030003u << (2 * s);
          A[j] = and_or(w[m][j], msk, BF16_128x2);
          B[j] = and_or(w[m][j] >> 8, msk, BF16_128x2);
        } else {
          A[j] = and_or(w[m][j] >> 2, 0x00300030u, BF16_128x2);
          B[j] = and_or(w[m][j] >> 10, 0x00300030u, BF16_128x2);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int part = 0; part < PARTS; ++part) {
          acc = dot2_bf16(A[0], xa[t][part].x, acc);
          acc = dot2_bf16(B[0], xb[t][part].x, acc);
          acc = dot2_bf16(A[1], xa[t][part].y, acc);
          acc = dot2_bf16(B[1], xb[t][part].y, acc);
          acc = dot2_bf16(A[2], xa[t][part].z, acc);
          acc = dot2_bf16(B[2], xb[t][part].z, acc);
          acc = dot2_bf16(A[3], xa[t][part].w, acc);
          acc = dot2_bf16(B[3], xb[t][part].w, acc);
        }
        const float qx = __builtin_fmaf(acc, inv_f(s), xc[t]);
        yd[m][t] = __builtin_fmaf(scf, qx, yd[m][t]);
        ym[m][t] = __builtin_fmaf(mf, xs[t], ym[m][t]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) out[m][t] += d[m] * yd[m][t] - dmin[m] * ym[m][t];
}

// Q8_0 units (68 bytes: two 34-byte blocks) of NM matrices against NT tokens.
template <int NT, int PARTS, int NM>
BM_DEVICE void q8_dot(const uint8_t *const (&un)[NM], const uint4 *X, int LPR, float (&out)[NM][NT]) {
  constexpr int XG = xgroups<PARTS>();
  float acc[NM][2][NT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][0][t] = acc[m][1][t] = 0.f;
  float dA[NM], dB[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    dA[m] = half_to_f32(lds32(un[m], 0) & 0xFFFFu);
    dB[m] = half_to_f32(lds32(un[m], 32) >> 16);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint4 xp[NT][PARTS];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int part = 0; part < PARTS; ++part) xp[t][part] = X[(t * XG + 8 * part + 4 * b + g) * LPR];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        // codes 8g .. 8g+7 of block b: bytes 2 + 34b + 8g .. +7 of the unit
        const int o = 2 + 34 * b + 8 * g;  // even; the dwords holding them start at o & ~3
        const uint32_t u0 = lds32(un[m], o & ~3) ^ 0x80808080u, u1 = lds32(un[m], (o & ~3) + 4) ^ 0x80808080u,
                       u2 = lds32(un[m], (o & ~3) + 8) ^ 0x80808080u;
        const uint32_t uu[3] = {u0, u1, u2};
        uint32_t pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b0 = (o & 3) + 2 * e, b1 = b0 + 1;  // byte index within uu (q + 128 as unsigned)
          const float f0 = float((uu[b0 >> 2] >> (8 * (b0 & 3))) & 0xFFu);
          const float f1 = float((uu[b1 >> 2] >> (8 * (b1 & 3))) & 0xFFu);
          pr[e] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int part = 0; part < PARTS; ++part) {
            acc[m][b][t] = dot2_bf16(pr[0], xp[t][part].x, acc[m][b][t]);
            acc[m][b][t] = dot2_bf16(pr[1], xp[t][part].y, acc[m][b][t]);
            acc[m][b][t] = dot2_bf16(pr[2], xp[t][part].z, acc[m][b][t]);
            acc[m][b][t] = dot2_bf16(pr[3], xp[t][part].w, acc[m][b][t]);
          }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float *xc = reinterpret_cast<const float *>(X + (t * XG + 8 * PARTS) * LPR);
      out[m][t] += dA[m] * (acc[m][0][t] + xc[0]) + dB[m] * (acc[m][1][t] + xc[1]);
    }
}

// One block of the down GEMV: rows [r0, r0 + nrows) of the job's down matrix
// for its pairs (shared expert: tokens) t0 .. t0 + nt - 1.  smem: the rows'
// weight bytes (plus up to 12 bytes of lead), then the activation operands
// (h as hi + lo parts).
template <bool IS_Q8, int NT>
BM_DEVICE void down_block(const FfnArgs &a, const Job &job, int t0, int nt, int r0, int nrows, uint8_t *smem) {
  constexpr int PARTS = 2;
  const int K = a.F, LPR = K / 64, RPI = 64 / LPR;
  const size_t row_bytes = IS_Q8 ? size_t(K) / 32 * 34 : size_t(K) * 84 / 256;
  const uint8_t *mat = IS_Q8 ? a.sd : a.wd + size_t(job.e) * (size_t(a.F) * a.D / 256 * 84);
  const size_t chunk0 = size_t(r0) * row_bytes;  // chunk start inside the matrix
  const int cbytes = int(size_t(nrows) * row_bytes);
  const int stride = (cbytes + 16 + 15) & ~15;
  uint4 *XL = reinterpret_cast<uint4 *>(smem + stride);
  __syncthreads();  // the previous pass is done with the block's LDS
  const int pad = stage_bytes(smem, mat + chunk0, cbytes);
  stage_x<IS_Q8, PARTS, false>(XL, IS_Q8 ? a.hs : a.h, IS_Q8 ? a.hs_lo : a.h_lo, K, NT, [&](int t) {
    return IS_Q8 ? jtok(a, job, t0 + min(t, nt - 1)) : jpair(job, t0 + min(t, nt - 1));
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int jj = lane % LPR, rsub = lane / LPR;
  const uint4 *X = XL + jj;
  const int n_it = (nrows + RPI - 1) / RPI;
  for (int it = wave; it < n_it; it += 4) {
    const int rl = it * RPI + rsub;  // row within the chunk
    const bool active = rl < nrows;
    const size_t unit = size_t(r0 + (active ? rl : nrows - 1)) * LPR + jj;
    float acc[1][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[0][t] = 0.f;
    if constexpr (IS_Q8) {
      const uint8_t *un[1] = {smem + pad + (unit * 68 - chunk0)};
      q8_dot<NT, PARTS, 1>(un, X, LPR, acc);
    } else {
      const uint8_t *sb[1] = {smem + pad + ((unit >> 2) * 84 - chunk0)};
      q2_dot<NT, PARTS, 1>(sb, int(unit >> 1) & 1, int(unit) & 1, X, LPR, acc);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float ys = lane_group_sum(acc[0][t], LPR);  // sum over the LPR lanes of the row
      if (active && jj == 0 && t < nt) {
        const int r = r0 + rl;
        if constexpr (IS_Q8)
          a.ys[size_t(jtok(a, job, t0 + t)) * a.D + r] = ys;
        else
          a.y[size_t(jpair(job, t0 + t)) * a.D + r] = ys;
      }
    }
  }
}

// Grid: the shared expert's row chunks first, then u_max routed job slots x
// row chunks.  The shared job's tokens go in passes of NT_S; a routed job with
// one pair (the common case of a verify batch) takes the one-token code, else
// its pairs go in passes of NT_R.
template <int NT_S, int NT_R>
__global__ void __launch_bounds__(256) ffn_down_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_down[];
  Job job;
  const bool shared = int(blockIdx.x) < a.chunks_sd;
  int r0, nrows;
  if (shared) {
    shared_job(a, job);
    r0 = blockIdx.x * a.rows_sd;
    nrows = min(a.rows_sd, a.D - r0);
  } else {
    const int b = blockIdx.x - a.chunks_sd;
    if (!pair_job_wave(a, b / a.chunks_dn, job)) return;
    r0 = (b % a.chunks_dn) * a.rows_dn;
    nrows = min(a.rows_dn, a.D - r0);
  }
  if (shared) {
    for (int t0 = 0; t0 < job.n; t0 += NT_S) down_block<true, NT_S>(a, job, t0, min(NT_S, job.n - t0), r0, nrows, smem_down);
  } else if (NT_R == 1 || job.n == 1) {
    for (int t0 = 0; t0 < job.n; ++t0) down_block<false, 1>(a, job, t0, 1, r0, nrows, smem_down);
  } else {
    for (int t0 = 0; t0 < job.n; t0 += NT_R) down_block<false, NT_R>(a, job, t0, min(NT_R, job.n - t0), r0, nrows, smem_down);
  }
}

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
    const int t = jtok(a, job, t0 + min(i, nt - 1));
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
  using Raw = typename std::conditional<IS_Q8, Q8Unit, Q2Unit>::type;
  // raw bytes of the lane's unit in row iteration `it`
  auto load_it = [&](int it, Raw &rg, Raw &ru) {
    const int r = min(r_begin + it * RPI + rsub, r_end - 1);
    const int unit = r * LPR + jj;
    if constexpr (IS_Q8) {
      rg = q8_unit_load(a.sg + size_t(unit) * 68);
      ru = q8_unit_load(a.su + size_t(unit) * 68);
    } else {
      const int n = unit >> 2, q = unit & 3;
      rg = q2_unit_load(a.wg + size_t(job.e) * mat_bytes_q2 + size_t(n) * 84, q >> 1, q & 1);
      ru = q2_unit_load(a.wu + size_t(job.e) * mat_bytes_q2 + size_t(n) * 84, q >> 1, q & 1);
    }
  };
  const int n_it = (r_end - r_begin + RPI - 1) / RPI;
  // the wave's row iterations it = wave, wave + 4, ...: the weight loads of up
  // to DEPTH of them are issued before any arithmetic, so their memory
  // latencies overlap (two at most, so that the one-token kernel stays within
  // 128 VGPRs and every block of a decode launch is resident at once)
  constexpr int DEPTH = IS_Q8 ? 2 : (NT == 1 ? 2 : (NV <= 2 ? 2 : 1));
  for (int it0 = wave; it0 < n_it; it0 += 4 * DEPTH) {
    Raw rg[DEPTH], ru[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (it0 + 4 * d < n_it) load_it(it0 + 4 * d, rg[d], ru[d]);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int it = it0 + 4 * d;
      if (it >= n_it) break;
      const int r = r_begin + it * RPI + rsub;
      const bool active = r < r_end;
      float g[NV], u[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) g[v] = u[v] = 0.f;
      if constexpr (IS_Q8) {
        q8_unit_dot<NV>(rg[d], X, g);
        q8_unit_dot<NV>(ru[d], X, u);
      } else {
        const int unit = (active ? r : r_end - 1) * LPR + jj;
        q2_unit_dot<NV>(rg[d], unit & 1, X, g);
        q2_unit_dot<NV>(ru[d], unit & 1, X, u);
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
        gs = lane_group_sum(gs, LPR);  // sum over the LPR lanes of the row
        us = lane_group_sum(us, LPR);
        if (active && jj == 0 && i < nt) {
          const float hf = silu(gs) * us;
          const uint16_t hv = f32_to_bf16(hf);
          const size_t o = IS_Q8 ? size_t(jtok(a, job, t0 + i)) * a.F + r : size_t(jpair(job, t0 + i)) * a.F + r;
          // h travels as bf16 hi + lo parts (16 significant bits): a single bf16
          // rounding of h would dominate the layer's output error
          (IS_Q8 ? a.hs : a.h)[o] = hv;
          (IS_Q8 ? a.hs_lo : a.h_lo)[o] = f32_to_bf16(hf - bf16_to_f32(hv));
        }
      }
    }
  }
}

// Grid: the shared expert's row chunks first (its Q8_0 rows are the heaviest,
// so they start first), then u_max routed job slots x chunks_gu row chunks.
// Token passes as in the down kernel: NT_S for the shared job, one-token code
// for a routed job of one pair, else passes of NT_R.
template <int NT_S, int NT_R, bool XF32>
__global__ void __launch_bounds__(256) ffn_gateup_kernel(FfnArgs a) {
  Job job;
  int r_begin, r_end;
  const bool shared = int(blockIdx.x) < a.chunks_sg;
  if (shared) {
    shared_job(a, job);
    r_begin = blockIdx.x * a.rows_sg;
    r_end = min(a.F, r_begin + a.rows_sg);
  } else {
    const int b = blockIdx.x - a.chunks_sg;
    if (!pair_job_wave(a, b / a.chunks_gu, job)) return;
    r_begin = (b % a.chunks_gu) * a.rows_gu;
    r_end = min(a.F, r_begin + a.rows_gu);
  }
  if (shared) {
    for (int t0 = 0; t0 < job.n; t0 += NT_S)
      gateup_rows<NT_S, XF32, true>(a, job, t0, min(NT_S, job.n - t0), r_begin, r_end);
  } else if (NT_R == 1 || job.n == 1) {
    for (int t0 = 0; t0 < job.n; ++t0) gateup_rows<1, XF32, false>(a, job, t0, 1, r_begin, r_end);
  } else {
    for (int t0 = 0; t0 < job.n; t0 += NT_R)
      gateup_rows<NT_R, XF32, false>(a, job, t0, min(NT_R, job.n - t0), r_begin, r_end);
  }
}

// ---- launch configuration -----------------------------------------------------

// Down rows per block (a multiple of 4 waves x RPI rows) sized so that the
// rows' bytes plus the activation operands fit a 44 KB LDS budget (at least
// one wave iteration, at most four), and the block's LDS bytes.
static int down_rows(bool q8, int K, int N, int nt) {
  const int LPR = K / 64, RPI = 64 / LPR;
  const size_t row_bytes = q8 ? size_t(K) / 32 * 34 : size_t(K) * 84 / 256;
  const size_t x_bytes = size_t(nt) * xgroups<2>() * LPR * 16;
  const size_t budget = 44 * 1024 > x_bytes + 4096 ? 44 * 1024 - x_bytes : 4096;
  const int iters = int(std::max<size_t>(1, std::min<size_t>(4, budget / (4 * RPI * row_bytes))));
  return std::min(N, 4 * RPI * iters);
}
static size_t down_smem(bool q8, int K, int rows, int nt) {
  const size_t row_bytes = q8 ? size_t(K) / 32 * 34 : size_t(K) * 84 / 256;
  return ((size_t(rows) * row_bytes + 16 + 15) & ~size_t(15)) + size_t(nt) * xgroups<2>() * (K / 64) * 16;
}

// Gate/up GEMV launch over the shared expert's row chunks and u_max routed
// job slots: routed blocks hold 4 row iterations per wave, shared (Q8_0, 3.2x
// the bytes per row) blocks 2.
template <int NT_S, int NT_R, bool XF32>
static hipError_t launch_gateup_gemv(FfnArgs a, hipStream_t stream) {
  const int rpi = 64 / (a.D / 64);
  a.rows_gu = min(a.F, 16 * rpi);
  a.chunks_gu = (a.F + a.rows_gu - 1) / a.rows_gu;
  a.rows_sg = min(a.F, 8 * rpi);
  a.chunks_sg = a.sg ? (a.F + a.rows_sg - 1) / a.rows_sg : 0;
  const unsigned grid = unsigned(a.chunks_sg + a.u_max * a.chunks_gu);
  if (grid == 0) return hipSuccess;
  BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_kernel<NT_S, NT_R, XF32>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Down GEMV launch over the shared expert's row chunks and u_max routed job
// slots; raises the kernel's LDS limit when needed.
template <int NT_S, int NT_R>
static hipError_t launch_down_gemv(FfnArgs a, hipStream_t stream) {
  a.rows_dn = down_rows(false, a.F, a.D, NT_R);
  a.chunks_dn = (a.D + a.rows_dn - 1) / a.rows_dn;
  a.rows_sd = down_rows(true, a.F, a.D, NT_S);
  a.chunks_sd = a.sd ? (a.D + a.rows_sd - 1) / a.rows_sd : 0;
  const size_t smem = std::max(a.u_max ? down_smem(false, a.F, a.rows_dn, NT_R) : 0,
                               a.sd ? down_smem(true, a.F, a.rows_sd, NT_S) : 0);
  const unsigned grid = unsigned(a.chunks_sd + a.u_max * a.chunks_dn);
  if (grid == 0) return hipSuccess;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&ffn_down_kernel<NT_S, NT_R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
  }
  BM_LAUNCH("ffn_down_kernel", (ffn_down_kernel<NT_S, NT_R>), dim3(grid), dim3(256), smem, stream, a);
  return hipGetLastError();
}

// ---- streamed GEMV: each wave stages its rows through an LDS ring ------------
// A block is one wave that owns one job and a chunk of at most 64 consecutive
// output rows.  The weight bytes of the chunk are consumed in stages of 64
// units (RPI rows of one matrix: 1344 bytes of Q2 or 4352 bytes of Q8_0),
// copied into a wave-private LDS ring with 16-byte direct-to-LDS loads, so
// every load instruction reads 1 KB of contiguous HBM; up to NBUF stages are
// in flight.  Lane l computes unit l of the stage against its tokens'
// activation operands (registers), the LPR lanes of each row are summed, and
// the row's value is parked in lane (row - chunk start) until one coalesced
// store per token at the end.  The global loads of the wave complete in issue
// order, so waiting for all but the stages issued after stage j (NI loads per
// stage) makes stage j visible in LDS; no store is issued inside the loop.

constexpr int RING_BYTES = 13 * 1024;  // LDS ring per wave
constexpr int STREAM_ROWS_GU = 8, STREAM_ROWS_SG = 8;   // rows per chunk, gate/up (routed, shared)
constexpr int STREAM_ROWS_DN = 16, STREAM_ROWS_SD = 16;  // down

template <int K, bool IS_Q8>
struct StreamGeo {
  static constexpr int LPR = K / 64, RPI = 64 / LPR;
  static constexpr int ROWB = IS_Q8 ? K / 32 * 34 : K / 256 * 84;  // bytes per weight row
  static constexpr int STB = RPI * ROWB;                            // stage bytes (64 units)
  static constexpr int NI = (STB + 1023) / 1024;                    // loads per lane per stage
  static constexpr int NBUF = RING_BYTES / STB;                     // ring depth
  static_assert(STB % 16 == 0 && NBUF >= 2 && NI * (NBUF - 1) <= 63, "stream geometry");
};

// Rows [r_begin, r_end) (a multiple of RPI rows, at most 64) of one job for its
// tokens / pairs t0 .. t0 + nt - 1.  GATEUP: gate and up matrices, operands
// from x, h = silu(g) u stored as hi + lo; down: operands from h hi + lo, y.
template <int K, int NT, bool GATEUP, bool XF32, bool IS_Q8>
BM_DEVICE void stream_rows(const FfnArgs &a, const Job &job, int t0, int nt, int r_begin, int r_end, uint8_t *ring) {
  using G = StreamGeo<K, IS_Q8>;
  constexpr int PARTS = GATEUP ? (XF32 ? 2 : 1) : 2;
  constexpr int NV = NT * PARTS;
  constexpr int NM = GATEUP ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int jj = lane % G::LPR;
  // activation operands of the lane's unit (its columns do not depend on the row)
  const int c0 = IS_Q8 ? jj * 64 : q2_c0(jj >> 2, jj & 3, K);
  typename std::conditional<IS_Q8, XQ8, XQ2>::type X[NV];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int ti = t0 + min(i, nt - 1);
    if constexpr (GATEUP) {
      const size_t row = size_t(jtok(a, job, ti)) * K;
      if constexpr (IS_Q8) {
        if constexpr (XF32)
          load_xq8_f32(static_cast<const float *>(a.x) + row, c0, X[2 * i], X[2 * i + 1]);
        else
          load_xq8_bf16(static_cast<const uint16_t *>(a.x) + row, c0, X[i]);
      } else {
        if constexpr (XF32)
          load_xq2_f32(static_cast<const float *>(a.x) + row, c0, X[2 * i], X[2 * i + 1]);
        else
          load_xq2_bf16(static_cast<const uint16_t *>(a.x) + row, c0, X[i]);
      }
    } else {
      const size_t row = size_t(IS_Q8 ? jtok(a, job, ti) : jpair(job, ti)) * K;
      const uint16_t *hi = IS_Q8 ? a.hs : a.h, *lo = IS_Q8 ? a.hs_lo : a.h_lo;
      if constexpr (IS_Q8) {
        load_xq8_bf16(hi + row, c0, X[2 * i]);
        load_xq8_bf16(lo + row, c0, X[2 * i + 1]);
      } else {
        load_xq2_bf16(hi + row, c0, X[2 * i]);
        load_xq2_bf16(lo + row, c0, X[2 * i + 1]);
      }
    }
  }
  const uint8_t *m0, *m1 = nullptr;
  if constexpr (IS_Q8) {
    m0 = GATEUP ? a.sg : a.sd;
    if constexpr (GATEUP) m1 = a.su;
  } else {
    const size_t mat = size_t(a.F) * a.D / 256 * 84;
    m0 = (GATEUP ? a.wg : a.wd) + size_t(job.e) * mat;
    if constexpr (GATEUP) m1 = a.wu + size_t(job.e) * mat;
  }
  // stage j: row group j / NM (rows r_begin + (j / NM) RPI ..), matrix j % NM
  const int n_st = (r_end - r_begin) / G::RPI * NM;
  auto src = [&](int j) {
    return ((NM == 2 && (j & 1)) ? m1 : m0) + size_t(r_begin + (j / NM) * G::RPI) * G::ROWB;
  };
  for (int j = 0; j < G::NBUF && j < n_st; ++j) stream_issue<G::STB, G::NI>(ring + j * G::STB, src(j));
  float res[NT], gsum[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) res[i] = gsum[i] = 0.f;
  // SPI stages per iteration (two for Q2: a gate row with its up row, or two
  // row groups of down), so that their arithmetic and row sums interleave
  constexpr int SPI = IS_Q8 ? 1 : 2;
  for (int j = 0; j < n_st; j += SPI) {
    const int nj = min(SPI, n_st - j);
    // stages j .. j + nj - 1 have landed; later ones may still be in flight
    stream_wait<G::NI, G::NBUF - 1>(min(G::NBUF - nj, n_st - j - nj));
    float acc[SPI][NV];
#pragma unroll
    for (int q = 0; q < SPI; ++q) {
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[q][v] = 0.f;
      if (q < nj) {
        const uint8_t *slot = ring + ((j + q) % G::NBUF) * G::STB;
        if constexpr (IS_Q8) {
          const Q8Unit u = q8_unit_load(slot + lane * 68);
          q8_unit_dot<NV>(u, X, acc[q]);
        } else {
          const Q2Unit u = q2_unit_load(slot + (lane >> 2) * 84, (lane >> 1) & 1, lane & 1);
          q2_unit_dot<NV>(u, lane & 1, X, acc[q]);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slots' LDS reads are done before their refill
#pragma unroll
    for (int q = 0; q < SPI; ++q)
      if (q < nj && j + q + G::NBUF < n_st)
        stream_issue<G::STB, G::NI>(ring + ((j + q) % G::NBUF) * G::STB, src(j + q + G::NBUF));
    float vs[SPI][NT];
#pragma unroll
    for (int q = 0; q < SPI; ++q)
#pragma unroll
      for (int i = 0; i < NT; ++i)  // every lane of a row's group gets the row's sum
        vs[q][i] = lane_group_sum(PARTS == 2 ? acc[q][2 * i] + acc[q][2 * i + 1] : acc[q][i], G::LPR);
#pragma unroll
    for (int q = 0; q < SPI; ++q) {
      if (q >= nj) break;
      const int js = j + q, rg = js / NM;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (GATEUP && (js % NM) == 0) {
          gsum[i] = vs[q][i];
          continue;
        }
        const float rv = GATEUP ? silu(gsum[i]) * vs[q][i] : vs[q][i];
        // row rg * RPI + r lives in lanes r * LPR ..; park it in lane (row - r_begin)
#pragma unroll
        for (int r = 0; r < G::RPI; ++r) {
          const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), r * G::LPR));
          if (lane == rg * G::RPI + r) res[i] = s;
        }
      }
    }
  }
  const int nrows = r_end - r_begin;
  if (lane < nrows) {
    const int r = r_begin + lane;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i >= nt) break;
      if constexpr (GATEUP) {
        const size_t o = size_t(IS_Q8 ? jtok(a, job, t0 + i) : jpair(job, t0 + i)) * a.F + r;
        // h travels as bf16 hi + lo parts (h - hi is exact in float32)
        const uint16_t hv = f32_to_bf16(res[i]);
        (IS_Q8 ? a.hs : a.h)[o] = hv;
        (IS_Q8 ? a.hs_lo : a.h_lo)[o] = f32_to_bf16(res[i] - bf16_to_f32(hv));
      } else {
        if constexpr (IS_Q8)
          a.ys[size_t(jtok(a, job, t0 + i)) * a.D + r] = res[i];
        else
          a.y[size_t(jpair(job, t0 + i)) * a.D + r] = res[i];
      }
    }
  }
}

// Grid: the shared expert's row chunks first, then u_max routed job slots x
// row chunks (chunks_sg / rows_sg and chunks_gu / rows_gu for gate/up,
// chunks_sd / rows_sd and chunks_dn / rows_dn for down).  Token passes: NT_S
// for the shared job, the one-token code for a routed job of one pair, else
// passes of NT_R.
template <int K, int NT_S, int NT_R, bool GATEUP, bool XF32>
__global__ void __launch_bounds__(64) ffn_stream_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[RING_BYTES];
  const int chunks_s = GATEUP ? a.chunks_sg : a.chunks_sd, rows_s = GATEUP ? a.rows_sg : a.rows_sd;
  const int chunks_r = GATEUP ? a.chunks_gu : a.chunks_dn, rows_r = GATEUP ? a.rows_gu : a.rows_dn;
  const int N = GATEUP ? a.F : a.D;
  Job job;
  int r_begin, r_end;
  const bool shared = int(blockIdx.x) < chunks_s;
  if (shared) {
    shared_job(a, job);
    r_begin = blockIdx.x * rows_s;
    r_end = min(N, r_begin + rows_s);
  } else {
    const int b = blockIdx.x - chunks_s;
    if (!pair_job_wave(a, b / chunks_r, job)) return;
    r_begin = (b % chunks_r) * rows_r;
    r_end = min(N, r_begin + rows_r);
  }
  if (shared) {
    for (int t0 = 0; t0 < job.n; t0 += NT_S)
      stream_rows<K, NT_S, GATEUP, XF32, true>(a, job, t0, min(NT_S, job.n - t0), r_begin, r_end, ring);
  } else if (NT_R == 1 || job.n == 1) {
    for (int t0 = 0; t0 < job.n; ++t0) stream_rows<K, 1, GATEUP, XF32, false>(a, job, t0, 1, r_begin, r_end, ring);
  } else {
    for (int t0 = 0; t0 < job.n; t0 += NT_R)
      stream_rows<K, NT_R, GATEUP, XF32, false>(a, job, t0, min(NT_R, job.n - t0), r_begin, r_end, ring);
  }
}

// Streamed launch of one half of the FFN (gate/up or down) with chunks of
// rows_r routed and rows_s shared rows.
template <int K, int NT_S, int NT_R, bool GATEUP, bool XF32>
static hipError_t launch_stream(FfnArgs a, int rows_r, int rows_s, hipStream_t stream) {
  const int N = GATEUP ? a.F : a.D;
  const bool has_s = GATEUP ? a.sg != nullptr : a.sd != nullptr;
  const int cr = (N + rows_r - 1) / rows_r, cs = has_s ? (N + rows_s - 1) / rows_s : 0;
  if (GATEUP) {
    a.rows_gu = rows_r, a.chunks_gu = cr, a.rows_sg = rows_s, a.chunks_sg = cs;
  } else {
    a.rows_dn = rows_r, a.chunks_dn = cr, a.rows_sd = rows_s, a.chunks_sd = cs;
  }
  const unsigned grid = unsigned(cs + a.u_max * cr);
  if (grid == 0) return hipSuccess;
  BM_LAUNCH(GATEUP ? "ffn_gateup_kernel" : "ffn_down_kernel", (ffn_stream_kernel<K, NT_S, NT_R, GATEUP, XF32>),
            dim3(grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// ---- combine ----------------------------------------------------------------
// y is indexed by pair; pairs whose id is out of range contribute nothing.

template <int K>
__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ y, const float *__restrict__ ys,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ wts, int T, int D, int E,
                                                      void *out, int out_bf16, int64_t *status) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;  // one thread per 4 outputs
  const int64_t per_tok = D / 4;
  if (idx >= int64_t(T) * per_tok) return;
  const int t = int(idx / per_tok);
  const int c = int(idx % per_tok) * 4;
  store_out4(out, out_bf16, t, D, c, combine4<K>(y, ys, ids, wts, t, c, D, E, status));
}

// ---- launch -----------------------------------------------------------------

// Token passes: NT_GU / NT_DN for the shared job, NT_R (or one) for routed jobs.
template <int NT_GU, int NT_DN, int NT_R, bool XF32>
static hipError_t launch_decode_nt(const FfnArgs &a, hipStream_t stream) {
  hipError_t err = launch_gateup_gemv<NT_GU, NT_R, XF32>(a, stream);
  if (err != hipSuccess) return err;
  return launch_down_gemv<NT_DN, NT_R>(a, stream);
}

// Streamed gate/up (K = D) and down (K = F) with NT_S / NT_R token passes.
// NT_SG / NT_SD: tokens per pass of the shared expert's gate/up / down rows
template <int D, int F, int NT_SG, int NT_SD, int NT_R, bool XF32>
static hipError_t launch_stream_ffn(const FfnArgs &a, hipStream_t stream) {
  hipError_t err = launch_stream<D, NT_SG, NT_R, true, XF32>(a, STREAM_ROWS_GU, STREAM_ROWS_SG, stream);
  if (err != hipSuccess) return err;
  return launch_stream<F, NT_SD, NT_R, false, XF32>(a, STREAM_ROWS_DN, STREAM_ROWS_SD, stream);
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Routed experts and shared expert per launch:
//  T = 1: the register GEMV kernels (every wave loads its rows' bytes up
//         front; the one-token code has the fewest instructions per weight);
//  T >= 2 at d_model 4096, d_ff 2048 (weights 16-byte aligned): the streamed
//         kernels, routed jobs of one pair on the one-token code;
//  other shapes: the register GEMV kernels in token passes.
hipError_t launch_decode_ffn(FfnArgs a, bool xf32, hipStream_t stream) {
  a.u_max = a.T * a.k;  // one job slot per pair; repeated experts exit at once
  hipError_t err;
  const bool stream_ok = a.D == 4096 && a.F == 2048 && aligned16(a.wg) && aligned16(a.wu) && aligned16(a.wd) &&
                         aligned16(a.sg) && aligned16(a.su) && aligned16(a.sd);
  if (a.T == 1)
    err = xf32 ? launch_decode_nt<1, 1, 1, true>(a, stream) : launch_decode_nt<1, 1, 1, false>(a, stream);
  else if (stream_ok)
    // bf16 x from three tokens on: the shared gate/up rows in passes of three
    // (two passes at T = 5 instead of three; 156 VGPRs against 146, the same
    // three waves per SIMD); down keeps passes of two (three would take 256)
    err = xf32 ? launch_stream_ffn<4096, 2048, 2, 2, 2, true>(a, stream)
               : (a.T == 2 ? launch_stream_ffn<4096, 2048, 2, 2, 2, false>(a, stream)
                           : launch_stream_ffn<4096, 2048, 3, 2, 2, false>(a, stream));
  else if (a.T == 2 || xf32)
    err = xf32 ? launch_decode_nt<2, 2, 2, true>(a, stream) : launch_decode_nt<2, 2, 2, false>(a, stream);
  else
    err = launch_decode_nt<NTOK, 2, 2, false>(a, stream);
  if (err != hipSuccess) return err;
  return launch_combine(a.y, a.sd ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        a.x_res, a.x_next, stream);
}

// ---- one decode step of one token in four launches ---------------------------
// moe_layer at T = 1 runs moe_route + moe_expert_ffn (decode mode) as
//  (1) the router logits (router_gemv_kernel, one block per expert row);
//  (2) ffn_gateup_sel_kernel: the gate/up launch of moe_expert_ffn, whose
//      routed blocks first select the token's experts from the logits with the
//      top-k routine of moe_route (the same code on the same logits: every
//      block reaches the same selection; the first routed block stores it as
//      the call's ids and weights), while the shared expert's blocks, which
//      need no selection, start streaming at once;
//  (3) the down launch and (4) the combine, as moe_expert_ffn runs them.
// Every row and output goes through the same arithmetic as in the two
// separate calls, so ids, weights and y agree bit for bit; the top-k launch,
// whose latency the shared rows now cover, is gone.

template <int PER, bool XF32>
__global__ void __launch_bounds__(256) ffn_gateup_sel_kernel(FfnArgs a, const float *__restrict__ logits,
                                                             int32_t *__restrict__ ids_out,
                                                             float *__restrict__ wts_out) {
  const int b = int(blockIdx.x) - a.chunks_sg;
  if (b < 0) {  // shared expert: chunk blockIdx.x of its rows
    Job job;
    shared_job(a, job);
    const int r_begin = blockIdx.x * a.rows_sg;
    gateup_rows<1, XF32, true>(a, job, 0, 1, r_begin, min(a.F, r_begin + a.rows_sg));
    return;
  }
  __shared__ int32_t s_ids[8];
  __shared__ float s_wts[8];
  if (threadIdx.x < 64) topk_token<PER>(logits, a.E, a.k, s_ids, s_wts, threadIdx.x);
  __syncthreads();
  if (b == 0 && int(threadIdx.x) < a.k) {
    ids_out[threadIdx.x] = s_ids[threadIdx.x];
    wts_out[threadIdx.x] = s_wts[threadIdx.x];
  }
  a.ids = s_ids;
  a.wts = s_wts;
  Job job;
  if (!pair_job_wave(a, b / a.chunks_gu, job)) return;
  const int r_begin = (b % a.chunks_gu) * a.rows_gu;
  gateup_rows<1, XF32, false>(a, job, 0, 1, r_begin, min(a.F, r_begin + a.rows_gu));
}

// a: the moe_expert_ffn arguments for one token with a.ids / a.wts the call's
// outputs; wr, bias, logits: moe_route's router matrix, optional bias and
// logit buffer ([E] float32).
hipError_t launch_decode_layer(FfnArgs a, bool xf32, const float *wr, const float *bias, float *logits,
                               hipStream_t stream) {
  if (a.T != 1 || a.k > 8 || a.E > 16 * 64) return hipErrorNotSupported;
  hipError_t err = launch_route_logits(a.x, !xf32, 1, a.D, a.E, wr, bias, logits, stream);
  if (err != hipSuccess) return err;
  a.u_max = a.k;
  // row chunks as launch_gateup_gemv sets them (the same rows per block)
  const int rpi = 64 / (a.D / 64);
  a.rows_gu = min(a.F, 16 * rpi);
  a.chunks_gu = (a.F + a.rows_gu - 1) / a.rows_gu;
  a.rows_sg = min(a.F, 8 * rpi);
  a.chunks_sg = a.sg ? (a.F + a.rows_sg - 1) / a.rows_sg : 0;
  int32_t *ids_out = const_cast<int32_t *>(a.ids);
  float *wts_out = const_cast<float *>(a.wts);
  const dim3 grid(unsigned(a.chunks_sg + a.u_max * a.chunks_gu));
  if (a.E <= 6 * 64) {
    if (xf32)
      BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_sel_kernel<6, true>), grid, dim3(256), 0, stream, a, logits, ids_out,
                wts_out);
    else
      BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_sel_kernel<6, false>), grid, dim3(256), 0, stream, a, logits,
                ids_out, wts_out);
  } else {
    if (xf32)
      BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_sel_kernel<16, true>), grid, dim3(256), 0, stream, a, logits,
                ids_out, wts_out);
    else
      BM_LAUNCH("ffn_gateup_kernel", (ffn_gateup_sel_kernel<16, false>), grid, dim3(256), 0, stream, a, logits,
                ids_out, wts_out);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_down_gemv<1, 1>(a, stream)) != hipSuccess) return err;
  return launch_combine(a.y, a.sd ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        a.x_res, a.x_next, stream);
}

hipError_t launch_combine(const float *y, const float *ys, const int32_t *ids, const float *wts, int T, int k, int D,
                          int E, void *out, int out_bf16, int64_t *status, const uint16_t *x_res, uint16_t *x_next,
                          hipStream_t stream) {
  if (x_next) return launch_combine_residual(y, ys, ids, wts, T, k, D, E, out, out_bf16, status, x_res, x_next, stream);
  const int64_t n4 = int64_t(T) * (D / 4);
  return with_top_k(k, [&](auto kc) {
    BM_LAUNCH("combine_kernel", combine_kernel<decltype(kc)::value>, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0,
              stream, y, ys, ids, wts, T, D, E, out, out_bf16, status);
    return hipGetLastError();
  });
}

}  // namespace bm
