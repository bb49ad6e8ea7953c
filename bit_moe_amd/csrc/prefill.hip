// Prefill path: one MoE layer over a prompt chunk as grouped GEMMs on MFMA.
//
// "Strata-DSV4.1", §Results / §How it works: a prompt chunk runs each layer's
// routed experts as grouped expert matrix products (there on int8 tensor
// cores).  Here every product runs on v_mfma_f32_16x16x32_bf16 with float32
// accumulation and the weights enter the matrix cores exactly:
//  * routed Q2 experts: the grouped kernels of prefill_q2.hip (sc*q and m are
//    small integers, exact in bf16; d and dmin are applied per super-block);
//  * the Q8_0 shared expert (this file): the int8 codes are expanded once per
//    call to exact bf16 and one float scale per 32-weight block, then a dense
//    GEMM multiplies the codes and applies d once per 32-wide MFMA step.
// SwiGLU (gate is the SiLU operand, "run the DeepSeek-V4-Flash-Vision tower on
// CUDA" commit notes) is fused into the gate/up epilogues; h is stored as a
// bf16 hi + lo pair; the combine runs afterwards in the fixed slot order.
//
// Order of one call: optional float32 -> bf16 conversion of x, the plan
// (groups, pair permutation, tile lists), routed gate/up, routed down, shared
// gate/up, shared down, combine.
#include "common.h"
#include "internal.h"
#include "mfma_q2.h"

namespace bm {

constexpr int BM_ = 64;          // tokens per M-tile of the shared expert's dense GEMM
constexpr int BN_ = 64;          // output rows per block
constexpr int KS = 256;          // K per step
constexpr int LDS_ROW = KS + 8;  // bf16 elements per LDS activation row (16-byte pad)

struct GemmArgs {
  int T;                      // tokens (rows of A)
  // A: bf16 rows of length K, by token
  const uint16_t *a;
  const uint16_t *a_lo;       // down: bf16 lo parts of the A rows (A = a + a_lo), else null
  int K, N;
  // B: expanded Q8_0, bf16 codes [N][K] and float d [N][K/32]
  const uint8_t *b0, *b1;     // b1: up matrix (gate/up)
  const float *d0, *d1;
  // out
  uint16_t *h_out;            // gate/up: [T][N] bf16 hi part of h
  uint16_t *h_lo_out;         // gate/up: [T][N] bf16 lo part of h
  float *y_out;               // down: [T][N] float32
  int m_tiles;                // grid M-tile slots
};

// Shared expert (dense, Q8_0 expanded to exact int8 codes as bf16 + one float
// scale per 32 weights) on MFMA: 64-token M-tiles x 64 weight rows per block,
// K-steps of 256; each 32-wide MFMA step covers one Q8_0 block, so its result
// is scaled by d once.  ALO: the A rows arrive as bf16 hi + lo parts (the down
// projection's h); both parts multiply the same B operand.
template <bool GATEUP, bool ALO>
__global__ void __launch_bounds__(256) q8x_gemm_kernel(GemmArgs a) {
  __shared__ uint16_t As[BM_ * LDS_ROW];
  __shared__ uint16_t As_lo[ALO ? BM_ * LDS_ROW : 8];
  const int nt_n = a.N / BN_;
  // XCD-aware remap of the block index (grid is a multiple of 8)
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int mt = L / nt_n, ntile = L % nt_n;
  if (mt >= a.m_tiles) return;
  const int base = mt * BM_;
  if (base >= a.T) return;
  const int valid = min(BM_, a.T - base);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, nl = lane & 15;
  const int n = ntile * BN_ + wave * 16 + nl;  // this lane's weight row
  // A staging slice of this thread: row ar, 64 elements at 64*aq
  const int ar = tid >> 2, aq = tid & 3;
  const int a_row = ar < valid ? base + ar : -1;
  const uint16_t *a_src = a_row >= 0 ? a.a + size_t(a_row) * a.K : nullptr;
  const uint16_t *a_src_lo = (ALO && a_row >= 0) ? a.a_lo + size_t(a_row) * a.K : nullptr;
  const size_t b_off = size_t(n) * a.K * 2;
  f32x4_t acc0[4], acc1[4];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc0[i] = acc1[i] = zero;
  const int nsteps = a.K / KS;
  for (int kb = 0; kb < nsteps; ++kb) {
    uint4 av[8], al[ALO ? 8 : 1];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      av[i] = a_src ? *reinterpret_cast<const uint4 *>(a_src + kb * KS + aq * 64 + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        al[i] = a_src_lo ? *reinterpret_cast<const uint4 *>(a_src_lo + kb * KS + aq * 64 + 8 * i)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();  // the previous step's LDS reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4 *>(&As[ar * LDS_ROW + aq * 64 + 8 * i]) = av[i];
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4 *>(&As_lo[ar * LDS_ROW + aq * 64 + 8 * i]) = al[i];
    }
    __syncthreads();
    const uint16_t *r0 = reinterpret_cast<const uint16_t *>(a.b0 + b_off) + kb * KS;
    const uint16_t *r1 = GATEUP ? reinterpret_cast<const uint16_t *>(a.b1 + b_off) + kb * KS : nullptr;
    const float *s0 = a.d0 + size_t(n) * (a.K / 32) + kb * 8;
    const float *s1 = GATEUP ? a.d1 + size_t(n) * (a.K / 32) + kb * 8 : nullptr;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t B0[4], B1[4];
      ld16(r0 + 32 * t + 8 * g, B0);
      const float e0 = s0[t];
      float e1 = 0.f;
      if constexpr (GATEUP) {
        ld16(r1 + 32 * t + 8 * g, B1);
        e1 = s1[t];
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        uint32_t A[4];
        ld16(&As[(16 * mi + nl) * LDS_ROW + 32 * t + 8 * g], A);
        f32x4_t c0 = mfma16(A, B0, zero);
        if constexpr (ALO) {
          uint32_t Alo[4];
          ld16(&As_lo[(16 * mi + nl) * LDS_ROW + 32 * t + 8 * g], Alo);
          c0 = mfma16(Alo, B0, c0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc0[mi][r] = __builtin_fmaf(e0, c0[r], acc0[mi][r]);
        if constexpr (GATEUP) {
          const f32x4_t c1 = mfma16(A, B1, zero);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc1[mi][r] = __builtin_fmaf(e1, c1[r], acc1[mi][r]);
        }
      }
    }
  }
  // epilogue: lane holds rows 16 mi + 4 g + r of column n
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mi + 4 * g + r;
      if (m >= valid) continue;
      const size_t orow = size_t(base + m);
      if constexpr (GATEUP) {
        const float hf = silu(acc0[mi][r]) * acc1[mi][r];
        const uint16_t hb = f32_to_bf16(hf);
        a.h_out[orow * a.N + n] = hb;
        a.h_lo_out[orow * a.N + n] = f32_to_bf16(hf - bf16_to_f32(hb));
      } else {
        a.y_out[orow * a.N + n] = acc0[mi][r];
      }
    }
  }
}

// Q8_0 [N][K] -> exact bf16 codes [N][K] and float scales [N][K/32]
__global__ void __launch_bounds__(256) q8_expand_kernel(const uint8_t *__restrict__ blocks, int64_t n_blocks,
                                                        uint16_t *__restrict__ codes, float *__restrict__ scales) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // one thread per (block, 4 codes)
  if (i >= n_blocks * 8) return;
  const int64_t blk = i >> 3;
  const int c = int(i & 7) * 4;
  const uint8_t *bp = blocks + blk * 34;
  if (c == 0) scales[blk] = half_to_f32(bp[0] | (uint32_t(bp[1]) << 8));
  uint32_t o[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float f0 = float(int8_t(bp[2 + c + 2 * j])), f1 = float(int8_t(bp[3 + c + 2 * j]));
    o[j] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
  }
  *reinterpret_cast<uint2 *>(codes + blk * 32 + c) = make_uint2(o[0], o[1]);
}

__global__ void __launch_bounds__(256) f32_to_bf16_kernel(const float *__restrict__ x, uint16_t *__restrict__ y,
                                                          int64_t n) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 v = *reinterpret_cast<const float4 *>(x + i);
  *reinterpret_cast<uint2 *>(y + i) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

static hipError_t launch_q8x_gemm(const GemmArgs &g, bool gateup, hipStream_t stream) {
  int grid = g.m_tiles * (g.N / BN_);
  grid = (grid + 7) & ~7;
  if (gateup)
    BM_LAUNCH("shared_gateup_gemm_kernel", (q8x_gemm_kernel<true, false>), dim3(grid), dim3(256), 0, stream, g);
  else
    BM_LAUNCH("shared_down_gemm_kernel", (q8x_gemm_kernel<false, true>), dim3(grid), dim3(256), 0, stream, g);
  return hipGetLastError();
}

static hipError_t launch_q8_expand(const void *blocks, int64_t n_weights, uint16_t *codes, float *scales,
                                   hipStream_t stream) {
  const int64_t nb = n_weights / 32;
  BM_LAUNCH("q8_expand_kernel", q8_expand_kernel, dim3(unsigned((nb * 8 + 255) / 256)), dim3(256), 0, stream,
            static_cast<const uint8_t *>(blocks), nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t stream) {
  if (a.D % KS || a.F % KS) return hipErrorNotSupported;  // K-steps of 256, N-tiles of 64
  hipError_t err;
  const uint16_t *x = static_cast<const uint16_t *>(a.x);
  if (a.x_f32) {
    const int64_t n = int64_t(a.T) * a.D;
    BM_LAUNCH("f32_to_bf16_kernel", f32_to_bf16_kernel, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0, stream,
              static_cast<const float *>(a.x), a.xs, n);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    x = a.xs;
  }
  PlanBufs p = a.plan;
  if ((err = launch_plan(a.ids, a.T, a.k, a.E, PREFILL_BM, PREFILL_BM_DOWN, p, stream)) != hipSuccess) return err;
  const int P = a.T * a.k;
  const size_t q2_stride = size_t(a.F) * a.D / 256 * 84;

  // routed gate/up (A = x rows by token, N = F), then down (A = h hi + lo rows by pair, N = D)
  if ((err = launch_q2_group(true, a, x, a.xsum, a.xtot, stream)) != hipSuccess) return err;
  if ((err = launch_q2_group(false, a, x, a.xsum, a.xtot, stream)) != hipSuccess) return err;

  if (a.sg) {
    // shared expert: expand Q8_0 to exact bf16 codes + float scales, then dense GEMMs
    const int64_t nw = int64_t(a.F) * a.D;
    float *sd = reinterpret_cast<float *>(a.sw_bf16 + 3 * nw);
    if ((err = launch_q8_expand(a.sg, nw, a.sw_bf16, sd, stream)) != hipSuccess) return err;
    if ((err = launch_q8_expand(a.su, nw, a.sw_bf16 + nw, sd + nw / 32, stream)) != hipSuccess) return err;
    if ((err = launch_q8_expand(a.sd, nw, a.sw_bf16 + 2 * nw, sd + 2 * nw / 32, stream)) != hipSuccess) return err;
    GemmArgs s{};
    s.T = a.T;
    s.m_tiles = (a.T + BM_ - 1) / BM_;
    s.a = x;
    s.K = a.D;
    s.N = a.F;
    s.b0 = reinterpret_cast<const uint8_t *>(a.sw_bf16);
    s.b1 = reinterpret_cast<const uint8_t *>(a.sw_bf16 + nw);
    s.d0 = sd;
    s.d1 = sd + nw / 32;
    s.h_out = a.hs;
    s.h_lo_out = a.hs_lo;
    if ((err = launch_q8x_gemm(s, true, stream)) != hipSuccess) return err;
    s.a = a.hs;
    s.a_lo = a.hs_lo;
    s.K = a.F;
    s.N = a.D;
    s.b0 = reinterpret_cast<const uint8_t *>(a.sw_bf16 + 2 * nw);
    s.b1 = nullptr;
    s.d0 = sd + 2 * nw / 32;
    s.d1 = nullptr;
    s.y_out = a.ys;
    if ((err = launch_q8x_gemm(s, false, stream)) != hipSuccess) return err;
  }
  return launch_combine(a.y, a.sg ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        stream);
}

}  // namespace bm
