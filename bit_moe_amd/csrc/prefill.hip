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

constexpr int KS = 256;          // K per step of the shared expert's dense GEMM
constexpr int ROWP = KS + 8;     // bf16 per LDS activation row (16-byte pad)

// ---- shared expert (Q8_0): exact bf16 codes in MFMA operand order ------------
// The Q8_0 matrix [N][K] is expanded once per call to exact bf16 codes (int8
// values are exact in bf16) laid out in the lane order of the B operand of
// v_mfma_f32_16x16x32_bf16, each 16-row group and 32-column block (one Q8_0
// block per row) in a chunk of 1,088 bytes at (G * K/32 + t) * 1088:
//   bytes 0 .. 1023   : lane L = 16 g + r holds codes 32 t + 8 g .. + 7 of row
//                       16 G + r as bf16, so one wave's B operand of one MFMA
//                       step is one contiguous 1 KB load;
//   bytes 1024 .. 1087: the 16 rows' scales d as float32.
constexpr int Q8X_CHUNK = 1088;  // bytes of one expanded (16-row group, 32-column block) chunk

__global__ void __launch_bounds__(256) q8_expand_kernel(const uint8_t *__restrict__ blocks, int N, int K,
                                                        uint8_t *__restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // (chunk, lane)
  const int KT = K / 32;
  if (i >= int64_t(N / 16) * KT * 64) return;
  const int lane = int(i & 63), g = lane >> 4, r = lane & 15;
  const int64_t chunk = i >> 6;
  const int t = int(chunk % KT);
  const int64_t G = chunk / KT;
  const uint8_t *bp = blocks + ((G * 16 + r) * KT + t) * 34;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float f0 = float(int8_t(bp[2 + 8 * g + 2 * j])), f1 = float(int8_t(bp[3 + 8 * g + 2 * j]));
    o[j] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
  }
  uint8_t *c = out + chunk * Q8X_CHUNK;
  *reinterpret_cast<uint4 *>(c + 16 * lane) = make_uint4(o[0], o[1], o[2], o[3]);
  if (g == 0) reinterpret_cast<float *>(c + 1024)[r] = half_to_f32(bp[0] | (uint32_t(bp[1]) << 8));
}

struct DenseArgs {
  int T, K, N;
  const uint16_t *a, *a_lo;  // activation rows [T][K] bf16 (a_lo: the lo parts of down's h)
  const uint8_t *c0, *c1;    // expanded codes and scales (c1: up matrix)
  uint16_t *h, *h_lo;        // gate/up out [T][N]: h = silu(g) u as bf16 hi + lo
  float *y;                  // down out [T][N]
};

// A block owns BM tokens and BN weight rows (8 waves x NG groups of 16 rows,
// both matrices for gate/up).  Per 256-wide K-step the block stages its
// activation rows in LDS (through registers, one step ahead); each wave
// keeps the codes and scales of its rows in registers, loaded one MFMA step
// ahead, applies each to the block's MT 16-token tiles and scales
// each MFMA result (one Q8_0 block: 16 rows x 16 tokens) by d into float32
// accumulators.  Down multiplies the hi and lo parts of h by the same codes.
template <bool GATEUP>
struct DenseGeo {
  static constexpr int NM = GATEUP ? 2 : 1;     // matrices
  static constexpr int PARTS = GATEUP ? 1 : 2;  // activation parts
  static constexpr int MT = GATEUP ? 4 : 2;     // 16-token tiles per block
  static constexpr int NG = GATEUP ? 2 : 4;     // 16-row groups per wave
  static constexpr int W = 8;                   // waves
  static constexpr int BN = 16 * NG * W;        // weight rows per block
  static constexpr int BM = 16 * MT;            // tokens per block
  static constexpr int AROWS = PARTS * BM;      // LDS activation rows per step
  static constexpr int ABUF = AROWS * ROWP * 2;
  static constexpr int SMEM = 2 * ABUF;
  static_assert(AROWS * 8 == 64 * W, "one staging slice per thread");
};

template <bool GATEUP>
__global__ void __launch_bounds__(512) q8_dense_kernel(DenseArgs g) {
  using Gm = DenseGeo<GATEUP>;
  constexpr int NM = Gm::NM, PARTS = Gm::PARTS, MT = Gm::MT, NG = Gm::NG;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_d[];
  const int n_m = (g.T + Gm::BM - 1) / Gm::BM, n_n = g.N / Gm::BN;
  const int G_ = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G_ >> 3) + (b >> 3);  // XCD-aware: blocks sharing weight rows run together
  const int mc = L % n_m, ntile = L / n_m;
  if (ntile >= n_n) return;
  const int m0 = mc * Gm::BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nl = lane & 15;
  const int KT = g.K / 32, nsteps = g.K / KS;
  const int G0 = ntile * (Gm::BN / 16);  // first row group of the block
  uint8_t *abuf = smem_d;
  // staging slice: activation row ar (part ap), 64 bytes at column 32 aq of the step
  const int ar = tid >> 3, aq = tid & 7;
  const int ap = ar / Gm::BM, atok = min(m0 + ar % Gm::BM, g.T - 1);
  const uint16_t *asrc = (ap ? g.a_lo : g.a) + size_t(atok) * g.K + 32 * aq;
  auto stage_load = [&](int s, uint4 (&av)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = reinterpret_cast<const uint4 *>(asrc + size_t(s) * KS)[i];
  };
  auto stage_store = [&](int half, const uint4 (&av)[4]) __attribute__((always_inline)) {
    uint16_t *ad = reinterpret_cast<uint16_t *>(abuf + half * Gm::ABUF) + ar * ROWP + 32 * aq;
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<uint4 *>(ad)[i] = av[i];
  };
  // this wave's codes and scales of MFMA step t (group ng = rows 16 (wave NG +
  // ng) of the block; the lane's row is 16 (wave NG + ng) + nl)
  uint32_t B0[NG][NM][4], B1[NG][NM][4];  // codes of the even and odd MFMA steps
  float S0[NG][NM], S1[NG][NM];           // and their scales
  auto load_b = [&](int t, uint32_t (&B)[NG][NM][4], float (&S)[NG][NM]) __attribute__((always_inline)) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint8_t *c = (m ? g.c1 : g.c0) + (size_t(G0 + wave * NG + ng) * KT + t) * Q8X_CHUNK;
        ld16(reinterpret_cast<const uint16_t *>(c) + 8 * lane, B[ng][m]);
        S[ng][m] = reinterpret_cast<const float *>(c + 1024)[nl];
      }
  };
  f32x4_t acc[MT][NG][NM];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[mi][ng][m] = zero;
  load_b(0, B0, S0);
  {
    uint4 av[4];
    stage_load(0, av);
    stage_store(0, av);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int half = s & 1;
    // next step's slices (the last step re-reads its own: loads and stores
    // stay unconditional, which keeps these values in registers)
    uint4 av[4];
    stage_load(min(s + 1, nsteps - 1), av);
    const uint16_t *Ah = reinterpret_cast<const uint16_t *>(abuf + half * Gm::ABUF);
    // one MFMA step (32 columns): codes of step t from `use`, the codes of
    // step t + 1 loaded into `nxt` first
    auto mstep = [&](int tt, const uint32_t (&use)[NG][NM][4], const float (&sc)[NG][NM], uint32_t (&nxt)[NG][NM][4],
                     float (&nsc)[NG][NM]) __attribute__((always_inline)) {
      const int t = 8 * s + tt;
      if (t + 1 < KT) load_b(t + 1, nxt, nsc);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        uint32_t A[PARTS][4];
#pragma unroll
        for (int part = 0; part < PARTS; ++part)
          ld16(Ah + (part * Gm::BM + 16 * mi + nl) * ROWP + 32 * tt + 8 * gq, A[part]);
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            f32x4_t c = mfma16(A[0], use[ng][m], zero);
            if constexpr (PARTS == 2) c = mfma16(A[1], use[ng][m], c);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][ng][m][r] = __builtin_fmaf(sc[ng][m], c[r], acc[mi][ng][m][r]);
          }
      }
    };
#pragma unroll 1
    for (int tq = 0; tq < 8; tq += 2) {
      mstep(tq, B0, S0, B1, S1);
      mstep(tq + 1, B1, S1, B0, S0);
    }
    stage_store(half ^ 1, av);  // the buffer read in step s - 1 (every wave passed the barrier since)
    __syncthreads();
  }
  // epilogue: lane holds tokens 16 mi + 4 gq + r of row n of group ng
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = m0 + 16 * mi + 4 * gq + r;
      if (tok >= g.T) continue;
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        const int n = ntile * Gm::BN + (wave * NG + ng) * 16 + nl;
        if constexpr (GATEUP) {
          const float hf = silu(acc[mi][ng][0][r]) * acc[mi][ng][1][r];
          const uint16_t hb = f32_to_bf16(hf);
          g.h[size_t(tok) * g.N + n] = hb;
          g.h_lo[size_t(tok) * g.N + n] = f32_to_bf16(hf - bf16_to_f32(hb));
        } else {
          g.y[size_t(tok) * g.N + n] = acc[mi][ng][0][r];
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) f32_to_bf16_kernel(const float *__restrict__ x, uint16_t *__restrict__ y,
                                                          int64_t n) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 v = *reinterpret_cast<const float4 *>(x + i);
  *reinterpret_cast<uint2 *>(y + i) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

template <bool GATEUP>
static hipError_t launch_q8_dense(const DenseArgs &g, hipStream_t stream) {
  using Gm = DenseGeo<GATEUP>;
  if (g.N % Gm::BN || g.K % KS) return hipErrorNotSupported;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&q8_dense_kernel<GATEUP>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Gm::SMEM);
  if (err != hipSuccess) return err;
  int grid = (g.T + Gm::BM - 1) / Gm::BM * (g.N / Gm::BN);
  grid = (grid + 7) & ~7;
  BM_LAUNCH(GATEUP ? "shared_gateup_gemm_kernel" : "shared_down_gemm_kernel", q8_dense_kernel<GATEUP>, dim3(grid),
            dim3(512), Gm::SMEM, stream, g);
  return hipGetLastError();
}

static hipError_t launch_q8_expand(const void *blocks, int N, int K, uint8_t *out, hipStream_t stream) {
  const int64_t n = int64_t(N / 16) * (K / 32) * 64;
  BM_LAUNCH("q8_expand_kernel", q8_expand_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
            static_cast<const uint8_t *>(blocks), N, K, out);
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
    // shared expert: expand Q8_0 to exact bf16 codes (MFMA operand order) + float scales, then dense GEMMs
    const size_t xb = size_t(a.F) * a.D / 512 * Q8X_CHUNK;  // expanded bytes per matrix
    uint8_t *sw = reinterpret_cast<uint8_t *>(a.sw_bf16);
    if ((err = launch_q8_expand(a.sg, a.F, a.D, sw, stream)) != hipSuccess) return err;
    if ((err = launch_q8_expand(a.su, a.F, a.D, sw + xb, stream)) != hipSuccess) return err;
    if ((err = launch_q8_expand(a.sd, a.D, a.F, sw + 2 * xb, stream)) != hipSuccess) return err;
    DenseArgs s{};
    s.T = a.T;
    s.K = a.D;
    s.N = a.F;
    s.a = x;
    s.c0 = sw;
    s.c1 = sw + xb;
    s.h = a.hs;
    s.h_lo = a.hs_lo;
    if ((err = launch_q8_dense<true>(s, stream)) != hipSuccess) return err;
    s.K = a.F;
    s.N = a.D;
    s.a = a.hs;
    s.a_lo = a.hs_lo;
    s.c0 = sw + 2 * xb;
    s.c1 = nullptr;
    s.y = a.ys;
    if ((err = launch_q8_dense<false>(s, stream)) != hipSuccess) return err;
  }
  return launch_combine(a.y, a.sg ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        a.x_res, a.x_next, stream);
}

}  // namespace bm
