// Prefill path: grouped GEMM over the experts' token groups on MFMA.
//
// "Strata-DSV4.1", §Results / §How it works: a prompt chunk runs each layer's
// routed experts as grouped expert matrix products (there on int8 tensor
// cores).  Here they run on v_mfma_f32_16x16x32_bf16 with float32
// accumulation, and the weights enter the matrix cores exactly:
//   w_k = d*sc_s*q_k - dmin*m_s   (k in sub-block s of a super-block)
//   sum_k w_k x_k = d * sum_k (sc_s q_k) x_k  -  dmin * sum_s m_s X_s
// with X_s the sub-block sums of x.  sc*q (0..45) and m (0..15) are small
// integers, exact in bf16, so per 256-wide K-step (one super-block of every
// weight row) the block runs 8 MFMAs on B = sc*q and one MFMA on B = m against
// A = X_s split into bf16 hi + lo parts, then applies d and dmin in float32.
// The Q8_0 shared expert likewise multiplies exact int8 codes and applies d
// once per 32-weight block.  SwiGLU (gate is the SiLU operand, "run the
// DeepSeek-V4-Flash-Vision tower on CUDA" commit notes) is fused into the
// gate/up epilogue; h is stored as bf16; the combine runs afterwards in the
// fixed slot order.
//
// Tiling.  A block owns one 64-token M-tile of one expert (tiles listed by the
// plan, 64 tokens each) and 64 output rows (N); each of its 4 waves owns 16
// weight rows.  Per K-step of 256:
//  * the 64 activation rows of the M-tile (gathered through the plan's pair
//    permutation) are staged in LDS with their 16 sub-block sums;
//  * each lane expands the 16 code bytes of one quarter of its weight row's
//    super-block into B operands by table lookup (v_perm_b32 on a 4-entry
//    table of bf16(sc*q), low bytes, high bytes, interleave);
//  * lane k-slots: lane group g = l/16 owns half h = g/2 and sub-block parity
//    p = g%2; MFMA step t covers sub-block s = t/2, 8 weights from 8*(t%2), so
//    one lane's 8 values are 8 consecutive weights of one sub-block and the
//    matching activations are 16 contiguous bytes of LDS.
// MFMA 16x16x32 lane layout: A lane l holds row l%16, k = 8*(l/16)+0..7; B
// lane l holds column l%16, the same k; D lane l holds rows 4*(l/16)+0..3 of
// column l%16.
//
// Blocks are remapped so that each of the 8 XCDs (blocks are dealt to XCDs
// round-robin) takes a contiguous range of tiles: the N-tiles of one M-tile
// then share that XCD's L2 for the activation rows.
#include "common.h"
#include "internal.h"
#include "mfma_q2.h"

namespace bm {

constexpr int BM_ = PREFILL_BM;  // 64 tokens per M-tile
constexpr int BN_ = 64;          // output rows per block
constexpr int KS = 256;          // K per step
constexpr int LDS_ROW = KS + 8;  // bf16 elements per LDS activation row (16-byte pad)
constexpr int XS_ROW = 32 + 8;   // bf16 per LDS row of sub-block sums (16 hi, 16 lo, pad)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 __attribute__((aligned(4))) u32x4_a4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 __attribute__((aligned(4))) u32x2_a4;

enum { BF_Q2 = 0, BF_Q8X = 1 };

struct GemmArgs {
  // M side
  int dense;                  // 1: rows are tokens 0..T-1 (shared expert)
  int T, k, E;
  const int32_t *perm;        // grouped: pair indices by expert
  const int32_t *offsets;     // [E+1]
  const int32_t *counts;      // [E]
  const int32_t *tile_off;    // [E+1]
  // A: bf16 rows of length K; row index = token (gate/up) or pair/token (down)
  const uint16_t *a;
  const uint16_t *a_lo;       // down: bf16 lo parts of the A rows (A = a + a_lo), else null
  int a_by_pair;              // grouped down: A row = pair index
  int K, N;
  // B: Q2 super-blocks [E][N][K/256], or expanded Q8_0 (bf16 codes [N][K], float d [N][K/32])
  const uint8_t *b0, *b1;     // b1: up matrix (gate/up)
  const float *d0, *d1;       // Q8X scales
  size_t b_expert_stride;     // bytes per expert matrix (Q2)
  // out
  uint16_t *h_out;            // gate/up: [rows][N] bf16 hi part of h
  uint16_t *h_lo_out;         // gate/up: [rows][N] bf16 lo part of h
  float *y_out;               // down: [rows][N] float32
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

// ---- routed Q2 grouped GEMM with asynchronous activation staging ---------------
// Block tile: BMt = 16 MI rows (tokens or pairs of one expert) x BNt = 4 waves x
// 16 NG weight rows; K-steps of one super-block (256).  While step kb
// computes, the BMt activation rows of step kb+1 (and their lo parts for the
// down projection) are copied into the other half of a double LDS buffer with
// direct-to-LDS loads (one 512-byte row per instruction), and each lane's
// weight bytes of kb+1 are loaded into registers; the block waits for both
// once per step.  The sub-block sums of the step's rows are formed from LDS.
// Per wave and step: 8 x MI x NG x NM main MFMAs (+ the lo parts) on exact
// B = bf16(128 + sc*q), MI MFMAs for the offset and MI x NG x NM min MFMAs
// against the sums.
// One K-step of the routed grouped GEMM for a block's wave: the sub-block
// sums of the step's BMt activation rows (all parts, from the LDS half cb) into
// Xs as bf16 hi + lo, then per wave: -128 x the rows' super-block sums as the
// start of the main accumulators, eight MFMA steps on the offset operands of
// the weight bytes cur, the min term against the sums, and d, dmin into acc.
// Contains one block barrier (the sums are shared by the block's waves).
template <int MI, int NG, int NM, bool ALO>
BM_DEVICE void q2_step(const uint8_t *cb, uint16_t *Xs, const Q2Raw (&cur)[NG][NM], f32x4_t (&acc)[MI][NG][NM]) {
  constexpr int BMt = 16 * MI, PARTS = ALO ? 2 : 1;
  constexpr int ROWB = LDS_ROW * 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 4, nl = lane & 15, p = g & 1;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  // sub-block sums of the step's rows (all parts), split into bf16 hi + lo
  for (int idx = tid; idx < BMt * 16; idx += 256) {
    const int r = idx >> 4, sb = idx & 15;
    float sum = 0.f;
#pragma unroll
    for (int part = 0; part < PARTS; ++part) {
      const uint4 *v = reinterpret_cast<const uint4 *>(cb + (part * BMt + r) * ROWB + sb * 32);
      const uint4 v0 = v[0], v1 = v[1];
      const uint32_t w8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) sum = dot2_bf16(w8[i], 0x3F803F80u, sum);  // + lo + hi (bf16 1.0 pair)
    }
    const uint16_t shi = f32_to_bf16(sum);
    Xs[r * XS_ROW + q2_sum_slot(sb, 0)] = shi;
    Xs[r * XS_ROW + q2_sum_slot(sb, 1)] = f32_to_bf16(sum - bf16_to_f32(shi));
  }
  __syncthreads();
  // the step's sub-block sums (hi + lo, min-slot order) and -128 times the
  // sum of each row's activations over the super-block: the main
  // accumulators start from it, which removes the 128 offset of the main
  // operands without a subtraction per output
  uint32_t As[MI][4];
  f32x4_t cm[MI][NG][NM];
  {
    const uint32_t Bm128[4] = {0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u};  // bf16 -128
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      ld16(Xs + (16 * mi + nl) * XS_ROW + 8 * g, As[mi]);
      const f32x4_t cx = mfma16(As[mi], Bm128, zero);
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) cm[mi][ng][m] = cx;
    }
  }
  const uint16_t *Ah = reinterpret_cast<const uint16_t *>(cb);
  const uint16_t *Al = reinterpret_cast<const uint16_t *>(cb + BMt * ROWB);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int ko = q2_kofs(t, g);
    uint32_t B[NG][NM][4];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) q2_main_operand(cur[ng][m], p, t, B[ng][m]);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      uint32_t A[4];
      ld16(Ah + (16 * mi + nl) * LDS_ROW + ko, A);
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) cm[mi][ng][m] = mfma16(A, B[ng][m], cm[mi][ng][m]);
      if constexpr (ALO) {
        ld16(Al + (16 * mi + nl) * LDS_ROW + ko, A);
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) cm[mi][ng][0] = mfma16(A, B[ng][0], cm[mi][ng][0]);
      }
    }
  }
  // min term against the sums, then d and dmin of the super-block
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      uint32_t Bn[4];
      q2_min_operand(cur[ng][m], p, Bn);
      const float d = q2_d(cur[ng][m]), dm = q2_dmin(cur[ng][m]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const f32x4_t cn = mfma16(As[mi], Bn, zero);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[mi][ng][m][r] = __builtin_fmaf(d, cm[mi][ng][m][r], __builtin_fmaf(-dm, cn[r], acc[mi][ng][m][r]));
      }
    }
  }
}

template <bool GATEUP, int MI, int NG, bool ALO>
__global__ void __launch_bounds__(256, 2) q2_gemm_kernel(GemmArgs a) {
  constexpr int BMt = 16 * MI, BNt = 64 * NG, PARTS = ALO ? 2 : 1, NM = GATEUP ? 2 : 1;
  constexpr int ROWB = LDS_ROW * 2;        // bytes per LDS activation row
  constexpr int BUF = PARTS * BMt * ROWB;  // bytes per buffer half
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_q2[];
  uint16_t *Xs = reinterpret_cast<uint16_t *>(smem_q2 + 2 * BUF);  // [BMt][XS_ROW]
  int32_t *rows = reinterpret_cast<int32_t *>(Xs + BMt * XS_ROW);  // [BMt] activation row, -1: none
  const int nt_n = a.N / BNt;
  // XCD-aware remap of the block index (grid is a multiple of 8)
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int mt = L / nt_n, ntile = L % nt_n;
  if (mt >= a.m_tiles || mt >= a.tile_off[a.E]) return;
  int lo = 0, hi = a.E;  // largest e with tile_off[e] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int m0 = (mt - a.tile_off[e]) * BMt;
  const int valid = min(BMt, a.counts[e] - m0);
  const int base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, nl = lane & 15;
  for (int i = tid; i < BMt; i += 256) {
    int r = -1;
    if (i < valid) {
      const int pr = a.perm[base + i];
      r = a.a_by_pair ? pr : pr / a.k;
    }
    rows[i] = r;
  }
  __syncthreads();
  const size_t row_bytes = size_t(a.K) / 256 * 84;
  const uint8_t *wb[2] = {a.b0 + size_t(e) * a.b_expert_stride, NM > 1 ? a.b1 + size_t(e) * a.b_expert_stride : nullptr};
  const int n_w = ntile * BNt + wave * 16 * NG + nl;  // weight row of group 0; group ng adds 16 ng
  auto issue_a = [&](int kb, int half) {
    uint8_t *dst = smem_q2 + half * BUF;
    for (int i = wave; i < PARTS * BMt; i += 4) {
      const int part = i / BMt, r = i % BMt;
      const int src_row = rows[r];
      if (src_row >= 0 && lane < 32) {
        const uint16_t *src = (part ? a.a_lo : a.a) + size_t(src_row) * a.K + kb * KS + 8 * lane;
        lds_dma16(src, lds_offset(dst + (part * BMt + r) * ROWB));
      }
    }
  };
  auto load_b = [&](int kb, Q2Raw (&raw)[NG][NM]) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) raw[ng][m] = q2_load(wb[m] + size_t(n_w + 16 * ng) * row_bytes + size_t(kb) * 84, g);
  };
  f32x4_t acc[MI][NG][NM];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[mi][ng][m] = zero;
  Q2Raw cur[NG][NM];
  issue_a(0, 0);
  load_b(0, cur);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int ng = 0; ng < NG; ++ng)
#pragma unroll
    for (int m = 0; m < NM; ++m) q2_settle(cur[ng][m]);
  __syncthreads();
  const int nsteps = a.K / KS;
  for (int kb = 0; kb < nsteps; ++kb) {
    Q2Raw nxt[NG][NM];
    if (kb + 1 < nsteps) {
      issue_a(kb + 1, (kb + 1) & 1);
      load_b(kb + 1, nxt);
    }
    q2_step<MI, NG, NM, ALO>(smem_q2 + (kb & 1) * BUF, Xs, cur, acc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // step kb+1's rows and weight bytes have landed
    __syncthreads();  // ... and this step's buffer half and sums are no longer read
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        cur[ng][m] = nxt[ng][m];
        q2_settle(cur[ng][m]);
      }
  }
  // epilogue: lane holds rows 16 mi + 4 g + r of column n_w + 16 ng
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mrow = 16 * mi + 4 * g + r;
      if (mrow >= valid) continue;
      const size_t orow = size_t(a.perm[base + mrow]);
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        const int n = n_w + 16 * ng;
        if constexpr (GATEUP) {
          const float hf = silu(acc[mi][ng][0][r]) * acc[mi][ng][NM - 1][r];
          const uint16_t hb = f32_to_bf16(hf);
          a.h_out[orow * a.N + n] = hb;
          a.h_lo_out[orow * a.N + n] = f32_to_bf16(hf - bf16_to_f32(hb));
        } else {
          a.y_out[orow * a.N + n] = acc[mi][ng][0][r];
        }
      }
    }
  }
}

// Routed gate/up grouped GEMM with the weight bytes two steps ahead.  Same
// tiles, operands and arithmetic as q2_gemm_kernel<true, ...>; the activation
// rows of step kb+1 are loaded into registers at the start of step kb and
// written to the other LDS half at its end, and the weight bytes of step kb+2
// are loaded into the third of three register sets.  Every load is a plain
// one, so the compiler's waits count them exactly: computing step kb waits
// only for its own weight bytes (requested two steps earlier), writing the
// activations of kb+1 only for those.  The K loop is unrolled by three so the
// register sets rotate without copies.
template <int MI, int NG>
__global__ void __launch_bounds__(256, 2) q2_gemm_p3_kernel(GemmArgs a) {
  constexpr int BMt = 16 * MI, BNt = 64 * NG, NM = 2;
  constexpr int ROWB = LDS_ROW * 2;              // bytes per LDS activation row
  constexpr int BUF = BMt * ROWB;                // bytes per buffer half
  constexpr int APT = BMt * KS * 2 / 256 / 16;   // 16-byte activation slices per thread and step
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_q2[];
  uint16_t *Xs = reinterpret_cast<uint16_t *>(smem_q2 + 2 * BUF);  // [BMt][XS_ROW]
  int32_t *rows = reinterpret_cast<int32_t *>(Xs + BMt * XS_ROW);  // [BMt] activation row, -1: none
  const int nt_n = a.N / BNt;
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);  // XCD-aware remap (grid is a multiple of 8)
  const int mt = L / nt_n, ntile = L % nt_n;
  if (mt >= a.m_tiles || mt >= a.tile_off[a.E]) return;
  int lo = 0, hi = a.E;  // largest e with tile_off[e] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int m0 = (mt - a.tile_off[e]) * BMt;
  const int valid = min(BMt, a.counts[e] - m0);
  const int base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, nl = lane & 15;
  for (int i = tid; i < BMt; i += 256) {
    int r = -1;
    if (i < valid) r = a.perm[base + i] / a.k;
    rows[i] = r;
  }
  __syncthreads();
  const size_t row_bytes = size_t(a.K) / 256 * 84;
  const uint8_t *wb[2] = {a.b0 + size_t(e) * a.b_expert_stride, a.b1 + size_t(e) * a.b_expert_stride};
  const int n_w = ntile * BNt + wave * 16 * NG + nl;
  // this thread's activation slices: 16 bytes each; slice sl is 16-byte piece
  // sl % 32 of row sl / 32 (a step's row is 512 bytes)
  const uint16_t *asrc[APT];
  int adst[APT];
#pragma unroll
  for (int j = 0; j < APT; ++j) {
    const int sl = tid * APT + j, r = sl >> 5, c = sl & 31;
    const int src_row = rows[r];
    asrc[j] = src_row >= 0 ? a.a + size_t(src_row) * a.K + 8 * c : nullptr;
    adst[j] = r * ROWB + 16 * c;
  }
  auto load_a = [&](int kb, uint4 (&av)[APT]) {
#pragma unroll
    for (int j = 0; j < APT; ++j)
      av[j] = asrc[j] ? *reinterpret_cast<const uint4 *>(asrc[j] + kb * KS) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto store_a = [&](int half, const uint4 (&av)[APT]) {
#pragma unroll
    for (int j = 0; j < APT; ++j) *reinterpret_cast<uint4 *>(smem_q2 + half * BUF + adst[j]) = av[j];
  };
  auto load_b = [&](int kb, Q2Raw (&raw)[NG][NM]) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) raw[ng][m] = q2_load(wb[m] + size_t(n_w + 16 * ng) * row_bytes + size_t(kb) * 84, g);
  };
  f32x4_t acc[MI][NG][NM];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[mi][ng][m] = zero;
  const int nsteps = a.K / KS;
  // one K-step: compute with cur (weights of kb), request the weights of kb+2
  // into fill and the activations of kb+1, write those to the other LDS half
  auto step = [&](int kb, const Q2Raw (&cur)[NG][NM], Q2Raw (&fill)[NG][NM]) {
    uint4 av[APT];
    if (kb + 1 < nsteps) load_a(kb + 1, av);
    if (kb + 2 < nsteps) load_b(kb + 2, fill);
    q2_step<MI, NG, NM, false>(smem_q2 + (kb & 1) * BUF, Xs, cur, acc);
    __syncthreads();  // this step's buffer half and sums are no longer read
    if (kb + 1 < nsteps) store_a((kb + 1) & 1, av);
    __syncthreads();  // the next step's activation rows are in LDS
  };
  Q2Raw s0[NG][NM], s1[NG][NM], s2[NG][NM];
  {
    uint4 av[APT];
    load_a(0, av);
    load_b(0, s0);
    if (nsteps > 1) load_b(1, s1);
    store_a(0, av);
    __syncthreads();
  }
  for (int kb = 0; kb < nsteps; kb += 3) {
    step(kb, s0, s2);
    if (kb + 1 < nsteps) step(kb + 1, s1, s0);
    if (kb + 2 < nsteps) step(kb + 2, s2, s1);
  }
  // epilogue: lane holds rows 16 mi + 4 g + r of column n_w + 16 ng
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mrow = 16 * mi + 4 * g + r;
      if (mrow >= valid) continue;
      const size_t orow = size_t(a.perm[base + mrow]);
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        const int n = n_w + 16 * ng;
        const float hf = silu(acc[mi][ng][0][r]) * acc[mi][ng][1][r];
        const uint16_t hb = f32_to_bf16(hf);
        a.h_out[orow * a.N + n] = hb;
        a.h_lo_out[orow * a.N + n] = f32_to_bf16(hf - bf16_to_f32(hb));
      }
    }
  }
}

template <bool GATEUP, int MI, int NG, bool ALO>
static size_t q2_gemm_smem() {
  return size_t(2) * (ALO ? 2 : 1) * 16 * MI * LDS_ROW * 2 + size_t(16) * MI * XS_ROW * 2 + size_t(16) * MI * 4;
}

template <bool GATEUP, int MI, int NG, bool ALO>
static hipError_t launch_q2_gemm(const GemmArgs &g, hipStream_t stream) {
  const size_t smem = q2_gemm_smem<GATEUP, MI, NG, ALO>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&q2_gemm_kernel<GATEUP, MI, NG, ALO>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int grid = g.m_tiles * (g.N / (64 * NG));
  grid = (grid + 7) & ~7;
  BM_LAUNCH(GATEUP ? "routed_gateup_gemm_kernel" : "routed_down_gemm_kernel", (q2_gemm_kernel<GATEUP, MI, NG, ALO>),
            dim3(grid), dim3(256), smem, stream, g);
  return hipGetLastError();
}

template <int MI, int NG>
static hipError_t launch_q2_gemm_p3(const GemmArgs &g, hipStream_t stream) {
  const size_t smem = q2_gemm_smem<true, MI, NG, false>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&q2_gemm_p3_kernel<MI, NG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int grid = g.m_tiles * (g.N / (64 * NG));
  grid = (grid + 7) & ~7;
  BM_LAUNCH("routed_gateup_gemm_kernel", (q2_gemm_p3_kernel<MI, NG>), dim3(grid), dim3(256), smem, stream, g);
  return hipGetLastError();
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

// Routed grouped-GEMM tiles: 16 MI tokens (pairs) x 64 NG weight rows per
// block (MI = 2 or 4: the plan's 32- and 64-row tile lists).  Measured on the
// 4096-token chunk (gate/up, down): MI 2, NG 2 / MI 2, NG 4 take 2.71 / 1.98
// ms; gate/up with 64-token tiles (MI 4, NG 1 or 2) 3.8-4.1 ms; down with
// 64-pair tiles 6.3-10.5 ms (its double-buffered hi + lo rows then leave LDS
// for one block per CU); gate/up NG 1 (4 waves per SIMD) 2.66 ms; down NG 2
// or 1 3.0 / 4.7 ms.
#ifndef BM_PF_GU_MI
#define BM_PF_GU_MI 2
#endif
#ifndef BM_PF_GU_NG
#define BM_PF_GU_NG 2
#endif
#ifndef BM_PF_DN_MI
#define BM_PF_DN_MI 2
#endif
#ifndef BM_PF_DN_NG
#define BM_PF_DN_NG 4
#endif
constexpr int GU_MI = BM_PF_GU_MI, GU_NG = BM_PF_GU_NG, DN_MI = BM_PF_DN_MI, DN_NG = BM_PF_DN_NG;
static_assert((GU_MI == 2 || GU_MI == 4) && (DN_MI == 2 || DN_MI == 4), "M-tiles of 32 or 64 rows");
static_assert(16 * 4 == PREFILL_BM && 16 * 2 == PREFILL_BM_DOWN, "tile lists of the plan");

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
  if ((err = launch_plan(a.ids, a.T, a.k, a.E, BM_, PREFILL_BM_DOWN, p, stream)) != hipSuccess) return err;
  const int P = a.T * a.k;
  const size_t q2_stride = size_t(a.F) * a.D / 256 * 84;

  GemmArgs g{};
  g.dense = 0;
  g.T = a.T;
  g.k = a.k;
  g.E = a.E;
  g.perm = p.perm;
  g.offsets = p.offsets;
  g.counts = p.counts;
  // routed gate/up: A = x rows by token, N = F; tiles of 16 GU_MI tokens x 64 GU_NG rows
  g.tile_off = GU_MI == 4 ? p.tile_off : p.tile_off2;
  g.m_tiles = (P + 16 * GU_MI - 1) / (16 * GU_MI) + min(a.E, P);
  g.a = x;
  g.a_by_pair = 0;
  g.K = a.D;
  g.N = a.F;
  g.b0 = a.wg;
  g.b1 = a.wu;
  g.b_expert_stride = q2_stride;
  g.h_out = a.h;
  g.h_lo_out = a.h_lo;
  if ((err = launch_q2_gemm_p3<GU_MI, GU_NG>(g, stream)) != hipSuccess) return err;
  // routed down: A = h rows (hi + lo) by pair, N = D; tiles of 16 DN_MI pairs x 64 DN_NG rows
  g.tile_off = DN_MI == 4 ? p.tile_off : p.tile_off2;
  g.m_tiles = (P + 16 * DN_MI - 1) / (16 * DN_MI) + min(a.E, P);
  g.a = a.h;
  g.a_lo = a.h_lo;
  g.a_by_pair = 1;
  g.K = a.F;
  g.N = a.D;
  g.b0 = a.wd;
  g.b1 = nullptr;
  g.y_out = a.y;
  if ((err = launch_q2_gemm<false, DN_MI, DN_NG, true>(g, stream)) != hipSuccess) return err;

  if (a.sg) {
    // shared expert: expand Q8_0 to exact bf16 codes + float scales, then dense GEMMs
    const int64_t nw = int64_t(a.F) * a.D;
    float *sd = reinterpret_cast<float *>(a.sw_bf16 + 3 * nw);
    if ((err = launch_q8_expand(a.sg, nw, a.sw_bf16, sd, stream)) != hipSuccess) return err;
    if ((err = launch_q8_expand(a.su, nw, a.sw_bf16 + nw, sd + nw / 32, stream)) != hipSuccess) return err;
    if ((err = launch_q8_expand(a.sd, nw, a.sw_bf16 + 2 * nw, sd + 2 * nw / 32, stream)) != hipSuccess) return err;
    GemmArgs s{};
    s.dense = 1;
    s.T = a.T;
    s.k = a.k;
    s.E = 1;
    s.m_tiles = (a.T + BM_ - 1) / BM_;
    s.a = x;
    s.K = a.D;
    s.N = a.F;
    s.b0 = reinterpret_cast<const uint8_t *>(a.sw_bf16);
    s.b1 = reinterpret_cast<const uint8_t *>(a.sw_bf16 + nw);
    s.d0 = sd;
    s.d1 = sd + nw / 32;
    s.b_expert_stride = 0;
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
