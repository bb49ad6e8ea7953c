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

// four codes (bytes 0..3, each 0..3) -> two bf16 pairs via a 4-entry table
BM_DEVICE void lookup4(uint32_t codes, uint32_t tlo, uint32_t thi, uint32_t &p01, uint32_t &p23) {
  const uint32_t lo = __builtin_amdgcn_perm(0u, tlo, codes);
  const uint32_t hi = __builtin_amdgcn_perm(0u, thi, codes);
  p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// bf16 bits of a small non-negative integer (exact)
BM_DEVICE uint32_t bf16_of_small(uint32_t v) { return __float_as_uint(float(v)) >> 16; }

// Q2 step operands of one lane for one weight row's super-block:
//   Bm[t]: exact bf16 sc*q for MFMA step t; Bn: exact bf16 m for the min MFMA;
//   d, dmin.  `tab` holds per scale value sc the table (tlo, thi) of sc*q.
BM_DEVICE void q2_operands(const uint8_t *sb, int g, const uint2 *tab, uint32_t (&Bm)[8][4], uint32_t (&Bn)[4],
                           float &d, float &dmin) {
  const int h = g >> 1, p = g & 1;
  const u32x4 q = *reinterpret_cast<const u32x4_a4 *>(sb + 16 + 32 * h + 16 * p);
  const u32x2 sc = *reinterpret_cast<const u32x2_a4 *>(sb + 8 * h);
  const u32x2 mn = *reinterpret_cast<const u32x2_a4 *>(sb + 8 * p);
  const uint32_t dd = *reinterpret_cast<const uint32_t *>(sb + 80);
  d = half_to_f32(dd & 0xFFFFu);
  dmin = half_to_f32(dd >> 16);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  const uint32_t sw0 = sc.x >> (8 * p), sw1 = sc.y >> (8 * p);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t scv = ((s < 2 ? sw0 : sw1) >> (16 * (s & 1))) & 0xFu;
    const uint2 t = tab[scv];
#pragma unroll
    for (int j8 = 0; j8 < 2; ++j8) {
      uint32_t *o = Bm[2 * s + j8];
      lookup4((w[2 * j8] >> (2 * s)) & 0x03030303u, t.x, t.y, o[0], o[1]);
      lookup4((w[2 * j8 + 1] >> (2 * s)) & 0x03030303u, t.x, t.y, o[2], o[3]);
    }
  }
  // min nibbles of sub-blocks 8p .. 8p+7
  const uint32_t m0 = (mn.x >> 4) & 0x0F0F0F0Fu, m1 = (mn.y >> 4) & 0x0F0F0F0Fu;
  Bn[0] = bf16_of_small(m0 & 0xFFu) | (bf16_of_small((m0 >> 8) & 0xFFu) << 16);
  Bn[1] = bf16_of_small((m0 >> 16) & 0xFFu) | (bf16_of_small(m0 >> 24) << 16);
  Bn[2] = bf16_of_small(m1 & 0xFFu) | (bf16_of_small((m1 >> 8) & 0xFFu) << 16);
  Bn[3] = bf16_of_small((m1 >> 16) & 0xFFu) | (bf16_of_small(m1 >> 24) << 16);
}

BM_DEVICE f32x4_t mfma(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c) {
  u32x4 av = {a[0], a[1], a[2], a[3]};
  u32x4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                 c, 0, 0, 0);
}

BM_DEVICE void lds_a(const uint16_t *p, uint32_t (&A)[4]) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  A[0] = v.x;
  A[1] = v.y;
  A[2] = v.z;
  A[3] = v.w;
}

// ALO: the A rows arrive as bf16 hi + lo parts (the down projection's h); both
// parts multiply the same B operand into the same accumulator.
template <bool GATEUP, int BF, bool ALO>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(GemmArgs a) {
  __shared__ uint16_t As[BM_ * LDS_ROW];
  __shared__ uint16_t As_lo[ALO ? BM_ * LDS_ROW : 8];
  __shared__ uint16_t Xs[BM_ * XS_ROW];
  __shared__ uint2 tab[16];
  const int nt_n = a.N / BN_;
  // XCD-aware remap of the block index (grid is a multiple of 8)
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int mt = L / nt_n, ntile = L % nt_n;
  if (mt >= a.m_tiles) return;
  int e = 0, valid, base;
  if (a.dense) {
    const int m0 = mt * BM_;
    if (m0 >= a.T) return;
    valid = min(BM_, a.T - m0);
    base = m0;
  } else {
    if (mt >= a.tile_off[a.E]) return;
    int lo = 0, hi = a.E;  // largest e with tile_off[e] <= mt
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_off[mid] <= mt) lo = mid; else hi = mid;
    }
    e = lo;
    const int m0 = (mt - a.tile_off[e]) * BM_;
    valid = min(BM_, a.counts[e] - m0);
    base = a.offsets[e] + m0;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, nl = lane & 15;
  const int n = ntile * BN_ + wave * 16 + nl;  // this lane's weight row
  if (BF == BF_Q2 && tid < 16) {
    // table of bf16(sc*q), q = 0..3, for scale sc = tid: low bytes, high bytes
    uint32_t lo = 0, hi = 0;
    for (int q = 1; q < 4; ++q) {
      const uint32_t v = bf16_of_small(uint32_t(tid * q));
      lo |= (v & 0xFFu) << (8 * q);
      hi |= (v >> 8) << (8 * q);
    }
    tab[tid] = make_uint2(lo, hi);
  }
  // A staging slice of this thread: row ar, 64 elements at 64*aq
  const int ar = tid >> 2, aq = tid & 3;
  int a_row = -1;
  if (ar < valid) {
    if (a.dense) {
      a_row = base + ar;
    } else {
      const int pr = a.perm[base + ar];
      a_row = a.a_by_pair ? pr : pr / a.k;
    }
  }
  const uint16_t *a_src = a_row >= 0 ? a.a + size_t(a_row) * a.K : nullptr;
  const uint16_t *a_src_lo = (ALO && a_row >= 0) ? a.a_lo + size_t(a_row) * a.K : nullptr;
  size_t row_bytes, b_off;
  if (BF == BF_Q2) {
    row_bytes = size_t(a.K) / 256 * 84;
    b_off = size_t(e) * a.b_expert_stride + size_t(n) * row_bytes;
  } else {
    row_bytes = size_t(a.K) * 2;
    b_off = size_t(n) * row_bytes;
  }

  f32x4_t acc0[4], acc1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc0[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
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
    if (BF == BF_Q2) {
      // sub-block sums (16 values each) of this slice, split into bf16 hi + lo
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s = 0.f;
        const uint4 u0 = av[2 * j], u1 = av[2 * j + 1];
        const uint32_t w8[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) s += bf16_lo(w8[i]) + bf16_hi(w8[i]);
        if constexpr (ALO) {
          const uint4 l0 = al[2 * j], l1 = al[2 * j + 1];
          const uint32_t v8[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) s += bf16_lo(v8[i]) + bf16_hi(v8[i]);
        }
        const uint16_t shi = f32_to_bf16(s);
        Xs[ar * XS_ROW + 4 * aq + j] = shi;
        Xs[ar * XS_ROW + 16 + 4 * aq + j] = f32_to_bf16(s - bf16_to_f32(shi));
      }
    }
    __syncthreads();
    if constexpr (BF == BF_Q2) {
      const int h = g >> 1, p = g & 1;
      uint32_t Bm0[8][4], Bn0[4], Bm1[8][4], Bn1[4];
      float d0, dm0, d1 = 0.f, dm1 = 0.f;
      q2_operands(a.b0 + b_off + size_t(kb) * 84, g, tab, Bm0, Bn0, d0, dm0);
      if constexpr (GATEUP) q2_operands(a.b1 + b_off + size_t(kb) * 84, g, tab, Bm1, Bn1, d1, dm1);
      f32x4_t cm0[4], cm1[4], cn0[4], cn1[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) cm0[mi] = cm1[mi] = zero;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ko = 128 * h + 32 * (t >> 1) + 16 * p + 8 * (t & 1);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          uint32_t A[4];
          lds_a(&As[(16 * mi + nl) * LDS_ROW + ko], A);
          cm0[mi] = mfma(A, Bm0[t], cm0[mi]);
          if constexpr (GATEUP) cm1[mi] = mfma(A, Bm1[t], cm1[mi]);
          if constexpr (ALO) {
            lds_a(&As_lo[(16 * mi + nl) * LDS_ROW + ko], A);
            cm0[mi] = mfma(A, Bm0[t], cm0[mi]);
          }
        }
      }
      // min term: k-slot (g, i) = part g/2 (hi, lo) of sub-block sum 8p + i
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        uint32_t A[4];
        lds_a(&Xs[(16 * mi + nl) * XS_ROW + 16 * (g >> 1) + 8 * p], A);
        cn0[mi] = mfma(A, Bn0, zero);
        if constexpr (GATEUP) cn1[mi] = mfma(A, Bn1, zero);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc0[mi][r] = __builtin_fmaf(d0, cm0[mi][r], __builtin_fmaf(-dm0, cn0[mi][r], acc0[mi][r]));
          if constexpr (GATEUP)
            acc1[mi][r] = __builtin_fmaf(d1, cm1[mi][r], __builtin_fmaf(-dm1, cn1[mi][r], acc1[mi][r]));
        }
      }
    } else {
      // expanded Q8_0: exact int8 codes as bf16, one float d per 32 weights
      const uint16_t *r0 = reinterpret_cast<const uint16_t *>(a.b0 + b_off) + kb * KS;
      const uint16_t *r1 = GATEUP ? reinterpret_cast<const uint16_t *>(a.b1 + b_off) + kb * KS : nullptr;
      const float *s0 = a.d0 + size_t(n) * (a.K / 32) + kb * 8;
      const float *s1 = GATEUP ? a.d1 + size_t(n) * (a.K / 32) + kb * 8 : nullptr;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t B0[4], B1[4];
        lds_a(r0 + 32 * t + 8 * g, B0);
        const float e0 = s0[t];
        float e1 = 0.f;
        if constexpr (GATEUP) {
          lds_a(r1 + 32 * t + 8 * g, B1);
          e1 = s1[t];
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          uint32_t A[4];
          lds_a(&As[(16 * mi + nl) * LDS_ROW + 32 * t + 8 * g], A);
          f32x4_t c0 = mfma(A, B0, zero);
          if constexpr (ALO) {
            uint32_t Al[4];
            lds_a(&As_lo[(16 * mi + nl) * LDS_ROW + 32 * t + 8 * g], Al);
            c0 = mfma(Al, B0, c0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc0[mi][r] = __builtin_fmaf(e0, c0[r], acc0[mi][r]);
          if constexpr (GATEUP) {
            const f32x4_t c1 = mfma(A, B1, zero);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc1[mi][r] = __builtin_fmaf(e1, c1[r], acc1[mi][r]);
          }
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
      const int orow = a.dense ? base + m : a.perm[base + m];
      if constexpr (GATEUP) {
        const float hf = silu(acc0[mi][r]) * acc1[mi][r];
        const uint16_t hb = f32_to_bf16(hf);
        a.h_out[size_t(orow) * a.N + n] = hb;
        a.h_lo_out[size_t(orow) * a.N + n] = f32_to_bf16(hf - bf16_to_f32(hb));
      } else {
        a.y_out[size_t(orow) * a.N + n] = acc0[mi][r];
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

static hipError_t launch_gemm(const GemmArgs &g, bool gateup, bool q2, hipStream_t stream) {
  int grid = g.m_tiles * (g.N / BN_);
  grid = (grid + 7) & ~7;
  if (gateup && q2)
    BM_LAUNCH("grouped_gemm_kernel", (grouped_gemm_kernel<true, BF_Q2, false>), dim3(grid), dim3(256), 0, stream, g);
  else if (gateup)
    BM_LAUNCH("grouped_gemm_kernel", (grouped_gemm_kernel<true, BF_Q8X, false>), dim3(grid), dim3(256), 0, stream, g);
  else if (q2)
    BM_LAUNCH("grouped_gemm_kernel", (grouped_gemm_kernel<false, BF_Q2, true>), dim3(grid), dim3(256), 0, stream, g);
  else
    BM_LAUNCH("grouped_gemm_kernel", (grouped_gemm_kernel<false, BF_Q8X, true>), dim3(grid), dim3(256), 0, stream, g);
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
  if ((err = launch_plan(a.ids, a.T, a.k, a.E, BM_, p, stream)) != hipSuccess) return err;
  const int P = a.T * a.k;
  const int m_slots = (P + BM_ - 1) / BM_ + min(a.E, P);
  const size_t q2_stride = size_t(a.F) * a.D / 256 * 84;

  GemmArgs g{};
  g.dense = 0;
  g.T = a.T;
  g.k = a.k;
  g.E = a.E;
  g.perm = p.perm;
  g.offsets = p.offsets;
  g.counts = p.counts;
  g.tile_off = p.tile_off;
  g.m_tiles = m_slots;
  // routed gate/up: A = x rows by token, N = F
  g.a = x;
  g.a_by_pair = 0;
  g.K = a.D;
  g.N = a.F;
  g.b0 = a.wg;
  g.b1 = a.wu;
  g.b_expert_stride = q2_stride;
  g.h_out = a.h;
  g.h_lo_out = a.h_lo;
  if ((err = launch_gemm(g, true, true, stream)) != hipSuccess) return err;
  // routed down: A = h rows (hi + lo) by pair, N = D
  g.a = a.h;
  g.a_lo = a.h_lo;
  g.a_by_pair = 1;
  g.K = a.F;
  g.N = a.D;
  g.b0 = a.wd;
  g.b1 = nullptr;
  g.y_out = a.y;
  if ((err = launch_gemm(g, false, true, stream)) != hipSuccess) return err;

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
    if ((err = launch_gemm(s, true, false, stream)) != hipSuccess) return err;
    s.a = a.hs;
    s.a_lo = a.hs_lo;
    s.K = a.F;
    s.N = a.D;
    s.b0 = reinterpret_cast<const uint8_t *>(a.sw_bf16 + 2 * nw);
    s.b1 = nullptr;
    s.d0 = sd + 2 * nw / 32;
    s.d1 = nullptr;
    s.y_out = a.ys;
    if ((err = launch_gemm(s, false, false, stream)) != hipSuccess) return err;
  }
  return launch_combine(a.y, a.sg ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        stream);
}

}  // namespace bm
