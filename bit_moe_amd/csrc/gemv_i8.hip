// Int8 activation numerics of the expert FFN on the decode path (T <= 8).
//
// Page: "Strata-DSV4.1", §Results and the decode notes of its DeepSeek-V4-Flash
// engine section: the expert products run as integer dot products (dp4a at
// decode) against activations quantised to 8-bit blocks of 32 values with one
// scale each (q8_1), which moves results slightly against the float path.
// The pages name the block format but print neither the quantiser nor the
// integer formulation; the readings taken here:
//
//   quantiser, per block of 32 float32 values v (x of a token, or h of a
//   pair): d = float32(max|v| / 127), q = rint-half-even(float32(v / d)), all
//   q = 0 when the block is zero; per 16-value half b the stored sum
//   s_b = float32(d * sum_{k in b} q_k).  Only IEEE division, rounding and
//   multiplication decide q, d and s, so the result is the same bit for bit on
//   any conforming implementation.
//   Q2 row x quantised activations, per super-block:
//     d_w * sum_b sc_b dx_c(b) (sum_{k in b} q2_k q_k) - dmin_w * sum_b m_b s_b
//   (sub-block b of 16 weights lies in activation block c(b) = b / 2);
//   Q8_0 row: sum over 32-blocks of d_w dx (sum qw qx);
//   h = silu(g) * u in float32, quantised again before the down rows.
//
// Kernels (one wave = 64 lanes; a unit is 64 weights of one row, lane jj of a
// row owns unit jj of every row it visits, LPR = K/64 lanes per row):
//  ffn_i8_kernel<GATEUP>  one block = one job (an expert of the union, or the
//                         shared expert) and a chunk of output rows.  The block
//                         first quantises the job's activation rows into LDS
//                         (two lanes per 32-value block), then each lane takes
//                         its unit's int8 operands, scales and half sums into
//                         registers and streams its rows: codes are masked in
//                         place (codes at bit 2s read 4^s q, s = 3 pre-shifted
//                         to 16 q) and multiplied by the int8 activations with
//                         v_dot4_i32_i8, four weights per instruction; the
//                         integer sub-block sums are exact and get sc (integer
//                         multiply), then dx / 4^s and d in float32.
//  q8_quantize_kernel     the same quantiser over arbitrary rows (test export).
#include "common.h"
#include "decode_job.h"
#include "internal.h"

#include <algorithm>

namespace bm {

namespace {

typedef uint32_t i8u32x4 __attribute__((ext_vector_type(4)));
typedef i8u32x4 __attribute__((aligned(4))) i8u32x4_a4;
typedef uint32_t i8u32x2 __attribute__((ext_vector_type(2)));
typedef i8u32x2 __attribute__((aligned(4))) i8u32x2_a4;

constexpr int QBLK = 32;     // activation values per quantisation block
constexpr int HALF = 16;     // values per stored sum
constexpr int MAX_SLOTS = 8; // activation rows a block quantises at most (tokens or pairs of its job)

// Tokens per pass for calls of T >= 2 (the pass's operands live in registers,
// so it sets the kernel's register budget: at 4 tokens the kernels need ~200
// VGPRs, two waves per SIMD) and row-iteration groups per chunk (routed;
// shared: half) of the gate/up and down launches.  Measured at T = 5 (verify
// batch, ~29 experts): gate/up 49 us with passes of 2 and 32-row chunks
// against 68 us with passes of 4 and 16-row chunks; down 29.5 us with passes
// of 1 (the shared job re-reads its chunk from L2) against 41 us.
#ifndef BM_I8_NT_GU
#define BM_I8_NT_GU 2
#endif
#ifndef BM_I8_NT_DN
#define BM_I8_NT_DN 1
#endif
#ifndef BM_I8_GU_ITERS
#define BM_I8_GU_ITERS 32
#endif
#ifndef BM_I8_DN_ITERS
#define BM_I8_DN_ITERS 16
#endif

BM_DEVICE int sdot4(uint32_t a, uint32_t b, int c) { return __builtin_amdgcn_sdot4(int(a), int(b), c, false); }

// ---- quantiser --------------------------------------------------------------

// One 16-value half of a 32-value block; lane ^ 1 holds the other half, and
// both lanes of the pair must execute this together (the block maximum is
// exchanged between them).  q: the 16 codes as int8 bytes in order; d: the
// block's scale; s: the half's stored sum.
BM_DEVICE void quant_half(const float (&v)[HALF], uint32_t (&q)[4], float &d, float &s) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < HALF; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  d = amax / 127.0f;  // IEEE division (correctly rounded)
  int sum = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t packed = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int qi = d > 0.f ? int(rintf(v[4 * w + b] / d)) : 0;
      sum += qi;
      packed |= (uint32_t(qi) & 0xFFu) << (8 * b);
    }
    q[w] = packed;
  }
  s = d * float(sum);  // sum is an exact integer: one rounding of d * sum
}

// 16 consecutive activations as float32 from a bf16 or float32 row
template <bool SRC_F32>
BM_DEVICE void load_half(const void *row, int c, float (&v)[HALF]) {
  if constexpr (SRC_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(row) + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(row) + c);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 u = p[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_lo(w[j]);
        v[8 * i + 2 * j + 1] = bf16_hi(w[j]);
      }
    }
  }
}

// LDS image of the quantised activation rows of a job: codes Q[slot][K] int8,
// scales DX[slot][K/32], stored sums SX[slot][K/16].
struct QAct {
  uint8_t *Q;
  float *DX, *SX;
};

// slots: rows of the image, min(T * k, MAX_SLOTS): a job has at most T tokens
// (shared) or, like every decode job, at most MAX_SLOTS pairs
BM_HOST_DEVICE inline size_t qact_bytes(int K, int slots) { return size_t(slots) * (K + K / QBLK * 4 + K / HALF * 4); }

BM_DEVICE QAct qact_carve(uint8_t *smem, int K, int slots) {
  QAct r;
  r.Q = smem;
  r.DX = reinterpret_cast<float *>(smem + slots * K);
  r.SX = r.DX + slots * K / QBLK;
  return r;
}

// ---- per-lane operands -------------------------------------------------------

struct XI2 {  // Q2 unit at columns c0 + 32 s + 0..15, s = 0..3
  uint32_t q[4][4];
  float dx[4];  // dx of block (c0 + 32 s) / 32, divided by the code factor 1, 4, 16, 16
  float sx[4];  // stored sum of half (c0 + 32 s) / 16
};

struct XI8 {  // Q8_0 unit at columns c0 .. c0 + 63 (two 32-blocks)
  uint32_t q[16];
  float dx[2];
};

BM_DEVICE float code_factor_inv(int s) { return s == 0 ? 1.f : (s == 1 ? 0.25f : 0.0625f); }

BM_DEVICE void xi2_load(const QAct &A, int K, int slot, int c0, XI2 &X) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = c0 + 32 * s;
    const uint4 v = *reinterpret_cast<const uint4 *>(A.Q + slot * K + c);
    X.q[s][0] = v.x;
    X.q[s][1] = v.y;
    X.q[s][2] = v.z;
    X.q[s][3] = v.w;
    X.dx[s] = A.DX[slot * (K / QBLK) + c / QBLK] * code_factor_inv(s);
    X.sx[s] = A.SX[slot * (K / HALF) + c / HALF];
  }
}

BM_DEVICE void xi8_load(const QAct &A, int K, int slot, int c0, XI8 &X) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = *reinterpret_cast<const uint4 *>(A.Q + slot * K + c0 + 16 * i);
    X.q[4 * i] = v.x;
    X.q[4 * i + 1] = v.y;
    X.q[4 * i + 2] = v.z;
    X.q[4 * i + 3] = v.w;
  }
  X.dx[0] = A.DX[slot * (K / QBLK) + c0 / QBLK];
  X.dx[1] = A.DX[slot * (K / QBLK) + c0 / QBLK + 1];
}

// ---- raw weight units ----------------------------------------------------------

struct RawQ2 {  // quarter q of a super-block: h = q / 2, p = q % 2
  i8u32x4 q;    // code bytes 16 + 32h + 16p .. +15 (sub-blocks 8h + 2s + p at bit 2s)
  i8u32x2 sc;   // scale bytes 8h .. 8h+7
  uint32_t dd;  // d | dmin << 16
};

BM_DEVICE RawQ2 raw_q2(const uint8_t *sb, int h, int p) {
  RawQ2 r;
  r.q = *reinterpret_cast<const i8u32x4_a4 *>(sb + 16 + 32 * h + 16 * p);
  r.sc = *reinterpret_cast<const i8u32x2_a4 *>(sb + 8 * h);
  r.dd = *reinterpret_cast<const uint32_t *>(sb + 80);
  return r;
}

struct RawQ8 {  // two Q8_0 blocks (68 bytes: d0, 32 codes, d1, 32 codes)
  uint32_t dw[17];
};

BM_DEVICE RawQ8 raw_q8(const uint8_t *u68) {
  RawQ8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const i8u32x4 v = *reinterpret_cast<const i8u32x4_a4 *>(u68 + 16 * i);
    r.dw[4 * i] = v.x;
    r.dw[4 * i + 1] = v.y;
    r.dw[4 * i + 2] = v.z;
    r.dw[4 * i + 3] = v.w;
  }
  r.dw[16] = *reinterpret_cast<const uint32_t *>(u68 + 64);
  return r;
}

// One Q2 unit against NT tokens: out[v] += unit's share of the row dot.
template <int NT>
BM_DEVICE void q2_i8_dot(const RawQ2 &u, int p, const XI2 *X, float *out) {
  const float d = half_to_f32(u.dd & 0xFFFFu), dmin = half_to_f32(u.dd >> 16);
  const uint32_t w[4] = {u.q.x, u.q.y, u.q.z, u.q.w};
  const uint32_t sw0 = u.sc.x >> (8 * p), sw1 = u.sc.y >> (8 * p);
  float yd[NT], ym[NT];
#pragma unroll
  for (int v = 0; v < NT; ++v) yd[v] = ym[v] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t sbyte = ((s < 2 ? sw0 : sw1) >> (16 * (s & 1))) & 0xFFu;
    const int sc = int(sbyte & 15u);
    const float mf = float(sbyte >> 4);
    uint32_t M[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) M[j] = s < 3 ? (w[j] & (0x03030303u << (2 * s))) : ((w[j] >> 2) & 0x30303030u);
#pragma unroll
    for (int v = 0; v < NT; ++v) {
      int acc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = sdot4(M[j], X[v].q[s][j], acc);
      // |acc| <= 16 * 48 * 127 and |acc * sc| < 2^24: a 24-bit multiply, exact in float32
      yd[v] = __builtin_fmaf(float(__mul24(acc, sc)), X[v].dx[s], yd[v]);
      ym[v] = __builtin_fmaf(mf, X[v].sx[s], ym[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < NT; ++v) out[v] += d * yd[v] - dmin * ym[v];
}

// One Q8_0 unit (two blocks) against NT tokens.
template <int NT>
BM_DEVICE void q8_i8_dot(const RawQ8 &u, const XI8 *X, float *out) {
  const float dA = half_to_f32(u.dw[0] & 0xFFFFu), dB = half_to_f32(u.dw[8] >> 16);
  uint32_t qa[8];  // codes of block 0 start at byte 2: realign to dwords
#pragma unroll
  for (int i = 0; i < 8; ++i) qa[i] = __builtin_amdgcn_alignbit(u.dw[i + 1], u.dw[i], 16);
#pragma unroll
  for (int v = 0; v < NT; ++v) {
    int a0 = 0, a1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a0 = sdot4(qa[i], X[v].q[i], a0);
      a1 = sdot4(u.dw[9 + i], X[v].q[8 + i], a1);
    }
    out[v] += dA * (float(a0) * X[v].dx[0]) + dB * (float(a1) * X[v].dx[1]);
  }
}

// ---- rows of one job ---------------------------------------------------------

// Rows [r_begin, r_end) of one job for the activation slots t0 .. t0+nt-1 of
// the block's LDS image.  GATEUP: gate and up rows together, h = silu(g) u to
// hf / hsf (float32); else down rows to y / ys.  IS_Q8: shared expert.
template <int NT, bool IS_Q8, bool GATEUP>
BM_DEVICE void i8_rows(const FfnArgs &a, const Job &job, const QAct &A, int t0, int nt, int r_begin, int r_end) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = GATEUP ? a.D : a.F, N = GATEUP ? a.F : a.D;
  const int LPR = K / 64, RPI = 64 / LPR;
  const int jj = lane % LPR, rsub = lane / LPR;
  // the lane's columns do not depend on the row (K is a multiple of 256)
  const int c0 = IS_Q8 ? jj * 64 : 256 * (jj >> 2) + 128 * ((jj & 3) >> 1) + 16 * (jj & 1);
  typename std::conditional<IS_Q8, XI8, XI2>::type X[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int slot = t0 + min(i, nt - 1);
    if constexpr (IS_Q8) xi8_load(A, K, slot, c0, X[i]);
    else xi2_load(A, K, slot, c0, X[i]);
  }
  const size_t mat_bytes = IS_Q8 ? size_t(N) * K / 32 * 34 : size_t(N) * K / 256 * 84;
  const uint8_t *m0, *m1 = nullptr;
  if constexpr (GATEUP) {
    m0 = IS_Q8 ? a.sg : a.wg + size_t(job.e) * mat_bytes;
    m1 = IS_Q8 ? a.su : a.wu + size_t(job.e) * mat_bytes;
  } else {
    m0 = IS_Q8 ? a.sd : a.wd + size_t(job.e) * mat_bytes;
  }
  using Raw = typename std::conditional<IS_Q8, RawQ8, RawQ2>::type;
  constexpr int NM = GATEUP ? 2 : 1;
  auto load_it = [&](int it, Raw (&raw)[NM]) {
    const int r = min(r_begin + it * RPI + rsub, r_end - 1);
    const int unit = r * LPR + jj;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint8_t *base = m ? m1 : m0;
      if constexpr (IS_Q8) raw[m] = raw_q8(base + size_t(unit) * 68);
      else raw[m] = raw_q2(base + size_t(unit >> 2) * 84, (unit & 3) >> 1, unit & 1);
    }
  };
  const int n_it = (r_end - r_begin + RPI - 1) / RPI;
  // the weight loads of DEPTH row iterations of the wave (it, it + 4, ...) are
  // issued before their arithmetic so that their latencies overlap
  constexpr int DEPTH = 2;
  for (int it0 = wave; it0 < n_it; it0 += 4 * DEPTH) {
    Raw raw[DEPTH][NM];
#pragma unroll
    for (int dd = 0; dd < DEPTH; ++dd)
      if (it0 + 4 * dd < n_it) load_it(it0 + 4 * dd, raw[dd]);
#pragma unroll
    for (int dd = 0; dd < DEPTH; ++dd) {
      const int it = it0 + 4 * dd;
      if (it >= n_it) break;
      const int r = r_begin + it * RPI + rsub;
      const bool active = r < r_end;
      float acc[NM][NT];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int v = 0; v < NT; ++v) acc[m][v] = 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if constexpr (IS_Q8) q8_i8_dot<NT>(raw[dd][m], X, acc[m]);
        else q2_i8_dot<NT>(raw[dd][m], jj & 1, X, acc[m]);
      }
#pragma unroll
      for (int v = 0; v < NT; ++v) {
        float s0 = lane_group_sum(acc[0][v], LPR);
        if constexpr (GATEUP) {
          const float s1 = lane_group_sum(acc[1][v], LPR);
          if (active && jj == 0 && v < nt) {
            const int i = t0 + v;
            // slot i: token i of the shared job, pair i of a routed job
            (IS_Q8 ? a.hsf : a.hf)[size_t(jpair(job, i)) * a.F + r] = silu(s0) * s1;
          }
        } else {
          if (active && jj == 0 && v < nt) {
            const int i = t0 + v;
            (IS_Q8 ? a.ys : a.y)[size_t(jpair(job, i)) * a.D + r] = s0;
          }
        }
      }
    }
  }
}

// Quantise the job's activation rows into the block's LDS image: slot i is
// token i of the shared job or pair i of a routed job; its row is x of that
// token (gate/up), or h of that pair / token (down).
template <bool GATEUP, bool XF32>
BM_DEVICE void quantize_job(const FfnArgs &a, const Job &job, const QAct &A) {
  const int K = GATEUP ? a.D : a.F;
  const int halves = K / HALF, total = job.n * halves;
  for (int base = 0; base < total; base += 256) {  // uniform trip count: lane pairs stay together
    const int hidx = base + int(threadIdx.x);
    const bool ok = hidx < total;
    const int slot = ok ? hidx / halves : 0, c = (hidx % halves) * HALF;
    float v[HALF];
    if (ok) {
      if constexpr (GATEUP) {
        const size_t tok = size_t(jtok(a, job, slot));
        load_half<XF32>(XF32 ? static_cast<const void *>(static_cast<const float *>(a.x) + tok * K)
                             : static_cast<const void *>(static_cast<const uint16_t *>(a.x) + tok * K),
                        c, v);
      } else {
        const float *row = (job.e < 0 ? a.hsf : a.hf) + size_t(jpair(job, slot)) * K;
        load_half<true>(row, c, v);
      }
    } else {
#pragma unroll
      for (int i = 0; i < HALF; ++i) v[i] = 0.f;
    }
    uint32_t q[4];
    float d, s;
    quant_half(v, q, d, s);
    if (ok) {
      *reinterpret_cast<uint4 *>(A.Q + slot * K + c) = make_uint4(q[0], q[1], q[2], q[3]);
      if ((hidx & 1) == 0) A.DX[slot * (K / QBLK) + c / QBLK] = d;
      A.SX[slot * halves + c / HALF] = s;
    }
  }
}

// Passes of at most NT tokens over the rows (the operands of a pass live in
// registers).
template <int NT, bool IS_Q8, bool GATEUP>
BM_DEVICE void i8_passes(const FfnArgs &a, const Job &job, const QAct &A, int r_begin, int r_end) {
  for (int t0 = 0; t0 < job.n; t0 += NT) {
    const int nt = min(NT, job.n - t0);
    if (NT == 1 || nt == 1) i8_rows<1, IS_Q8, GATEUP>(a, job, A, t0, 1, r_begin, r_end);
    else if (NT == 2 || nt == 2) i8_rows<(NT >= 2 ? 2 : 1), IS_Q8, GATEUP>(a, job, A, t0, nt, r_begin, r_end);
    else i8_rows<NT, IS_Q8, GATEUP>(a, job, A, t0, nt, r_begin, r_end);
  }
}

// Grid: the shared expert's row chunks first, then u_max routed job slots x
// row chunks (a slot whose expert an earlier pair already chose exits).
// NTMAX: tokens per pass (1 for one-token calls, whose kernel then needs the
// fewest registers).
template <bool GATEUP, bool XF32, int NTMAX>
__global__ void __launch_bounds__(256) ffn_i8_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_i8[];
  const int N = GATEUP ? a.F : a.D;
  const int chunks_s = GATEUP ? a.chunks_sg : a.chunks_sd, rows_s = GATEUP ? a.rows_sg : a.rows_sd;
  const int chunks_r = GATEUP ? a.chunks_gu : a.chunks_dn, rows_r = GATEUP ? a.rows_gu : a.rows_dn;
  Job job;
  int r_begin, r_end;
  if (int(blockIdx.x) < chunks_s) {
    shared_job(a, job);
    r_begin = blockIdx.x * rows_s;
    r_end = min(N, r_begin + rows_s);
  } else {
    const int b = blockIdx.x - chunks_s;
    if (!pair_job_wave(a, b / chunks_r, job)) return;  // uniform over the block
    r_begin = (b % chunks_r) * rows_r;
    r_end = min(N, r_begin + rows_r);
  }
  const QAct A = qact_carve(smem_i8, GATEUP ? a.D : a.F, min(MAX_SLOTS, a.T * a.k));
  quantize_job<GATEUP, XF32>(a, job, A);
  __syncthreads();
  if (job.e < 0) i8_passes<NTMAX, true, GATEUP>(a, job, A, r_begin, r_end);
  else i8_passes<NTMAX, false, GATEUP>(a, job, A, r_begin, r_end);
}

// Quantiser over rows of a [rows][cols] matrix (cols a multiple of 32): one
// lane per 16-value half.
template <bool SRC_F32>
__global__ void __launch_bounds__(256) q8_quantize_kernel(const void *x, int64_t rows, int cols, uint8_t *q,
                                                          float *d, float *s) {
  const int halves = cols / HALF;
  const int64_t total = rows * halves;
  const int64_t hidx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool ok = hidx < total;  // total is even: both lanes of a pair agree
  const int64_t r = ok ? hidx / halves : 0;
  const int c = ok ? int(hidx % halves) * HALF : 0;
  float v[HALF];
  if (ok) {
    load_half<SRC_F32>(SRC_F32 ? static_cast<const void *>(static_cast<const float *>(x) + r * cols)
                               : static_cast<const void *>(static_cast<const uint16_t *>(x) + r * cols),
                       c, v);
  } else {
#pragma unroll
    for (int i = 0; i < HALF; ++i) v[i] = 0.f;
  }
  uint32_t qw[4];
  float dd, ss;
  quant_half(v, qw, dd, ss);
  if (ok) {
    *reinterpret_cast<uint4 *>(q + r * cols + c) = make_uint4(qw[0], qw[1], qw[2], qw[3]);
    if ((hidx & 1) == 0) d[r * (cols / QBLK) + c / QBLK] = dd;
    s[r * halves + c / HALF] = ss;
  }
}

}  // namespace

// Routed chunks of BM_I8_GU_ITERS (gate/up) and BM_I8_DN_ITERS (down) row
// iterations, shared chunks (Q8_0, 3.2x the bytes per row) of half that.
hipError_t launch_decode_ffn_i8(FfnArgs a, bool xf32, hipStream_t stream) {
  a.u_max = a.T * a.k;
  const int rpi_gu = 64 / (a.D / 64), rpi_dn = 64 / (a.F / 64);
  a.rows_gu = std::min(a.F, BM_I8_GU_ITERS * rpi_gu);
  a.chunks_gu = (a.F + a.rows_gu - 1) / a.rows_gu;
  a.rows_sg = std::min(a.F, BM_I8_GU_ITERS / 2 * rpi_gu);
  a.chunks_sg = a.sg ? (a.F + a.rows_sg - 1) / a.rows_sg : 0;
  a.rows_dn = std::min(a.D, BM_I8_DN_ITERS * rpi_dn);
  a.chunks_dn = (a.D + a.rows_dn - 1) / a.rows_dn;
  a.rows_sd = std::min(a.D, BM_I8_DN_ITERS / 2 * rpi_dn);
  a.chunks_sd = a.sd ? (a.D + a.rows_sd - 1) / a.rows_sd : 0;
  if (a.T > MAX_SLOTS) return hipErrorInvalidValue;
  const int slots = std::min(MAX_SLOTS, a.T * a.k);
  const size_t smem_gu = qact_bytes(a.D, slots), smem_dn = qact_bytes(a.F, slots);
  const unsigned grid_gu = unsigned(a.chunks_sg + a.u_max * a.chunks_gu);
  const unsigned grid_dn = unsigned(a.chunks_sd + a.u_max * a.chunks_dn);
  hipError_t err;
  if (a.T == 1) {
    if (xf32) BM_LAUNCH("ffn_i8_gateup_kernel", (ffn_i8_kernel<true, true, 1>), dim3(grid_gu), dim3(256), smem_gu, stream, a);
    else BM_LAUNCH("ffn_i8_gateup_kernel", (ffn_i8_kernel<true, false, 1>), dim3(grid_gu), dim3(256), smem_gu, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    BM_LAUNCH("ffn_i8_down_kernel", (ffn_i8_kernel<false, false, 1>), dim3(grid_dn), dim3(256), smem_dn, stream, a);
  } else {
    if (xf32) BM_LAUNCH("ffn_i8_gateup_kernel", (ffn_i8_kernel<true, true, BM_I8_NT_GU>), dim3(grid_gu), dim3(256), smem_gu, stream, a);
    else BM_LAUNCH("ffn_i8_gateup_kernel", (ffn_i8_kernel<true, false, BM_I8_NT_GU>), dim3(grid_gu), dim3(256), smem_gu, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    BM_LAUNCH("ffn_i8_down_kernel", (ffn_i8_kernel<false, false, BM_I8_NT_DN>), dim3(grid_dn), dim3(256), smem_dn, stream, a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_combine(a.y, a.sd ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        a.x_res, a.x_next, stream);
}

hipError_t launch_quantize_q8(const void *x, bool xf32, int64_t rows, int cols, uint8_t *q, float *d, float *s,
                              hipStream_t stream) {
  const int64_t total = rows * (cols / HALF);
  if (total == 0) return hipSuccess;
  const unsigned grid = unsigned((total + 255) / 256);
  if (xf32)
    BM_LAUNCH("q8_quantize_kernel", q8_quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, x, rows, cols, q, d,
              s);
  else
    BM_LAUNCH("q8_quantize_kernel", q8_quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, x, rows, cols, q, d,
              s);
  return hipGetLastError();
}

}  // namespace bm
