// Int8 numerics of the prefill path: grouped int8 MFMA over the experts' token
// chunks, against activations quantised to 8-bit blocks of 32 (q8_1).
//
// "Strata-DSV4.1", §Results and §How fast: a prompt chunk runs the expert
// products as int8 tensor-core matrix products (MMQ) against q8_1 activations.
// The quantiser and the integer formulation are the int8 decode mode's (the
// readings are at the top of gemv_i8.hip):
//   Q2 row x quantised activations, per super-block:
//     d_w * sum_c dx_c (sum_{b in c} sc_b sum_{k in b} q2_k q_k) - dmin_w * sum_b m_b s_b
//   (activation block c of 32 values holds sub-blocks 2c, 2c + 1); Q8_0 row:
//   sum over 32-blocks of d_w dx (sum qw qx); h = silu(g) * u in float32,
//   quantised again before the down rows.
// On v_mfma_i32_16x16x32_i8 one instruction covers exactly one activation
// block: B holds the int8 products sc_b * q2_k (0..45, exact), A the block's
// int8 activations, so the instruction's int32 result is the block's integer
// sum, exact; dx_c scales it in float32, d_w the super-block's total.  The
// minimum term is one bf16 MFMA of m against the stored sums s_b (bf16 hi + lo
// parts), as in the bf16 path.
//
// Lane layout (16x16x32 i8: A lane l holds row l%16, k = 8*(l/16) .. +7 of the
// instruction's 32; B lane l holds column l%16, the same k): step c of a
// super-block covers its activation block c, so lane group g = l/16 owns
// positions 8*(g%2) .. +7 of sub-block 2c + g/2, i.e. code bytes 16*(g/2) +
// 8*(g%2) .. +7 of half c/4 at shift 2*(c%4): each lane reads 16 code bytes
// (8 per half), the 16 scale bytes and d/dmin of its rows' super-blocks.
//
// Blocking, plan and staging are those of the bf16 grouped GEMM
// (prefill_q2.hip): chunks of up to 48 tokens (gate/up) or 32 pairs (down) of
// one expert x 128 weight rows per block (8 waves x 16 rows); activation rows, their block
// scales and stored sums, and the step's weight bytes (both matrices of gate/up) staged in LDS
// one K-step ahead with direct-to-LDS copies.
#include "common.h"
#include "internal.h"
#include "mfma_q2.h"

namespace bm {

namespace {

constexpr int KS = 256;        // K per step (one super-block of every weight row)
constexpr int ROWB = KS + 16;  // bytes per LDS activation row (int8, 16-byte pad)
constexpr int SUMS = 32;       // bf16 sums per (row, step): 16 sub-blocks x (hi, lo)
constexpr int DXN = KS / 32;   // activation block scales per (row, step)
constexpr int MT_GU = BM_PF_CHUNK_GU, MT_DN = BM_PF_CHUNK_DN;
constexpr int WAVES = 8;

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

template <bool GATEUP>
struct GeoI8 {
  static constexpr int NG = 1;                       // 16-row groups per wave (two would not fit the registers)
  static constexpr int NM = GATEUP ? 2 : 1;          // matrices (gate, up)
  static constexpr int MT = GATEUP ? MT_GU : MT_DN;  // M-tiles per chunk at most
  static constexpr int BN = 16 * NG * WAVES;         // weight rows per block (128)
  static constexpr int BUF = 16 * MT * ROWB;         // bytes of one activation buffer
  static constexpr int SBUF = 16 * MT * SUMS * 2;    // bytes of one sums buffer
  static constexpr int DBUF = 16 * MT * DXN * 4;     // bytes of one scales buffer
  // Each step's weights are staged per matrix in LDS, as the bf16 gate/up
  // kernel does: bytes 0..79 of every row's super-block as 5 16-byte pieces
  // per row, then the rows' d|dmin words (one int8 activation part leaves the
  // LDS room for it in down too).
  static constexpr int WMAT = BN * 84;               // bytes per matrix and step
  static constexpr int WBUF = NM * WMAT;
  static constexpr int WX4 = BN * 5 / 64;            // 64-lane 16-byte copies per matrix and step
  static constexpr int WX1 = BN / 64;                // 64-lane dword copies (d|dmin) per matrix and step
  static constexpr int WPM = WAVES / NM;             // waves copying one matrix
  static constexpr int WC4 = (WX4 + WPM - 1) / WPM;  // 16-byte copies per wave and step
  static constexpr int WC1 = (WX1 + WPM - 1) / WPM;  // dword copies per wave and step
  static constexpr int ROWS_OFF = 2 * (BUF + SBUF + DBUF) + 2 * WBUF;
  static constexpr size_t SMEM = size_t(ROWS_OFF) + 16 * MT * 4;
  static_assert(BN * 5 % 64 == 0 && BN % 64 == 0 && WAVES % NM == 0, "weight copies of whole 64-lane rows");
  static_assert(SMEM <= 160 * 1024, "LDS of one CU");
};

// One lane's bytes of a super-block: 8 code bytes of each half, the 16 scale
// bytes, d | dmin << 16.
struct Q2RawI8 {
  uint32_t q[4];   // half 0: q[0], q[1]; half 1: q[2], q[3]
  uint32_t sc[4];  // scale bytes 0..15
  uint32_t dd;
};

// the step image in LDS holds 80 bytes per row: the code bytes of a lane group
// start 8-byte aligned, the scale bytes 16-byte aligned
typedef uint32_t i8u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t i8u32x4 __attribute__((ext_vector_type(4)));

// One half (h) of a lane's super-block bytes: its 8 code bytes and the scale
// bytes of sub-blocks 8h .. 8h + 7.
struct HalfI8 {
  uint32_t q0, q1, sc0, sc1;
};
BM_DEVICE HalfI8 q2i8_half(const Q2RawI8 &r, int h) {
  return HalfI8{h ? r.q[2] : r.q[0], h ? r.q[3] : r.q[1], h ? r.sc[2] : r.sc[0], h ? r.sc[3] : r.sc[1]};
}

// B operand of step c = 4h + cc (activation block c): the 8 int8 products
// sc * q of sub-block 2c + g/2, positions 8*(g%2) .. +7, from a byte table
// sc * 0x03020100.
BM_DEVICE int64_t q2i8_operand(const HalfI8 &r, int g, int cc) {
  const int sbl = 2 * cc + (g >> 1);  // sub-block within the half
  const uint32_t scb = ((sbl < 4 ? r.sc0 : r.sc1) >> (8 * (sbl & 3))) & 0xFu;
  const uint32_t tab = scb * 0x03020100u;  // bytes 0, sc, 2 sc, 3 sc (3 * 15 < 128)
  const int sh = 2 * cc;
  const uint32_t w0 = __builtin_amdgcn_perm(0u, tab, (r.q0 >> sh) & 0x03030303u);
  const uint32_t w1 = __builtin_amdgcn_perm(0u, tab, (r.q1 >> sh) & 0x03030303u);
  return int64_t(uint64_t(w0) | (uint64_t(w1) << 32));
}

// Min operand (bf16, the bf16 path's slot order): slot i = 2s + part holds m
// of sub-block 8h + 2s + p for lane group g = 2h + p.
BM_DEVICE void q2i8_min_operand(const Q2RawI8 &r, int g, uint32_t (&B)[4]) {
  const bool h = (g >> 1) != 0;
  const int p = g & 1;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t w = h ? r.sc[2 + (s >> 1)] : r.sc[s >> 1];  // selects, no indexing by a lane value
    const uint32_t scw = w >> (8 * p + 16 * (s & 1));
    const uint32_t m = bf16_of_small((scw >> 4) & 0xFu);
    B[s] = m | (m << 16);
  }
}

BM_DEVICE i32x4_t mfma_i8(int64_t a, int64_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
}

}  // namespace

// ---- stored sums of quantised activations in the min-term layout ------------
// out[row][kb][slot]: the 16 stored sums s_b of columns [256 kb, 256 kb + 256)
// of row `row` (s: [rows][K/16] float32), each split into bf16 hi + lo and
// placed at q2_sum_slot(sub-block, part).  One thread per sub-block.
__global__ void __launch_bounds__(256) i8_sums_kernel(const float *__restrict__ s, int64_t rows, int K,
                                                      uint16_t *__restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int nsb = K / 16;
  if (i >= rows * nsb) return;
  const int64_t row = i / nsb;
  const int c = int(i % nsb), kb = c >> 4, sb = c & 15;
  const float v = s[i];
  const uint16_t hi = f32_to_bf16(v);
  uint16_t *o = out + (row * (K / KS) + kb) * SUMS;
  o[q2_sum_slot(sb, 0)] = hi;
  o[q2_sum_slot(sb, 1)] = f32_to_bf16(v - bf16_to_f32(hi));
}

struct GroupI8Args {
  int E, k, K, N;
  const int32_t *perm, *offsets, *counts, *tile_off;  // plan: pairs by expert; chunks of 16 MT rows per expert
  int n_chunks;                                       // grid chunk slots
  const int8_t *a;                                    // quantised activation rows [rows][K]
  const float *dx;                                    // their block scales [rows][K/32]
  const uint16_t *sums;                               // their stored sums, min-term layout [rows][K/256][32]
  int a_by_pair;                                      // row index = pair (down) or token (gate/up)
  const uint8_t *b0, *b1;                             // Q2 matrices [E][N][K/256] (b1: up)
  size_t b_stride;                                    // bytes per expert matrix
  float *h;                                           // gate/up out [pairs][N] float32
  float *y;                                           // down out [pairs][N] float32
};

template <bool GATEUP, int NT>
BM_DEVICE void group_i8_body(const GroupI8Args &g, int e, int valid, int base, int ntile, uint8_t *smem,
                             const int32_t *rows) {
  using Gm = GeoI8<GATEUP>;
  constexpr int NM = Gm::NM, MT = Gm::MT, NG = Gm::NG, W = WAVES;
  uint8_t *abuf = smem;
  uint8_t *sbuf = smem + 2 * Gm::BUF;
  uint8_t *dbuf = sbuf + 2 * Gm::SBUF;
  uint8_t *wbuf = dbuf + 2 * Gm::DBUF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nl = lane & 15;
  const int nsteps = g.K / KS;
  const size_t row_bytes = size_t(nsteps) * 84;
  const int n_w = ntile * Gm::BN + wave * 16 * NG + nl;  // weight row of group 0; group ng adds 16 ng
  // weight copies: wave `wave` copies matrix wm; its 16-byte copy c
  // moves pieces 64 j + l (lane l, j = wj0 + WPM c) of the step image, piece i
  // being bytes 16 (i % 5) .. +15 of row i / 5's super-block; its dword copy
  // moves the d|dmin words of rows 64 j + l.  The source offsets (from the
  // block's first row, step 0) do not depend on the step.
  const int wm = wave / Gm::WPM, wj0 = wave % Gm::WPM;
  const uint8_t *wsrc = (wm ? g.b1 : g.b0) + size_t(e) * g.b_stride + size_t(ntile) * Gm::BN * row_bytes;
  uint32_t woff4[Gm::WC4], woff1[Gm::WC1];
#pragma unroll
  for (int c = 0; c < Gm::WC4; ++c) {
    const int i = 64 * min(wj0 + Gm::WPM * c, Gm::WX4 - 1) + lane;
    const int row = i / 5;
    woff4[c] = uint32_t(row) * uint32_t(row_bytes) + 16u * uint32_t(i - 5 * row);
  }
#pragma unroll
  for (int c = 0; c < Gm::WC1; ++c)
    woff1[c] = uint32_t(64 * min(wj0 + Gm::WPM * c, Gm::WX1 - 1) + lane) * uint32_t(row_bytes) + 80u;
  // copies of step kb into buffer half: activation rows (256 B: 16 lanes, one
  // row per instruction so that the rows keep their padded LDS stride), their
  // stored sums (64 B: 4 lanes per row) and block scales (32 B: 2 lanes per row)
  auto issue = [&](int kb, int half) {
    for (int r = wave; r < 16 * NT; r += W) {
      const int src = rows[r];
      if (src >= 0 && lane < 16)
        lds_dma16(g.a + size_t(src) * g.K + kb * KS + 16 * lane, lds_offset(abuf + half * Gm::BUF + r * ROWB));
    }
    for (int i = wave; i < NT; i += W) {  // rows 16 i .. 16 i + 15
      const int r = 16 * i + (lane >> 2), src = rows[r];
      if (src >= 0)
        lds_dma16(g.sums + (size_t(src) * nsteps + kb) * SUMS + 8 * (lane & 3),
                  lds_offset(sbuf + half * Gm::SBUF + (16 * i) * SUMS * 2));
    }
    if (wave == W - 1) {  // rows 0 .. 16 NT - 1, two lanes each, 32 rows per instruction
      for (int b0 = 0; b0 < 32 * NT; b0 += 64) {
        const int l = b0 + lane, src = rows[min(l >> 1, 16 * NT - 1)];
        if (l < 32 * NT && src >= 0)
          lds_dma16(g.dx + (size_t(src) * nsteps + kb) * DXN + 4 * (l & 1),
                    lds_offset(dbuf + half * Gm::DBUF + 16 * b0));
      }
    }
    uint8_t *wd = wbuf + half * Gm::WBUF + wm * Gm::WMAT;
    const uint8_t *ws = wsrc + size_t(kb) * 84;
#pragma unroll
    for (int c = 0; c < Gm::WC4; ++c) {
      const int j = wj0 + Gm::WPM * c;
      if (Gm::WX4 % Gm::WPM == 0 || j < Gm::WX4) lds_dma16(ws + woff4[c], lds_offset(wd + 1024 * j));
    }
#pragma unroll
    for (int c = 0; c < Gm::WC1; ++c) {
      const int j = wj0 + Gm::WPM * c;
      if (Gm::WX1 % Gm::WPM == 0 || j < Gm::WX1) lds_dma4(ws + woff1[c], lds_offset(wd + Gm::BN * 80 + 256 * j));
    }
  };
  // this lane's bytes of group ng, matrix m from the step image: lane group gq
  // reads code bytes 16 + 16 (gq / 2) + 8 (gq % 2) .. +7 of each half, the 16
  // scale bytes and d|dmin of its row's super-block
  auto read_b = [&](int half, Q2RawI8 (&raw)[NG][NM]) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint8_t *wm_ = wbuf + half * Gm::WBUF + m * Gm::WMAT;
        const int r = wave * 16 * NG + 16 * ng + nl;
        const uint8_t *sb = wm_ + 80 * r;
        const int o = 16 + 16 * (gq >> 1) + 8 * (gq & 1);
        const i8u32x2 h0 = *reinterpret_cast<const i8u32x2 *>(sb + o);
        const i8u32x2 h1 = *reinterpret_cast<const i8u32x2 *>(sb + o + 32);
        const i8u32x4 sc = *reinterpret_cast<const i8u32x4 *>(sb);
        raw[ng][m].q[0] = h0.x, raw[ng][m].q[1] = h0.y, raw[ng][m].q[2] = h1.x, raw[ng][m].q[3] = h1.y;
        raw[ng][m].sc[0] = sc.x, raw[ng][m].sc[1] = sc.y, raw[ng][m].sc[2] = sc.z, raw[ng][m].sc[3] = sc.w;
        raw[ng][m].dd = *reinterpret_cast<const uint32_t *>(wm_ + Gm::BN * 80 + 4 * r);
      }
  };
  f32x4_t acc[NT][NG][NM];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  const i32x4_t izero = {0, 0, 0, 0};
#pragma unroll
  for (int mi = 0; mi < NT; ++mi)
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[mi][ng][m] = zero;
  Q2RawI8 cur[NG][NM];
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kb = 0; kb < nsteps; ++kb) {
    const int half = kb & 1;
    if (kb + 1 < nsteps) issue(kb + 1, half ^ 1);
    read_b(half, cur);
    const int8_t *Ab = reinterpret_cast<const int8_t *>(abuf + half * Gm::BUF);
    const uint16_t *Sx = reinterpret_cast<const uint16_t *>(sbuf + half * Gm::SBUF);
    const float *Dx = reinterpret_cast<const float *>(dbuf + half * Gm::DBUF);
    f32x4_t cf[NT][NG][NM];  // sum over the step's activation blocks of dx * (integer block sum)
#pragma unroll
    for (int mi = 0; mi < NT; ++mi)
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) cf[mi][ng][m] = zero;
    // the two halves of the super-block in turn (a loop: its eight blocks
    // unrolled at once would not fit the registers)
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      HalfI8 hb[NG][NM];
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) hb[ng][m] = q2i8_half(cur[ng][m], h);
#pragma unroll 2  // fully unrolled, the four blocks' operands would not fit the registers
    for (int cc = 0; cc < 4; ++cc) {
      const int c = 4 * h + cc;
      int64_t B[NG][NM];
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) B[ng][m] = q2i8_operand(hb[ng][m], gq, cc);
#pragma unroll
      for (int mi = 0; mi < NT; ++mi) {
        const int64_t A = *reinterpret_cast<const int64_t *>(Ab + (16 * mi + nl) * ROWB + 32 * c + 8 * gq);
        // block scales of this lane's output rows 16 mi + 4 gq + r
        float dxr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) dxr[r] = Dx[(16 * mi + 4 * gq + r) * DXN + c];
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const i32x4_t ci = mfma_i8(A, B[ng][m], izero);
#pragma unroll
            for (int r = 0; r < 4; ++r) cf[mi][ng][m][r] = __builtin_fmaf(dxr[r], float(ci[r]), cf[mi][ng][m][r]);
          }
      }
    }
    }
    // min term against the stored sums, then d and dmin of the super-block
#pragma unroll
    for (int mi = 0; mi < NT; ++mi) {
      uint32_t As[4];
      ld16(Sx + (16 * mi + nl) * SUMS + 8 * gq, As);
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          uint32_t Bn[4];
          q2i8_min_operand(cur[ng][m], gq, Bn);
          const float d = half_to_f32(cur[ng][m].dd & 0xFFFFu), dm = half_to_f32(cur[ng][m].dd >> 16);
          const f32x4_t cn = mfma16(As, Bn, zero);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[mi][ng][m][r] = __builtin_fmaf(d, cf[mi][ng][m][r], __builtin_fmaf(-dm, cn[r], acc[mi][ng][m][r]));
        }
    }
    if (kb + 1 < nsteps) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // step kb+1's rows, sums, scales and weight bytes have landed
      __syncthreads();                                  // ... and this step's buffers are no longer read
    }
  }
  // epilogue: lane holds rows 16 mi + 4 gq + r of column n_w + 16 ng
#pragma unroll
  for (int mi = 0; mi < NT; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mrow = 16 * mi + 4 * gq + r;
      if (mrow >= valid) continue;
      const size_t orow = size_t(g.perm[base + mrow]);
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        const int n = n_w + 16 * ng;
        if constexpr (GATEUP)
          g.h[orow * g.N + n] = silu(acc[mi][ng][0][r]) * acc[mi][ng][1][r];
        else
          g.y[orow * g.N + n] = acc[mi][ng][0][r];
      }
    }
  }
}

template <bool GATEUP>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(GATEUP ? 2 : 4)))
q2_group_i8_kernel(GroupI8Args g) {
  using Gm = GeoI8<GATEUP>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_i8[];
  int32_t *rows = reinterpret_cast<int32_t *>(smem_i8 + Gm::ROWS_OFF);  // activation row, -1: padding
  const int nt_n = g.N / Gm::BN;
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);  // XCD-aware: each XCD takes a contiguous range
  const int ch = L / nt_n, ntile = L % nt_n;
  if (ch >= g.n_chunks || ch >= g.tile_off[g.E]) return;
  int lo = 0, hi = g.E;  // largest e with tile_off[e] <= ch
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.tile_off[mid] <= ch) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int m0 = (ch - g.tile_off[e]) * 16 * Gm::MT;
  const int valid = min(16 * Gm::MT, g.counts[e] - m0);
  const int base = g.offsets[e] + m0;
  for (int i = threadIdx.x; i < 16 * Gm::MT; i += 64 * WAVES) {
    int r = -1;
    if (i < valid) {
      const int pr = g.perm[base + i];
      r = g.a_by_pair ? pr : pr / g.k;
    }
    rows[i] = r;
  }
  __syncthreads();
  switch ((valid + 15) >> 4) {  // M-tiles of the chunk
    case 1: group_i8_body<GATEUP, 1>(g, e, valid, base, ntile, smem_i8, rows); break;
    case 2: group_i8_body<GATEUP, 2>(g, e, valid, base, ntile, smem_i8, rows); break;
    case 3: if constexpr (Gm::MT >= 3) group_i8_body<GATEUP, 3>(g, e, valid, base, ntile, smem_i8, rows); break;
    default: if constexpr (Gm::MT >= 4) group_i8_body<GATEUP, 4>(g, e, valid, base, ntile, smem_i8, rows); break;
  }
  static_assert(Gm::MT >= 1 && Gm::MT <= 4, "chunks of 1 to 4 M-tiles");
}

// ---- shared expert: Q8_0 codes x q8_1 activations, dense ---------------------
// 64-token M-tiles x 64 weight rows per block (4 waves x 16 rows), K-steps of
// 256 (8 blocks of 32).  The Q8_0 rows are expanded once per call to int8
// codes [N][K] and float32 scales [N][K/32]; each v_mfma_i32_16x16x32_i8
// covers one block of both sides, its integer result scaled by d_w * dx.
constexpr int SD_BM = 64, SD_BN = 64;

struct DenseI8Args {
  int T, K, N;
  const int8_t *a;        // quantised activations [T][K]
  const float *dx;        // [T][K/32]
  const int8_t *b0, *b1;  // int8 codes [N][K] (b1: up)
  const float *d0, *d1;   // their scales [N][K/32]
  float *h_out;           // gate/up: [T][N] float32
  float *y_out;           // down: [T][N] float32
  int m_tiles;
};

template <bool GATEUP>
__global__ void __launch_bounds__(256) q8_i8_gemm_kernel(DenseI8Args a) {
  constexpr int NM = GATEUP ? 2 : 1;
  __shared__ __attribute__((aligned(16))) int8_t As[SD_BM * ROWB];
  __shared__ float Dxs[DXN * SD_BM];  // [block][row]
  const int nt_n = a.N / SD_BN;
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);  // XCD-aware remap (grid is a multiple of 8)
  const int mt = L / nt_n, ntile = L % nt_n;
  if (mt >= a.m_tiles) return;
  const int base = mt * SD_BM;
  const int valid = min(SD_BM, a.T - base);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nl = lane & 15;
  const int n = ntile * SD_BN + wave * 16 + nl;  // this lane's weight row
  const int8_t *bw[NM];
  const float *dw[NM];
  bw[0] = a.b0 + size_t(n) * a.K;
  dw[0] = a.d0 + size_t(n) * (a.K / 32);
  if constexpr (GATEUP) {
    bw[1] = a.b1 + size_t(n) * a.K;
    dw[1] = a.d1 + size_t(n) * (a.K / 32);
  }
  f32x4_t acc[4][NM];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  const i32x4_t izero = {0, 0, 0, 0};
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[mi][m] = zero;
  const int nsteps = a.K / KS;
  // staging slice of this thread: row ar, 64 bytes at 64 aq; scales of row ar
  const int ar = tid >> 2, aq = tid & 3;
  const int a_row = ar < valid ? base + ar : -1;
  for (int kb = 0; kb < nsteps; ++kb) {
    uint4 av[4];
    float dxv[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      av[i] = a_row >= 0 ? *reinterpret_cast<const uint4 *>(a.a + size_t(a_row) * a.K + kb * KS + 64 * aq + 16 * i)
                         : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < 2; ++i) dxv[i] = a_row >= 0 ? a.dx[size_t(a_row) * (a.K / 32) + kb * DXN + 2 * aq + i] : 0.f;
    __syncthreads();  // the previous step's LDS reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&As[ar * ROWB + 64 * aq + 16 * i]) = av[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) Dxs[(2 * aq + i) * SD_BM + ar] = dxv[i];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < DXN; ++c) {
      int64_t B[NM];
      float dwc[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        B[m] = *reinterpret_cast<const int64_t *>(bw[m] + kb * KS + 32 * c + 8 * gq);
        dwc[m] = dw[m][kb * DXN + c];
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int64_t A = *reinterpret_cast<const int64_t *>(&As[(16 * mi + nl) * ROWB + 32 * c + 8 * gq]);
        const float4 dxr = *reinterpret_cast<const float4 *>(&Dxs[c * SD_BM + 16 * mi + 4 * gq]);
        const float dxa[4] = {dxr.x, dxr.y, dxr.z, dxr.w};
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const i32x4_t ci = mfma_i8(A, B[m], izero);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mi][m][r] = __builtin_fmaf(dwc[m] * dxa[r], float(ci[r]), acc[mi][m][r]);
        }
      }
    }
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mi + 4 * gq + r;
      if (m >= valid) continue;
      const size_t orow = size_t(base + m);
      if constexpr (GATEUP)
        a.h_out[orow * a.N + n] = silu(acc[mi][0][r]) * acc[mi][1][r];
      else
        a.y_out[orow * a.N + n] = acc[mi][0][r];
    }
  }
}

// Q8_0 [N][K] -> int8 codes [N][K] and float32 scales [N][K/32]
__global__ void __launch_bounds__(256) q8_expand_i8_kernel(const uint8_t *__restrict__ blocks, int64_t n_blocks,
                                                           int8_t *__restrict__ codes, float *__restrict__ scales) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // one thread per (block, 8 codes)
  if (i >= n_blocks * 4) return;
  const int64_t blk = i >> 2;
  const int c = int(i & 3) * 8;
  const uint8_t *bp = blocks + blk * 34;
  if (c == 0) scales[blk] = half_to_f32(bp[0] | (uint32_t(bp[1]) << 8));
  uint32_t o[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    o[j] = uint32_t(bp[2 + c + 4 * j]) | (uint32_t(bp[3 + c + 4 * j]) << 8) | (uint32_t(bp[4 + c + 4 * j]) << 16) |
           (uint32_t(bp[5 + c + 4 * j]) << 24);
  *reinterpret_cast<uint2 *>(codes + blk * 32 + c) = make_uint2(o[0], o[1]);
}

// ---- launch -----------------------------------------------------------------

static hipError_t launch_group_i8(bool gateup, const PrefillI8Args &a, const int8_t *xq, const float *dx,
                                  const uint16_t *sums, hipStream_t stream) {
  GroupI8Args g{};
  g.E = a.E;
  g.k = a.k;
  g.perm = a.plan.perm;
  g.offsets = a.plan.offsets;
  g.counts = a.plan.counts;
  const int mt = gateup ? MT_GU : MT_DN;
  static_assert(16 * MT_GU == PREFILL_BM && 16 * MT_DN == PREFILL_BM_DOWN, "chunk lists of the plan");
  g.tile_off = gateup ? a.tile_off : a.tile_off2;
  const int P = a.T * a.k;
  g.n_chunks = (P + 16 * mt - 1) / (16 * mt) + min(a.E, P);
  g.a = xq;
  g.dx = dx;
  g.sums = sums;
  const int bn = gateup ? GeoI8<true>::BN : GeoI8<false>::BN;
  if (gateup) {
    g.K = a.D, g.N = a.F, g.a_by_pair = 0;
    g.b0 = a.wg, g.b1 = a.wu;
    g.h = a.hf;
  } else {
    g.K = a.F, g.N = a.D, g.a_by_pair = 1;
    g.b0 = a.wd, g.b1 = nullptr;
    g.y = a.y;
  }
  g.b_stride = size_t(a.F) * a.D / 256 * 84;
  if (g.N % bn || g.K % KS) return hipErrorNotSupported;
  const size_t smem = gateup ? GeoI8<true>::SMEM : GeoI8<false>::SMEM;
  hipError_t err = gateup ? hipFuncSetAttribute(reinterpret_cast<const void *>(&q2_group_i8_kernel<true>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem))
                          : hipFuncSetAttribute(reinterpret_cast<const void *>(&q2_group_i8_kernel<false>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
  if (err != hipSuccess) return err;
  int grid = g.n_chunks * (g.N / bn);
  grid = (grid + 7) & ~7;
  if (gateup)
    BM_LAUNCH("routed_i8_gateup_gemm_kernel", q2_group_i8_kernel<true>, dim3(grid), dim3(64 * WAVES), smem, stream, g);
  else
    BM_LAUNCH("routed_i8_down_gemm_kernel", q2_group_i8_kernel<false>, dim3(grid), dim3(64 * WAVES), smem, stream, g);
  return hipGetLastError();
}

static hipError_t launch_sums_i8(const float *s, int64_t rows, int K, uint16_t *out, hipStream_t stream) {
  const int64_t n = rows * (K / 16);
  if (n == 0) return hipSuccess;
  BM_LAUNCH("i8_sums_kernel", i8_sums_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, s, rows, K, out);
  return hipGetLastError();
}

static hipError_t launch_dense_i8(bool gateup, const DenseI8Args &d, hipStream_t stream) {
  int grid = d.m_tiles * (d.N / SD_BN);
  grid = (grid + 7) & ~7;
  if (gateup)
    BM_LAUNCH("shared_i8_gateup_gemm_kernel", q8_i8_gemm_kernel<true>, dim3(grid), dim3(256), 0, stream, d);
  else
    BM_LAUNCH("shared_i8_down_gemm_kernel", q8_i8_gemm_kernel<false>, dim3(grid), dim3(256), 0, stream, d);
  return hipGetLastError();
}

hipError_t launch_prefill_ffn_i8(const PrefillI8Args &a, hipStream_t stream) {
  if (a.D % KS || a.F % KS) return hipErrorNotSupported;
  if (a.F % GeoI8<true>::BN || a.D % GeoI8<false>::BN || a.F % SD_BN || a.D % SD_BN) return hipErrorNotSupported;
  hipError_t err;
  const int P = a.T * a.k;
  // x quantised per token (shared by the routed and the shared gate/up)
  if ((err = launch_quantize_q8(a.x, a.x_f32, a.T, a.D, reinterpret_cast<uint8_t *>(a.xq), a.xd, a.xs, stream)) !=
      hipSuccess)
    return err;
  if ((err = launch_sums_i8(a.xs, a.T, a.D, a.sums, stream)) != hipSuccess) return err;
  PlanBufs p = a.plan;
  if ((err = launch_plan(a.ids, a.T, a.k, a.E, PREFILL_BM, PREFILL_BM_DOWN, p, stream)) != hipSuccess) return err;
  if ((err = launch_group_i8(true, a, a.xq, a.xd, a.sums, stream)) != hipSuccess) return err;
  // h of every served pair quantised (rows of unserved pairs are never read)
  if ((err = launch_quantize_q8(a.hf, true, P, a.F, reinterpret_cast<uint8_t *>(a.hq), a.hd, a.hs, stream)) !=
      hipSuccess)
    return err;
  if ((err = launch_sums_i8(a.hs, P, a.F, a.sums, stream)) != hipSuccess) return err;
  if ((err = launch_group_i8(false, a, a.hq, a.hd, a.sums, stream)) != hipSuccess) return err;
  if (a.sg) {
    const int64_t nw = int64_t(a.F) * a.D;
    int8_t *codes = a.sw_i8;
    float *sd = a.sw_d;
    const int64_t nb = nw / 32;
    const unsigned g = unsigned((nb * 4 + 255) / 256);
    BM_LAUNCH("q8_expand_i8_kernel", q8_expand_i8_kernel, dim3(g), dim3(256), 0, stream, a.sg, nb, codes, sd);
    BM_LAUNCH("q8_expand_i8_kernel", q8_expand_i8_kernel, dim3(g), dim3(256), 0, stream, a.su, nb, codes + nw, sd + nb);
    BM_LAUNCH("q8_expand_i8_kernel", q8_expand_i8_kernel, dim3(g), dim3(256), 0, stream, a.sd, nb, codes + 2 * nw,
              sd + 2 * nb);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    DenseI8Args s{};
    s.T = a.T;
    s.m_tiles = (a.T + SD_BM - 1) / SD_BM;
    s.a = a.xq;
    s.dx = a.xd;
    s.K = a.D;
    s.N = a.F;
    s.b0 = codes;
    s.b1 = codes + nw;
    s.d0 = sd;
    s.d1 = sd + nb;
    s.h_out = a.hsf;
    if ((err = launch_dense_i8(true, s, stream)) != hipSuccess) return err;
    if ((err = launch_quantize_q8(a.hsf, true, a.T, a.F, reinterpret_cast<uint8_t *>(a.hsq), a.hsd, a.hss, stream)) !=
        hipSuccess)
      return err;
    s.a = a.hsq;
    s.dx = a.hsd;
    s.K = a.F;
    s.N = a.D;
    s.b0 = codes + 2 * nw;
    s.b1 = nullptr;
    s.d0 = sd + 2 * nb;
    s.d1 = nullptr;
    s.h_out = nullptr;
    s.y_out = a.ys;
    if ((err = launch_dense_i8(false, s, stream)) != hipSuccess) return err;
  }
  return launch_combine(a.y, a.sg ? a.ys : nullptr, a.ids, a.wts, a.T, a.k, a.D, a.E, a.out, a.out_bf16, a.status,
                        a.x_res, a.x_next, stream);
}

}  // namespace bm
