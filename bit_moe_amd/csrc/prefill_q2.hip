// Routed grouped GEMM of the prefill path with each weight operand built once
// per chunk of up to 48 tokens (gate/up) or 32 pairs (down) of its expert.
//
// "Strata-DSV4.1", §Results / §How it works: a prompt chunk runs each layer's
// routed experts as grouped expert matrix products.  Here on
// v_mfma_f32_16x16x32_bf16 with float32 accumulation and exact weights (the
// offset form of mfma_q2.h: B = 128 + sc*q per weight, the sub-block sums of
// the activations against B = m, d and dmin on the float32 sums).  The main
// accumulators start from -128 times the row's float32 super-block sum (the
// same for every output column, so no MFMA is needed for it): the sum is
// exact for bf16 data of ordinary range, where a bf16 hi + lo split of it
// would leave 2^-17 of it, times 128, in every output.
//
// The operand build (code unpack and table lookup, ~11 VALU instructions per
// 8 weights and lane) is the costly part, so a block owns one chunk of an
// expert's tokens -- up to three 16-token M-tiles for gate/up, two for down,
// as many as the chunk needs -- and one N-tile of 256 weight rows (8 waves of
// 2 x 16 rows); each wave builds the operands of its weight rows for a whole
// 256-wide K-step once and applies them to every M-tile of the chunk.  The
// chunk's activation rows and their sub-block sums (precomputed once per call
// by xsum_kernel) are staged in LDS with direct-to-LDS copies one K-step
// ahead, double-buffered.  Gate/up stages the step's weight bytes the same
// way (16-byte copies of consecutive rows' super-blocks: each copy instruction
// reads about four contiguous 84-byte runs, where per-lane loads of a lane's
// own 28 bytes touch sixteen rows per instruction, and were measured 0.25 ms
// slower on the 4096-token chunk); down, whose two activation parts take
// twice the LDS per row, loads each lane's weight bytes into registers and
// keeps two blocks per CU.  Padding is per 16-token tile: a group of n tokens
// runs ceil(n / 16) tiles.
//
//  gate/up  (GATEUP): weight rows of the gate and up matrices alike, h =
//           silu(g) u stored as bf16 hi + lo parts per pair.
//  down     : A = h (hi and lo parts each multiply the operands: two MFMAs per
//           step), y stored in float32 per pair.
#include "common.h"
#include "internal.h"
#include "mfma_q2.h"

namespace bm {

namespace {

constexpr int KS = 256;               // K per step (one super-block of every weight row)
#ifndef BM_PF_ROWPAD
#define BM_PF_ROWPAD 8
#endif
constexpr int ROWP = KS + BM_PF_ROWPAD;  // bf16 per LDS activation row (16-byte pad)
constexpr int SUMS = 32;              // bf16 sums per (row, step): 16 sub-blocks x (hi, lo)
constexpr int MT_GU = BM_PF_CHUNK_GU;  // gate/up: M-tiles of 16 per chunk
constexpr int MT_DN = BM_PF_CHUNK_DN;  // down: M-tiles of 16 pairs per chunk (hi and lo rows: twice the LDS per row)

}  // namespace

// ---- activation sub-block sums --------------------------------------------
// out[row][kb][slot]: the 16 sub-block sums of columns [256 kb, 256 kb + 256)
// of row `row` (over both parts when a_lo is given), each split into bf16 hi +
// lo and placed at q2_sum_slot(sub-block, part); tot[row][kb]: -128 times their float32
// total.  One thread per sub-block; the 16 threads of a super-block are 16
// consecutive lanes of one wave.
__global__ void __launch_bounds__(256) xsum_kernel(const uint16_t *__restrict__ a, const uint16_t *__restrict__ a_lo,
                                                   int64_t rows, int K, uint16_t *__restrict__ out,
                                                   float *__restrict__ tot) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // (row, sub-block of the row)
  const int nsb = K / 16;
  // rows * nsb is a multiple of 16: a super-block's 16 lanes are all in range or all out
  if (i >= rows * nsb) return;
  const int64_t row = i / nsb;
  const int c = int(i % nsb), kb = c >> 4, sb = c & 15;
  float sum = 0.f;
  for (int part = 0; part < (a_lo ? 2 : 1); ++part) {
    const uint4 *v = reinterpret_cast<const uint4 *>((part ? a_lo : a) + row * K + 16 * c);
    const uint4 v0 = v[0], v1 = v[1];
    const uint32_t w8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) sum = dot2_bf16(w8[j], 0x3F803F80u, sum);  // + lo + hi (bf16 1.0 pair)
  }
  const uint16_t shi = f32_to_bf16(sum);
  uint16_t *o = out + (row * (K / KS) + kb) * SUMS;
  o[q2_sum_slot(sb, 0)] = shi;
  o[q2_sum_slot(sb, 1)] = f32_to_bf16(sum - bf16_to_f32(shi));
  float t = sum;
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) t += __shfl_xor(t, m, 16);
  if (sb == 0) tot[row * (K / KS) + kb] = -128.f * t;  // exact: a power of two
}

// ---- grouped GEMM ---------------------------------------------------------------

struct GroupArgs {
  int E, k, K, N;
  const int32_t *perm, *offsets, *counts, *tile_off;  // plan: pairs by expert; chunks of 16 MT rows per expert
  int n_chunks;                                       // grid chunk slots
  const uint16_t *a, *a_lo;                           // activation rows (a_lo: down's lo parts)
  int a_by_pair;                                      // row index = pair (down) or token (gate/up)
  const uint16_t *sums;                               // xsum_kernel output for the same rows
  const float *tot;                                   // and their super-block totals
  const uint8_t *b0, *b1;                             // Q2 matrices [E][N][K/256] (b1: up)
  size_t b_stride;                                    // bytes per expert matrix
  uint16_t *h, *h_lo;                                 // gate/up out [pairs][N]
  float *y;                                           // down out [pairs][N]
};

// Per wave: NG groups of 16 weight rows (gate and up alike for gate/up); per
// K-step and MFMA step t the wave builds the NG x NM operands once and feeds
// each activation operand it reads from LDS to all of them, for each of the
// chunk's NT M-tiles (NT known at compile time: one instantiation per count).
template <bool GATEUP>
struct GroupGeo {
  static constexpr int NM = GATEUP ? 2 : 1;          // matrices (gate, up)
  static constexpr int PARTS = GATEUP ? 1 : 2;       // activation parts (h hi, lo)
  static constexpr int MT = GATEUP ? MT_GU : MT_DN;  // M-tiles per chunk at most
#ifndef BM_GRP_NG_GU
#define BM_GRP_NG_GU 2
#endif
#ifndef BM_GRP_NG_DN
#define BM_GRP_NG_DN 2
#endif
#ifndef BM_GRP_WAVES
#define BM_GRP_WAVES 8
#endif
  static constexpr int NG = GATEUP ? BM_GRP_NG_GU : BM_GRP_NG_DN;  // 16-row groups per wave
  static constexpr int WAVES = BM_GRP_WAVES;                       // waves per block
  static constexpr int BN = 16 * NG * WAVES;                       // weight rows per block
  static constexpr int BUF = PARTS * 16 * MT * ROWP * 2;  // bytes of one activation buffer
  static constexpr int SBUF = 16 * MT * SUMS * 2;         // bytes of one sums buffer
  static constexpr int TBUF = 16 * MT * 4;                // bytes of one buffer of super-block totals
  // gate/up stages one step's weights per matrix in LDS: bytes 0..79 of every
  // row's super-block (codes and scales) as 5 16-byte pieces per row, then the
  // rows' d|dmin words.  Down loads them into registers instead (its LDS then
  // holds two blocks per CU, four waves per SIMD).
  static constexpr bool WLDS = GATEUP;
  static constexpr int WMAT = BN * 84;                    // bytes per matrix and step
  static constexpr int WBUF = WLDS ? NM * WMAT : 0;
  static constexpr int WX4 = BN * 5 / 64;                 // 64-lane 16-byte copies per matrix and step
  static constexpr int WX1 = BN / 64;                     // 64-lane dword copies (d|dmin) per matrix and step
  static constexpr int WPM = WAVES / NM;                  // waves copying one matrix
  static constexpr int WC4 = (WX4 + WPM - 1) / WPM;       // 16-byte copies per wave and step
  static constexpr int WC1 = (WX1 + WPM - 1) / WPM;       // dword copies per wave and step
  static constexpr int ROWS_OFF = 2 * BUF + 2 * SBUF + 2 * TBUF + 2 * WBUF;  // chunk row table
  static constexpr size_t SMEM = size_t(ROWS_OFF) + 16 * MT * 4;
  static_assert(BN * 5 % 64 == 0 && BN % 64 == 0 && WAVES % NM == 0, "weight copies of whole 64-lane rows");
  static_assert(SMEM <= 160 * 1024, "LDS of one CU");
};

template <bool GATEUP, int NT>
BM_DEVICE void group_body(const GroupArgs &g, int e, int valid, int base, int ntile, uint8_t *smem, const int32_t *rows) {
  using Gm = GroupGeo<GATEUP>;
  constexpr int NM = Gm::NM, PARTS = Gm::PARTS, MT = Gm::MT, NG = Gm::NG;
  uint8_t *abuf = smem;
  uint8_t *sbuf = smem + 2 * Gm::BUF;
  uint8_t *tbuf = sbuf + 2 * Gm::SBUF;
  uint8_t *wbuf = tbuf + 2 * Gm::TBUF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nl = lane & 15, p = gq & 1;
  const int nsteps = g.K / KS;
  const size_t row_bytes = size_t(nsteps) * 84;
  const int n_w = ntile * Gm::BN + wave * 16 * NG + nl;  // weight row of group 0; group ng adds 16 ng
  constexpr int W = Gm::WAVES;
  // weight copies: wave `wave` copies matrix wm; its 16-byte copy c moves
  // pieces 64 j + l (lane l, j = wj0 + WPM c) of the step image, piece i being
  // bytes 16 (i % 5) .. +15 of row i / 5's super-block; its dword copy moves
  // the d|dmin words of rows 64 j + l.  Source offsets (from the block's first
  // row, step 0) do not depend on the step.
  const int wm = wave / Gm::WPM, wj0 = wave % Gm::WPM;
  const uint8_t *wsrc = (wm ? g.b1 : g.b0) + size_t(e) * g.b_stride + size_t(ntile) * Gm::BN * row_bytes;
  uint32_t woff4[Gm::WC4], woff1[Gm::WC1];
  // register path (down): the lane's own rows
  const uint8_t *wb[NM];
  wb[0] = g.b0 + size_t(e) * g.b_stride + size_t(n_w) * row_bytes;
  if constexpr (GATEUP) wb[1] = g.b1 + size_t(e) * g.b_stride + size_t(n_w) * row_bytes;
#pragma unroll
  for (int c = 0; c < Gm::WC4; ++c) {
    const int i = 64 * min(wj0 + Gm::WPM * c, Gm::WX4 - 1) + lane;
    const int row = i / 5;
    woff4[c] = uint32_t(row) * uint32_t(row_bytes) + 16u * uint32_t(i - 5 * row);
  }
#pragma unroll
  for (int c = 0; c < Gm::WC1; ++c)
    woff1[c] = uint32_t(64 * min(wj0 + Gm::WPM * c, Gm::WX1 - 1) + lane) * uint32_t(row_bytes) + 80u;
  // copies of step kb into buffer half: activation rows (512 B each, half a
  // wave per row; this wave's rows wave, wave + W, ..) and their sums (64 B
  // per row, 16 rows per instruction).  Addresses are formed in vector
  // registers: a variant with wave-uniform row bases in scalar registers
  // gave wrong rows, run to run, in builds where those registers spilled.
  auto issue = [&](int kb, int half) {
    uint8_t *ad = abuf + half * Gm::BUF;
    for (int i = wave; i < PARTS * 16 * NT; i += W) {
      const int part = i / (16 * NT), r = i % (16 * NT);
      const int src = rows[r];
      if (src >= 0 && lane < 32)
        lds_dma16((part ? g.a_lo : g.a) + size_t(src) * g.K + kb * KS + 8 * lane,
                  lds_offset(ad + (part * 16 * MT + r) * ROWP * 2));
    }
    uint8_t *sd = sbuf + half * Gm::SBUF;
    for (int i = wave; i < NT; i += W) {  // rows 16 i .. 16 i + 15, four lanes (64 B) each
      const int r = 16 * i + (lane >> 2), src = rows[r];
      if (src >= 0)
        lds_dma16(g.sums + (size_t(src) * nsteps + kb) * SUMS + 8 * (lane & 3), lds_offset(sd + (16 * i) * SUMS * 2));
    }
    if (wave == W - 1 && lane < 16 * NT) {  // totals: one dword per row
      const int src = rows[lane];
      if (src >= 0) lds_dma4(g.tot + size_t(src) * nsteps + kb, lds_offset(tbuf + half * Gm::TBUF));
    }
    if constexpr (!Gm::WLDS) return;
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
  auto load_b = [&](int kb, Q2Raw (&raw)[NG][NM]) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) raw[ng][m] = q2_load(wb[m] + size_t(16 * ng) * row_bytes + size_t(kb) * 84, gq);
  };
  // this lane's raw bytes of group ng, matrix m from the step image
  auto read_b = [&](int half, Q2Raw (&raw)[NG][NM]) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint8_t *wm_ = wbuf + half * Gm::WBUF + m * Gm::WMAT;
        const int r = wave * 16 * NG + 16 * ng + nl, h = gq >> 1;
        raw[ng][m].q = *reinterpret_cast<const q2u32x4 *>(wm_ + 80 * r + 16 + 32 * h + 16 * p);
        raw[ng][m].sc = *reinterpret_cast<const q2u32x2 *>(wm_ + 80 * r + 8 * h);
        raw[ng][m].dd = *reinterpret_cast<const uint32_t *>(wm_ + Gm::BN * 80 + 4 * r);
      }
  };
  f32x4_t acc[NT][NG][NM];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mi = 0; mi < NT; ++mi)
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[mi][ng][m] = zero;
  Q2Raw cur[NG][NM];
  issue(0, 0);
  if constexpr (!Gm::WLDS) load_b(0, cur);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (!Gm::WLDS) {
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int m = 0; m < NM; ++m) q2_settle(cur[ng][m]);
  }
  __syncthreads();
  for (int kb = 0; kb < nsteps; ++kb) {
    const int half = kb & 1;
    Q2Raw nxt[NG][NM];
    if (kb + 1 < nsteps) {
      issue(kb + 1, half ^ 1);
      if constexpr (!Gm::WLDS) load_b(kb + 1, nxt);
    }
    if constexpr (Gm::WLDS) read_b(half, cur);
    const uint16_t *Ah = reinterpret_cast<const uint16_t *>(abuf + half * Gm::BUF);
    const uint16_t *Sx = reinterpret_cast<const uint16_t *>(sbuf + half * Gm::SBUF);
    const float *Xt = reinterpret_cast<const float *>(tbuf + half * Gm::TBUF);
    // the main accumulators start from -128 x the rows' super-block sums
    // (rows 4 gq .. 4 gq + 3 of the tile in this lane), which removes the 128
    // offset of the main operands
    uint32_t As[NT][4];
    f32x4_t cm[NT][NG][NM];
#pragma unroll
    for (int mi = 0; mi < NT; ++mi) {
      ld16(Sx + (16 * mi + nl) * SUMS + 8 * gq, As[mi]);
      const float4 xt = *reinterpret_cast<const float4 *>(Xt + 16 * mi + 4 * gq);
      const f32x4_t cx = {xt.x, xt.y, xt.z, xt.w};
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) cm[mi][ng][m] = cx;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int ko = q2_kofs(t, gq);
      uint32_t B[NG][NM][4];
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NM; ++m) q2_main_operand(cur[ng][m], p, t, B[ng][m]);
#pragma unroll
      for (int mi = 0; mi < NT; ++mi) {
#pragma unroll
        for (int part = 0; part < PARTS; ++part) {
          uint32_t A[4];
          ld16(Ah + (part * 16 * MT + 16 * mi + nl) * ROWP + ko, A);
#pragma unroll
          for (int ng = 0; ng < NG; ++ng)
#pragma unroll
            for (int m = 0; m < NM; ++m) cm[mi][ng][m] = mfma16(A, B[ng][m], cm[mi][ng][m]);
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
        for (int mi = 0; mi < NT; ++mi) {
          const f32x4_t cn = mfma16(As[mi], Bn, zero);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[mi][ng][m][r] = __builtin_fmaf(d, cm[mi][ng][m][r], __builtin_fmaf(-dm, cn[r], acc[mi][ng][m][r]));
        }
      }
    }
    if (kb + 1 < nsteps) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // step kb+1's rows, sums, totals and weights have landed
      __syncthreads();                                  // ... and this step's buffers are no longer read
      if constexpr (!Gm::WLDS) {
        // the weight bytes count as produced by the wait above, so the
        // compiler keeps no load of them pending (a pending load would make it
        // wait again in the next step, behind that step's copies)
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            q2_settle(nxt[ng][m]);
            cur[ng][m] = nxt[ng][m];
          }
      }
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
        if constexpr (GATEUP) {
          const float hf = silu(acc[mi][ng][0][r]) * acc[mi][ng][1][r];
          const uint16_t hb = f32_to_bf16(hf);
          g.h[orow * g.N + n] = hb;
          g.h_lo[orow * g.N + n] = f32_to_bf16(hf - bf16_to_f32(hb));
        } else {
          g.y[orow * g.N + n] = acc[mi][ng][0][r];
        }
      }
    }
  }
}

template <bool GATEUP>
__global__ void __launch_bounds__(64 * BM_GRP_WAVES) __attribute__((amdgpu_waves_per_eu(GATEUP ? 2 : 4)))
q2_group_kernel(GroupArgs g) {
  using Gm = GroupGeo<GATEUP>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_g[];
  int32_t *rows = reinterpret_cast<int32_t *>(smem_g + Gm::ROWS_OFF);  // activation row, -1: padding
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
  for (int i = threadIdx.x; i < 16 * Gm::MT; i += 64 * Gm::WAVES) {
    int r = -1;
    if (i < valid) {
      const int pr = g.perm[base + i];
      r = g.a_by_pair ? pr : pr / g.k;
    }
    rows[i] = r;
  }
  __syncthreads();
  switch ((valid + 15) >> 4) {  // M-tiles of the chunk
    case 1: group_body<GATEUP, 1>(g, e, valid, base, ntile, smem_g, rows); break;
    case 2: group_body<GATEUP, 2>(g, e, valid, base, ntile, smem_g, rows); break;
    case 3: if constexpr (Gm::MT >= 3) group_body<GATEUP, 3>(g, e, valid, base, ntile, smem_g, rows); break;
    case 4: if constexpr (Gm::MT >= 4) group_body<GATEUP, 4>(g, e, valid, base, ntile, smem_g, rows); break;
    case 5: if constexpr (Gm::MT >= 5) group_body<GATEUP, 5>(g, e, valid, base, ntile, smem_g, rows); break;
    case 6: if constexpr (Gm::MT >= 6) group_body<GATEUP, 6>(g, e, valid, base, ntile, smem_g, rows); break;
    case 7: if constexpr (Gm::MT >= 7) group_body<GATEUP, 7>(g, e, valid, base, ntile, smem_g, rows); break;
    default: if constexpr (Gm::MT >= 8) group_body<GATEUP, 8>(g, e, valid, base, ntile, smem_g, rows); break;
  }
  static_assert(Gm::MT >= 1 && Gm::MT <= 8, "chunks of 1 to 8 M-tiles");
}

size_t q2_group_smem(bool gateup) { return gateup ? GroupGeo<true>::SMEM : GroupGeo<false>::SMEM; }

// Routed gate/up (gateup) or down over the plan's chunks of 48 tokens
// (tile_off) or 32 pairs (tile_off2) per expert, 256 weight rows per block.
// sums, tot: workspace for the activations' sub-block sums (K / 4 bytes per
// row) and super-block totals (K / 64 bytes per row), rows being tokens for
// gate/up and pairs for down.  hipErrorNotSupported when N is not a multiple
// of the block's rows (nothing is launched then).
hipError_t launch_q2_group(bool gateup, const PrefillArgs &a, const uint16_t *x, uint16_t *sums, float *tot,
                           hipStream_t stream) {
  GroupArgs g{};
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
  g.sums = sums;
  g.tot = tot;
  const int bn = gateup ? GroupGeo<true>::BN : GroupGeo<false>::BN;
  if (gateup) {
    g.K = a.D, g.N = a.F;
    g.a = x, g.a_lo = nullptr, g.a_by_pair = 0;
    g.b0 = a.wg, g.b1 = a.wu;
    g.h = a.h, g.h_lo = a.h_lo;
  } else {
    g.K = a.F, g.N = a.D;
    g.a = a.h, g.a_lo = a.h_lo, g.a_by_pair = 1;
    g.b0 = a.wd, g.b1 = nullptr;
    g.y = a.y;
  }
  g.b_stride = size_t(a.F) * a.D / 256 * 84;
  if (g.N % bn || g.K % KS) return hipErrorNotSupported;
  // sums of the activation rows (tokens for gate/up, pairs for down)
  const int64_t rows = gateup ? a.T : P;
  const int64_t nthreads = rows * (g.K / 16);
  BM_LAUNCH("xsum_kernel", xsum_kernel, dim3(unsigned((nthreads + 255) / 256)), dim3(256), 0, stream, g.a, g.a_lo,
            rows, g.K, sums, tot);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t smem = q2_group_smem(gateup);
  // set on every call: the attribute is per device and the call is cheap
  err = gateup ? hipFuncSetAttribute(reinterpret_cast<const void *>(&q2_group_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(smem))
               : hipFuncSetAttribute(reinterpret_cast<const void *>(&q2_group_kernel<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
  if (err != hipSuccess) return err;
  int grid = g.n_chunks * (g.N / bn);
  grid = (grid + 7) & ~7;
  if (gateup)
    BM_LAUNCH("routed_gateup_gemm_kernel", q2_group_kernel<true>, dim3(grid), dim3(64 * BM_GRP_WAVES), smem, stream, g);
  else
    BM_LAUNCH("routed_down_gemm_kernel", q2_group_kernel<false>, dim3(grid), dim3(64 * BM_GRP_WAVES), smem, stream, g);
  return hipGetLastError();
}

}  // namespace bm
