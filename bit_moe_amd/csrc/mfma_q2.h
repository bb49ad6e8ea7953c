// Exact 2-bit super-block operands for v_mfma_f32_16x16x32_bf16 (gfx950).
//
// A weight of sub-block s is w_k = d*sc_s*q_k - dmin*m_s, so a row's dot
// product with activations x over one 256-weight super-block is
//   d * sum_k (sc_s q_k) x_k  -  dmin * sum_s m_s X_s,   X_s = sum_{k in s} x_k.
// sc*q (0..45) and m (0..15) are small integers, and 128 + sc*q is exact in
// bf16 too: eight MFMAs on B = 128 + sc*q, one MFMA on B = m and one on B =
// 128 (both against X_s split into bf16 hi + lo) give the sums in float32 (the
// last one removes the offset), and d, dmin scale them afterwards.
//
// Lane k-slots (MFMA 16x16x32: A lane l holds row l%16 and k = 8*(l/16)+0..7,
// B lane l holds column l%16 and the same k, D lane l holds rows 4*(l/16)+0..3
// of column l%16).  Lane group g = l/16 owns half h = g/2 and sub-block parity
// p = g%2 of every super-block:
//   main step t (0..7): sub-block 8h + 2*(t/2) + p, weights 8*(t%2) .. +7 of it,
//                       k offset 128h + 32*(t/2) + 16p + 8*(t%2) inside the block
//   min slot i (0..7):  sub-block 8h + 2*(i/2) + p, bf16 part i%2 (hi, lo)
// so each lane reads its 16 code bytes, its 8 scale bytes and d/dmin only, and
// its activation operands are 16 contiguous bytes.  The sub-block sums are
// stored per row in min-slot order: index 8g + i.
#pragma once

#include "common.h"

namespace bm {

typedef uint32_t q2u32x4 __attribute__((ext_vector_type(4)));
typedef q2u32x4 __attribute__((aligned(4))) q2u32x4_a4;
typedef uint32_t q2u32x2 __attribute__((ext_vector_type(2)));
typedef q2u32x2 __attribute__((aligned(4))) q2u32x2_a4;

// bf16 bits of a small non-negative integer (exact)
BM_DEVICE uint32_t bf16_of_small(uint32_t v) { return __float_as_uint(float(v)) >> 16; }

// Raw bytes of one lane's quarter of a super-block.
struct Q2Raw {
  q2u32x4 q;    // 16 code bytes at 16 + 32h + 16p
  q2u32x2 sc;   // scale bytes 8h .. 8h+7
  uint32_t dd;  // d | dmin << 16
};

// Hands r over as if produced here.  For loads already completed by an
// explicit s_waitcnt in asm (which the compiler's wait insertion cannot see),
// this keeps the compiler from waiting again at the first use, where its
// count would also cover later loads issued from asm.
BM_DEVICE void q2_settle(Q2Raw &r) { asm volatile("" : "+v"(r.q), "+v"(r.sc), "+v"(r.dd)); }

BM_DEVICE Q2Raw q2_load(const uint8_t *sb, int g) {
  const int h = g >> 1, p = g & 1;
  Q2Raw r;
  r.q = *reinterpret_cast<const q2u32x4_a4 *>(sb + 16 + 32 * h + 16 * p);
  r.sc = *reinterpret_cast<const q2u32x2_a4 *>(sb + 8 * h);
  r.dd = *reinterpret_cast<const uint32_t *>(sb + 80);
  return r;
}

// Main operands for MFMA step t (8 weights) from the raw bytes, in offset
// form: bf16 bits 0x43vv are the value 128 + vv for vv < 128, so the bytes v
// = sc*q (0..45) of a per-scale byte table (one multiply) become bf16
// operands 128 + sc*q with one byte interleave per pair: two table perms and
// four interleave perms per 8 weights.  The MFMA then sums (128 + sc q) x;
// the caller removes 128 * (sum of x over the super-block).
BM_DEVICE void q2_main_operand(const Q2Raw &r, int p, int t, uint32_t (&B)[4]) {
  const int s = t >> 1, j8 = t & 1;
  const uint32_t scw = (s < 2 ? r.sc.x : r.sc.y) >> (8 * p + 16 * (s & 1));
  const uint32_t tab = (scw & 0xFu) * 0x03020100u;  // bytes 0, sc, 2 sc, 3 sc (3 * 15 < 256: no carries)
  const uint32_t w0 = j8 ? r.q.z : r.q.x, w1 = j8 ? r.q.w : r.q.y;
  const uint32_t v0 = __builtin_amdgcn_perm(0u, tab, (w0 >> (2 * s)) & 0x03030303u);
  const uint32_t v1 = __builtin_amdgcn_perm(0u, tab, (w1 >> (2 * s)) & 0x03030303u);
  B[0] = __builtin_amdgcn_perm(0x43434343u, v0, 0x04010400u);  // (v0.b0, v0.b1) as 0x43vv words
  B[1] = __builtin_amdgcn_perm(0x43434343u, v0, 0x04030402u);
  B[2] = __builtin_amdgcn_perm(0x43434343u, v1, 0x04010400u);
  B[3] = __builtin_amdgcn_perm(0x43434343u, v1, 0x04030402u);
}

// Min operand: slot i = 2s + part holds m of sub-block 8h + 2s + p.
BM_DEVICE void q2_min_operand(const Q2Raw &r, int p, uint32_t (&B)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t scw = (s < 2 ? r.sc.x : r.sc.y) >> (8 * p + 16 * (s & 1));
    const uint32_t f = __float_as_uint(float((scw >> 4) & 0xFu));  // m, exact
    B[s] = __builtin_amdgcn_perm(f, f, 0x03020302u);               // its bf16 bits (the high half) twice
  }
}

BM_DEVICE float q2_d(const Q2Raw &r) { return half_to_f32(r.dd & 0xFFFFu); }
BM_DEVICE float q2_dmin(const Q2Raw &r) { return half_to_f32(r.dd >> 16); }

// k offset inside the super-block of main step t for lane group g
BM_DEVICE int q2_kofs(int t, int g) { return 128 * (g >> 1) + 32 * (t >> 1) + 16 * (g & 1) + 8 * (t & 1); }

// index (min-slot order) of the sums of sub-block sb: 8g + 2s + part
BM_DEVICE int q2_sum_slot(int sb, int part) {
  const int h = sb >> 3, s = (sb >> 1) & 3, p = sb & 1;
  return 8 * (2 * h + p) + 2 * s + part;
}

BM_DEVICE f32x4_t mfma16(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  v4u av = {a[0], a[1], a[2], a[3]};
  v4u bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                 c, 0, 0, 0);
}

BM_DEVICE void ld16(const uint16_t *p, uint32_t (&v)[4]) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  v[0] = u.x;
  v[1] = u.y;
  v[2] = u.z;
  v[3] = u.w;
}

}  // namespace bm
