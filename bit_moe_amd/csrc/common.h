// Internal helpers shared by the HIP kernels of libbitmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define BM_DEVICE __device__ __forceinline__
#define BM_HOST_DEVICE __host__ __device__

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

namespace bm {

constexpr int WAVE = 64;

// ---- bf16 ---------------------------------------------------------------

BM_DEVICE float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
BM_DEVICE float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
BM_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even; NaN stays NaN.
BM_DEVICE uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

BM_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

BM_DEVICE float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

BM_DEVICE float half_to_f32(uint32_t h16) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h16)));
}

// ---- reductions -----------------------------------------------------------

template <int WIDTH>
BM_DEVICE float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}

// Wave-wide reductions on DPP: within each quad (lane ^ 1, lane ^ 2), then
// half-row and row mirrors give every lane of a 16-lane row the row's result;
// the four rows are combined from lanes 0, 16, 32, 48 (uniform result).
BM_DEVICE int dpp_quad_swap1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
BM_DEVICE int dpp_quad_swap2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
BM_DEVICE int dpp_half_mirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
BM_DEVICE int dpp_row_mirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); }

BM_DEVICE uint32_t wave_max_u32(uint32_t v) {
  v = max(v, uint32_t(dpp_quad_swap1(int(v))));
  v = max(v, uint32_t(dpp_quad_swap2(int(v))));
  v = max(v, uint32_t(dpp_half_mirror(int(v))));
  v = max(v, uint32_t(dpp_row_mirror(int(v))));
  const uint32_t r0 = __builtin_amdgcn_readlane(int(v), 0), r1 = __builtin_amdgcn_readlane(int(v), 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(int(v), 32), r3 = __builtin_amdgcn_readlane(int(v), 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sum over aligned groups of `lpr` lanes (lpr = 1, 2, 4, ..., 64), the result
// in every lane of the group: DPP within rows of 16 lanes, then the gfx950
// row swaps (v_permlane16_swap, v_permlane32_swap).  Each step adds the same
// two operands in the same order in both partner lanes, so all lanes agree.
BM_DEVICE float swap_add16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
BM_DEVICE float swap_add32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
BM_DEVICE float lane_group_sum(float v, int lpr) {
  if (lpr >= 2) v += __int_as_float(dpp_quad_swap1(__float_as_int(v)));
  if (lpr >= 4) v += __int_as_float(dpp_quad_swap2(__float_as_int(v)));
  if (lpr >= 8) v += __int_as_float(dpp_half_mirror(__float_as_int(v)));
  if (lpr >= 16) v += __int_as_float(dpp_row_mirror(__float_as_int(v)));
  if (lpr >= 32) v = swap_add16(v);
  if (lpr >= 64) v = swap_add32(v);
  return v;
}

// (a & mask) | c in one v_and_or_b32 (the compiler splits it in two when both
// constants are literals); mask comes from an SGPR, c from a VGPR
BM_DEVICE uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}

BM_DEVICE float wave_sum(float v) {
  v += __int_as_float(dpp_quad_swap1(__float_as_int(v)));
  v += __int_as_float(dpp_quad_swap2(__float_as_int(v)));
  v += __int_as_float(dpp_half_mirror(__float_as_int(v)));
  v += __int_as_float(dpp_row_mirror(__float_as_int(v)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

BM_DEVICE float silu(float g) { return g / (1.0f + __expf(-g)); }

// bf16 bits of a float64 value, rounded to nearest-even once: the float32
// conversion (RNE) is exact to 29 extra bits, so it only misleads the second
// rounding when it lands on a bf16 halfway point; then the float64 value
// decides the direction.
BM_DEVICE uint16_t bf16_from_f64(double v) {
  const float f = float(v);
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return uint16_t((b >> 16) | ((b & 0x007FFFFFu) ? 0x0040u : 0u));
  if ((b & 0xFFFFu) == 0x8000u && double(f) != v) {
    const bool away = fabs(v) > fabs(double(f));  // the true value lies beyond the halfway point
    return uint16_t((b >> 16) + (away ? 1u : 0u));
  }
  return f32_to_bf16(f);
}


// ---- direct-to-LDS copies ----------------------------------------------------
// 16 bytes per lane from global p into LDS at byte offset lds + 16 * lane
// (global_load_lds_dwordx4; M0 holds the wave's LDS base and is set here).
// Issued from asm on purpose: for the builtin the compiler waits for every
// load in flight before any later LDS read, which would serialise a
// prefetch with the reads of the buffer before it.  Completion is therefore
// the caller's business: an explicit s_waitcnt vmcnt (loads of one wave
// complete in issue order), plus a barrier when other waves read the data.
BM_DEVICE void lds_dma16(const void *p, uint32_t lds) {
  // lds is wave-uniform; readfirstlane puts it in an SGPR when the compiler cannot tell
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(base) : "memory");
}
// 4-byte variant: lane l's dword lands at LDS byte lds + 4 l.
BM_DEVICE void lds_dma4(const void *p, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(p), "s"(base) : "memory");
}
// LDS byte offset of a generic pointer into shared memory
BM_DEVICE uint32_t lds_offset(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// ---- sticky device status record (int64 code flags, int64 detail) --------
// detail stores INT64_MAX - index so that atomicMax keeps the smallest index
// while a zero-filled record means "nothing recorded".
BM_DEVICE void record_fault(int64_t *status, int64_t flag, int64_t index) {
  if (!status) return;
  atomicOr(reinterpret_cast<unsigned long long *>(status), (unsigned long long)flag);
  atomicMax(reinterpret_cast<unsigned long long *>(status + 1),
            (unsigned long long)(INT64_MAX - index));
}

// Status flags (the values of BITMOE_DEV_* in the public header).
constexpr int64_t FAULT_BAD_EXPERT = 1, FAULT_BAD_ROW = 2, FAULT_BAD_TOKEN = 4, FAULT_DUP_EXPERT = 8;

// A pair (t, j) is served only if its expert id e lies in [0, E) and no
// earlier slot j' < j of the same token holds e: a token that names an expert
// twice gets that expert once, at its first slot.  row = the token's k ids.
BM_DEVICE bool repeats_earlier(const int32_t *row, int j, int e) {
  for (int i = 0; i < j; ++i)
    if (row[i] == e) return true;
  return false;
}

}  // namespace bm
