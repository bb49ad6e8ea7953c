// Launch functions of the kernel translation units (internal to libbitmoe).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bm {

// Launch timing (off unless bitmoe_profile_start() was called): prof_events
// hands out a start/stop event pair for the launch, or nulls when timing is
// off.  The pair goes to hipExtLaunchKernel, which stamps it from the kernel's
// own dispatch (start and end of its execution, no queue gaps).
void prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop);

#define BM_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                                        \
  do {                                                                                                  \
    hipEvent_t bm_ev_a_ = nullptr, bm_ev_b_ = nullptr;                                                  \
    ::bm::prof_events(name, &bm_ev_a_, &bm_ev_b_);                                                      \
    if (bm_ev_a_)                                                                                       \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, bm_ev_a_, bm_ev_b_, 0u, __VA_ARGS__);   \
    else                                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                              \
  } while (0)

// Engram tables of one gather launch (up to four; by value as a kernel argument)
constexpr int ENGRAM_MAX_TABLES = 4;
struct EngramTables {
  const uint8_t *table[ENGRAM_MAX_TABLES];
  int64_t rows[ENGRAM_MAX_TABLES];
  int32_t n;
};
// id i of row_ids reads tabs.table[(i / per) % tabs.n]
hipError_t launch_engram_gather(const EngramTables &tabs, int32_t per, const int64_t *row_ids, int64_t n,
                                uint16_t *out, int64_t *status, hipStream_t stream);
// kv: [T][5 W] float32 scratch
hipError_t launch_engram_inject(const uint16_t *rows, int T, int n_rows, const uint16_t *w_kv, int W,
                                const float *q_norm, const float *k_norm, float eps, const uint8_t *mask,
                                uint16_t *residual, float *gate_out, float *kv, hipStream_t stream);
hipError_t launch_dequant(const void *blocks, int wfmt, int64_t n_weights, void *out, int out_bf16,
                          hipStream_t stream);
hipError_t launch_fill(void *dst, int64_t n_bytes, uint64_t key, int kind, const uint16_t *lut,
                       hipStream_t stream);
hipError_t launch_probe_read(const void *src, int64_t n_bytes, uint32_t *sink, int blocks, hipStream_t stream);
// wsplit: router_split_bytes(E, D) of scratch for T > 8 (the router matrix's
// exact bf16 parts), or null (then T > 8 runs the float32 tile kernel)
size_t router_split_bytes(int E, int D);
hipError_t launch_route(const void *x, bool xbf16, int T, int D, int E, int k, const float *wr, const float *bias,
                        float *logits, int32_t *ids, float *wts, uint16_t *wsplit, hipStream_t stream);

// score: 0 softmax, 1 sqrt(softplus); select_bias and hash_table/token_ids
// optional (see moe_route_ex)
hipError_t launch_route_variant(const void *x, bool xbf16, int T, int D, int E, int k, const float *wr,
                                const float *logit_bias, int score, const float *select_bias,
                                const int32_t *hash_table, const int32_t *token_ids, int64_t vocab, float *logits,
                                int32_t *ids, float *wts, int64_t *status, uint16_t *wsplit, hipStream_t stream);

struct PlanBufs {
  int32_t *counts;
  int32_t *offsets;
  int32_t *perm;
  int32_t *union_ids;
  int32_t *n_union;
  int32_t *chunk_counts;
  int32_t *tile_off;   // [E+1] prefix of ceil(count / bm_tile), or null
  int32_t *tile_off2;  // [E+1] prefix of ceil(count / bm_tile2), or null
  int64_t *status;
};
hipError_t launch_plan(const int32_t *ids, int T, int k, int E, int bm_tile, int bm_tile2, PlanBufs p,
                       hipStream_t stream);
size_t plan_scratch_bytes(int T, int E);

struct FfnArgs {
  int D, F, E, k, T;
  const uint8_t *wg, *wu, *wd;
  const uint8_t *sg, *su, *sd;
  const void *x;
  const int32_t *ids;
  const float *wts;
  uint16_t *h;     // [T*k][F] bf16 (hi part in float32 mode)
  uint16_t *hs;    // [T][F]
  uint16_t *h_lo;  // float32 mode: lo parts, else unused
  uint16_t *hs_lo;
  float *hf;       // int8 numerics: [T*k][F] float32 h (pair order)
  float *hsf;      // int8 numerics: [T][F] float32 h of the shared expert
  float *y;
  float *ys;
  void *out;
  int out_bf16;
  int64_t *status;
  const uint16_t *x_res;  // with x_next: the combine also runs the residual step of x_res (bf16)
  uint16_t *x_next;
  int chunks_gu, rows_gu;   // routed gate/up: row chunks per job, rows per chunk
  int chunks_dn, rows_dn;   // routed down
  int chunks_sg, rows_sg;   // shared gate/up (0 chunks: no shared blocks in the launch)
  int chunks_sd, rows_sd;   // shared down
  int u_max;
};
hipError_t launch_decode_ffn(FfnArgs a, bool xf32, hipStream_t stream);
// router logits alone for T <= 8 tokens (the router_gemv_kernel launch of launch_route)
hipError_t launch_route_logits(const void *x, bool xbf16, int T, int D, int E, const float *wr, const float *bias,
                               float *logits, hipStream_t stream);
// router + experts + combine of one token (T = 1) in four launches; a.ids and
// a.wts receive the selection (hipErrorNotSupported for T != 1, k > 8, E > 1024)
hipError_t launch_decode_layer(FfnArgs a, bool xf32, const float *wr, const float *bias, float *logits,
                               hipStream_t stream);
// int8 activation numerics (T <= 8; d_model, d_ff multiples of 256): a.hf /
// a.hsf carry h, a.h* are unused
hipError_t launch_decode_ffn_i8(FfnArgs a, bool xf32, hipStream_t stream);
// the int8 mode's quantiser over [rows][cols] (cols a multiple of 32)
hipError_t launch_quantize_q8(const void *x, bool xf32, int64_t rows, int cols, uint8_t *q, float *d, float *s,
                              hipStream_t stream);
// The combine of every path (out = the layer output); with x_next set, the
// same launch also runs the stack's residual step x_next = rescale(x_res + out)
// (x_res bf16 [T][D], D a multiple of 16 up to 4096; stack.hip).
hipError_t launch_combine(const float *y, const float *ys, const int32_t *ids, const float *wts, int T, int k, int D,
                          int E, void *out, int out_bf16, int64_t *status, const uint16_t *x_res, uint16_t *x_next,
                          hipStream_t stream);
hipError_t launch_combine_residual(const float *y, const float *ys, const int32_t *ids, const float *wts, int T, int k,
                                   int D, int E, void *out, int out_bf16, int64_t *status, const uint16_t *x,
                                   uint16_t *x_next, hipStream_t stream);

struct PrefillArgs {
  int D, F, E, k, T;
  const uint8_t *wg, *wu, *wd;
  const uint8_t *sg, *su, *sd;
  const void *x;
  int x_f32;
  const int32_t *ids;
  const float *wts;
  PlanBufs plan;
  int32_t *tile_off;   // [E+1] chunks of PREFILL_BM tokens per expert, prefix
  int32_t *tile_off2;  // [E+1] chunks of PREFILL_BM_DOWN pairs per expert, prefix
  uint16_t *xs;        // [T][D] bf16 copy of x (x_f32 only)
  uint16_t *h;         // [T*k][F] bf16 hi part of h, pair order
  uint16_t *hs;        // [T][F] bf16 hi part (shared expert)
  uint16_t *h_lo;      // lo parts
  uint16_t *hs_lo;
  uint16_t *sw_bf16;   // the shared expert expanded for its dense GEMMs (gate, up, down): 3 x F*D*17/8 bytes
  uint16_t *xsum;      // activation sub-block sums of the grouped GEMMs: max(T*D, T*k*F) / 8 bf16
  float *xtot;         // -128 x the activation super-block sums (float32): max(T*D, T*k*F) / 256
  float *y;            // [T*k][D] float32, pair order
  float *ys;           // [T][D]
  void *out;
  int out_bf16;
  int64_t *status;
  const uint16_t *x_res;  // with x_next: the combine also runs the residual step of x_res (bf16)
  uint16_t *x_next;
};
hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t stream);
// routed grouped GEMM (gate/up with h out, or down with y out) over the plan's
// chunks, after the activation rows' sub-block sums (into sums)
// Int8 numerics of the prefill path (prefill_i8.hip)
struct PrefillI8Args {
  int D, F, E, k, T;
  const uint8_t *wg, *wu, *wd;
  const uint8_t *sg, *su, *sd;
  const void *x;
  bool x_f32;
  const int32_t *ids;
  const float *wts;
  PlanBufs plan;
  int32_t *tile_off, *tile_off2;  // chunk lists of the plan (PREFILL_BM, PREFILL_BM_DOWN rows)
  int8_t *xq;                     // [T][D] quantised x, with its block scales [T][D/32] and stored sums [T][D/16]
  float *xd, *xs;
  uint16_t *sums;                 // stored sums in the min-term layout: max(T*D, T*k*F) / 8 bf16
  float *hf;                      // [T*k][F] h in float32 (pair order)
  int8_t *hq;                     // [T*k][F] quantised h, scales [T*k][F/32], sums [T*k][F/16]
  float *hd, *hs;
  int8_t *sw_i8;                  // [3][F*D] int8 codes of the shared expert (gate, up, down)
  float *sw_d;                    // [3][F*D/32] their scales
  float *hsf;                     // [T][F] shared h in float32
  int8_t *hsq;                    // [T][F] quantised, scales [T][F/32], sums [T][F/16]
  float *hsd, *hss;
  float *y;                       // [T*k][D] float32, pair order
  float *ys;                      // [T][D]
  void *out;
  int out_bf16;
  int64_t *status;
  const uint16_t *x_res;  // with x_next: the combine also runs the residual step of x_res (bf16)
  uint16_t *x_next;
};
hipError_t launch_prefill_ffn_i8(const PrefillI8Args &a, hipStream_t stream);
hipError_t launch_probe_mfma(int blocks, int iters, uint32_t *sink, hipStream_t stream);
hipError_t launch_q2_group(bool gateup, const PrefillArgs &a, const uint16_t *x, uint16_t *sums, float *tot,
                           hipStream_t stream);
hipError_t launch_residual_rescale(const uint16_t *x, const void *y, bool y_f32, int T, int D, uint16_t *out,
                                   hipStream_t stream);
// 16-row M-tiles per chunk of the routed grouped GEMMs
#ifndef BM_PF_CHUNK_GU
#define BM_PF_CHUNK_GU 3
#endif
#ifndef BM_PF_CHUNK_DN
#define BM_PF_CHUNK_DN 2
#endif
constexpr int PREFILL_BM = 16 * BM_PF_CHUNK_GU;       // tokens per chunk of the gate/up grouped GEMM (tile_off)
constexpr int PREFILL_BM_DOWN = 16 * BM_PF_CHUNK_DN;  // pairs per chunk of the down grouped GEMM (tile_off2)

}  // namespace bm
