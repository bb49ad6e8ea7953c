// Residual step between the layers of a resident multi-layer MoE stack.
//
// "Strata-DSV4.1", §DeepSeek-V4.1-Flash: the model stacks its MoE layers (40
// in the 40-layer resident configuration measured here).  Between two layers
// the stack forms r = x + y (x the layer input, y its MoE output) and rescales
// it to unit RMS without a learned weight: x' = bf16(r / sqrt(mean(r^2) + 1e-6)).
// This is a harness step of the stack, not a step of the MoE method.
//
// One block per token row; r, the sum of squares and the quotient are formed in
// float64 (r = x + y is exact), and the quotient is rounded once to bf16.  The
// sum of squares is added in a different order than a pairwise or sequential
// float64 sum; the orders agree to ~1e-16 relative, far inside bf16 rounding.
//
// combine_residual_kernel runs the layer's combine and this step in one launch:
// each thread combines its four columns exactly as the combine launch does,
// stores them as the layer output, and feeds the stored values to the step.
#include "common.h"
#include "internal.h"

#include "combine_units.h"

namespace bm {

// Thread i of the block owns the 4 consecutive elements 4 i .. 4 i + 3 of the
// row (D / 4 <= 1024 threads busy): sixteen waves share the float64 divisions
// of the row, so their latencies overlap.  r: the thread's r = x + y (busy
// threads); writes x' to out_row.
BM_DEVICE void rescale_row(const double (&r)[4], bool busy, int D, uint16_t *__restrict__ out_row) {
  __shared__ double part[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double ss = 0.0;
  if (busy) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = fma(r[i], r[i], ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  if (!busy) return;
  double total = 0.0;
#pragma unroll
  for (int w = 0; w < 16; ++w) total += part[w];
  const double rms = sqrt(total / D + 1e-6);
  const uint32_t o0 = uint32_t(bf16_from_f64(r[0] / rms)) | (uint32_t(bf16_from_f64(r[1] / rms)) << 16);
  const uint32_t o1 = uint32_t(bf16_from_f64(r[2] / rms)) | (uint32_t(bf16_from_f64(r[3] / rms)) << 16);
  *reinterpret_cast<uint2 *>(out_row + 4 * tid) = make_uint2(o0, o1);
}

// r = x + y for the thread's four columns (x bf16, y widened)
BM_DEVICE void residual_sum4(const uint16_t *__restrict__ xrow, int c, const float (&yv)[4], double (&r)[4]) {
  const uint2 xw = *reinterpret_cast<const uint2 *>(xrow + c);
  r[0] = double(bf16_lo(xw.x)) + double(yv[0]);
  r[1] = double(bf16_hi(xw.x)) + double(yv[1]);
  r[2] = double(bf16_lo(xw.y)) + double(yv[2]);
  r[3] = double(bf16_hi(xw.y)) + double(yv[3]);
}

template <bool Y_F32>
__global__ void __launch_bounds__(1024) residual_rescale_kernel(const uint16_t *__restrict__ x, const void *__restrict__ y,
                                                                int D, uint16_t *__restrict__ out) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const size_t row = size_t(t) * D;
  const bool busy = 4 * tid < D;
  double r[4] = {0.0, 0.0, 0.0, 0.0};
  if (busy) {
    const size_t c = row + 4 * size_t(tid);
    float yv[4];
    if constexpr (Y_F32) {
      const float4 v = *reinterpret_cast<const float4 *>(static_cast<const float *>(y) + c);
      yv[0] = v.x, yv[1] = v.y, yv[2] = v.z, yv[3] = v.w;
    } else {
      const uint2 yw = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(y) + c);
      yv[0] = bf16_lo(yw.x), yv[1] = bf16_hi(yw.x), yv[2] = bf16_lo(yw.y), yv[3] = bf16_hi(yw.y);
    }
    residual_sum4(x + row, 4 * tid, yv, r);
  }
  rescale_row(r, busy, D, out + row);
}

// One block per token: the combine of its row (out, bf16 or float32), then
// x_next = the residual step of x and the stored out.  x_next may alias x
// (each thread reads its x columns before the block's barrier and writes
// after it).
template <int K>
__global__ void __launch_bounds__(1024) combine_residual_kernel(const float *__restrict__ y, const float *__restrict__ ys,
                                                                const int32_t *__restrict__ ids,
                                                                const float *__restrict__ wts, int D, int E,
                                                                void *out, int out_bf16, int64_t *status,
                                                                const uint16_t *x, uint16_t *x_next) {
  const int t = blockIdx.x, c = 4 * int(threadIdx.x);
  const bool busy = c < D;
  double r[4] = {0.0, 0.0, 0.0, 0.0};
  if (busy) {
    const float4 o = store_out4(out, out_bf16, t, D, c, combine4<K>(y, ys, ids, wts, t, c, D, E, status));
    const float yv[4] = {o.x, o.y, o.z, o.w};
    residual_sum4(x + size_t(t) * D, c, yv, r);
  }
  rescale_row(r, busy, D, x_next + size_t(t) * D);
}

hipError_t launch_residual_rescale(const uint16_t *x, const void *y, bool y_f32, int T, int D, uint16_t *out,
                                   hipStream_t stream) {
  if (y_f32)
    BM_LAUNCH("residual_rescale_kernel", residual_rescale_kernel<true>, dim3(T), dim3(1024), 0, stream, x, y, D, out);
  else
    BM_LAUNCH("residual_rescale_kernel", residual_rescale_kernel<false>, dim3(T), dim3(1024), 0, stream, x, y, D, out);
  return hipGetLastError();
}

hipError_t launch_combine_residual(const float *y, const float *ys, const int32_t *ids, const float *wts, int T, int k,
                                   int D, int E, void *out, int out_bf16, int64_t *status, const uint16_t *x,
                                   uint16_t *x_next, hipStream_t stream) {
  if (D % 16 || D > 4096) return hipErrorNotSupported;
  return with_top_k(k, [&](auto kc) {
    BM_LAUNCH("combine_residual_kernel", combine_residual_kernel<decltype(kc)::value>, dim3(T), dim3(1024), 0, stream,
              y, ys, ids, wts, D, E, out, out_bf16, status, x, x_next);
    return hipGetLastError();
  });
}

}  // namespace bm
