// Residual step between the layers of a resident multi-layer MoE stack.
//
// "Strata-DSV4.1", §DeepSeek-V4.1-Flash: the model stacks its MoE layers (40
// in the 40-layer resident configuration measured here).  Between two layers
// the stack forms r = x + y (x the layer input, y its MoE output) and rescales
// it to unit RMS without a learned weight: x' = bf16(r / sqrt(mean(r^2) + 1e-6)).
// This is a harness step of the stack, not a step of the MoE method.
//
// One block per token row; r, the sum of squares and the quotient are formed in
// float64 (r = x + y is exact), and the quotient is rounded once to bf16.
#include "common.h"
#include "internal.h"

namespace bm {

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

template <bool Y_F32>
__global__ void __launch_bounds__(256) residual_rescale_kernel(const uint16_t *__restrict__ x, const void *__restrict__ y,
                                                               int D, uint16_t *__restrict__ out) {
  constexpr int MAXE = 16;  // D <= 4096
  __shared__ double part[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = size_t(t) * D;
  double r[MAXE];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < MAXE; ++i) {
    const int c = tid + 256 * i;
    r[i] = 0.0;
    if (c < D) {
      const double yv = Y_F32 ? double(static_cast<const float *>(y)[row + c])
                              : double(bf16_to_f32(static_cast<const uint16_t *>(y)[row + c]));
      r[i] = double(bf16_to_f32(x[row + c])) + yv;
      ss = fma(r[i], r[i], ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const double total = (part[0] + part[1]) + (part[2] + part[3]);
  const double rms = sqrt(total / D + 1e-6);
#pragma unroll
  for (int i = 0; i < MAXE; ++i) {
    const int c = tid + 256 * i;
    if (c < D) out[row + c] = bf16_from_f64(r[i] / rms);
  }
}

hipError_t launch_residual_rescale(const uint16_t *x, const void *y, bool y_f32, int T, int D, uint16_t *out,
                                   hipStream_t stream) {
  if (y_f32)
    BM_LAUNCH("residual_rescale_kernel", residual_rescale_kernel<true>, dim3(T), dim3(256), 0, stream, x, y, D, out);
  else
    BM_LAUNCH("residual_rescale_kernel", residual_rescale_kernel<false>, dim3(T), dim3(256), 0, stream, x, y, D, out);
  return hipGetLastError();
}

}  // namespace bm
