// Prefill path (grouped GEMM on MFMA) -- placeholder until the kernels land.
#include "common.h"
#include "internal.h"

namespace bm {

hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t stream) {
  (void)a;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace bm
