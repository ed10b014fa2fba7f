// Chunked prefill on bf16 matrix cores with the state stored as bf16 or OCP
// FP8 E4M3 codes of state / scale: instantiations of the kernel in
// prefill_bf16_kernel.hpp.
#include "prefill_bf16_kernel.hpp"

namespace lal {

hipError_t prefill_bf16_scaled_launch(PrefillArgs a, int64_t BH, int d, int state_fmt, hipStream_t stream) {
  if (state_fmt == kStBF16) return prefill_bf16_dispatch<kPsBF16>(a, BH, d, stream);
  if (state_fmt == kStE4M3) return prefill_bf16_dispatch<kPsE4M3>(a, BH, d, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
