// The chunked kernel in the roles the gradients need: forward order with a
// (transposed) initial state that is not written back, and reversed order,
// where the causal mask becomes a suffix sum.  Instantiations of the kernel
// in prefill_bf16_kernel.hpp.
#include "prefill_bf16_kernel.hpp"

namespace lal {

hipError_t prefill_bf16_grad_launch(PrefillArgs a, int64_t BH, int d, bool reverse, hipStream_t stream) {
  return reverse ? prefill_bf16_dispatch<kPsGradRev>(a, BH, d, stream) : prefill_bf16_dispatch<kPsGrad>(a, BH, d, stream);
}

}  // namespace lal
