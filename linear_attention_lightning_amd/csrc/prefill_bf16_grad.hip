// The chunked kernel in the roles the gradients need: forward order with a
// (transposed) initial state that is not written back, and reversed order,
// where the causal mask becomes a suffix sum.  Instantiations of the kernel
// in prefill_bf16_kernel.hpp.
#include "prefill_bf16_kernel.hpp"

namespace lal {

hipError_t prefill_bf16_grad_launch(PrefillArgs a, int64_t BH, int d, bool reverse, hipStream_t stream) {
  return reverse ? prefill_bf16_dispatch<kPsGradRev>(a, BH, d, stream) : prefill_bf16_dispatch<kPsGrad>(a, BH, d, stream);
}

hipError_t prefill_bf16_grad_pair_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  // two "slices" per sequence, whose workgroup ids share an XCD when the grid
  // allows it (see the kernel's workgroup mapping); each covers all columns
  a.nsplit = 2;
  a.xcd_map = (BH % 8 == 0) ? 1 : 0;
  if (d == 128) return launch_nt<128, 128, kPsGradRevPair>(a, BH, stream);
  if (d == 64) return launch_nt<64, 64, kPsGradRevPair>(a, BH, stream);
  return hipErrorInvalidValue;
}

hipError_t prefill_bf16_grad_fused_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  a.nsplit = 1;
  a.xcd_map = 0;
  if (d == 128) return launch_nt<128, 128, kPsGradFused>(a, BH, stream);
  if (d == 64) return launch_nt<64, 64, kPsGradFused>(a, BH, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
