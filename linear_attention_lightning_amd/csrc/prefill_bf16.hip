// Chunked prefill on bf16 matrix cores with an fp32 state (and optional
// state snapshots): instantiations of the kernel in prefill_bf16_kernel.hpp.
#include "prefill_bf16_kernel.hpp"

namespace lal {

int prefill_bf16_max_block(int) { return kBlkMax; }

int prefill_bf16_max_split(int d) { return d == 128 ? 4 : 2; }

hipError_t prefill_bf16_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  return a.snap ? prefill_bf16_dispatch<kPsF32Snap>(a, BH, d, stream) : prefill_bf16_dispatch<kPsF32>(a, BH, d, stream);
}

hipError_t prefill_bf16_part_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  return prefill_bf16_dispatch<kPsPart>(a, BH, d, stream);
}

// d = 128 only: at d = 64 the two-launch form is the faster one
hipError_t prefill_bf16_part_lb_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  return prefill_bf16_dispatch<kPsPartLB, false>(a, BH, d, stream);
}

}  // namespace lal
