// One share of the forward scan's kernels (the general kernel (d_state 1..15), bf16 io),
// instantiated in a translation unit of its own so the library builds in parallel.
#include "scan_fwd_kernels.h"

namespace ssm {

hipError_t scan_general_bf16(const ScanArgs &a, hipStream_t s) { return dispatch_general<bf16_t, bf16_t>(a, s); }

}  // namespace ssm
