// One share of the forward scan's kernels (the general kernel (d_state 1..15), bf16 io with an fp32 x: the fused prologue's filtered x),
// instantiated in a translation unit of its own so the library builds in parallel.
#include "scan_fwd_kernels.h"

namespace ssm {

hipError_t scan_general_bf16_xf32(const ScanArgs &a, hipStream_t s) { return dispatch_general<bf16_t, float>(a, s); }

}  // namespace ssm
