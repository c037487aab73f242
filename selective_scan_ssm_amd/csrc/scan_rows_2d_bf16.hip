// One share of the forward scan's kernels (the d_state-16 row kernel, bf16 io: the 2-D orders visited in place),
// instantiated in a translation unit of its own so the library builds in parallel.
#include "scan_fwd_kernels.h"

namespace ssm {

hipError_t scan_rows_2d_bf16(const ScanArgs &a, hipStream_t s) { return dispatch_rows_2d<bf16_t>(a, s); }

}  // namespace ssm
