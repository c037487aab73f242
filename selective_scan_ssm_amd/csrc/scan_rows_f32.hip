// One share of the forward scan's kernels (the d_state-16 row kernel, fp32 io: the forward, its checkpointing form and the fused prologue),
// instantiated in a translation unit of its own so the library builds in parallel.
#include "scan_fwd_kernels.h"

namespace ssm {

hipError_t scan_rows_main_f32(const ScanArgs &a, hipStream_t s) { return dispatch_rows_main<float>(a, s); }

}  // namespace ssm
