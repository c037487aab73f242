// d_state = 1 ("SM1", the scalar-state Mamba-1 scan of the "Windows SM1
// (Scalar Mamba1)" page) forward scan.
#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {

size_t sm1_workspace(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_sm1_scan(const ScanArgs &a, hipStream_t s) {
    ScanArgs g = a;
    g.dstate = 1;
    return launch_scan_fwd(g, s);
}

}  // namespace ssm
