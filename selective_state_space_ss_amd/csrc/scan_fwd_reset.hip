// Prompt / prefill selective scan for gfx950: the chunked kernel's instances
// with a reset mask (packed sequences, "s6_reset" post, Enforced Boundary
// Resetting), in a file of their own so that they are built with the machine
// scheduler that measured faster for them (iterative ILP; the instances
// without a reset mask measured faster with the default scheduler). The tokens
// per lane are chosen by the caller, launch_scan_fwd in scan_fwd.hip.
#include "scan_chunked.h"

namespace ss {

hipError_t launch_scan_fwd_reset(const ScanParams& p, bool io_bf16, int K, hipStream_t stream) {
  if (io_bf16)
    return K == 32 ? launch_n<bf16_t, 32, kNoStates, 1>(p, stream) : launch_n<bf16_t, 16, kNoStates, 1>(p, stream);
  return K == 32 ? launch_n<float, 32, kNoStates, 1>(p, stream) : launch_n<float, 16, kNoStates, 1>(p, stream);
}

}  // namespace ss
