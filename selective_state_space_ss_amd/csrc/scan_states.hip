// Prompt / prefill selective scan that also writes per-token states, for
// gfx950: the chunked kernel (scan_chunked.h) with its state store enabled.
// The nnterp "selective_scan" page exposes the state after every token of a
// scan (the `states` attribute); the TransformerLens "ssm_mixer" page's
// compute_ssm_state returns every step or one selected time_step. Both are
// the walk's h after a token, stored as it is computed. Every token's states
// are laid out [batch, channels, N, L] (seq fastest, as the kernel's x and y):
// the 16 lanes of a row then store contiguous runs of one coordinate, where the
// [.., L, N] order would scatter 4-byte stores across a row's whole chunk.
#include "scan_chunked.h"

namespace ss {

hipError_t launch_scan_states(const ScanParams& p, bool io_bf16, hipStream_t stream) {
  const bool all = p.time_step < 0;
  if (io_bf16)
    return all ? launch_n<bf16_t, 16, kAllStates, 2>(p, stream) : launch_n<bf16_t, 16, kOneState, 2>(p, stream);
  return all ? launch_n<float, 16, kAllStates, 2>(p, stream) : launch_n<float, 16, kOneState, 2>(p, stream);
}

}  // namespace ss
