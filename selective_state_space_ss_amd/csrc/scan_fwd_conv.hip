// Prompt / prefill selective scan for gfx950 with the input-side producer
// fused in: x = silu(conv1d(x_pre)) is formed per lane from x_pre in
// registers (conv_silu_lane in scan_chunked.h) and never written to memory,
// where the two-kernel path writes x and reads it back (2 x 2 bytes per
// channel-token for bf16). 16 tokens per lane; state_dim up to 16 takes the
// 16-coordinate instances (coordinates past N run as the identity), up to 64
// the 64-coordinate ones; conv widths up to 4 take a 4-tap window, up to 8 an
// 8-tap one.
#include "scan_chunked.h"

namespace ss {
namespace {

template <typename IoT, int NMAX, int CW>
hipError_t launch_conv_resets(const ScanParams& p, hipStream_t stream) {
  if (p.reset) return launch_flags<IoT, 16, NMAX, kNoStates, 1, CW>(p, stream);
  return launch_flags<IoT, 16, NMAX, kNoStates, 0, CW>(p, stream);
}

template <typename IoT>
hipError_t launch_conv_io(const ScanParams& p, hipStream_t stream) {
  if (p.N <= 16)
    return p.conv_width <= 4 ? launch_conv_resets<IoT, 16, 4>(p, stream) : launch_conv_resets<IoT, 16, 8>(p, stream);
  return p.conv_width <= 4 ? launch_conv_resets<IoT, 64, 4>(p, stream) : launch_conv_resets<IoT, 64, 8>(p, stream);
}

}  // namespace

hipError_t launch_scan_fwd_conv(const ScanParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_conv_io<bf16_t>(p, stream) : launch_conv_io<float>(p, stream);
}

}  // namespace ss
