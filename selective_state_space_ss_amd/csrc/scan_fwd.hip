// Prompt / prefill selective scan for gfx950: launch of the plain scan (the
// kernels are in scan_chunked.h and scan_rows.hip) and the choice between them.
#include "scan_chunked.h"

#include <cstdlib>
#include <string>

namespace ss {
namespace {

int pick_k() {
  const char* e = std::getenv("SS_SCAN_TOKENS_PER_LANE");
  return (e && std::atoi(e) == 32) ? 32 : 16;
}

// 1 = row-parallel walk, 2 = chunked scan. The chunked scan is the default:
// on the shapes measured so far it is the faster of the two. SS_SCAN_KERNEL=
// rows or =chunked, read at every call, picks one where the walk supports the
// shape (a tuning knob and the way the tests reach both kernels).
int pick_kernel(const ScanParams& p, bool io_bf16) {
  if (!scan_rows_supported(p, io_bf16)) return 2;
  if (const char* e = std::getenv("SS_SCAN_KERNEL")) {
    if (std::string(e) == "rows") return 1;
  }
  return 2;
}

}  // namespace

hipError_t launch_scan_fwd(const ScanParams& p, bool io_bf16, hipStream_t stream) {
  if (pick_kernel(p, io_bf16) == 1) return launch_scan_rows(p, io_bf16, stream);
  const int K = pick_k();
  if (io_bf16)
    return K == 32 ? launch_n<bf16_t, 32, kNoStates>(p, stream) : launch_n<bf16_t, 16, kNoStates>(p, stream);
  return K == 32 ? launch_n<float, 32, kNoStates>(p, stream) : launch_n<float, 16, kNoStates>(p, stream);
}

int64_t scan_fwd_blocks(int64_t batch, int64_t channels) {
  // the smallest channel block of the instantiations (16 channels)
  return batch * ((channels + 15) / 16);
}

}  // namespace ss
