// Prompt / prefill selective scan for gfx950: launch of the plain scan (the
// kernels are in scan_chunked.h and scan_rows.hip) and the choice between them.
#include "scan_chunked.h"

#include <atomic>
#include <cstdlib>
#include <string>

namespace ss {
namespace {

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tokens per lane. K = 16 is the default. With a reset mask the kernel's
// blocks are 16 channels at 3 per CU (K = 16) or 2 per CU (K = 32, half the
// per-chunk scan work). K = 32 wins where its grid fits one round of 2 blocks
// per CU, so that the K = 16 grid would leave slots empty, and the sequence
// is long. Measured at 4 x 2048 channels (512 blocks), reset mask, seq 8192:
// 316.5 against 332.7 us (354.9 against 370.5 with a gate). At seq 4096 the
// two were even, and at 2048 K = 16 was faster (90.1 against 92.5 us). At
// 8 x 5120 channels x 2048 (2560 blocks) K = 16 was far faster (371.8 against
// 415.2 us). SS_SCAN_TOKENS_PER_LANE=16|32 (read at every call) overrides the
// choice.
int pick_k(const ScanParams& p) {
  if (const char* e = std::getenv("SS_SCAN_TOKENS_PER_LANE")) return std::atoi(e) == 32 ? 32 : 16;
  const int64_t blocks = p.batch * ((p.channels + 15) / 16);
  return (p.reset != nullptr && p.L >= 8192 && blocks <= 2 * static_cast<int64_t>(device_cus())) ? 32 : 16;
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
  const int K = pick_k(p);
  if (io_bf16)
    return K == 32 ? launch_n<bf16_t, 32, kNoStates>(p, stream) : launch_n<bf16_t, 16, kNoStates>(p, stream);
  return K == 32 ? launch_n<float, 32, kNoStates>(p, stream) : launch_n<float, 16, kNoStates>(p, stream);
}

int64_t scan_fwd_blocks(int64_t batch, int64_t channels) {
  // the smallest channel block of the instantiations (16 channels)
  return batch * ((channels + 15) / 16);
}

}  // namespace ss
