// Prompt / prefill selective scan for gfx950: launch of the plain scan (the
// kernels are in scan_chunked.h and scan_rows.hip) and the choice between them.
// This file instantiates the chunked kernel without a reset mask; the
// instances with one are in scan_fwd_reset.hip.
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
// 415.2 us). SS_SCAN_TOKENS_PER_LANE=16 or =32 (read at every call) overrides
// the choice; any other value leaves it to the rule.
int pick_k(const ScanParams& p) {
  if (const char* e = std::getenv("SS_SCAN_TOKENS_PER_LANE")) {
    const std::string v(e);
    if (v == "16") return 16;
    if (v == "32") return 32;
    // anything else: the shape rule below
  }
  const int64_t blocks = p.batch * ((p.channels + 15) / 16);
  return (p.reset != nullptr && p.L >= 8192 && blocks <= 2 * static_cast<int64_t>(device_cus())) ? 32 : 16;
}

// The launch form for few rows (scan_chunked.h, Form): rows of 32 or 64
// lanes (a wave on 2 channels or 1), for launches whose plain grid would give
// each SIMD at most about two waves: there a wave's dependent chains leave
// the SIMD idle between issues, and the work does not spread evenly (6144
// rows are 1536 waves on 1024 SIMDs). The form is the first whose grid fits
// one round: 64-lane rows in 4-wave blocks (3 per CU, by LDS), 32-lane rows
// in 4-wave blocks, 32-lane rows in 8-wave blocks (2 per CU). Measured on
// MI355X, bf16 with gate, seq 2048: 4 x 1536 channels 82.7 -> 61.7 us
// (32 lanes, 4 waves; 64 lanes: 67.5); 1 x 3072: 80.7 -> 39.8 (64 lanes);
// 2 x 2048: 81.8 -> 49.1 (32 lanes, 4 waves); 4 x 2048: 85.9 -> 77.9 (32
// lanes, 8 waves). Only for K = 16 without a reset mask and N <= 16.
// SS_SCAN_FORM=plain, =r32w4, =r32w8 or =r64w4 (read at every call)
// overrides the rule.
int few_rows_form(const ScanParams& p) {
  if (p.N > 16) return kPlain;
  if (const char* e = std::getenv("SS_SCAN_FORM")) {
    const std::string v(e);
    if (v == "plain") return kPlain;
    if (v == "r32w4") return kRows32w4;
    if (v == "r32w8") return kRows32w8;
    if (v == "r64w4") return kRows64w4;
  }
  const int64_t cus = device_cus();
  if (p.batch * ((p.channels + 3) / 4) <= 3 * cus) return kRows64w4;  // 4-wave blocks, 3 per CU
  if (p.batch * ((p.channels + 7) / 8) <= 3 * cus) return kRows32w4;
  if (p.batch * ((p.channels + 15) / 16) <= 2 * cus) return kRows32w8;  // 8-wave blocks, 2 per CU
  return kPlain;
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
  if (p.reset) return launch_scan_fwd_reset(p, io_bf16, K, stream);
  const int form = K == 16 ? few_rows_form(p) : kPlain;
  if (io_bf16)
    return K == 32 ? launch_n<bf16_t, 32, kNoStates, 0>(p, stream)
                   : launch_n<bf16_t, 16, kNoStates, 0>(p, stream, form);
  return K == 32 ? launch_n<float, 32, kNoStates, 0>(p, stream) : launch_n<float, 16, kNoStates, 0>(p, stream, form);
}

int64_t scan_fwd_blocks(int64_t batch, int64_t channels) {
  // the smallest channel block of the instantiations (16 channels)
  return batch * ((channels + 15) / 16);
}

}  // namespace ss
