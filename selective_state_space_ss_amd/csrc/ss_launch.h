// Kernel parameter blocks and launchers shared by the C ABI (ss_abi.hip) and
// the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

struct ScanParams {
  int64_t batch, channels, L;
  int64_t chan_blocks;  // ceil(channels / channels per block)
  int N;
  int dt_softplus;
  int vec_ok;    // x, dt, z, y, B, C are 16-byte aligned and L is a multiple of the vector width
  int reset_vec; // reset is 16-byte aligned and L is a multiple of 16
  const void* x;
  const void* dt;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* h0;
  const uint8_t* reset;
  void* y;
  float* h_last;
  float* states;      // per-token states (launch_scan_states only)
  int64_t time_step;  // < 0: every token's state; else the state after this token
  int states_vec;     // states 16-byte aligned and L a multiple of 4
  // fused conv1d + SiLU (launch_scan_fwd_conv only): x is then x_pre
  const float* conv_w;  // [channels, conv_width]
  const float* conv_b;  // [channels] or nullptr
  int conv_width;
};

struct UpdateParams {
  int64_t batch, channels;
  int N;
  int dt_softplus;
  int vec_ok;  // N is 16, 32 or 64, state and A 16-byte aligned, B and C aligned to 4 elements
  float* state;
  const void* x;
  const void* dt;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* dt_bias;
  void* y;
};

struct GatedParams {
  int64_t batch, L, dv;
  int dk;
  int64_t col_blocks;  // ceil(dv / columns per block)
  const void* q;       // [batch, L, dk]
  const void* k;       // [batch, L, dk]
  const void* v;       // [batch, L, dv]
  const float* gamma;  // [batch, L]
  const void* s0;      // [batch, dk, dv] or nullptr, state dtype
  void* y;             // [batch, L, dv]
  void* final_state;   // [batch, dk, dv] or nullptr, state dtype
};

// io_bf16: element type of x, dt, z, B, C, y (false = float32).
// launch_scan_fwd picks between the chunked scan (scan_fwd.hip) and the
// row-parallel walk (scan_rows.hip, launch_scan_rows) by shape.
hipError_t launch_scan_fwd(const ScanParams& p, bool io_bf16, hipStream_t stream);
// The prompt scan with its x made in the kernel from x_pre (p.x) by the
// causal conv1d + SiLU (scan_fwd_conv.hip): 16 tokens per lane, N <= 16 or
// <= 64 instances, conv width <= 8.
hipError_t launch_scan_fwd_conv(const ScanParams& p, bool io_bf16, hipStream_t stream);
// The chunked scan's instances with a reset mask (scan_fwd_reset.hip), at K
// tokens per lane (16 or 32).
hipError_t launch_scan_fwd_reset(const ScanParams& p, bool io_bf16, int K, hipStream_t stream);
hipError_t launch_scan_rows(const ScanParams& p, bool io_bf16, hipStream_t stream);
// The scan that also writes per-token states (scan_states.hip): p.states
// receives [batch, channels, N, L] (p.time_step < 0) or the state after token
// p.time_step, [batch, channels, N].
hipError_t launch_scan_states(const ScanParams& p, bool io_bf16, hipStream_t stream);
// The row-parallel walk needs L a multiple of 4, N <= 16, x, dt, z, y, B, C
// aligned to two elements and reset to 4 bytes.
bool scan_rows_supported(const ScanParams& p, bool io_bf16);
hipError_t launch_state_update(const UpdateParams& p, bool io_bf16, hipStream_t stream);
// The scalar-gated state scan (gated_scan.hip); io_bf16: element type of q, k, v, y.
// Input-side producers; see ss_conv1d_silu and ss_dt_proj in ss_scan.h.
struct ConvParams {
  int64_t rows, channels, L;   // rows = batch * channels
  int W;
  const void* x_pre;           // [batch, channels, L]
  const float* conv_w;         // [channels, W]
  const float* conv_b;         // [channels] or nullptr
  const uint8_t* reset;        // [batch, L] or nullptr
  void* x;                     // [batch, channels, L]
};

struct ProjParams {
  int64_t batch, channels, L, R;
  const void* w_dt;            // [channels, R]
  const void* delta;           // [batch, L, R]
  const float* dt_bias;        // [channels] or nullptr
  int apply;                   // softplus(dt + dt_bias)
  void* dt;                    // [batch, channels, L]
};

hipError_t launch_conv1d_silu(const ConvParams& p, bool io_bf16, hipStream_t stream);
hipError_t launch_dt_proj(const ProjParams& p, bool io_bf16, hipStream_t stream);

// Effective attention; see ss_effective_attention in ss_scan.h.
struct AttnParams {
  int64_t batch, channels, L;
  int N;
  int64_t jblocks;      // ceil(L / columns per block)
  const void* dt;       // [batch, channels, L]
  const float* A;       // [channels, N]
  const void* B;        // [batch, N, L]
  const void* C;        // [batch, N, L]
  const float* dt_bias; // [channels] or nullptr
  int dt_softplus, include_dt, per_state;
  float* M;             // [batch, channels, L, L] or [batch, channels, N, L, L]
  int out_vec;          // rows of M are whole 16-byte vectors (set by the launcher)
};

hipError_t launch_effective_attention(const AttnParams& p, bool io_bf16, hipStream_t stream);

// io_bf16: element type of q, k, v, y; state_bf16: that of s0 and final_state.
hipError_t launch_gated_scan(const GatedParams& p, bool io_bf16, bool state_bf16, hipStream_t stream);

}  // namespace ss

namespace ss {
// Every kernel of the library is launched through launch_kernel (no dynamic
// LDS). A call made through ss_scan_fwd_timed or ss_state_update_timed first
// sets the calling thread's event pair; launch_kernel then gives the events
// to the dispatch itself (hipExtLaunchKernel), which records them when the
// kernel starts and when it ends, and counts the launch.
struct TimedLaunch {
  hipEvent_t start = nullptr, stop = nullptr;
  int launches = 0;
};
TimedLaunch& timed_launch();  // the calling thread's
hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream);

// Launch-geometry limits, checked by the C ABI before launching.
int64_t scan_fwd_blocks(int64_t batch, int64_t channels);
bool state_update_grid_ok(int64_t batch, int64_t channels, int64_t state_dim);
int64_t gated_scan_blocks(int64_t batch, int64_t dv);
int64_t effective_attention_blocks(int64_t batch, int64_t channels, int64_t L);
bool producer_grids_ok(int64_t batch, int64_t channels, int64_t L);
}  // namespace ss
