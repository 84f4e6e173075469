// C ABI entry points: validate, pick the kernel instantiation, enqueue.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "ss_scan.h"
#include "ss_launch.h"
#include "ss_validate.h"

namespace ss {

TimedLaunch& timed_launch() {
  static thread_local TimedLaunch t;
  return t;
}

hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream) {
  TimedLaunch& t = timed_launch();
  if (t.start || t.stop) {
    ++t.launches;
    return hipExtLaunchKernel(fn, grid, block, args, 0, stream, t.start, t.stop, 0);
  }
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace ss

namespace {

bool vec16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Runs one entry point with the calling thread's event pair set, so that its
// kernel's dispatch records them (launch_kernel). A call that launches
// nothing (an empty shape) records them on the stream instead, so that they
// still mark the call's place; a call that fails leaves them unrecorded.
template <typename F>
ss_status timed_call(F&& call, void* stream, void* start, void* stop) {
  ss::TimedLaunch& t = ss::timed_launch();
  t = ss::TimedLaunch{static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop), 0};
  const ss_status st = call();
  const int launched = t.launches;
  t = ss::TimedLaunch{};
  if (st == SS_OK && launched == 0) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((start && hipEventRecord(static_cast<hipEvent_t>(start), s) != hipSuccess) ||
        (stop && hipEventRecord(static_cast<hipEvent_t>(stop), s) != hipSuccess))
      return SS_ERR_HIP;
  }
  return st;
}

struct ConvArgs {
  const float* w;
  const float* b;
  int64_t width;
};

// The shared body of ss_scan_fwd, ss_scan_fwd_states (states != nullptr) and
// ss_scan_fwd_conv (conv != nullptr).
int scan_entry(const ss::ScanArgs& a, float* states, int64_t time_step, const ConvArgs* conv, void* stream) {
  const int64_t batch = a.batch, channels = a.channels, state_dim = a.state_dim, seqlen = a.seqlen;
  const int io_dtype = a.io_dtype;
  const void *x = a.x, *dt = a.dt, *z = a.z, *B = a.B, *C = a.C;
  const uint8_t* reset = a.reset;
  void* y = a.y;
  bool noop = false;
  ss_status st = ss::validate_scan(a, &noop);
  if (st == SS_OK && states) st = ss::validate_scan_states(a, states, time_step);
  if (st == SS_OK && !noop && conv) st = ss::validate_scan_conv(a, conv->w, conv->b, conv->width);
  if (st != SS_OK || noop) return st;
  if (seqlen == 0 && a.h_last == nullptr) return SS_OK;
  if (ss::scan_fwd_blocks(batch, channels) > 0x7fffffff) return SS_ERR_SHAPE;

  const bool bf16 = io_dtype == SS_BF16;
  const int64_t vec = bf16 ? 8 : 4;
  ss::ScanParams p{};
  p.batch = batch;
  p.channels = channels;
  p.L = seqlen;
  p.N = (int)state_dim;
  p.dt_softplus = a.dt_softplus != 0;
  p.vec_ok = (seqlen % vec == 0) && vec16(x) && vec16(dt) && vec16(z) && vec16(y) && vec16(B) && vec16(C);
  p.reset_vec = (seqlen % 16 == 0) && vec16(reset);
  p.x = x;
  p.dt = dt;
  p.z = z;
  p.B = B;
  p.C = C;
  p.A = a.A;
  p.D = a.D;
  p.dt_bias = a.dt_bias;
  p.h0 = a.h0;
  p.reset = reset;
  p.y = y;
  p.h_last = a.h_last;
  p.states = states;
  p.time_step = time_step;
  p.states_vec = (seqlen % 4 == 0) && vec16(states);
  if (conv) {
    p.conv_w = conv->w;
    p.conv_b = conv->b;
    p.conv_width = (int)conv->width;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = states ? ss::launch_scan_states(p, bf16, s)
                       : conv ? ss::launch_scan_fwd_conv(p, bf16, s)
                              : ss::launch_scan_fwd(p, bf16, s);
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace

extern "C" {

ss_status ss_scan_fwd(const ss_scan_args* args, void* stream) {
  if (!args) return SS_ERR_NULL;
  return static_cast<ss_status>(scan_entry(*args, nullptr, -1, nullptr, stream));
}

ss_status ss_scan_fwd_states(const ss_scan_args* args, float* states, int64_t time_step, void* stream) {
  if (!args || !states) return SS_ERR_NULL;
  return static_cast<ss_status>(scan_entry(*args, states, time_step, nullptr, stream));
}

ss_status ss_scan_fwd_conv(const ss_scan_args* args, const float* conv_w, const float* conv_b, int64_t width,
                           void* stream) {
  if (!args) return SS_ERR_NULL;
  const ConvArgs conv{conv_w, conv_b, width};
  return static_cast<ss_status>(scan_entry(*args, nullptr, -1, &conv, stream));
}

ss_status ss_state_update(const ss_update_args* args, void* stream) {
  if (!args) return SS_ERR_NULL;
  const ss_update_args& a = *args;
  bool noop = false;
  const ss_status st = ss::validate_update(a, &noop);
  if (st != SS_OK || noop) return st;
  if (!ss::state_update_grid_ok(a.batch, a.channels, a.state_dim)) return SS_ERR_SHAPE;
  ss::UpdateParams p{};
  p.batch = a.batch;
  p.channels = a.channels;
  p.N = (int)a.state_dim;
  p.dt_softplus = a.dt_softplus != 0;
  const uintptr_t bc_align = a.io_dtype == SS_BF16 ? 8 : 16;
  p.vec_ok = (a.state_dim == 16 || a.state_dim == 32 || a.state_dim == 64) && vec16(a.state) && vec16(a.A) &&
             (reinterpret_cast<uintptr_t>(a.B) % bc_align) == 0 && (reinterpret_cast<uintptr_t>(a.C) % bc_align) == 0;
  p.state = a.state;
  p.x = a.x;
  p.dt = a.dt;
  p.z = a.z;
  p.B = a.B;
  p.C = a.C;
  p.A = a.A;
  p.D = a.D;
  p.dt_bias = a.dt_bias;
  p.y = a.y;
  const hipError_t e = ss::launch_state_update(p, a.io_dtype == SS_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

ss_status ss_scan_fwd_timed(const ss_scan_args* args, void* stream, void* start_event, void* stop_event) {
  return timed_call([&] { return ss_scan_fwd(args, stream); }, stream, start_event, stop_event);
}

ss_status ss_state_update_timed(const ss_update_args* args, void* stream, void* start_event, void* stop_event) {
  return timed_call([&] { return ss_state_update(args, stream); }, stream, start_event, stop_event);
}

int ss_gated_scan(int64_t batch, int64_t seqlen, int64_t dk, int64_t dv, int io_dtype, int state_dtype,
                  const void* q, const void* k, const void* v, const float* gamma, const void* s0, void* y,
                  void* final_state, void* stream) {
  const ss::GatedArgs a{batch, seqlen, dk, dv, io_dtype, state_dtype, q, k, v, gamma, s0, y, final_state};
  bool noop = false;
  const ss_status st = ss::validate_gated(a, &noop);
  if (st != SS_OK || noop) return st;
  if (seqlen == 0 && final_state == nullptr) return SS_OK;
  if (ss::gated_scan_blocks(batch, dv) > 0x7fffffff) return SS_ERR_SHAPE;
  ss::GatedParams p{};
  p.batch = batch;
  p.L = seqlen;
  p.dk = (int)dk;
  p.dv = dv;
  p.q = q;
  p.k = k;
  p.v = v;
  p.gamma = gamma;
  p.s0 = s0;
  p.y = y;
  p.final_state = final_state;
  const hipError_t e = ss::launch_gated_scan(p, io_dtype == SS_BF16, state_dtype == SS_BF16,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

int ss_effective_attention(int64_t batch, int64_t channels, int64_t state_dim, int64_t seqlen, int io_dtype,
                           const void* dt, const float* A, const void* B, const void* C, const float* dt_bias,
                           int dt_softplus, int include_dt_scaling, int per_state_coord, float* M, void* stream) {
  const ss::AttnArgs a{batch, channels, state_dim, seqlen, io_dtype, dt, A, B, C, dt_bias,
                       dt_softplus, include_dt_scaling, per_state_coord, M};
  bool noop = false;
  const ss_status st = ss::validate_attention(a, &noop);
  if (st != SS_OK || noop) return st;
  if (ss::effective_attention_blocks(batch, channels, seqlen) > 0x7fffffff) return SS_ERR_SHAPE;
  ss::AttnParams p{};
  p.batch = batch;
  p.channels = channels;
  p.L = seqlen;
  p.N = (int)state_dim;
  p.dt = dt;
  p.A = A;
  p.B = B;
  p.C = C;
  p.dt_bias = dt_bias;
  p.dt_softplus = dt_softplus != 0;
  p.include_dt = include_dt_scaling != 0;
  p.per_state = per_state_coord != 0;
  p.M = M;
  const hipError_t e = ss::launch_effective_attention(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

int ss_conv1d_silu(int64_t batch, int64_t channels, int64_t seqlen, int64_t width, int io_dtype,
                   const void* x_pre, const float* conv_w, const float* conv_b, const uint8_t* reset,
                   void* x, void* stream) {
  const ss::ConvArgs a{batch, channels, seqlen, width, io_dtype, x_pre, conv_w, conv_b, reset, x};
  bool noop = false;
  const ss_status st = ss::validate_conv(a, &noop);
  if (st != SS_OK || noop) return st;
  if (!ss::producer_grids_ok(batch, channels, seqlen)) return SS_ERR_SHAPE;
  ss::ConvParams p{};
  p.rows = batch * channels;
  p.channels = channels;
  p.L = seqlen;
  p.W = (int)width;
  p.x_pre = x_pre;
  p.conv_w = conv_w;
  p.conv_b = conv_b;
  p.reset = reset;
  p.x = x;
  const hipError_t e = ss::launch_conv1d_silu(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

int ss_dt_proj(int64_t batch, int64_t channels, int64_t seqlen, int64_t rank, int io_dtype,
               const void* w_dt, const void* delta, const float* dt_bias, int apply_softplus,
               void* dt, void* stream) {
  const ss::ProjArgs a{batch, channels, seqlen, rank, io_dtype, w_dt, delta, dt_bias, apply_softplus, dt};
  bool noop = false;
  const ss_status st = ss::validate_proj(a, &noop);
  if (st != SS_OK || noop) return st;
  if (!ss::producer_grids_ok(batch, channels, seqlen)) return SS_ERR_SHAPE;
  ss::ProjParams p{};
  p.batch = batch;
  p.channels = channels;
  p.L = seqlen;
  p.R = rank;
  p.w_dt = w_dt;
  p.delta = delta;
  p.dt_bias = dt_bias;
  p.apply = apply_softplus != 0;
  p.dt = dt;
  const hipError_t e = ss::launch_dt_proj(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

const char* ss_status_str(int status) {
  switch (status) {
    case SS_OK: return "SS_OK";
    case SS_ERR_NULL: return "SS_ERR_NULL: a required pointer is NULL";
    case SS_ERR_SHAPE: return "SS_ERR_SHAPE: a size is negative or too large";
    case SS_ERR_DTYPE: return "SS_ERR_DTYPE: io_dtype is not SS_F32 or SS_BF16";
    case SS_ERR_UNSUPPORTED:
      return "SS_ERR_UNSUPPORTED: state_dim outside [1, 64] (gated scan: dk outside [1, 256] or dv < 1; conv width "
             "outside [1, 8]; dt_proj rank < 1)";
    case SS_ERR_ALIAS: return "SS_ERR_ALIAS: an output overlaps an input";
    case SS_ERR_HIP: return "SS_ERR_HIP: the HIP runtime failed to launch the kernel";
    case SS_ERR_ALIGN: return "SS_ERR_ALIGN: a pointer is not aligned to its element size";
    default: return "unknown ss_status";
  }
}

int ss_abi_version(void) { return SS_ABI_VERSION; }

}  // extern "C"
