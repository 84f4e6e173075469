// Single-token decode update of a cached fp32 state, in place, for gfx950
// (nnterp "selective_scan" page: the state-update call on one token).
//
// Four lanes own one (b, c) row: lane q holds state coordinates 4q..4q+3 as a
// float4, so a wavefront reads and writes 16 rows = 1 KiB of state as one
// contiguous stream. A thread walks kRowsB batch rows of the same channel,
// keeping A[c, :], D[c] and dt_bias[c] in registers, and issues all of its
// state loads before the arithmetic. y is the sum over the quad (two DPP
// quad_perm adds), finished by lane 0 of the quad.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsB = 4;  // batch rows per thread

template <typename IoT, bool GATE, bool VEC>
__global__ __launch_bounds__(kThreads) void state_update_kernel(const UpdateParams p) {
  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int64_t c_raw = (int64_t)blockIdx.x * (kThreads / 4) + (tid >> 2);
  const bool c_ok = c_raw < p.channels;
  const int64_t c = c_ok ? c_raw : p.channels - 1;
  const int64_t b0 = (int64_t)blockIdx.y * kRowsB;
  const int N = p.N;

  float a2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 4 * q + i;
    a2[i] = n < N ? p.A[c * N + n] * kLog2e : 0.0f;
  }
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;
  const IoT* __restrict__ xg = static_cast<const IoT*>(p.x);
  const IoT* __restrict__ dg = static_cast<const IoT*>(p.dt);
  const IoT* __restrict__ zg = static_cast<const IoT*>(p.z);
  const IoT* __restrict__ Bg = static_cast<const IoT*>(p.B);
  const IoT* __restrict__ Cg = static_cast<const IoT*>(p.C);

  float s[kRowsB][4];
  bool ok[kRowsB];
  int64_t rb[kRowsB], bb[kRowsB];
#pragma unroll
  for (int k = 0; k < kRowsB; ++k) {
    const int64_t b = b0 + k;
    ok[k] = c_ok && b < p.batch;
    bb[k] = b < p.batch ? b : p.batch - 1;
    rb[k] = bb[k] * p.channels + c;
    float* st = p.state + rb[k] * N + 4 * q;
    if constexpr (VEC) {
      const float4 v = *reinterpret_cast<const float4*>(st);
      s[k][0] = v.x; s[k][1] = v.y; s[k][2] = v.z; s[k][3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[k][i] = (4 * q + i < N) ? st[i] : 0.0f;
    }
  }

#pragma unroll
  for (int k = 0; k < kRowsB; ++k) {
    const int64_t r = rb[k];
    const int64_t b = bb[k];
    const float xv = Io<IoT>::to_f32(xg[r]);
    const float v = Io<IoT>::to_f32(dg[r]) + bias;
    const float d = p.dt_softplus ? softplus_f32(v) : v;
    const float dx = d * xv;
    float yp = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 4 * q + i;
      const bool nin = n < N;
      const float Bn = nin ? Io<IoT>::to_f32(Bg[b * N + n]) : 0.0f;
      const float Cn = nin ? Io<IoT>::to_f32(Cg[b * N + n]) : 0.0f;
      s[k][i] = __builtin_fmaf(fast_exp2(d * a2[i]), s[k][i], dx * Bn);
      yp = __builtin_fmaf(Cn, s[k][i], yp);
    }
    yp += dpp_or<kDppQuadXor1>(0.0f, yp);
    yp += dpp_or<kDppQuadXor2>(0.0f, yp);
    if (ok[k]) {
      float* st = p.state + r * N + 4 * q;
      if constexpr (VEC) {
        *reinterpret_cast<float4*>(st) = make_float4(s[k][0], s[k][1], s[k][2], s[k][3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * q + i < N) st[i] = s[k][i];
      }
      if (q == 0) {
        float yv = __builtin_fmaf(Dc, xv, yp);
        if constexpr (GATE) yv *= silu_f32(Io<IoT>::to_f32(zg[r]));
        static_cast<IoT*>(p.y)[r] = Io<IoT>::from_f32(yv);
      }
    }
  }
}

template <typename IoT, bool GATE, bool VEC>
hipError_t launch_t(const UpdateParams& p, hipStream_t stream) {
  UpdateParams q = p;
  void* args[] = {&q};
  const dim3 grid((unsigned)((p.channels + kThreads / 4 - 1) / (kThreads / 4)),
                  (unsigned)((p.batch + kRowsB - 1) / kRowsB));
  return hipLaunchKernel(reinterpret_cast<const void*>(&state_update_kernel<IoT, GATE, VEC>), grid,
                         dim3(kThreads), args, 0, stream);
}

template <typename IoT>
hipError_t launch_io(const UpdateParams& p, hipStream_t stream) {
  const bool gate = p.z != nullptr;
  if (p.vec_ok) return gate ? launch_t<IoT, true, true>(p, stream) : launch_t<IoT, false, true>(p, stream);
  return gate ? launch_t<IoT, true, false>(p, stream) : launch_t<IoT, false, false>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const UpdateParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

bool state_update_grid_ok(int64_t batch, int64_t channels) {
  return (channels + kThreads / 4 - 1) / (kThreads / 4) <= 0x7fffffff &&
         (batch + kRowsB - 1) / kRowsB <= 65535;
}

}  // namespace ss
