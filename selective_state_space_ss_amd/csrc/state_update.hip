// Single-token decode update of a cached fp32 state, in place, for gfx950
// (nnterp "selective_scan" page: the state-update call on one token).
//
// The step reads and writes the whole [batch, channels, state_dim] fp32
// state once, so it is bound by HBM bandwidth. Four lanes own one (b, c) row:
// lane q holds state coordinates 4q..4q+3 as a float4, so a wavefront reads
// and writes 16 rows = 1 KiB of state as one contiguous stream. A thread
// walks kRowsB batch rows of one channel (A[c, :], D[c] and dt_bias[c] stay in
// registers) in three phases -- every load issued, then the arithmetic, then
// every store -- so its loads are all in flight at once. y is the sum over
// the quad (two DPP quad_perm adds), finished by lane 0 of the quad.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsB = 4;  // batch rows per thread

// Four consecutive I/O elements starting at p (8 bytes of bf16 or 16 of fp32).
__device__ __forceinline__ void load4(const bf16_t* p, float* out) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  out[0] = __builtin_bit_cast(float, v.x << 16);
  out[1] = __builtin_bit_cast(float, v.x & 0xffff0000u);
  out[2] = __builtin_bit_cast(float, v.y << 16);
  out[3] = __builtin_bit_cast(float, v.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float* out) { load_vec16(p, out); }

// VEC: state_dim == 16 and 16-byte aligned state / 8-byte (bf16) or 16-byte
// (fp32) aligned B and C, so each lane moves its 4 coordinates as vectors.
template <typename IoT, bool GATE, bool VEC>
__global__ __launch_bounds__(kThreads) void state_update_kernel(const UpdateParams p) {
  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int64_t c_raw = (int64_t)blockIdx.x * (kThreads / 4) + (tid >> 2);
  const bool c_ok = c_raw < p.channels;
  const int64_t c = c_ok ? c_raw : p.channels - 1;  // lanes past the end compute, never store
  const int64_t b0 = (int64_t)blockIdx.y * kRowsB;
  const int N = p.N;
  const IoT* __restrict__ xg = static_cast<const IoT*>(p.x);
  const IoT* __restrict__ dg = static_cast<const IoT*>(p.dt);
  const IoT* __restrict__ zg = static_cast<const IoT*>(p.z);
  const IoT* __restrict__ Bg = static_cast<const IoT*>(p.B);
  const IoT* __restrict__ Cg = static_cast<const IoT*>(p.C);
  float* __restrict__ sg = p.state;

  // phase 1: every load
  float a2[4];  // A[c, 4q..4q+3] * log2(e)
  if constexpr (VEC) {
    load_vec16(p.A + c * N + 4 * q, a2);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a2[i] = 4 * q + i < N ? p.A[c * N + 4 * q + i] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) a2[i] *= kLog2e;
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;
  float s[kRowsB][4], Bv[kRowsB][4], Cv[kRowsB][4], xv[kRowsB], dv[kRowsB], zv[kRowsB];
  int64_t rr[kRowsB];
  bool ok[kRowsB];
#pragma unroll
  for (int k = 0; k < kRowsB; ++k) {
    const int64_t b_raw = b0 + k;
    ok[k] = c_ok && b_raw < p.batch;
    const int64_t b = b_raw < p.batch ? b_raw : p.batch - 1;
    const int64_t r = b * p.channels + c;
    rr[k] = r;
    if constexpr (VEC) {
      load_vec16(sg + r * N + 4 * q, s[k]);
      load4(Bg + b * N + 4 * q, Bv[k]);
      load4(Cg + b * N + 4 * q, Cv[k]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * q + i;
        const bool nin = n < N;
        s[k][i] = nin ? sg[r * N + n] : 0.0f;
        Bv[k][i] = nin ? Io<IoT>::to_f32(Bg[b * N + n]) : 0.0f;
        Cv[k][i] = nin ? Io<IoT>::to_f32(Cg[b * N + n]) : 0.0f;
      }
    }
    xv[k] = Io<IoT>::to_f32(xg[r]);
    dv[k] = Io<IoT>::to_f32(dg[r]);
    zv[k] = GATE ? Io<IoT>::to_f32(zg[r]) : 0.0f;
  }

  // phase 2: arithmetic
  float yv[kRowsB];
#pragma unroll
  for (int k = 0; k < kRowsB; ++k) {
    const float v = dv[k] + bias;
    const float d = p.dt_softplus ? softplus_f32(v) : v;
    const float dx = d * xv[k];
    float yp = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[k][i] = __builtin_fmaf(fast_exp2(d * a2[i]), s[k][i], dx * Bv[k][i]);
      yp = __builtin_fmaf(Cv[k][i], s[k][i], yp);
    }
    yp += dpp_or<kDppQuadXor1>(0.0f, yp);
    yp += dpp_or<kDppQuadXor2>(0.0f, yp);
    float yo = __builtin_fmaf(Dc, xv[k], yp);
    if constexpr (GATE) yo *= silu_f32(zv[k]);
    yv[k] = yo;
  }

  // phase 3: every store
#pragma unroll
  for (int k = 0; k < kRowsB; ++k) {
    if (!ok[k]) continue;
    const int64_t r = rr[k];
    if constexpr (VEC) {
      *reinterpret_cast<float4*>(sg + r * N + 4 * q) = make_float4(s[k][0], s[k][1], s[k][2], s[k][3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < N) sg[r * N + 4 * q + i] = s[k][i];
    }
    if (q == 0) static_cast<IoT*>(p.y)[r] = Io<IoT>::from_f32(yv[k]);
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
