// Single-token decode update of a cached fp32 state, in place, for gfx950
// (nnterp "selective_scan" page: the state-update call on one token).
//
// The step reads and writes the whole [batch, channels, state_dim] fp32
// state once, so it is bound by HBM bandwidth. Four lanes own one (b, c) row:
// lane q holds state coordinates 16k + 4q .. 16k + 4q + 3 (k < G, G = 1, 2
// or 4 groups of 16 for state_dim up to 16, 32, 64) as float4s, so a
// wavefront reads and writes 16 rows of state as one contiguous stream. A
// thread walks kRowsB batch rows of one channel (A[c, :], D[c] and dt_bias[c]
// stay in registers) in three phases -- every load issued, then the
// arithmetic, then every store -- so its loads are all in flight at once. y
// is the sum over the quad (two DPP quad_perm adds), finished by lane 0.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kThreads = 256;

// batch rows per thread: 4 at G = 1, fewer for wider states (registers)
template <int G>
constexpr int rows_per_thread() {
  return G == 1 ? 4 : (G == 2 ? 2 : 1);
}

// Four consecutive I/O elements starting at p (8 bytes of bf16 or 16 of fp32).
__device__ __forceinline__ void load4(const bf16_t* p, float* out) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  out[0] = __builtin_bit_cast(float, v.x << 16);
  out[1] = __builtin_bit_cast(float, v.x & 0xffff0000u);
  out[2] = __builtin_bit_cast(float, v.y << 16);
  out[3] = __builtin_bit_cast(float, v.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float* out) { load_vec16(p, out); }

// VEC: state_dim == 16 G (the launcher picks G from state_dim, so vec_ok,
// set for 16, 32 and 64, implies it), 16-byte aligned state and A, 8-byte
// (bf16) or 16-byte (fp32) aligned B and C: each lane moves its coordinates as
// vectors; else element by element with bounds checks.
template <typename IoT, int G, bool GATE, bool VEC>
__global__ __launch_bounds__(kThreads) void state_update_kernel(const UpdateParams p) {
  constexpr int R = rows_per_thread<G>();
  constexpr int NC = 4 * G;  // coordinates per lane
  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int64_t c_raw = (int64_t)blockIdx.x * (kThreads / 4) + (tid >> 2);
  const bool c_ok = c_raw < p.channels;
  const int64_t c = c_ok ? c_raw : p.channels - 1;  // lanes past the end compute, never store
  const int64_t b0 = (int64_t)blockIdx.y * R;
  const int N = p.N;
  const IoT* __restrict__ xg = static_cast<const IoT*>(p.x);
  const IoT* __restrict__ dg = static_cast<const IoT*>(p.dt);
  const IoT* __restrict__ zg = static_cast<const IoT*>(p.z);
  const IoT* __restrict__ Bg = static_cast<const IoT*>(p.B);
  const IoT* __restrict__ Cg = static_cast<const IoT*>(p.C);
  float* __restrict__ sg = p.state;
  // this lane's coordinate i of group k
  auto coord = [&](int k, int i) { return 16 * k + 4 * q + i; };

  // phase 1: every load
  float a2[NC];  // A[c, n] * log2(e)
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if constexpr (VEC) {
      load_vec16(p.A + c * N + coord(k, 0), a2 + 4 * k);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a2[4 * k + i] = coord(k, i) < N ? p.A[c * N + coord(k, i)] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) a2[i] *= kLog2e;
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;
  float s[R][NC], Bv[R][NC], Cv[R][NC], xv[R], dv[R], zv[R];
  int64_t rr[R];
  bool ok[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t b_raw = b0 + j;
    ok[j] = c_ok && b_raw < p.batch;
    const int64_t b = b_raw < p.batch ? b_raw : p.batch - 1;
    const int64_t r = b * p.channels + c;
    rr[j] = r;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if constexpr (VEC) {
        load_vec16(sg + r * N + coord(k, 0), s[j] + 4 * k);
        load4(Bg + b * N + coord(k, 0), Bv[j] + 4 * k);
        load4(Cg + b * N + coord(k, 0), Cv[j] + 4 * k);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = coord(k, i);
          const bool nin = n < N;
          s[j][4 * k + i] = nin ? sg[r * N + n] : 0.0f;
          Bv[j][4 * k + i] = nin ? Io<IoT>::to_f32(Bg[b * N + n]) : 0.0f;
          Cv[j][4 * k + i] = nin ? Io<IoT>::to_f32(Cg[b * N + n]) : 0.0f;
        }
      }
    }
    xv[j] = Io<IoT>::to_f32(xg[r]);
    dv[j] = Io<IoT>::to_f32(dg[r]);
    zv[j] = GATE ? Io<IoT>::to_f32(zg[r]) : 0.0f;
  }

  // phase 2: arithmetic
  float yv[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float v = dv[j] + bias;
    const float d = p.dt_softplus ? softplus_f32(v) : v;
    const float dx = d * xv[j];
    float yp = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      s[j][i] = __builtin_fmaf(fast_exp2(d * a2[i]), s[j][i], dx * Bv[j][i]);
      yp = __builtin_fmaf(Cv[j][i], s[j][i], yp);
    }
    yp += dpp_or<kDppQuadXor1>(0.0f, yp);
    yp += dpp_or<kDppQuadXor2>(0.0f, yp);
    float yo = __builtin_fmaf(Dc, xv[j], yp);
    if constexpr (GATE) yo *= silu_f32(zv[j]);
    yv[j] = yo;
  }

  // phase 3: every store
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (!ok[j]) continue;
    const int64_t r = rr[j];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if constexpr (VEC) {
        stream_store16(make_float4(s[j][4 * k], s[j][4 * k + 1], s[j][4 * k + 2], s[j][4 * k + 3]),
                       sg + r * N + coord(k, 0));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (coord(k, i) < N) sg[r * N + coord(k, i)] = s[j][4 * k + i];
      }
    }
    if (q == 0) static_cast<IoT*>(p.y)[r] = Io<IoT>::from_f32(yv[j]);
  }
}

template <typename IoT, int G, bool GATE, bool VEC>
hipError_t launch_t(const UpdateParams& p, hipStream_t stream) {
  constexpr int R = rows_per_thread<G>();
  UpdateParams q = p;
  void* args[] = {&q};
  const dim3 grid((unsigned)((p.channels + kThreads / 4 - 1) / (kThreads / 4)), (unsigned)((p.batch + R - 1) / R));
  return launch_kernel(reinterpret_cast<const void*>(&state_update_kernel<IoT, G, GATE, VEC>), grid,
                       dim3(kThreads), args, stream);
}

template <typename IoT, int G>
hipError_t launch_g(const UpdateParams& p, hipStream_t stream) {
  const bool gate = p.z != nullptr;
  if (p.vec_ok) return gate ? launch_t<IoT, G, true, true>(p, stream) : launch_t<IoT, G, false, true>(p, stream);
  return gate ? launch_t<IoT, G, true, false>(p, stream) : launch_t<IoT, G, false, false>(p, stream);
}

template <typename IoT>
hipError_t launch_io(const UpdateParams& p, hipStream_t stream) {
  if (p.N <= 16) return launch_g<IoT, 1>(p, stream);
  if (p.N <= 32) return launch_g<IoT, 2>(p, stream);
  return launch_g<IoT, 4>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const UpdateParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

bool state_update_grid_ok(int64_t batch, int64_t channels, int64_t state_dim) {
  const int64_t rows = state_dim <= 16 ? rows_per_thread<1>() : (state_dim <= 32 ? rows_per_thread<2>() : rows_per_thread<4>());
  return (channels + kThreads / 4 - 1) / (kThreads / 4) <= 0x7fffffff && (batch + rows - 1) / rows <= 65535;
}

}  // namespace ss
