// Effective attention of the selective scan for gfx950 (TransformerLens
// "ssm_mixer" page, compute_effective_attention): per batch item b and
// channel c,
//
//   M[i, j] = sum_n C[b, n, i] * prod_{k=j+1..i} exp(A[c, n] dt[b, c, k]) * B[b, n, j]
//
// for j <= i and 0 above the diagonal, with dt the scan's step size
// (softplus(dt + dt_bias) or dt + dt_bias); optionally column j scaled by
// dt[b, c, j], or the terms kept per state coordinate n.
//
// Work and bound. Every (i, j) element of the lower triangle needs the N
// running products of its column, so a lane owns one column j and carries
// d[n] = B[b, n, j] (* dt_j) * prod_{k=j+1..i} exp(A[c, n] dt_k) down the
// rows: one multiply to extend each product and one FMA to contract it with
// C per state coordinate and row, 2 N VALU operations per element, and no
// transcendental in the row loop. The output (4 L^2 bytes per channel, N
// times that unsummed) is the dominant traffic; each row step of a wave
// stores 64 consecutive columns (256 contiguous bytes).
//
// Layout. A block is (b, c) and 256 columns, one wave per 64 columns (which
// wave takes which 64 rotates with the block index, to balance the SIMDs). Rows
// are walked in tiles of 64 tokens: the block stages exp(A[c, n] dt_i) and
// C[b, n, i] for the tile in LDS ([token][n], so a lane reads four
// coordinates per 16-byte broadcast read), then each wave walks the tile's
// rows. Because tiles and waves are 64-aligned, a tile is for a given wave
// either entirely above the diagonal (zeros), entirely below it (no masks),
// or its diagonal tile (the only masked one). Rows above a block's first
// column are zeros written without staging.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kTile = 64;    // rows per staged tile
constexpr int kThreads = 256;
constexpr int kCols = 256;   // columns per block

template <typename IoT, int NMAX, bool PER_STATE>
__global__ __launch_bounds__(kThreads) void effective_attention_kernel(const AttnParams p) {
  __shared__ __align__(16) float sa[kTile][NMAX];  // exp(A[c, n] dt_i)
  __shared__ __align__(16) float sc[kTile][NMAX];  // C[b, n, i]

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int64_t L = p.L;
  const int N = p.N;
  const int64_t bc = blockIdx.x / p.jblocks;
  const int64_t jb = (blockIdx.x - bc * p.jblocks) * kCols;  // block's first column
  const int64_t b = bc / p.channels;
  const int64_t c = bc - b * p.channels;
  // Wave w of a block runs on SIMD w, and the triangle gives the first column
  // group four times the rows of the last; rotating the group a wave takes
  // by the block index spreads heavy and light groups over the SIMDs.
  const int grp = (w + static_cast<int>(blockIdx.x & 3)) & 3;
  const int64_t jw = jb + 64 * grp;    // this wave's first column
  const int64_t j = jw + (tid & 63);   // this lane's column
  const bool live = j < L;
  const IoT* __restrict__ dtg = static_cast<const IoT*>(p.dt) + bc * L;
  const IoT* __restrict__ Bg = static_cast<const IoT*>(p.B) + b * N * L;
  const IoT* __restrict__ Cg = static_cast<const IoT*>(p.C) + b * N * L;
  const float* __restrict__ Ac = p.A + c * N;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;
  const bool softplus = p.dt_softplus != 0;
  auto step_size = [&](int64_t t) {
    const float v = Io<IoT>::to_f32(dtg[t]) + bias;
    return softplus ? softplus_f32(v) : v;
  };

  // d[n] = B[b, n, j] (* dt_j); coordinates past N stay 0 and add nothing
  float d[NMAX];
  {
    const float scale = (p.include_dt && live) ? step_size(j) : 1.0f;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) d[n] = (live && n < N) ? Io<IoT>::to_f32(Bg[n * L + j]) * scale : 0.0f;
  }
  float* __restrict__ Mo = p.M + bc * (PER_STATE ? N : 1) * L * L;
  const int64_t plane = L * L;  // per_state: distance between coordinates n and n + 1
  auto store = [&](int64_t i, const float* term, float m) {
    float* q = Mo + i * L + j;
    if constexpr (PER_STATE) {
#pragma unroll
      for (int n = 0; n < NMAX; ++n) {
        if (n < N) *q = term[n];
        q += plane;
      }
    } else {
      *q = m;
    }
  };
  auto store_zero = [&](int64_t i) {
    float* q = Mo + i * L + j;
    if constexpr (PER_STATE) {
#pragma unroll
      for (int n = 0; n < NMAX; ++n) {
        if (n < N) *q = 0.0f;
        q += plane;
      }
    } else {
      *q = 0.0f;
    }
  };

  // rows above the block's first column
  if (live)
    for (int64_t i = 0; i < jb; ++i) store_zero(i);

  const int64_t ntiles = (L + kTile - 1) / kTile;
  for (int64_t tile = jb / kTile; tile < ntiles; ++tile) {
    const int64_t i0 = tile * kTile;
    __syncthreads();  // the previous tile's readers are done
    for (int e = tid; e < kTile * NMAX; e += kThreads) {
      const int ii = e % kTile, n = e / kTile;
      const int64_t i = i0 + ii;
      float a = 1.0f, cv = 0.0f;
      if (i < L && n < N) {
        a = fast_exp2(Ac[n] * kLog2e * step_size(i));
        cv = Io<IoT>::to_f32(Cg[n * L + i]);
      }
      sa[ii][n] = a;
      sc[ii][n] = cv;
    }
    __syncthreads();
    const int rows = static_cast<int>(L - i0 < kTile ? L - i0 : kTile);
    // One row step: extend the products by row ii's factors (where the row
    // is past the column, when masked) and contract with C. Reads are
    // unconditional 16-byte broadcasts and the masks are selects, so the
    // step has no branches; the contraction runs as two partial sums.
    auto row_step = [&](int ii, bool masked, bool extend, bool on) {
      float m0 = 0.0f, m1 = 0.0f;
      float term[PER_STATE ? NMAX : 1];
#pragma unroll
      for (int n = 0; n < NMAX; n += 4) {
        float4 a4 = *reinterpret_cast<const float4*>(&sa[ii][n]);
        const float4 c4 = *reinterpret_cast<const float4*>(&sc[ii][n]);
        if (masked) {
          a4.x = extend ? a4.x : 1.0f; a4.y = extend ? a4.y : 1.0f;
          a4.z = extend ? a4.z : 1.0f; a4.w = extend ? a4.w : 1.0f;
        }
        d[n] *= a4.x; d[n + 1] *= a4.y; d[n + 2] *= a4.z; d[n + 3] *= a4.w;
        if constexpr (PER_STATE) {
          term[n] = c4.x * d[n]; term[n + 1] = c4.y * d[n + 1];
          term[n + 2] = c4.z * d[n + 2]; term[n + 3] = c4.w * d[n + 3];
          if (masked && !on) term[n] = term[n + 1] = term[n + 2] = term[n + 3] = 0.0f;
        } else {
          m0 = __builtin_fmaf(c4.x, d[n], m0);
          m1 = __builtin_fmaf(c4.y, d[n + 1], m1);
          m0 = __builtin_fmaf(c4.z, d[n + 2], m0);
          m1 = __builtin_fmaf(c4.w, d[n + 3], m1);
        }
      }
      const float m = (masked && !on) ? 0.0f : m0 + m1;
      if (live) store(i0 + ii, term, m);
    };
    if (i0 + kTile <= jw) {  // above the diagonal for every column of this wave
      if (live)
        for (int ii = 0; ii < rows; ++ii) store_zero(i0 + ii);
    } else if (i0 >= jw + 64) {  // below it for every column of this wave
#pragma unroll 2
      for (int ii = 0; ii < rows; ++ii) row_step(ii, false, true, true);
    } else {  // the wave's diagonal tile: rows i0 .. i0 + 63 against columns jw .. jw + 63
      for (int ii = 0; ii < rows; ++ii) row_step(ii, true, i0 + ii > j, i0 + ii >= j);
    }
  }
}

template <typename IoT, bool PER_STATE>
hipError_t launch_ps(const AttnParams& p0, hipStream_t stream) {
  AttnParams p = p0;
  p.jblocks = (p.L + kCols - 1) / kCols;
  const int64_t blocks = p.batch * p.channels * p.jblocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  const void* fn;
  if (p.N <= 4) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 4, PER_STATE>);
  else if (p.N <= 8) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 8, PER_STATE>);
  else if (p.N <= 16) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 16, PER_STATE>);
  else if (p.N <= 32) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 32, PER_STATE>);
  else fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 64, PER_STATE>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

template <typename IoT>
hipError_t launch_io(const AttnParams& p, hipStream_t stream) {
  return p.per_state ? launch_ps<IoT, true>(p, stream) : launch_ps<IoT, false>(p, stream);
}

}  // namespace

hipError_t launch_effective_attention(const AttnParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

int64_t effective_attention_blocks(int64_t batch, int64_t channels, int64_t L) {
  return batch * channels * ((L + kCols - 1) / kCols);
}

}  // namespace ss
