// Prompt / prefill selective scan for gfx950, row-parallel form: every lane
// owns one channel row and walks the whole sequence token by token, for the
// two state coordinates of its wave.
//
// This form applies the recurrence of the nnterp "selective_scan" page, class
// docstring, token by token, with no fold and no cross-lane scan: one exp and
// four FMA-class operations per token and state coordinate (dt*A, dt*x*B,
// h = a h + b, y += C h), against five for the chunked scan. It has
// batch*channels*N/2 lanes of parallelism, so it serves shapes with many rows
// (the launcher decides).
//
// Layout. A block is 64 channel rows of one batch row times 8 waves; in the
// walk, lane r of every wave is row r and wave g holds state coordinates 2g
// and 2g+1. A wave's coordinates are the same in every lane, so B[b, n, t]
// and C[b, n, t] are wave-uniform: they come through scalar loads into SGPRs
// and feed the vector instructions directly. Tokens go in tiles of 16:
//   1. the block computes dt = softplus(dt + dt_bias) and dt*x for its
//      64 rows x 16 tokens and publishes them in LDS; here thread i owns row
//      i/8 and tokens 2(i%8), 2(i%8)+1, so 8 neighbouring lanes read one
//      contiguous tile row;
//   2. every wave walks the 16 tokens for its two coordinates and keeps the
//      partial y_t = sum over its coordinates of C[n,t] h_t;
//   3. the partials go to LDS; thread i sums the 8 waves' partials of its
//      (row, token pair), applies D*x and silu(z), and stores y.
// Two barriers per tile. Coordinates n >= N take no part: a wave whose
// coordinates are all >= N skips the walk, one with a single live coordinate
// walks that one only.
//
// Requirements (checked by the launcher, which otherwise takes the chunked
// kernel): L even and x, dt, z, y, B, C aligned to two elements, so token
// pairs move as one access and B, C rows start on a dword.
#include "ss_device.h"
#include "ss_launch.h"

#include <cmath>
#include <type_traits>

namespace ss {
namespace {

constexpr int kRowsPerBlock = 64;  // lanes of a wave
constexpr int kWaves = 8;          // 2 state coordinates each
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 16;                         // tokens per tile
constexpr int kPairs = kT / 2;                 // token pairs per row and tile
constexpr int kTokStride = kRowsPerBlock + 4;  // spreads the phase-1 writes over the LDS banks
constexpr int kYStride = kT + 4;               // floats per row of partial y (spreads LDS banks)
static_assert(kThreads == kRowsPerBlock * kPairs, "one thread per (row, token pair) of a tile");

using Two = std::integral_constant<bool, true>;
using One = std::integral_constant<bool, false>;

// Per-token values published for the walk: {dt, dt*x} or, with the reset
// mask, {dt, dt*x, m, 0} where m = -inf at a document's first token (the
// decay exp2(dt*A*log2e + m) is then 0) and 0 elsewhere.
template <bool RESET>
struct TokT;
template <>
struct TokT<false> {
  using type = float2;
};
template <>
struct TokT<true> {
  using type = float4;
};

// Two consecutive I/O elements (an aligned pair) widened to fp32, and back.
__device__ __forceinline__ float2 load_pair(const bf16_t* p) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u));
}
__device__ __forceinline__ float2 load_pair(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ void store_pair(bf16_t* p, float a, float b) {
  const uint32_t w = uint32_t(Io<bf16_t>::from_f32(a).bits) | (uint32_t(Io<bf16_t>::from_f32(b).bits) << 16);
  *reinterpret_cast<uint32_t*>(p) = w;
}
__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A wave-uniform address held in SGPRs, in the constant address space, so
// loads through it are scalar (B and C are never written by the kernel).
template <typename V>
__device__ __forceinline__ const __attribute__((address_space(4))) V* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return (const __attribute__((address_space(4))) V*)((static_cast<uint64_t>(hi) << 32) | lo);
}

// kT consecutive elements at a wave-uniform, dword-aligned address, through
// scalar loads, kept packed (bf16: two tokens per dword) until the walk
// widens each one where it is used, so they occupy few SGPRs.
template <typename IoT>
struct UniformTile;
template <>
struct UniformTile<bf16_t> {
  uint32_t w[kT / 2];
  __device__ __forceinline__ void load(const bf16_t* src) {
    const auto* q = uniform_ptr<u32x4>(src);
#pragma unroll
    for (int i = 0; i < kT / 8; ++i) {
      const u32x4 u = q[i];
      w[4 * i] = u.x;
      w[4 * i + 1] = u.y;
      w[4 * i + 2] = u.z;
      w[4 * i + 3] = u.w;
    }
  }
  __device__ __forceinline__ float operator[](int j) const {
    return (j & 1) ? __builtin_bit_cast(float, w[j >> 1] & 0xffff0000u) : __builtin_bit_cast(float, w[j >> 1] << 16);
  }
};
template <>
struct UniformTile<float> {
  float v[kT];
  __device__ __forceinline__ void load(const float* src) {
    const auto* q = uniform_ptr<f32x4>(src);
#pragma unroll
    for (int i = 0; i < kT / 4; ++i) {
      const f32x4 u = q[i];
      v[4 * i] = u.x;
      v[4 * i + 1] = u.y;
      v[4 * i + 2] = u.z;
      v[4 * i + 3] = u.w;
    }
  }
  __device__ __forceinline__ float operator[](int j) const { return v[j]; }
};

// The tile that ends the sequence: tokens past the end read as 0 (they are
// the identity anyway, dt = 0 there), loads clamped in bounds.
struct TailTile {
  float v[kT];
  template <typename IoT>
  __device__ __forceinline__ void load(const IoT* src, int64_t t0, int64_t L) {
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const bool tin = t0 + j < L;
      const float u = Io<IoT>::to_f32(src[tin ? t0 + j : L - 1]);
      v[j] = tin ? u : 0.0f;
    }
  }
  __device__ __forceinline__ float operator[](int j) const { return v[j]; }
};

template <typename IoT, bool GATE, bool RESET>
__global__ __launch_bounds__(kThreads) void scan_rows_kernel(const ScanParams p) {
  using Tok = typename TokT<RESET>::type;
  __shared__ __align__(16) Tok sTok[kT][kTokStride];                  // [token][row]
  __shared__ __align__(16) float sY[kWaves][kRowsPerBlock * kYStride];  // partial y[wave][row][token]

  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.chan_blocks;
  const int64_t cbase = (blk - b * p.chan_blocks) * kRowsPerBlock;
  const int N = p.N;
  const int64_t L = p.L;

  // ---- phases 1 and 3: row pr, tokens 2pt, 2pt+1 of each tile
  const int pr = tid >> 3, pt = tid & 7;
  const bool prow_ok = cbase + pr < p.channels;
  const int64_t cp = prow_ok ? cbase + pr : p.channels - 1;  // rows past the end compute, never store
  const int64_t rowoff = (b * p.channels + cp) * L;
  const IoT* __restrict__ xg = static_cast<const IoT*>(p.x) + rowoff;
  const IoT* __restrict__ dg = static_cast<const IoT*>(p.dt) + rowoff;
  const IoT* __restrict__ zg = GATE ? static_cast<const IoT*>(p.z) + rowoff : nullptr;
  IoT* __restrict__ yg = static_cast<IoT*>(p.y) + rowoff;
  const uint8_t* __restrict__ rg = RESET ? p.reset + b * L : nullptr;
  const float Dc = p.D ? p.D[cp] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[cp] : 0.0f;

  // ---- phase 2: row r, coordinates n0 = 2g, n1 = 2g+1
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int r = tid & 63;
  const bool wrow_ok = cbase + r < p.channels;
  const int64_t cw = wrow_ok ? cbase + r : p.channels - 1;
  const int n0 = 2 * g, n1 = 2 * g + 1;
  const bool live0 = n0 < N, live1 = n1 < N;
  const IoT* __restrict__ B0 = static_cast<const IoT*>(p.B) + (b * N + (live0 ? n0 : 0)) * L;
  const IoT* __restrict__ B1 = static_cast<const IoT*>(p.B) + (b * N + (live1 ? n1 : 0)) * L;
  const IoT* __restrict__ C0 = static_cast<const IoT*>(p.C) + (b * N + (live0 ? n0 : 0)) * L;
  const IoT* __restrict__ C1 = static_cast<const IoT*>(p.C) + (b * N + (live1 ? n1 : 0)) * L;
  const float a20 = live0 ? p.A[cw * N + n0] * kLog2e : 0.0f;
  const float a21 = live1 ? p.A[cw * N + n1] * kLog2e : 0.0f;
  float h0 = (live0 && p.h0) ? p.h0[(b * p.channels + cw) * N + n0] : 0.0f;
  float h1 = (live1 && p.h0) ? p.h0[(b * p.channels + cw) * N + n1] : 0.0f;

  // The walk over one tile, for both coordinates (TWO) or n0 only.
  float yp[kT];
  auto walk = [&](auto two, const auto& bb0, const auto& bb1, const auto& cc0, const auto& cc1) {
    constexpr bool TWO = decltype(two)::value;
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const Tok tk = sTok[j][r];
      float e0, e1;
      if constexpr (RESET) {
        e0 = __builtin_fmaf(tk.x, a20, tk.z);
        e1 = __builtin_fmaf(tk.x, a21, tk.z);
      } else {
        e0 = tk.x * a20;
        e1 = tk.x * a21;
      }
      h0 = __builtin_fmaf(fast_exp2(e0), h0, tk.y * bb0[j]);
      if constexpr (TWO) {
        h1 = __builtin_fmaf(fast_exp2(e1), h1, tk.y * bb1[j]);
        yp[j] = __builtin_fmaf(cc1[j], h1, cc0[j] * h0);
      } else {
        yp[j] = cc0[j] * h0;
      }
    }
  };

  auto tile = [&](int64_t t0, auto full) {
    constexpr bool FULL = decltype(full)::value;

    // 1. dt and dt*x of this thread's token pair
    const int64_t t = t0 + 2 * pt;
    const bool tin = FULL || t < L;  // L is even: a pair is wholly in or out
    float2 xo = make_float2(0.0f, 0.0f), zo = make_float2(0.0f, 0.0f), dr = make_float2(0.0f, 0.0f);
    if (tin) {
      xo = load_pair(xg + t);
      dr = load_pair(dg + t);
      if constexpr (GATE) zo = load_pair(zg + t);
    }
    float d[2] = {dr.x + bias, dr.y + bias};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (p.dt_softplus) d[e] = softplus_f32(d[e]);
      d[e] = tin ? d[e] : 0.0f;  // tokens past the end: a = 1, b = 0
    }
    const float dx[2] = {d[0] * xo.x, d[1] * xo.y};
    if constexpr (RESET) {
      uint32_t rr = 0;
      if (tin) rr = *reinterpret_cast<const uint16_t*>(rg + t);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float m = ((rr >> (8 * e)) & 0xffu) ? -INFINITY : 0.0f;
        sTok[2 * pt + e][pr] = make_float4(d[e], dx[e], m, 0.0f);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) sTok[2 * pt + e][pr] = make_float2(d[e], dx[e]);
    }
    __syncthreads();

    // 2. the walk
    if (!live0) {
#pragma unroll
      for (int j = 0; j < kT; ++j) yp[j] = 0.0f;
    } else if constexpr (FULL) {
      UniformTile<IoT> bb0, bb1, cc0, cc1;
      bb0.load(B0 + t0);
      cc0.load(C0 + t0);
      if (live1) {
        bb1.load(B1 + t0);
        cc1.load(C1 + t0);
        walk(Two{}, bb0, bb1, cc0, cc1);
      } else {
        walk(One{}, bb0, bb0, cc0, cc0);
      }
    } else {
      TailTile bb0, bb1, cc0, cc1;
      bb0.load(B0, t0, L);
      cc0.load(C0, t0, L);
      if (live1) {
        bb1.load(B1, t0, L);
        cc1.load(C1, t0, L);
        walk(Two{}, bb0, bb1, cc0, cc1);
      } else {
        walk(One{}, bb0, bb0, cc0, cc0);
      }
    }

    // 3. partials to LDS; thread (pr, pt) sums its pair over the 8 waves
    float* ys = &sY[g][r * kYStride];
#pragma unroll
    for (int j = 0; j < kT; j += 4)
      *reinterpret_cast<float4*>(ys + j) = make_float4(yp[j], yp[j + 1], yp[j + 2], yp[j + 3]);
    __syncthreads();
    float ysum[2] = {0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 q = *reinterpret_cast<const float2*>(&sY[w][pr * kYStride + 2 * pt]);
      ysum[0] += q.x;
      ysum[1] += q.y;
    }
    float yo[2] = {__builtin_fmaf(Dc, xo.x, ysum[0]), __builtin_fmaf(Dc, xo.y, ysum[1])};
    if constexpr (GATE) {
      yo[0] *= silu_f32(zo.x);
      yo[1] *= silu_f32(zo.y);
    }
    if (prow_ok && tin) store_pair(yg + t, yo[0], yo[1]);
  };

  const int64_t nfull = L / kT;
  for (int64_t k = 0; k < nfull; ++k) tile(k * kT, Two{});
  if (nfull * kT < L) tile(nfull * kT, One{});

  if (p.h_last && wrow_ok) {
    if (live0) p.h_last[(b * p.channels + cw) * N + n0] = h0;
    if (live1) p.h_last[(b * p.channels + cw) * N + n1] = h1;
  }
}

template <typename IoT, bool GATE, bool RESET>
hipError_t launch_t(const ScanParams& p0, hipStream_t stream) {
  ScanParams p = p0;
  p.chan_blocks = (p.channels + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = p.batch * p.chan_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_rows_kernel<IoT, GATE, RESET>), dim3((unsigned)blocks),
                         dim3(kThreads), args, 0, stream);
}

template <typename IoT>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  const bool gate = p.z != nullptr, reset = p.reset != nullptr;
  if (gate && reset) return launch_t<IoT, true, true>(p, stream);
  if (gate) return launch_t<IoT, true, false>(p, stream);
  if (reset) return launch_t<IoT, false, true>(p, stream);
  return launch_t<IoT, false, false>(p, stream);
}

}  // namespace

bool scan_rows_supported(const ScanParams& p, bool io_bf16) {
  const uintptr_t pair = io_bf16 ? 4 : 8;
  auto ok = [&](const void* q) { return reinterpret_cast<uintptr_t>(q) % pair == 0; };  // nullptr passes
  return p.L % 2 == 0 && ok(p.x) && ok(p.dt) && ok(p.z) && ok(p.y) && ok(p.B) && ok(p.C) &&
         reinterpret_cast<uintptr_t>(p.reset) % 2 == 0;
}

hipError_t launch_scan_rows(const ScanParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace ss
