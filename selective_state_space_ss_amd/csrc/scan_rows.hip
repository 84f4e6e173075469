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
// walk, lane r of every wave is row r and wave g holds state coordinates
// 2g, 2g+1. A wave's coordinates are the same in every lane, so B[b, n, t]
// and C[b, n, t] are wave-uniform: they come through scalar loads into SGPRs
// (widened there from bf16) and feed the vector instructions directly, and
// so do the reset flags, which depend on (b, t) only. Tokens go in tiles of
// kT (16 for bf16, 8 for fp32: a tile's B and C for two coordinates fill 32
// SGPRs either way):
//   1. the block computes dt = softplus(dt + dt_bias) and dt*x for its
//      64 rows x kT tokens and publishes them in LDS; here thread i owns row
//      i/8 and the token pairs i%8 + 8k, so 8 neighbouring lanes read 8
//      contiguous pairs of a row;
//   2. every wave walks the tile for its two coordinates and keeps the
//      partial y_t = sum over its coordinates of C[n,t] h_t;
//   3. the partials go to LDS; thread i sums the 8 waves' partials of its
//      (row, token pairs), applies D*x and silu(z), and stores y.
// Two barriers per tile, each over 8 waves. The next tile's x, dt, z are
// loaded one tile ahead, and its B, C and flags are loaded right after the
// second barrier, so their latency hides behind phase 3 and the next phase 1.
// Coordinates n >= N take no part (B = C = 0, A = 0: the state stays 0); a
// wave whose coordinates are all >= N skips the walk.
//
// Requirements (checked by the launcher, which otherwise takes the chunked
// kernel): L a multiple of 4, x, dt, z, y, B, C aligned to two elements and
// reset to 4 bytes, so token pairs move as one access and scalar loads of B,
// C and the flags start on a dword.
#include "ss_device.h"
#include "ss_launch.h"

#include <cmath>
#include <type_traits>

namespace ss {
namespace {

constexpr int kRowsPerBlock = 64;  // lanes of a wave
constexpr int kCoords = 2;         // state coordinates per wave
constexpr int kWaves = 8;          // 16 coordinates per block
constexpr int kThreads = 64 * kWaves;
constexpr int kRowThreads = kThreads / kRowsPerBlock;  // threads per row in phases 1 and 3
constexpr int kTokStride = kRowsPerBlock + 4;  // spreads the phase-1 writes over the LDS banks
// s_waitcnt operand: LDS and scalar loads done (lgkmcnt 0), others not waited
constexpr int kWaitLdsAndScalar = 0xc07f;

template <typename IoT>
struct Tiling {
  static constexpr int kT = sizeof(IoT) == 2 ? 16 : 8;  // tokens per tile
  static constexpr int kPairs = kT / 2;                  // token pairs per row and tile
  static constexpr int kPairsPerThread = (kPairs + kRowThreads - 1) / kRowThreads;
  static constexpr int kYStride = kT + 4;                    // floats per row of partial y
  static constexpr int kDwords = kT * (int)sizeof(IoT) / 4;  // dwords of one row's tile
};

// Two consecutive fp32 values stored as an aligned pair of I/O elements.
__device__ __forceinline__ void store_pair(bf16_t* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

// One thread's raw pair of consecutive I/O elements, widened on use.
template <typename IoT>
struct Pair;
template <>
struct Pair<bf16_t> {
  uint32_t w = 0;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float2 get() const {
    return make_float2(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u));
  }
};
template <>
struct Pair<float> {
  float2 v = make_float2(0.0f, 0.0f);
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ float2 get() const { return v; }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A wave-uniform address held in SGPRs, in the constant address space, so
// loads through it are scalar (B, C and the flags are never written by the
// kernel).
template <typename V>
__device__ __forceinline__ const __attribute__((address_space(4))) V* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return (const __attribute__((address_space(4))) V*)((static_cast<uint64_t>(hi) << 32) | lo);
}

// NW consecutive dwords of a row at a wave-uniform address, in SGPRs.
//   load:      the whole span is in bounds and dword aligned;
//   load_tail: dword d covers row elements [e0 + d*EPD, e0 + (d+1)*EPD) and
//              is read only if they lie below `end` and `live`, else is 0
//              (`end` is a multiple of EPD, so a dword is wholly in or out).
template <int NW>
struct UniformDwords {
  static_assert(NW % 4 == 0 || NW == 2, "whole 16-byte loads, or one 8-byte load");
  uint32_t w[NW];
  __device__ __forceinline__ void load(const void* src) {
    if constexpr (NW % 4 == 0) {
      const auto* q = uniform_ptr<u32x4>(src);
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) {
        const u32x4 u = q[i];
        w[4 * i] = u.x;
        w[4 * i + 1] = u.y;
        w[4 * i + 2] = u.z;
        w[4 * i + 3] = u.w;
      }
    } else {
      const u32x2 u = *uniform_ptr<u32x2>(src);
      w[0] = u.x;
      w[1] = u.y;
    }
  }
  template <int EPD, typename T>
  __device__ __forceinline__ void load_tail(const T* row, int64_t e0, int64_t end, bool live) {
#pragma unroll
    for (int d = 0; d < NW; ++d) {
      const int64_t e = e0 + (int64_t)d * EPD;
      const bool in = live && e < end;
      const uint32_t v = *uniform_ptr<uint32_t>(row + (e < end ? e : end - EPD));
      w[d] = in ? v : 0u;
    }
  }
};

// A tile of B or C for one coordinate: kT values, widened where used.
template <typename IoT>
struct BCTile : UniformDwords<Tiling<IoT>::kDwords> {
  __device__ __forceinline__ float operator[](int j) const {
    if constexpr (sizeof(IoT) == 2)
      return (j & 1) ? __builtin_bit_cast(float, this->w[j >> 1] & 0xffff0000u)
                     : __builtin_bit_cast(float, this->w[j >> 1] << 16);
    else
      return __builtin_bit_cast(float, this->w[j]);
  }
};

// B, C and reset flags of one tile for one wave's coordinates, in SGPRs.
template <typename IoT>
struct BCBuf {
  BCTile<IoT> B[kCoords], C[kCoords];
  UniformDwords<Tiling<IoT>::kT / 4> R;  // one flag byte per token
};

template <typename IoT, bool GATE, bool RESET>
__global__ __launch_bounds__(kThreads, 4) void scan_rows_kernel(const ScanParams p) {
  using Tl = Tiling<IoT>;
  constexpr int kT = Tl::kT;
  constexpr int kPT = Tl::kPairsPerThread;
  constexpr int kYS = Tl::kYStride;
  constexpr int EPD = 4 / (int)sizeof(IoT);  // elements per dword
  __shared__ __align__(16) float2 sTok[kT][kTokStride];            // {dt, dt*x}[token][row]
  __shared__ __align__(16) float sY[kWaves][kRowsPerBlock * kYS];  // partial y[wave][row][token]

  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.chan_blocks;
  const int64_t cbase = (blk - b * p.chan_blocks) * kRowsPerBlock;
  const int N = p.N;
  const int64_t L = p.L;

  // ---- phases 1 and 3: row pr, token pairs pq + kRowThreads*k of each tile
  const int pr = tid / kRowThreads, pq = tid % kRowThreads;
  // with fp32 tiles a row has fewer pairs than threads: the rest idle here
  auto pair_active = [&](int q) { return Tl::kPairs % kRowThreads == 0 || pq + kRowThreads * q < Tl::kPairs; };
  const bool prow_ok = cbase + pr < p.channels;
  const int64_t cp = prow_ok ? cbase + pr : p.channels - 1;  // rows past the end compute, never store
  const int64_t rowoff = (b * p.channels + cp) * L;
  const IoT* __restrict__ xg = static_cast<const IoT*>(p.x) + rowoff;
  const IoT* __restrict__ dg = static_cast<const IoT*>(p.dt) + rowoff;
  const IoT* __restrict__ zg = GATE ? static_cast<const IoT*>(p.z) + rowoff : nullptr;
  IoT* __restrict__ yg = static_cast<IoT*>(p.y) + rowoff;
  const float Dc = p.D ? p.D[cp] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[cp] : 0.0f;

  // ---- phase 2: row r, coordinates 4g..4g+3
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int r = tid & 63;
  const bool wrow_ok = cbase + r < p.channels;
  const int64_t cw = wrow_ok ? cbase + r : p.channels - 1;
  const int nlive = N - kCoords * g;  // live coordinates of this wave (may be <= 0)
  const IoT* __restrict__ Bw = static_cast<const IoT*>(p.B) + b * N * L;
  const IoT* __restrict__ Cw = static_cast<const IoT*>(p.C) + b * N * L;
  const uint8_t* __restrict__ rg = RESET ? p.reset + b * L : nullptr;
  float a2[kCoords], h[kCoords];
#pragma unroll
  for (int i = 0; i < kCoords; ++i) {
    const int n = kCoords * g + i;
    a2[i] = i < nlive ? p.A[cw * N + n] * kLog2e : 0.0f;
    h[i] = (i < nlive && p.h0) ? p.h0[(b * p.channels + cw) * N + n] : 0.0f;
  }

  // B, C and reset flags of a tile, wave-uniform. load_full: a whole tile of
  // live coordinates; load_tail: the last tile or a wave with coordinates
  // past state_dim (rows of coordinate 0 stand in for those: in bounds, read
  // as 0). Two buffers take alternate tiles, so that a tile's scalar loads
  // are issued two tiles ahead of its walk.
  BCBuf<IoT> bufA, bufB;
  const int64_t rowstep = L;  // elements between the rows of consecutive coordinates
  auto load_full = [&](BCBuf<IoT>& u, int64_t t0) {
    const IoT* bt = Bw + (int64_t)(kCoords * g) * L + t0;
    const IoT* ct = Cw + (int64_t)(kCoords * g) * L + t0;
#pragma unroll
    for (int i = 0; i < kCoords; ++i) {
      u.B[i].load(bt + i * rowstep);
      u.C[i].load(ct + i * rowstep);
    }
    if constexpr (RESET) u.R.load(rg + t0);
  };
  auto load_tail = [&](BCBuf<IoT>& u, int64_t t0) {
#pragma unroll
    for (int i = 0; i < kCoords; ++i) {
      const bool live = i < nlive;
      const int64_t ro = (int64_t)(live ? kCoords * g + i : 0) * L;
      u.B[i].template load_tail<EPD>(Bw + ro, t0, L, live);
      u.C[i].template load_tail<EPD>(Cw + ro, t0, L, live);
    }
    if constexpr (RESET) u.R.template load_tail<4>(rg, t0, L, true);
  };

  // This thread's raw x, dt, z pairs of the next tile, loaded one tile ahead
  // so that HBM latency hides behind the current one. Pairs past the end
  // load the last pair instead and the tile zeroes them.
  Pair<IoT> px[kPT], pd[kPT], pz[kPT];
  auto load_tok = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < kPT; ++k) {
      const int64_t t = t0 + 2 * (pq + kRowThreads * k) < L ? t0 + 2 * (pq + kRowThreads * k) : L - 2;
      px[k].load(xg + t);
      pd[k].load(dg + t);
      if constexpr (GATE) pz[k].load(zg + t);
    }
  };

  // The walk over one tile; M: with document starts. The tile's
  // {dt, dt*x} come from LDS first; once they are in registers the next
  // tile's scalar loads are issued (issue_next), so that no LDS wait of the
  // walk waits for them too (LDS and scalar loads share one counter) and
  // their latency hides behind the walk's arithmetic. The partial y goes to
  // LDS four tokens at a time.
  float* ys = &sY[g][r * kYS];
  auto walk = [&](const BCBuf<IoT>& u, auto with_reset, auto issue_next) {
    constexpr bool M = decltype(with_reset)::value;
    float2 tk[kT];
#pragma unroll
    for (int j = 0; j < kT; ++j) tk[j] = sTok[j][r];
    __builtin_amdgcn_s_waitcnt(kWaitLdsAndScalar);
    __builtin_amdgcn_sched_barrier(0);
    issue_next();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j4 = 0; j4 < kT; j4 += 4) {
      float yp[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = j4 + jj;
        float m = 0.0f;
        if constexpr (M) m = ((u.R.w[j >> 2] >> (8 * (j & 3))) & 0xffu) ? -INFINITY : 0.0f;
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < kCoords; ++i) {
          const float e = M ? __builtin_fmaf(tk[j].x, a2[i], m) : tk[j].x * a2[i];
          h[i] = __builtin_fmaf(fast_exp2(e), h[i], tk[j].y * u.B[i][j]);
          y = i == 0 ? u.C[i][j] * h[i] : __builtin_fmaf(u.C[i][j], h[i], y);
        }
        yp[jj] = y;
      }
      *reinterpret_cast<float4*>(ys + j4) = make_float4(yp[0], yp[1], yp[2], yp[3]);
    }
  };

  // One tile, walked with the B, C, flags in u. FULL: in bounds. issue_next
  // issues the next tile's scalar loads (from inside the walk).
  auto tile = [&](int64_t t0, const BCBuf<IoT>& u, auto full, auto issue_next) {
    constexpr bool FULL = decltype(full)::value;

    // 1. dt and dt*x of this thread's token pairs
    float2 xo[kPT], zo[kPT];
    bool tin[kPT];
#pragma unroll
    for (int q = 0; q < kPT; ++q) {
      const int64_t t = t0 + 2 * (pq + kRowThreads * q);
      tin[q] = FULL || t < L;  // L is even: a pair is wholly in or out
      const float2 xr = px[q].get(), dr = pd[q].get();
      xo[q] = tin[q] ? xr : make_float2(0.0f, 0.0f);
      zo[q] = GATE ? pz[q].get() : make_float2(0.0f, 0.0f);
      float d[2] = {dr.x + bias, dr.y + bias};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (p.dt_softplus) d[e] = softplus_f32(d[e]);
        d[e] = tin[q] ? d[e] : 0.0f;  // tokens past the end: a = 1, b = 0
      }
      const int j0 = 2 * (pq + kRowThreads * q);
      if (pair_active(q)) {
        sTok[j0][pr] = make_float2(d[0], d[0] * xo[q].x);
        sTok[j0 + 1][pr] = make_float2(d[1], d[1] * xo[q].y);
      }
    }
    if (t0 + kT < L) load_tok(t0 + kT);
    __syncthreads();

    // 2. the walk
    if (nlive <= 0) {
      issue_next();
#pragma unroll
      for (int j = 0; j < kT; j += 4) *reinterpret_cast<float4*>(ys + j) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
      walk(u, std::integral_constant<bool, RESET>{}, issue_next);
    }

    // 3. thread (pr, pq) sums its pairs' partials over the waves
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPT; ++q) {
      if (!pair_active(q)) continue;
      const int j0 = 2 * (pq + kRowThreads * q);
      float2 ys2 = make_float2(0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float2 v = *reinterpret_cast<const float2*>(&sY[w][pr * kYS + j0]);
        ys2.x += v.x;
        ys2.y += v.y;
      }
      float yo[2] = {__builtin_fmaf(Dc, xo[q].x, ys2.x), __builtin_fmaf(Dc, xo[q].y, ys2.y)};
      if constexpr (GATE) {
        yo[0] *= silu_f32(zo[q].x);
        yo[1] *= silu_f32(zo[q].y);
      }
      if (prow_ok && tin[q]) store_pair(yg + t0 + j0, yo[0], yo[1]);
    }
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  auto nothing = [] {};

  const int64_t nfull = L / kT;
  if (L > 0) load_tok(0);
  if (nlive >= kCoords) {
    // all coordinates live: whole tiles in pairs, tile k with buffer A and
    // tile k+1 with buffer B, each walk filling the other buffer
    if (nfull > 0) load_full(bufA, 0);
    int64_t k = 0;
    for (; k + 2 <= nfull; k += 2) {
      tile(k * kT, bufA, True{}, [&] { load_full(bufB, (k + 1) * kT); });
      tile((k + 1) * kT, bufB, True{}, [&] {
        if (k + 2 < nfull) load_full(bufA, (k + 2) * kT);
      });
    }
    if (k < nfull) tile(k * kT, bufA, True{}, nothing);
  } else {
    for (int64_t k = 0; k < nfull; ++k) {
      load_tail(bufA, k * kT);
      tile(k * kT, bufA, True{}, nothing);
    }
  }
  if (nfull * kT < L) {
    load_tail(bufA, nfull * kT);
    tile(nfull * kT, bufA, False{}, nothing);
  }

  if (p.h_last && wrow_ok) {
#pragma unroll
    for (int i = 0; i < kCoords; ++i)
      if (i < nlive) p.h_last[(b * p.channels + cw) * N + kCoords * g + i] = h[i];
  }
}

template <typename IoT, bool GATE, bool RESET>
hipError_t launch_t(const ScanParams& p0, hipStream_t stream) {
  ScanParams p = p0;
  p.chan_blocks = (p.channels + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = p.batch * p.chan_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  return launch_kernel(reinterpret_cast<const void*>(&scan_rows_kernel<IoT, GATE, RESET>), dim3((unsigned)blocks),
                       dim3(kThreads), args, stream);
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
  auto ok = [&](const void* q, uintptr_t a) { return reinterpret_cast<uintptr_t>(q) % a == 0; };  // nullptr passes
  return p.L % 4 == 0 && p.N <= kCoords * kWaves && ok(p.x, pair) && ok(p.dt, pair) && ok(p.z, pair) &&
         ok(p.y, pair) && ok(p.B, pair) && ok(p.C, pair) && ok(p.reset, 4);
}

hipError_t launch_scan_rows(const ScanParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace ss
