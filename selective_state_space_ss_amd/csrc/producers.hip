// Input-side producers of the scan for gfx950 (nnterp "selective_scan" page,
// class docstring: the scan's x is the causal conv1d output after SiLU and
// its dt the dt_proj output; TransformerLens "ssm_mixer" page: x is the
// post-conv SiLU input, dt is read from dt_proj's output).
//
// conv1d_silu: x[b, c, t] = silu(conv_b[c] + sum_k conv_w[c, k] x_pre[b, c, t - (W-1) + k]),
// a depthwise causal convolution of width W <= 8; a tap before position 0 or
// before the current document's first token (reset[b, s] != 0) reads 0.
// Bound by HBM (one read of x_pre, one write of x). A wave makes a segment of
// 2048 tokens of one row, each load and store instruction covering 64
// consecutive 8-token runs (see the kernel).
//
// dt_proj: dt[b, c, t] = sum_k w_dt[c, k] delta[b, t, k] (optionally
// softplus(dt + dt_bias[c])), a GEMM of channels x tokens over the rank k on
// the matrix cores: bf16 16x16x32 MFMAs for bf16 I/O, fp32 16x16x4 for fp32.
// Both operands are contiguous in k (w_dt row-major [channels, R], delta
// token-major [batch, L, R]), so each lane loads its operand slice with one
// 16-byte load per 32 (bf16) or 16 (fp32) values of k, straight from L2
// (w_dt and delta are small next to the dt it writes). Bound by writing dt.
// Ranks of up to 8 chunks with whole 16-byte rows take the streaming form
// below; other shapes a plain tile-per-block form.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ conv1d + SiLU
constexpr int kConvRun = 8;        // tokens per run (one 16-byte bf16 vector)
constexpr int kConvRuns = 4;       // runs per thread
constexpr int kConvSeg = 64 * kConvRuns * kConvRun;  // tokens per wave: a segment of a row
constexpr int kConvThreads = 256;

// Wave layout: a wave owns a segment of kConvSeg tokens of one row; run n
// of lane l is the 8 tokens at seg + (64 n + l) * 8, so every load and store
// instruction of the wave covers 64 consecutive runs (1 KiB of bf16). The 8
// tokens before a run (for the taps) are loaded the same way, from cache.
// MAXW: the width bound the tap loop is unrolled for (4 or 8); RESET: a
// reset mask is given (else the taps need no document bookkeeping).
template <typename IoT, bool VEC, int MAXW, bool RESET>
__global__ __launch_bounds__(kConvThreads) void conv1d_silu_kernel(const ConvParams p) {
  constexpr int E = 16 / sizeof(IoT);   // elements per 16-byte vector
  constexpr int RV = kConvRun / E;      // vectors per run
  const int64_t L = p.L;
  const int64_t segs = (L + kConvSeg - 1) / kConvSeg;
  const int64_t wv = (static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x) >> 6;
  if (wv >= p.rows * segs) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = wv / segs;               // b * channels + c
  const int64_t seg0 = (wv - row * segs) * kConvSeg;
  const int64_t b = row / p.channels, c = row - b * p.channels;
  const IoT* __restrict__ xp = static_cast<const IoT*>(p.x_pre) + row * L;
  IoT* __restrict__ xo = static_cast<IoT*>(p.x) + row * L;
  const int W = p.W;

  // wr[m]: the weight of the tap m tokens back (conv_w[c, W - 1 - m]), 0 past W
  float wr[MAXW];
#pragma unroll
  for (int m = 0; m < MAXW; ++m) wr[m] = m < W ? p.conv_w[c * W + (W - 1 - m)] : 0.0f;
  const float bias = p.conv_b ? p.conv_b[c] : 0.0f;

  // every load of the thread first: run n and the 8 tokens before it
  u32x4 cur[kConvRuns][RV], prv[kConvRuns][RV];
  float v[kConvRuns][2 * kConvRun];  // [0, 8): before the run, [8, 16): the run
  if constexpr (VEC) {
    // rows are whole 8-token runs (L % 8 == 0, 16-byte aligned): every run
    // is entirely inside or entirely past the row
#pragma unroll
    for (int n = 0; n < kConvRuns; ++n) {
      const int64_t t0 = seg0 + (64 * n + lane) * kConvRun;
#pragma unroll
      for (int h = 0; h < RV; ++h) {
        cur[n][h] = t0 < L ? *reinterpret_cast<const u32x4*>(xp + t0 + h * E) : u32x4{0, 0, 0, 0};
        prv[n][h] = (t0 > 0 && t0 < L) ? *reinterpret_cast<const u32x4*>(xp + t0 - kConvRun + h * E)
                                       : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int n = 0; n < kConvRuns; ++n)
#pragma unroll
      for (int h = 0; h < RV; ++h) {
        unpack_vec16<IoT>(uint4{prv[n][h][0], prv[n][h][1], prv[n][h][2], prv[n][h][3]}, &v[n][h * E]);
        unpack_vec16<IoT>(uint4{cur[n][h][0], cur[n][h][1], cur[n][h][2], cur[n][h][3]}, &v[n][kConvRun + h * E]);
      }
  } else {
#pragma unroll
    for (int n = 0; n < kConvRuns; ++n) {
      const int64_t t0 = seg0 + (64 * n + lane) * kConvRun;
#pragma unroll
      for (int u = 0; u < 2 * kConvRun; ++u) {
        const int64_t s = t0 - kConvRun + u;
        v[n][u] = (s >= 0 && s < L) ? Io<IoT>::to_f32(xp[s]) : 0.0f;
      }
    }
  }

#pragma unroll
  for (int n = 0; n < kConvRuns; ++n) {
    const int64_t t0 = seg0 + (64 * n + lane) * kConvRun;
    if (t0 >= L) continue;
    // reset flags of the run and the 8 tokens before it (bit u: position t0 - 8 + u)
    uint32_t start = 0;
    if constexpr (RESET) {
#pragma unroll
      for (int u = 0; u < 2 * kConvRun; ++u) {
        const int64_t s = t0 - kConvRun + u;
        if (s >= 0 && s < L && p.reset[b * L + s] != 0) start |= 1u << u;
      }
    }
    float out[kConvRun];
#pragma unroll
    for (int u = 0; u < kConvRun; ++u) {
      // token t0 + u is v[n][8 + u]; the tap m tokens back reads v[n][8 + u - m],
      // until a document start has been passed (weights past W are 0)
      float acc = bias;
      if constexpr (RESET) {
        bool open = true;
#pragma unroll
        for (int m = 0; m < MAXW; ++m) {
          acc = open ? __builtin_fmaf(wr[m], v[n][kConvRun + u - m], acc) : acc;
          open = open && !((start >> (kConvRun + u - m)) & 1u);
        }
      } else {
#pragma unroll
        for (int m = 0; m < MAXW; ++m) acc = __builtin_fmaf(wr[m], v[n][kConvRun + u - m], acc);
      }
      out[u] = silu_f32(acc);
    }
    if constexpr (VEC) {
#pragma unroll
      for (int h = 0; h < RV; ++h) store_vec16(reinterpret_cast<IoT*>(xo + t0 + h * E), out + h * E);
    } else {
#pragma unroll
      for (int u = 0; u < kConvRun; ++u)
        if (t0 + u < L) xo[t0 + u] = Io<IoT>::from_f32(out[u]);
    }
  }
}

// ------------------------------------------------------------------ dt_proj
constexpr int kProjThreads = 256;   // 4 waves
constexpr int kProjC = 64;          // channels per block: 16 per wave
constexpr int kProjT = 64;          // tokens per block: 4 MFMA tiles per wave

// One K chunk of operands for lane (row, G): 16 bytes = 8 bf16 or 4 fp32 values
template <typename IoT, bool VEC>
__device__ __forceinline__ u32x4 load_k16(const IoT* base, int64_t k0, int64_t R, bool row_ok) {
  constexpr int E = 16 / sizeof(IoT);
  if constexpr (VEC) {
    return (row_ok && k0 < R) ? *reinterpret_cast<const u32x4*>(base + k0) : u32x4{0, 0, 0, 0};
  } else {
    u32x4 r = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool in = row_ok && k0 + e < R;
      if constexpr (sizeof(IoT) == 2) {
        const uint32_t bits = in ? static_cast<const bf16_t*>(static_cast<const void*>(base))[k0 + e].bits : 0u;
        r[e >> 1] |= (e & 1) ? (bits << 16) : bits;
      } else {
        const float f = in ? base[k0 + e] : 0.0f;
        r[e] = __builtin_bit_cast(uint32_t, f);
      }
    }
    return r;
  }
}

template <typename IoT, bool VEC, bool APPLY>
__global__ __launch_bounds__(kProjThreads) void dt_proj_kernel(const ProjParams p) {
  constexpr int KC = sizeof(IoT) == 2 ? 32 : 16;   // k per 16-byte lane load x 4 lane groups
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, G = l >> 4, r16 = l & 15;
  const int64_t L = p.L, C = p.channels, R = p.R;
  const int64_t tblocks = (L + kProjT - 1) / kProjT, cblocks = (C + kProjC - 1) / kProjC;
  int64_t blk = blockIdx.x;
  const int64_t tb = blk % tblocks; blk /= tblocks;
  const int64_t cb = blk % cblocks;
  const int64_t b = blk / cblocks;
  const int64_t c0 = cb * kProjC + 16 * w;   // this wave's 16 channels
  const int64_t t0 = tb * kProjT;
  const IoT* __restrict__ Wg = static_cast<const IoT*>(p.w_dt);
  const IoT* __restrict__ Dg = static_cast<const IoT*>(p.delta) + b * L * R;

  // A operand rows: channel c0 + r16; B operand columns: token t0 + 16 n + r16
  const bool c_ok = c0 + r16 < C;
  const IoT* wrow = Wg + (c_ok ? (c0 + r16) * R : 0);
  v4f acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  for (int64_t k0 = 0; k0 < R; k0 += KC) {
    const int64_t kl = k0 + (KC / 4) * G;   // this lane group's slice of the chunk
    const u32x4 a = load_k16<IoT, VEC>(wrow, kl, R, c_ok);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int64_t t = t0 + 16 * n + r16;
      const bool t_ok = t < L;
      const u32x4 bv = load_k16<IoT, VEC>(Dg + (t_ok ? t * R : 0), kl, R, t_ok);
      if constexpr (sizeof(IoT) == 2) {
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bv),
                                                         acc[n], 0, 0, 0);
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t ag = a[g], bg = bv[g];
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, ag), __builtin_bit_cast(float, bg),
                                                         acc[n], 0, 0, 0);
        }
      }
    }
  }
  // D layout: register r at lane (column r16, G) is row 4 G + r, i.e.
  // channel c0 + 4 G + r and token t0 + 16 n + r16
  IoT* __restrict__ out = static_cast<IoT*>(p.dt) + b * C * L;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int64_t t = t0 + 16 * n + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t c = c0 + 4 * G + r;
      if (c < C && t < L) {
        float v = acc[n][r];
        if constexpr (APPLY) v = softplus_f32(v + (p.dt_bias ? p.dt_bias[c] : 0.0f));
        out[c * L + t] = Io<IoT>::from_f32(v);
      }
    }
  }
}

// Streaming form for ranks up to 8 chunks (R <= 256 bf16, 128 fp32) with
// whole 16-byte rows: a block owns 64 channels of one batch row, keeps their
// w_dt operand slices in registers, and walks the sequence in 64-token
// tiles. Each tile of delta ([token][k], k contiguous) is loaded with 16-byte
// loads one tile ahead into registers, written to one of two LDS buffers and
// read back as MFMA B operands; the 64 x 64 output tile goes through LDS so
// that every row of 64 tokens is written with whole 16-byte stores.
constexpr int kStreamT = 64;

template <typename IoT, int KCH>
struct ProjStage {
  static constexpr int E = 16 / sizeof(IoT);
  static constexpr int KP = KCH * 4 * E + E;   // k per staged row, padded by one vector
  IoT d[2][kStreamT][KP];
  IoT o[kProjC][kStreamT + E];
  float bias[kProjC];
};

template <typename IoT, int KCH, bool APPLY>
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(KCH <= 5 ? 3 : 1))) void
dt_proj_stream_kernel(const ProjParams p) {
  using St = ProjStage<IoT, KCH>;
  constexpr int E = St::E;
  constexpr int KC = 4 * E;                      // k per MFMA chunk
  constexpr int RV = KCH * 4;                    // 16-byte vectors per staged row
  constexpr int TV = kStreamT * RV;              // vectors per tile
  constexpr int NPF = (TV + kProjThreads - 1) / kProjThreads;
  __shared__ __align__(16) St st;

  // Wave w computes all 64 channels of the block against tokens
  // [16 w, 16 w + 16) of each tile: every B operand read from LDS feeds the
  // four channel tiles' MFMAs, whose A operands stay in registers.
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, G = l >> 4, r16 = l & 15;
  const int64_t L = p.L, C = p.channels, R = p.R;
  const int64_t cblocks = (C + kProjC - 1) / kProjC;
  const int64_t b = blockIdx.x / cblocks;
  const int64_t cbase = (blockIdx.x - b * cblocks) * kProjC;
  const IoT* __restrict__ Dg = static_cast<const IoT*>(p.delta) + b * L * R;
  IoT* __restrict__ out = static_cast<IoT*>(p.dt) + b * C * L;

  // A operands of channel tile m: w_dt[cbase + 16 m + r16][kc * KC + E * G .. + E - 1]
  u32x4 a[4][KCH];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t c = cbase + 16 * m + r16;
    const bool c_ok = c < C;
    const IoT* wrow = static_cast<const IoT*>(p.w_dt) + (c_ok ? c * R : 0);
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) a[m][kc] = load_k16<IoT, true>(wrow, kc * KC + E * G, R, c_ok);
  }

  if (APPLY && tid < kProjC) st.bias[tid] = (p.dt_bias && cbase + tid < C) ? p.dt_bias[cbase + tid] : 0.0f;

  u32x4 pf[NPF];
  auto prefetch = [&](int64_t t0) {
#pragma unroll
    for (int n = 0; n < NPF; ++n) {
      const int e = tid + n * kProjThreads;
      const int t = e / RV, kv = (e - t * RV) * E;
      const bool in = e < TV && t0 + t < L && kv < R;
      pf[n] = in ? *reinterpret_cast<const u32x4*>(Dg + (t0 + t) * R + kv) : u32x4{0, 0, 0, 0};
    }
  };
  const int64_t ntiles = (L + kStreamT - 1) / kStreamT;
  if (ntiles > 0) prefetch(0);
  for (int64_t it = 0; it < ntiles; ++it) {
    const int64_t t0 = it * kStreamT;
    const int buf = static_cast<int>(it & 1);
#pragma unroll
    for (int n = 0; n < NPF; ++n) {
      const int e = tid + n * kProjThreads;
      if (e < TV) {
        const int t = e / RV, kv = (e - t * RV) * E;
        *reinterpret_cast<u32x4*>(&st.d[buf][t][kv]) = pf[n];
      }
    }
    __syncthreads();
    if (it + 1 < ntiles) prefetch(t0 + kStreamT);
    v4f acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&st.d[buf][16 * w + r16][kc * KC + E * G]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (sizeof(IoT) == 2) {
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m][kc]),
                                                           __builtin_bit_cast(bf16x8, bv), acc[m], 0, 0, 0);
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t ag = a[m][kc][g], bg = bv[g];
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, ag),
                                                           __builtin_bit_cast(float, bg), acc[m], 0, 0, 0);
          }
        }
      }
    }
    // D: register r at lane (r16, G) of channel tile m is channel 16 m + 4 G + r,
    // token 16 w + r16 of the tile
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4f bm = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (APPLY) bm = *reinterpret_cast<const v4f*>(&st.bias[16 * m + 4 * G]);  // staged before
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[m][r];
        if constexpr (APPLY) v = softplus_f32(v + bm[r]);
        st.o[16 * m + 4 * G + r][16 * w + r16] = Io<IoT>::from_f32(v);
      }
    }
    __syncthreads();
    // rows of 64 tokens, E per 16-byte store
    constexpr int OV = kStreamT / E;               // vectors per output row
    for (int e = tid; e < kProjC * OV; e += kProjThreads) {
      const int cl = e / OV, tv = (e - cl * OV) * E;
      const int64_t c = cbase + cl, t = t0 + tv;
      if (c < C && t < L) {
        if (t + E <= L) {
          *reinterpret_cast<u32x4*>(out + c * L + t) = *reinterpret_cast<const u32x4*>(&st.o[cl][tv]);
        } else {
          for (int x = 0; x < E && t + x < L; ++x) out[c * L + t + x] = st.o[cl][tv + x];
        }
      }
    }
  }
}

template <typename IoT, int KCH>
hipError_t launch_stream(const ProjParams& p, hipStream_t stream) {
  const int64_t blocks = p.batch * ((p.channels + kProjC - 1) / kProjC);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {const_cast<ProjParams*>(&p)};
  const void* fn = p.apply ? reinterpret_cast<const void*>(&dt_proj_stream_kernel<IoT, KCH, true>)
                           : reinterpret_cast<const void*>(&dt_proj_stream_kernel<IoT, KCH, false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kProjThreads), args, 0, stream);
}

template <typename IoT>
hipError_t launch_conv_io(const ConvParams& p, hipStream_t stream) {
  const int64_t waves = p.rows * ((p.L + kConvSeg - 1) / kConvSeg);
  const int64_t blocks = (waves * 64 + kConvThreads - 1) / kConvThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bool vec = p.L % kConvRun == 0 && reinterpret_cast<uintptr_t>(p.x_pre) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.x) % 16 == 0;
  void* args[] = {const_cast<ConvParams*>(&p)};
  const bool reset = p.reset != nullptr, narrow = p.W <= 4;
  const void* fn;
  if (vec) {
    if (narrow) fn = reset ? reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, true, 4, true>)
                           : reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, true, 4, false>);
    else fn = reset ? reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, true, 8, true>)
                    : reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, true, 8, false>);
  } else {
    if (narrow) fn = reset ? reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, false, 4, true>)
                           : reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, false, 4, false>);
    else fn = reset ? reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, false, 8, true>)
                    : reinterpret_cast<const void*>(&conv1d_silu_kernel<IoT, false, 8, false>);
  }
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kConvThreads), args, 0, stream);
}

template <typename IoT, bool VEC>
hipError_t launch_proj_vec(const ProjParams& p, hipStream_t stream) {
  const int64_t blocks = p.batch * ((p.channels + kProjC - 1) / kProjC) * ((p.L + kProjT - 1) / kProjT);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {const_cast<ProjParams*>(&p)};
  const void* fn = p.apply ? reinterpret_cast<const void*>(&dt_proj_kernel<IoT, VEC, true>)
                           : reinterpret_cast<const void*>(&dt_proj_kernel<IoT, VEC, false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kProjThreads), args, 0, stream);
}

template <typename IoT>
hipError_t launch_proj_io(const ProjParams& p, hipStream_t stream) {
  constexpr int E = 16 / sizeof(IoT);
  constexpr int KC = 4 * E;
  const bool vec = p.R % E == 0 && reinterpret_cast<uintptr_t>(p.w_dt) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.delta) % 16 == 0;
  // the streaming kernel also needs whole 16-byte output rows
  const bool rows16 = p.L % E == 0 && reinterpret_cast<uintptr_t>(p.dt) % 16 == 0;
  const int64_t kch = (p.R + KC - 1) / KC;
  if (vec && rows16 && kch <= 8) {
    switch (kch) {
      case 1: return launch_stream<IoT, 1>(p, stream);
      case 2: return launch_stream<IoT, 2>(p, stream);
      case 3: return launch_stream<IoT, 3>(p, stream);
      case 4: return launch_stream<IoT, 4>(p, stream);
      case 5: return launch_stream<IoT, 5>(p, stream);
      case 6: return launch_stream<IoT, 6>(p, stream);
      case 7: return launch_stream<IoT, 7>(p, stream);
      default: return launch_stream<IoT, 8>(p, stream);
    }
  }
  return vec ? launch_proj_vec<IoT, true>(p, stream) : launch_proj_vec<IoT, false>(p, stream);
}

}  // namespace

hipError_t launch_conv1d_silu(const ConvParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_conv_io<bf16_t>(p, stream) : launch_conv_io<float>(p, stream);
}

hipError_t launch_dt_proj(const ProjParams& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_proj_io<bf16_t>(p, stream) : launch_proj_io<float>(p, stream);
}

bool producer_grids_ok(int64_t batch, int64_t channels, int64_t L) {
  const int64_t conv_blocks = (batch * channels * ((L + kConvSeg - 1) / kConvSeg) * 64 + kConvThreads - 1) / kConvThreads;
  const int64_t proj_blocks = batch * ((channels + kProjC - 1) / kProjC) * ((L + kProjT - 1) / kProjT);
  return conv_blocks <= 0x7fffffff && proj_blocks <= 0x7fffffff;
}

}  // namespace ss
