// Prompt / prefill selective scan for gfx950.
//
// Work decomposition. A channel row (b, c) is owned by one 16-lane DPP row of
// a wavefront: a wave holds 4 channels of one batch row, a 256-thread block
// 16 channels. The sequence is walked in chunks of 16*K tokens; inside a
// chunk lane l of a row owns the K consecutive tokens [l*K, (l+1)*K).
// Per chunk:
//   1. each lane loads its K tokens of x, dt (and z), coalesced along seq;
//   2. the block stages the chunk's B and C (shared by all its channels:
//      one group, nnterp "selective_scan" page) into LDS as fp32;
//   3. per token: dt = softplus(dt + dt_bias), dt*x, D*x (nnterp page, class
//      docstring);
//   4. for every state coordinate n:
//        a_t = exp(dt_t A[c,n]) (0 at a reset token), b_t = dt_t x_t B[n,t];
//        the lane folds its K pairs from a zero state into (A_l, B_l), with
//        A_l = exp(A[c,n] * sum dt) (0 if the lane holds a reset);
//        a 16-lane DPP inclusive scan of (A_l, B_l) under the combine
//        (a1,b1),(a2,b2) -> (a2 a1, a2 b1 + b2) ("s6_reset" post,
//        Associative Boundary Resetting) gives each lane the map of all
//        earlier lanes; applied to the carry from the previous chunk it is
//        the lane's incoming state; the row total advances the carry;
//        the lane then walks its K tokens, h = a h + b, y += C[n,t] h;
//   5. y = (y + D x) * silu(z), rounded to the I/O type and stored.
// The per-token state never leaves registers (the hardware-aware point of the
// "s6_reset" post, Performance Implications). After the last chunk the carry
// is the final state, written to h_last.
#include "ss_device.h"
#include "ss_launch.h"

#include <cmath>
#include <cstdlib>

namespace ss {
namespace {

constexpr int kRowLanes = 16;
constexpr int kRowsPerWave = 4;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;
constexpr int kChanPerBlock = kRowsPerWave * kWavesPerBlock;

template <typename IoT, int K, int NMAX, bool GATE, bool RESET>
__global__ __launch_bounds__(kThreads, 2) void scan_fwd_kernel(const ScanParams p) {
  constexpr int T = kRowLanes * K;  // tokens of one chunk of one row
  constexpr int KP = K + 4;         // LDS stride of one lane's K values (bank spread)
  constexpr int VEC = Io<IoT>::kVec;
  static_assert(K % VEC == 0 && K % 16 == 0, "K must hold whole 16-byte vectors");
  __shared__ float sB[NMAX][kRowLanes][KP];
  __shared__ float sC[NMAX][kRowLanes][KP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int tl = lane & 15;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.chan_blocks;
  const int64_t c_raw = (blk - b * p.chan_blocks) * kChanPerBlock + wave * kRowsPerWave + row;
  const bool row_ok = c_raw < p.channels;
  const int64_t c = row_ok ? c_raw : p.channels - 1;  // rows past the end compute, never store
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t rowoff = (b * p.channels + c) * L;

  const IoT* __restrict__ xg = static_cast<const IoT*>(p.x) + rowoff;
  const IoT* __restrict__ dg = static_cast<const IoT*>(p.dt) + rowoff;
  const IoT* __restrict__ zg = GATE ? static_cast<const IoT*>(p.z) + rowoff : nullptr;
  IoT* __restrict__ yg = static_cast<IoT*>(p.y) + rowoff;
  const IoT* __restrict__ Bg = static_cast<const IoT*>(p.B) + b * N * L;
  const IoT* __restrict__ Cg = static_cast<const IoT*>(p.C) + b * N * L;
  const uint8_t* __restrict__ rg = RESET ? p.reset + b * L : nullptr;

  float a2[NMAX];     // A[c, n] * log2(e)
  float carry[NMAX];  // state entering the current chunk
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    a2[n] = n < N ? p.A[c * N + n] * kLog2e : 0.0f;
    carry[n] = (n < N && p.h0) ? p.h0[(b * p.channels + c) * N + n] : 0.0f;
  }
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;

  const int64_t nchunks = (L + T - 1) / T;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * T;
    const int64_t tb = t0 + tl * K;  // this lane's first token
    const bool full = p.vec_ok && (t0 + T <= L);

    // 1. this lane's tokens
    float xv[K], dv[K];
    uint32_t zraw[GATE ? (K * sizeof(IoT) / 4) : 1];
    if (full) {
#pragma unroll
      for (int v = 0; v < K / VEC; ++v) {
        load_vec16(xg + tb + v * VEC, xv + v * VEC);
        load_vec16(dg + tb + v * VEC, dv + v * VEC);
        if constexpr (GATE) {
          const uint4 w = *reinterpret_cast<const uint4*>(zg + tb + v * VEC);
          zraw[4 * v] = w.x; zraw[4 * v + 1] = w.y; zraw[4 * v + 2] = w.z; zraw[4 * v + 3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const bool in = tb + j < L;
        xv[j] = in ? Io<IoT>::to_f32(xg[tb + j]) : 0.0f;
        dv[j] = in ? Io<IoT>::to_f32(dg[tb + j]) : 0.0f;
      }
      if constexpr (GATE) {
#pragma unroll
        for (int w = 0; w < (int)(K * sizeof(IoT) / 4); ++w) {
          if constexpr (sizeof(IoT) == 4) {
            const bool in = tb + w < L;
            zraw[w] = in ? __builtin_bit_cast(uint32_t, Io<IoT>::to_f32(zg[tb + w])) : 0u;
          } else {
            const bool in0 = tb + 2 * w < L, in1 = tb + 2 * w + 1 < L;
            const uint32_t lo = in0 ? reinterpret_cast<const uint16_t*>(zg)[tb + 2 * w] : 0u;
            const uint32_t hi = in1 ? reinterpret_cast<const uint16_t*>(zg)[tb + 2 * w + 1] : 0u;
            zraw[w] = lo | (hi << 16);
          }
        }
      }
    }
    uint32_t rbits = 0;  // bit j: token tb + j starts a document
    if constexpr (RESET) {
      if (full && p.reset_vec) {
#pragma unroll
        for (int v = 0; v < K / 16; ++v) {
          const uint4 w = *reinterpret_cast<const uint4*>(rg + tb + 16 * v);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int i = 0; i < 16; ++i)
            rbits |= (((ws[i >> 2] >> (8 * (i & 3))) & 0xffu) ? 1u : 0u) << (16 * v + i);
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j)
          if (tb + j < L && rg[tb + j]) rbits |= 1u << j;
      }
    }

    // 2. stage this chunk's B and C (fp32) for the whole block
    __syncthreads();  // previous chunk's readers are done
    {
      constexpr int kSegPerN = T / VEC;
      const int nseg = N * kSegPerN;
      for (int s = tid; s < nseg; s += kThreads) {
        const int n = s / kSegPerN;
        const int tpos = (s - n * kSegPerN) * VEC;
        const int sl = tpos / K, sj = tpos - sl * K;
        float vb[VEC], vc[VEC];
        const int64_t g = (int64_t)n * L + t0 + tpos;
        if (full) {
          load_vec16(Bg + g, vb);
          load_vec16(Cg + g, vc);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const bool in = t0 + tpos + e < L;
            vb[e] = in ? Io<IoT>::to_f32(Bg[g + e]) : 0.0f;
            vc[e] = in ? Io<IoT>::to_f32(Cg[g + e]) : 0.0f;
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          *reinterpret_cast<float4*>(&sB[n][sl][sj + e]) = make_float4(vb[e], vb[e + 1], vb[e + 2], vb[e + 3]);
          *reinterpret_cast<float4*>(&sC[n][sl][sj + e]) = make_float4(vc[e], vc[e + 1], vc[e + 2], vc[e + 3]);
        }
      }
    }
    __syncthreads();

    // 3. per-token step size, dt*x, skip term
    float dtv[K], dtx[K], yv[K], mj[RESET ? K : 1];
    float sdt = 0.0f, mlane = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool in = full || (tb + j < L);
      const float v = dv[j] + bias;
      float d = p.dt_softplus ? softplus_f32(v) : v;
      d = in ? d : 0.0f;  // tokens past the end: a = 1, b = 0 (identity)
      dtv[j] = d;
      dtx[j] = d * xv[j];
      yv[j] = Dc * xv[j];
      sdt += d;
      if constexpr (RESET) {
        const bool r = (rbits >> j) & 1u;
        mj[j] = r ? -INFINITY : 0.0f;
        mlane = r ? -INFINITY : mlane;
      }
    }

    // 4. state coordinates
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      if (n < N) {
        float av[K], bv[K];
        const float* bs = &sB[n][tl][0];
#pragma unroll
        for (int j = 0; j < K; j += 4) {
          const float4 q = *reinterpret_cast<const float4*>(bs + j);
          const float qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = RESET ? __builtin_fmaf(dtv[j + i], a2[n], mj[j + i]) : dtv[j + i] * a2[n];
            av[j + i] = fast_exp2(e);
            bv[j + i] = dtx[j + i] * qq[i];
          }
        }
        float Bl = bv[0];
#pragma unroll
        for (int j = 1; j < K; ++j) Bl = __builtin_fmaf(av[j], Bl, bv[j]);
        float Al = fast_exp2(RESET ? __builtin_fmaf(sdt, a2[n], mlane) : sdt * a2[n]);
        row16_inclusive_scan(Al, Bl);
        const float Ae = dpp_or<kDppRowShr1>(1.0f, Al);  // exclusive: lanes before this one
        const float Be = dpp_or<kDppRowShr1>(0.0f, Bl);
        const float At = dpp_or<kDppRowNewBcast15>(0.0f, Al);  // whole chunk of the row
        const float Bt = dpp_or<kDppRowNewBcast15>(0.0f, Bl);
        float h = __builtin_fmaf(Ae, carry[n], Be);
        carry[n] = __builtin_fmaf(At, carry[n], Bt);
        const float* cs = &sC[n][tl][0];
#pragma unroll
        for (int j = 0; j < K; j += 4) {
          const float4 q = *reinterpret_cast<const float4*>(cs + j);
          const float qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h = __builtin_fmaf(av[j + i], h, bv[j + i]);
            yv[j + i] = __builtin_fmaf(qq[i], h, yv[j + i]);
          }
        }
      }
    }

    // 5. gate and store
    if constexpr (GATE) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float zf;
        if constexpr (sizeof(IoT) == 4) {
          zf = __builtin_bit_cast(float, zraw[j]);
        } else {
          const uint32_t w = zraw[j >> 1];
          zf = __builtin_bit_cast(float, (j & 1) ? (w & 0xffff0000u) : (w << 16));
        }
        yv[j] *= silu_f32(zf);
      }
    }
    if (row_ok) {
      if (full) {
#pragma unroll
        for (int v = 0; v < K / VEC; ++v) store_vec16(yg + tb + v * VEC, yv + v * VEC);
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j)
          if (tb + j < L) yg[tb + j] = Io<IoT>::from_f32(yv[j]);
      }
    }
  }

  if (p.h_last && row_ok) {
    float v = 0.0f;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) v = (tl == n) ? carry[n] : v;
    if (tl < N) p.h_last[(b * p.channels + c) * N + tl] = v;
  }
}

template <typename IoT, int K, int NMAX, bool GATE, bool RESET>
hipError_t launch_t(const ScanParams& p, hipStream_t stream) {
  const int64_t blocks = p.batch * p.chan_blocks;
  ScanParams q = p;
  void* args[] = {&q};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_fwd_kernel<IoT, K, NMAX, GATE, RESET>),
                         dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

template <typename IoT, int K, int NMAX>
hipError_t launch_flags(const ScanParams& p, hipStream_t stream) {
  const bool gate = p.z != nullptr, reset = p.reset != nullptr;
  if (gate && reset) return launch_t<IoT, K, NMAX, true, true>(p, stream);
  if (gate) return launch_t<IoT, K, NMAX, true, false>(p, stream);
  if (reset) return launch_t<IoT, K, NMAX, false, true>(p, stream);
  return launch_t<IoT, K, NMAX, false, false>(p, stream);
}

template <typename IoT, int K>
hipError_t launch_n(const ScanParams& p, hipStream_t stream) {
  if (p.N <= 4) return launch_flags<IoT, K, 4>(p, stream);
  if (p.N <= 8) return launch_flags<IoT, K, 8>(p, stream);
  return launch_flags<IoT, K, 16>(p, stream);
}

// Tokens per lane: 32 halves the per-chunk scan overhead of 16 but nearly
// fills the 256 VGPRs of a 2-wave/SIMD occupancy; the reset mask and fp32 I/O
// need more registers than that (they would spill), and short sequences keep
// 16 so a chunk is not mostly padding.
// SS_SCAN_TOKENS_PER_LANE=16|32 overrides the choice (a tuning knob).
int pick_k(const ScanParams& p, bool io_bf16) {
  static const int forced = [] {
    const char* e = std::getenv("SS_SCAN_TOKENS_PER_LANE");
    return e ? std::atoi(e) : 0;
  }();
  if (forced == 16 || forced == 32) return forced;
  if (!io_bf16 || p.reset != nullptr) return 16;
  return p.L >= 16 * 32 ? 32 : 16;
}

}  // namespace

hipError_t launch_scan_fwd(const ScanParams& p0, bool io_bf16, hipStream_t stream) {
  ScanParams p = p0;
  p.chan_blocks = (p.channels + kChanPerBlock - 1) / kChanPerBlock;
  const int K = pick_k(p, io_bf16);
  if (io_bf16) return K == 32 ? launch_n<bf16_t, 32>(p, stream) : launch_n<bf16_t, 16>(p, stream);
  return K == 32 ? launch_n<float, 32>(p, stream) : launch_n<float, 16>(p, stream);
}

int64_t scan_fwd_blocks(int64_t batch, int64_t channels) {
  return batch * ((channels + kChanPerBlock - 1) / kChanPerBlock);
}

}  // namespace ss
