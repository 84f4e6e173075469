// Prompt / prefill selective scan for gfx950: the chunked kernel (included by
// scan_fwd.hip for the plain scan and by scan_states.hip for the variants that
// also write per-token states).
//
// Work decomposition. A channel row (b, c) is owned by one 16-lane DPP row of
// a wavefront: a wave holds 4 channels of one batch row, a block of W waves
// 4W channels of that batch row. The sequence is walked in chunks of 16*K
// tokens; inside a chunk lane l of a row owns the K consecutive tokens
// [l*K, (l+1)*K). Per chunk:
//   1. each lane loads its K tokens of x and dt, coalesced along seq;
//   2. the block stages the chunk's B and C (shared by all its channels:
//      one group, nnterp "selective_scan" page) into LDS as fp32;
//   3. per token: dt = softplus(dt + dt_bias), dt*x, D*x (nnterp page, class
//      docstring);
//   4. for every state coordinate n:
//        a_t = exp(dt_t A[c,n]) (0 at a reset token), b_t = dt_t x_t B[n,t];
//        the lane folds its K pairs from a zero state into (A_l, B_l), with
//        A_l = exp(A[c,n] * sum dt) (0 if the lane holds a reset); lane 0 of
//        the row also applies its map to the state carried in from the
//        previous chunk; a 16-lane DPP inclusive scan of the pairs under
//        the combine (a1,b1),(a2,b2) -> (a2 a1, a2 b1 + b2) ("s6_reset" post,
//        Associative Boundary Resetting) then leaves in each lane the state
//        at the end of its segment; shifted by one lane it is the state the
//        lane starts from, and lane 15's is the next chunk's carry; the lane
//        walks its K tokens, h = a h + b, y += C[n,t] h;
//   5. y = (y + D x) * silu(z), rounded to the I/O type and stored.
// The per-token state never leaves registers (the hardware-aware point of the
// "s6_reset" post, Performance Implications). After the last chunk the carry
// is the final state, written to h_last.
//
// The kernel is bound by VALU issue (one exp and five FMA-class operations
// per token and state coordinate), so its shape is chosen for occupancy: the
// state coordinates run in a rolled loop that keeps one coordinate's K-token
// arrays live, and the per-row constants and the carried state sit in LDS.
#pragma once

#include "ss_device.h"
#include "ss_launch.h"

#include <cmath>

namespace ss {
namespace {

// What the kernel writes besides y and h_last (ScanParams::states):
// nothing, the state after every token ([batch, channels, N, L], seq fastest
// like x and y) or the state after token ScanParams::time_step
// ([batch, channels, N]).
enum StatesOut { kNoStates = 0, kAllStates = 1, kOneState = 2 };

constexpr int kRowLanes = 16;
constexpr int kRowsPerWave = 4;

template <int K, int W>
struct Shape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kChan = kRowsPerWave * W;  // channels per block
  static constexpr int kT = kRowLanes * K;        // tokens per chunk
};

// Waves per SIMD the register budget is set for (launch bound). K = 16 with
// bf16 I/O and no reset mask fits 4 (<= 128 VGPRs); the reset mask and fp32
// z need more registers and run at 3; K = 32 at 2.
template <typename IoT, int K, bool RESET>
constexpr int min_waves_per_simd() {
  return K == 32 ? 2 : ((RESET || sizeof(IoT) == 4) ? 3 : 4);
}

template <typename IoT, int K, int W, int NMAX, bool GATE, bool RESET, int STATES>
__global__ __launch_bounds__(64 * W, (min_waves_per_simd<IoT, K, RESET>())) void scan_fwd_kernel(
    const ScanParams p) {
  using S = Shape<K, W>;
  constexpr int T = S::kT;
  constexpr int KP = K + 4;  // LDS stride of one lane's K values (spreads the banks)
  constexpr int VEC = Io<IoT>::kVec;
  static_assert(K % VEC == 0 && K % 16 == 0, "K must hold whole 16-byte vectors");
  // State coordinates go in groups of NG: a group's B and C are staged in LDS
  // at a time (one group when NMAX <= 16; LDS holds 16 coordinates' worth).
  constexpr int NG = NMAX < 16 ? NMAX : 16;
  constexpr int kGroups = NMAX / NG;
  static_assert(kGroups * NG == NMAX, "NMAX is a multiple of the group size");
  __shared__ float sB[NG][kRowLanes][KP];
  __shared__ float sC[NG][kRowLanes][KP];
  __shared__ float sA2[S::kChan * NMAX];     // A[c, n] * log2(e) per row of the block
  __shared__ float sCarry[S::kChan * NMAX];  // state entering the current chunk
  // kAllStates: one coordinate's states of the chunk per row, each lane's K
  // tokens padded to KP, re-read in token order for coalesced stores
  __shared__ __align__(16) float sSt[STATES == kAllStates ? S::kChan : 1][STATES == kAllStates ? kRowLanes * KP : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int tl = lane & 15;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.chan_blocks;
  const int64_t c_raw = (blk - b * p.chan_blocks) * S::kChan + wave * kRowsPerWave + row;
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

  // Per-row constants and the carried state live in LDS, indexed by the
  // row's slot; each 16-lane row only touches its own slot, and LDS accesses
  // of one wave complete in order, so no barrier guards them. Coordinates
  // n >= N get A2 = 0 and a zero state: they run as the identity.
  const int slot = (wave * kRowsPerWave + row) * NMAX;
  for (int n = tl; n < NMAX; n += kRowLanes) {
    sA2[slot + n] = n < N ? p.A[c * N + n] * kLog2e : 0.0f;
    sCarry[slot + n] = (n < N && p.h0) ? p.h0[(b * p.channels + c) * N + n] : 0.0f;
  }
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;

  const int64_t nchunks = (L + T - 1) / T;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * T;
    const int64_t tb = t0 + tl * K;  // this lane's first token
    const bool full = p.vec_ok && (t0 + T <= L);

    // 1. this lane's tokens of x and dt, and z (raw; it is needed only after
    // the state loop, and loading it here keeps its latency out of the way)
    float xv[K], dv[K];
    uint4 zraw[GATE ? K / VEC : 1];
    if (full) {
#pragma unroll
      for (int v = 0; v < K / VEC; ++v) {
        load_vec16(xg + tb + v * VEC, xv + v * VEC);
        load_vec16(dg + tb + v * VEC, dv + v * VEC);
        if constexpr (GATE) zraw[v] = *reinterpret_cast<const uint4*>(zg + tb + v * VEC);
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const bool in = tb + j < L;
        xv[j] = in ? Io<IoT>::to_f32(xg[tb + j]) : 0.0f;
        dv[j] = in ? Io<IoT>::to_f32(dg[tb + j]) : 0.0f;
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

    // 2. stage this chunk's B and C (fp32) of a group of coordinates for the
    // whole block, between two barriers (the first: the previous readers are
    // done). Coordinates n >= N are staged as zeros: with A2 = 0 they run as
    // the identity map and add nothing to y, so the n loop needs no bounds
    // check.
    auto stage = [&](int grp) {
      __syncthreads();
      {
        constexpr int kSegPerN = T / VEC;
        constexpr int kSeg = NG * kSegPerN;
        for (int s = tid; s < kSeg; s += S::kThreads) {
          const int nl = s / kSegPerN;
          const int n = grp * NG + nl;
          const int tpos = (s - nl * kSegPerN) * VEC;
          const int sl = tpos / K, sj = tpos - sl * K;
          float vb[VEC], vc[VEC];
          const int64_t g = (int64_t)n * L + t0 + tpos;
          if (n >= N) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) vb[e] = vc[e] = 0.0f;
          } else if (full) {
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
            *reinterpret_cast<float4*>(&sB[nl][sl][sj + e]) = make_float4(vb[e], vb[e + 1], vb[e + 2], vb[e + 3]);
            *reinterpret_cast<float4*>(&sC[nl][sl][sj + e]) = make_float4(vc[e], vc[e + 1], vc[e + 2], vc[e + 3]);
          }
        }
      }
      __syncthreads();
    };
    stage(0);

    // 3. per-token step size, dt*x, skip term
    float dtv[K], dtx[K], yv[K], mj[RESET ? K : 1];
    float sdt = 0.0f, mlane = 0.0f;
    // (uniform branches, so that whole chunks run neither a select per
    // token for the softplus switch nor the bounds mask)
    if (p.dt_softplus) {
#pragma unroll
      for (int j = 0; j < K; ++j) dtv[j] = softplus_f32(dv[j] + bias);
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) dtv[j] = dv[j] + bias;
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < K; ++j) dtv[j] = tb + j < L ? dtv[j] : 0.0f;  // past the end: a = 1, b = 0 (identity)
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float d = dtv[j];
      dtx[j] = d * xv[j];
      yv[j] = Dc * xv[j];
      sdt += d;
      if constexpr (RESET) {
        const bool r = (rbits >> j) & 1u;
        mj[j] = r ? -INFINITY : 0.0f;
        mlane = r ? -INFINITY : mlane;
      }
    }

    // 4. the group's state coordinates, one per iteration. With kOneState,
    // the lane whose tokens hold time_step keeps the state after it.
    int jsel = -1;
    if constexpr (STATES == kOneState) {
      const int64_t jd = p.time_step - tb;
      jsel = (jd >= 0 && jd < K) ? (int)jd : -1;
    }
    auto coords = [&](int grp) {
#pragma unroll 1
      for (int nl = 0; nl < NG; ++nl) {
        const int n = grp * NG + nl;
        const float a2n = sA2[slot + n];
        const float carry = sCarry[slot + n];
        float av[K], bv[K];
#pragma unroll
        for (int j = 0; j < K; j += 4) {
          const float4 qb = *reinterpret_cast<const float4*>(&sB[nl][tl][j]);
          bv[j] = qb.x; bv[j + 1] = qb.y; bv[j + 2] = qb.z; bv[j + 3] = qb.w;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float e = RESET ? __builtin_fmaf(dtv[j], a2n, mj[j]) : dtv[j] * a2n;
          av[j] = fast_exp2(e);
          bv[j] *= dtx[j];
        }
        float Al = fast_exp2(RESET ? __builtin_fmaf(sdt, a2n, mlane) : sdt * a2n);
        // fold from a zero state; lane 0 starts from the carried state instead
        float Bl = __builtin_fmaf(av[0], tl == 0 ? carry : 0.0f, bv[0]);
#pragma unroll
        for (int j = 1; j < K; ++j) Bl = __builtin_fmaf(av[j], Bl, bv[j]);
        row16_inclusive_scan(Al, Bl);                            // Bl: state after this lane's tokens
        float h = dpp_or<kDppRowShr1>(carry, Bl);                // state before them
        sCarry[slot + n] = dpp_or<kDppRowNewBcast15>(Bl, Bl);    // state after the chunk (in place)
        float hsel = 0.0f;  // kOneState: the state after the selected token
#pragma unroll
        for (int j = 0; j < K; j += 4) {
          const float4 qc = *reinterpret_cast<const float4*>(&sC[nl][tl][j]);
          const float cq[4] = {qc.x, qc.y, qc.z, qc.w};
          float h4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h = __builtin_fmaf(av[j + i], h, bv[j + i]);
            yv[j + i] = __builtin_fmaf(cq[i], h, yv[j + i]);
            h4[i] = h;
            if constexpr (STATES == kOneState) hsel = j + i == jsel ? h : hsel;
          }
          if constexpr (STATES == kAllStates)
            *reinterpret_cast<float4*>(&sSt[wave * kRowsPerWave + row][tl * KP + j]) =
                make_float4(h4[0], h4[1], h4[2], h4[3]);
        }
        if constexpr (STATES == kOneState) {
          if (jsel >= 0 && n < N && row_ok) p.states[(b * p.channels + c) * N + n] = hsel;
        }
        if constexpr (STATES == kAllStates) {
          // states [batch, channels, N, L]: the row's 16 K tokens of
          // coordinate n, read back in token order from this row's own LDS
          // slot (written by this wave just above; a wave's LDS accesses
          // complete in order), so that store q of the 16 lanes covers 64
          // consecutive tokens
          if (n < N && row_ok) {
            float* dst = p.states + ((b * p.channels + c) * N + n) * L + t0;
#pragma unroll
            for (int q = 0; q < K / 4; ++q) {
              const int tok = 64 * q + 4 * tl;  // within the chunk
              const float4 v4 = *reinterpret_cast<const float4*>(&sSt[wave * kRowsPerWave + row][(tok / K) * KP + tok % K]);
              if (full && p.states_vec) {
                // (plain stores: with the streaming hint this pattern measured slower)
                *reinterpret_cast<float4*>(dst + tok) = v4;
              } else {
                const float hv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (t0 + tok + i < L) dst[tok + i] = hv[i];
              }
            }
          }
        }
      }
    };
    coords(0);
#pragma unroll 1
    for (int grp = 1; grp < kGroups; ++grp) {
      stage(grp);
      coords(grp);
    }

    // 5. gate and store
    if constexpr (GATE) {
      float zv[K];
      if (full) {
#pragma unroll
        for (int v = 0; v < K / VEC; ++v) unpack_vec16<IoT>(zraw[v], zv + v * VEC);
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) zv[j] = tb + j < L ? Io<IoT>::to_f32(zg[tb + j]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < K; ++j) yv[j] *= silu_f32(zv[j]);
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

  if (p.h_last && row_ok)
    for (int n = tl; n < N; n += kRowLanes) p.h_last[(b * p.channels + c) * N + n] = sCarry[slot + n];
}

template <typename IoT, int K, int W, int NMAX, bool GATE, bool RESET, int STATES>
hipError_t launch_t(const ScanParams& p0, hipStream_t stream) {
  ScanParams p = p0;
  p.chan_blocks = (p.channels + Shape<K, W>::kChan - 1) / Shape<K, W>::kChan;
  const int64_t blocks = p.batch * p.chan_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_fwd_kernel<IoT, K, W, NMAX, GATE, RESET, STATES>),
                         dim3((unsigned)blocks), dim3(Shape<K, W>::kThreads), args, 0, stream);
}

// Block shapes. K = 16 tokens per lane keeps a lane's arrays small enough for
// 4 waves per SIMD (8-wave blocks share one B/C stage); the reset mask's
// per-token registers leave room for 3, so those blocks have 4 waves. K = 32
// halves the per-chunk scan overhead at 2 waves per SIMD.
// SS_SCAN_TOKENS_PER_LANE=16|32 overrides the choice (a tuning knob).
template <typename IoT, int K, int NMAX, int STATES>
hipError_t launch_flags(const ScanParams& p, hipStream_t stream) {
  const bool gate = p.z != nullptr, reset = p.reset != nullptr;
  // 8-wave blocks when 4 waves fit per SIMD (two blocks per CU), else 4-wave
  // blocks (three per CU at 3 waves per SIMD)
  // (the every-token states variant stages a 20 KB tile per 16 channels:
  // 4-wave blocks keep three blocks per CU)
  constexpr int W = (min_waves_per_simd<IoT, K, false>() == 4 && STATES != kAllStates) ? 8 : 4;
  constexpr int WR = 4;
  if (gate && reset) return launch_t<IoT, K, WR, NMAX, true, true, STATES>(p, stream);
  if (gate) return launch_t<IoT, K, W, NMAX, true, false, STATES>(p, stream);
  if (reset) return launch_t<IoT, K, WR, NMAX, false, true, STATES>(p, stream);
  return launch_t<IoT, K, W, NMAX, false, false, STATES>(p, stream);
}

// N_max instances: 4, 8, 16, 32, 64 (coordinates past N run as the identity).
// K = 32 is instantiated up to 16 coordinates only; wider states take K = 16.
template <typename IoT, int K, int STATES>
hipError_t launch_n(const ScanParams& p, hipStream_t stream) {
  if (p.N <= 4) return launch_flags<IoT, K, 4, STATES>(p, stream);
  if (p.N <= 8) return launch_flags<IoT, K, 8, STATES>(p, stream);
  if (p.N <= 16) return launch_flags<IoT, K, 16, STATES>(p, stream);
  if constexpr (K == 16) {
    if (p.N <= 32) return launch_flags<IoT, K, 32, STATES>(p, stream);
    return launch_flags<IoT, K, 64, STATES>(p, stream);
  } else {
    return launch_n<IoT, 16, STATES>(p, stream);
  }
}

}  // namespace
}  // namespace ss


