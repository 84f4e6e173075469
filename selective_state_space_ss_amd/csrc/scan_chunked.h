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
// per token and state coordinate, next to nothing else: on gfx950 an exp2
// occupies the issue port for two FMA slots and overlaps nothing), so every
// instruction outside that core is one too many. The state coordinates run
// one after another (unrolled, so every LDS offset is an immediate), keeping
// one coordinate's K-token arrays live; the per-row constants and the
// carried state sit in LDS.
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

// SPLIT = 2: two waves share each group of 4 rows, each taking half of the
// state coordinates (the split form below), so a block of W waves holds 2 W
// rows instead of 4 W.
template <int K, int W, int SPLIT = 1>
struct Shape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kChan = kRowsPerWave * W / SPLIT;  // channels per block
  static constexpr int kT = kRowLanes * K;                // tokens per chunk
};

// Waves per SIMD the register budget is set for (launch bound). K = 16 with
// bf16 I/O and no reset mask fits 4 (<= 128 VGPRs); the reset mask and fp32
// z need more registers and run at 3; K = 32 at 2. The split form in 4-wave
// blocks runs 3 blocks per CU (LDS), so 3 waves per SIMD.
template <typename IoT, int K, bool RESET, int SPLIT = 1, int W = 8>
constexpr int min_waves_per_simd() {
  return K == 32 ? 2 : ((RESET || sizeof(IoT) == 4 || (SPLIT == 2 && W == 4)) ? 3 : 4);
}

// The fused producer of x (nnterp "selective_scan" page, class docstring; the
// ssm_mixer page's x is the post-conv SiLU input): for this lane's K tokens,
//   x_t = silu(conv_b + sum_{k<W} conv_w[k] * x_pre[t - (W-1) + k]),
// a depthwise causal convolution, in fp32 and never rounded or stored. A tap
// before position 0, or before the current document's first token (a reset
// mask; bit 8 + j of `starts` marks token tb + j, bits 0..7 the 8 tokens
// before the lane), reads 0. The taps are taken through a window of the CW - 1
// previous x_pre values, which a document start clears, so each token costs
// CW FMAs (weights past W are 0) plus, with resets, CW - 1 selects.
template <typename IoT, int K, int CW, bool RESET>
__device__ __forceinline__ void conv_silu_lane(const IoT* __restrict__ xpg, int64_t tb, int64_t L, bool full,
                                               const float* __restrict__ wrow, int Wd, float cb, uint32_t starts,
                                               float* xv) {
  constexpr int VEC = Io<IoT>::kVec;
  float xp[K], hp[8];  // this lane's x_pre, and the 8 tokens before it
  if (full) {
#pragma unroll
    for (int v = 0; v < K / VEC; ++v) load_vec16(xpg + tb + v * VEC, xp + v * VEC);
    if (tb >= 8) {
#pragma unroll
      for (int v = 0; v < 8 / VEC; ++v) load_vec16(xpg + tb - 8 + v * VEC, hp + v * VEC);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) hp[u] = tb - 8 + u >= 0 ? Io<IoT>::to_f32(xpg[tb - 8 + u]) : 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) xp[j] = tb + j < L ? Io<IoT>::to_f32(xpg[tb + j]) : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t s = tb - 8 + u;
      hp[u] = (s >= 0 && s < L) ? Io<IoT>::to_f32(xpg[s]) : 0.0f;
    }
  }
  // wp[i]: the weight of the tap at t - (CW - 1) + i (conv_w[W - CW + i]), 0 for i < CW - W
  float wp[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) wp[i] = i >= CW - Wd ? wrow[Wd - CW + i] : 0.0f;
  // the window before token 0: positions -(CW - 1) .. -1, cleared at document starts
  float win[CW > 1 ? CW - 1 : 1];
#pragma unroll
  for (int i = 0; i < CW - 1; ++i) win[i] = 0.0f;
#pragma unroll
  for (int q = -(CW - 1); q < 0; ++q) {
    if constexpr (RESET) {
      if ((starts >> (8 + q)) & 1u) {
#pragma unroll
        for (int i = 0; i < CW - 1; ++i) win[i] = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i + 1 < CW - 1; ++i) win[i] = win[i + 1];
    if constexpr (CW > 1) win[CW - 2] = hp[8 + q];
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if constexpr (RESET) {
      if ((starts >> (8 + j)) & 1u) {
#pragma unroll
        for (int i = 0; i < CW - 1; ++i) win[i] = 0.0f;
      }
    }
    float acc = __builtin_fmaf(wp[CW - 1], xp[j], cb);
#pragma unroll
    for (int i = 0; i < CW - 1; ++i) acc = __builtin_fmaf(wp[i], win[i], acc);
    xv[j] = silu_f32(acc);
#pragma unroll
    for (int i = 0; i + 1 < CW - 1; ++i) win[i] = win[i + 1];
    if constexpr (CW > 1) win[CW - 2] = xp[j];
  }
}

// CW: 0, or the tap bound (4 or 8) of the fused causal conv1d + SiLU that
// makes x from x_pre (p.x is then x_pre; see conv_silu_lane).
//
// SPLIT: 1, or 2 for the split form used when a launch has few rows (a wave
// per SIMD or two): waves 2g and 2g + 1 share rows 4g..4g+3 of the block and
// the chunk's B/C stage, and take state coordinates [0, N/2) and [N/2, N)
// of every 16-coordinate group, so the launch has twice the waves for the
// same rows. Each wave forms every token's step size (the exponents need all
// of them), folds, scans and walks its own coordinates, and accumulates its
// part of every token's y; the two parts meet in LDS once per chunk
// (sYx, after a barrier), wave 2g finishing the first K/2 tokens of each
// lane (D x, the gate, the store) and wave 2g + 1 the rest.
template <typename IoT, int K, int W, int NMAX, bool GATE, bool RESET, int STATES, int CW = 0, int SPLIT = 1>
__global__ __launch_bounds__(64 * W, (min_waves_per_simd<IoT, K, RESET, SPLIT, W>())) void scan_fwd_kernel(
    const ScanParams p) {
  static_assert(CW == 0 || (K == 16 && STATES == kNoStates), "the fused conv runs at 16 tokens per lane");
  static_assert(SPLIT == 1 || (STATES == kNoStates && W % 2 == 0), "the split form writes y and h_last only");
  using S = Shape<K, W, SPLIT>;
  constexpr int KH = K / SPLIT;  // tokens per lane this wave finishes (y, gate, store)
  // PF: the split form in 4-wave blocks (bf16, 3 waves per SIMD, registers
  // to spare) loads the next chunk's x and dt and this chunk's z while it
  // computes. (B and C of the next chunk as well, 16 more registers per
  // lane, spilled and measured slower.)
  constexpr bool PF = SPLIT == 2 && W == 4 && sizeof(IoT) == 2 && CW == 0 && !RESET;
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
  __shared__ float sZero[NMAX];              // what lanes 1..15 read in place of the carry
  // SPLIT: each wave's part of y for the K/2 tokens per lane its partner
  // finishes, four tokens of a lane per float4, lanes adjacent (no bank
  // conflicts)
  __shared__ float4 sYx[SPLIT == 2 ? W : 1][SPLIT == 2 ? KH / 4 : 1][SPLIT == 2 ? 64 : 1];
  // kAllStates: one coordinate's states of the chunk per row, each lane's K
  // tokens padded to KP, re-read in token order for coalesced stores
  __shared__ __align__(16) float sSt[STATES == kAllStates ? S::kChan : 1][STATES == kAllStates ? kRowLanes * KP : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int gw = wave / SPLIT;    // the group of 4 rows this wave works on
  const int half = wave % SPLIT;  // SPLIT: which half of the coordinates (and which tokens it finishes)
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int tl = lane & 15;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.chan_blocks;
  const int64_t c_raw = (blk - b * p.chan_blocks) * S::kChan + gw * kRowsPerWave + row;
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
  const int slot = (gw * kRowsPerWave + row) * NMAX;
  for (int n = tl; n < NMAX; n += kRowLanes) {
    sA2[slot + n] = n < N ? p.A[c * N + n] * kLog2e : 0.0f;
    sCarry[slot + n] = (n < N && p.h0) ? p.h0[(b * p.channels + c) * N + n] : 0.0f;
  }
  for (int n = tid; n < NMAX; n += S::kThreads) sZero[n] = 0.0f;
  // The carried state enters a chunk at lane 0 of each row; the other lanes
  // read zeros in its place, so the first fold step needs no select. sZero is
  // only ever read after the first chunk's staging barrier.
  const float* __restrict__ carry_src = tl == 0 ? &sCarry[slot] : sZero;
  const bool carry_writer = tl == kRowLanes - 1;  // lane 15 ends the chunk
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;

  // PF: raw 16-byte vectors of this lane's x and dt in the next full chunk
  uint4 px[PF ? K / VEC : 1], pd[PF ? K / VEC : 1];
  auto prefetch = [&](int64_t t0n) {  // the chunk starting at t0n, which is full
#pragma unroll
    for (int v = 0; v < (PF ? K / VEC : 0); ++v) {
      px[v] = *reinterpret_cast<const uint4*>(xg + t0n + tl * K + v * VEC);
      pd[v] = *reinterpret_cast<const uint4*>(dg + t0n + tl * K + v * VEC);
    }
  };
  if constexpr (PF) {
    if (p.vec_ok && T <= L) prefetch(0);
  }

  const int64_t nchunks = (L + T - 1) / T;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * T;
    const int64_t tb = t0 + tl * K;  // this lane's first token
    const bool full = p.vec_ok && (t0 + T <= L);
    const bool next_full = p.vec_ok && (t0 + 2 * T <= L);

    // 1. this lane's tokens of x and dt. z is loaded after the state loop:
    // held in registers across the loop it costs registers the loop needs
    // (spills), and the other waves of the SIMD cover its latency. (Measured
    // on MI355X at batch 8 x 5120 x 2048: 334.4 us, against 348.8 us with z
    // held in registers and 348.1 us with z copied global -> LDS by
    // global_load_lds at the chunk's start.)
    float xv[K], dv[K];
    if (full) {
#pragma unroll
      for (int v = 0; v < K / VEC; ++v) {
        if constexpr (PF) {
          unpack_vec16<IoT>(px[v], xv + v * VEC);
          unpack_vec16<IoT>(pd[v], dv + v * VEC);
        } else {
          if constexpr (CW == 0) load_vec16(xg + tb + v * VEC, xv + v * VEC);
          load_vec16(dg + tb + v * VEC, dv + v * VEC);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const bool in = tb + j < L;
        if constexpr (CW == 0) xv[j] = in ? Io<IoT>::to_f32(xg[tb + j]) : 0.0f;
        dv[j] = in ? Io<IoT>::to_f32(dg[tb + j]) : 0.0f;
      }
    }
    uint32_t rbits = 0;  // bit j: token tb + j starts a document
    uint32_t hbits = 0;  // (fused conv) bit u: token tb - 8 + u starts a document
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
        if constexpr (CW > 0) {
          if (tb >= 8) {
            const uint2 w = *reinterpret_cast<const uint2*>(rg + tb - 8);
#pragma unroll
            for (int i = 0; i < 8; ++i) hbits |= ((((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xffu) ? 1u : 0u) << i;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j)
          if (tb + j < L && rg[tb + j]) rbits |= 1u << j;
        if constexpr (CW > 0) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int64_t s = tb - 8 + u;
            if (s >= 0 && s < L && rg[s]) hbits |= 1u << u;
          }
        }
      }
    }
    if constexpr (CW > 0)
      conv_silu_lane<IoT, K, CW, RESET>(xg, tb, L, full, p.conv_w + c * p.conv_width, p.conv_width,
                                        p.conv_b ? p.conv_b[c] : 0.0f, hbits | (rbits << 8), xv);

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
          // (each branch stores its own values: with one shared set the
          // compiler zero-fills it on the common path too)
          if (full && n < N) {
            load_vec16(Bg + g, vb);
            load_vec16(Cg + g, vc);
          } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const bool in = n < N && t0 + tpos + e < L;
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
    // PF: this chunk's z (the tokens this wave finishes), then the next
    // chunk's inputs, in flight during the state loop
    uint4 pz[PF && GATE ? KH / VEC : 1];
    if constexpr (PF && GATE) {
      if (full) {
#pragma unroll
        for (int v = 0; v < KH / VEC; ++v)
          pz[v] = *reinterpret_cast<const uint4*>(zg + tb + half * KH + v * VEC);
      }
    }
    if constexpr (PF) {
      if (next_full) prefetch(t0 + T);
    }

    // 3. per-token step size, dt*x, skip term
    float dtv[K], dtx[K], yv[K], mj[RESET ? K : 1];
    float sdt = 0.0f, mlane = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) dtv[j] = dv[j] + bias;
    // (uniform branches, so that whole chunks run neither a select per
    // token for the softplus switch nor the bounds mask)
    if (p.dt_softplus) {
#pragma unroll
      for (int j = 0; j < K; ++j) dtv[j] = softplus_f32(dtv[j]);
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < K; ++j) dtv[j] = tb + j < L ? dtv[j] : 0.0f;  // past the end: a = 1, b = 0 (identity)
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float d = dtv[j];
      dtx[j] = d * xv[j];
      // (SPLIT: D x only in the part of the wave that finishes the token;
      // then x is dead during the state loop)
      yv[j] = (SPLIT == 1 || (j < KH) == (half == 0)) ? Dc * xv[j] : 0.0f;
      sdt += d;
      if constexpr (RESET) {
        const bool r = (rbits >> j) & 1u;
        mj[j] = r ? -INFINITY : 0.0f;
        mlane = r ? -INFINITY : mlane;
      }
    }

    // 4. the group's state coordinates, one after another (unrolled: every
    // LDS offset is an immediate). With kOneState, the lane whose tokens hold
    // time_step keeps the state after it.
    int jsel = -1;
    if constexpr (STATES == kOneState) {
      const int64_t jd = p.time_step - tb;
      jsel = (jd >= 0 && jd < K) ? (int)jd : -1;
    }
    auto coords = [&](int grp) {
      constexpr int NGH = NG / SPLIT;  // coordinates of the group this wave takes
#pragma unroll
      for (int i = 0; i < NGH; ++i) {
        const int nl = half * NGH + i;
        const int n = grp * NG + nl;
        const float a2n = sA2[slot + n];
        const float carry_l = carry_src[n];
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
        const float Al = fast_exp2(RESET ? __builtin_fmaf(sdt, a2n, mlane) : sdt * a2n);
        // fold from a zero state; lane 0 starts from the carried state (the
        // other lanes read a zero carry, so their first step is exactly b0)
        const float f0 = __builtin_fmaf(av[0], carry_l, bv[0]);
        float Bl = f0;
#pragma unroll
        for (int j = 1; j < K; ++j) Bl = __builtin_fmaf(av[j], Bl, bv[j]);
        float h = f0;
        row16_scan_and_enter(Al, Bl, h, av[0]);  // Bl: state after this lane's tokens; h: after its first
        if (carry_writer) sCarry[slot + n] = Bl;  // state after the chunk (in place)
        float hsel = 0.0f;  // kOneState: the state after the selected token
#pragma unroll
        for (int j = 0; j < K; j += 4) {
          const float4 qc = *reinterpret_cast<const float4*>(&sC[nl][tl][j]);
          const float cq[4] = {qc.x, qc.y, qc.z, qc.w};
          float h4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (j + i > 0) h = __builtin_fmaf(av[j + i], h, bv[j + i]);
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
        // Pin this coordinate's walk here: y is only read after the loop, so
        // without this the compiler sinks every coordinate's walk to the end
        // (all their K-token arrays live at once, and spilled); and keep the
        // scheduler from interleaving coordinates for the same reason.
#pragma unroll
        for (int j = 0; j < K; ++j) asm volatile("" : "+v"(yv[j]));
        __builtin_amdgcn_sched_barrier(0);
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

    // 5. (SPLIT) the two waves' parts of y meet: each hands over the part
    // for the tokens its partner finishes and adds the partner's part to its
    // own. (Waves reach the next write of sYx only after the
    // next chunk's first staging barrier, so one barrier per chunk does.)
    float yo[KH];  // y of the tokens this wave finishes, tb + half * KH + i
    if constexpr (SPLIT == 2) {
      // (selects on the wave-uniform half, with constant register indexes)
      float ymine[KH], ygive[KH];
#pragma unroll
      for (int i = 0; i < KH; ++i) {
        ymine[i] = half ? yv[KH + i] : yv[i];
        ygive[i] = half ? yv[i] : yv[KH + i];
      }
#pragma unroll
      for (int q = 0; q < KH / 4; ++q)
        sYx[wave][q][lane] = make_float4(ygive[4 * q], ygive[4 * q + 1], ygive[4 * q + 2], ygive[4 * q + 3]);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < KH / 4; ++q) {
        const float4 o = sYx[wave ^ 1][q][lane];
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) yo[4 * q + i] = ymine[4 * q + i] + ov[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) yo[j] = yv[j];
    }

    // 6. gate and store
    const int64_t to = tb + half * KH;
    if constexpr (GATE) {
      float zv[KH];
      if (full) {
#pragma unroll
        for (int v = 0; v < KH / VEC; ++v) {
          if constexpr (PF) unpack_vec16<IoT>(pz[v], zv + v * VEC);
          else load_vec16(zg + to + v * VEC, zv + v * VEC);
        }
      } else {
#pragma unroll
        for (int j = 0; j < KH; ++j) zv[j] = to + j < L ? Io<IoT>::to_f32(zg[to + j]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < KH; ++j) yo[j] *= silu_f32(zv[j]);
    }
    if (row_ok) {
      if (full) {
#pragma unroll
        for (int v = 0; v < KH / VEC; ++v) store_vec16(yg + to + v * VEC, yo + v * VEC);
      } else {
#pragma unroll
        for (int j = 0; j < KH; ++j)
          if (to + j < L) yg[to + j] = Io<IoT>::from_f32(yo[j]);
      }
    }
  }

  // (SPLIT: each wave writes the coordinates it carried; its own LDS writes
  // of sCarry are complete in order, so no barrier is needed)
  if (p.h_last && row_ok)
    for (int n = tl; n < N; n += kRowLanes)
      if (SPLIT == 1 || (n % NG) / (NG / SPLIT) == half) p.h_last[(b * p.channels + c) * N + n] = sCarry[slot + n];
}

template <typename IoT, int K, int W, int NMAX, bool GATE, bool RESET, int STATES, int CW = 0, int SPLIT = 1>
hipError_t launch_t(const ScanParams& p0, hipStream_t stream) {
  using S = Shape<K, W, SPLIT>;
  ScanParams p = p0;
  p.chan_blocks = (p.channels + S::kChan - 1) / S::kChan;
  const int64_t blocks = p.batch * p.chan_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&scan_fwd_kernel<IoT, K, W, NMAX, GATE, RESET, STATES, CW, SPLIT>),
      dim3((unsigned)blocks), dim3(S::kThreads), args, 0, stream);
}

// Block shapes. K = 16 tokens per lane keeps a lane's arrays small enough for
// 4 waves per SIMD (8-wave blocks share one B/C stage); the reset mask's
// per-token registers leave room for 3, so those blocks have 4 waves. K = 32
// halves the per-chunk scan overhead at 2 waves per SIMD.
// SS_SCAN_TOKENS_PER_LANE=16|32 overrides the choice (a tuning knob).
// RESETS: which instantiations one call site compiles: 0 = without a reset
// mask, 1 = with one, 2 = both (picked at run time). The plain scan keeps the
// two sets in separate files, each built with the machine scheduler that
// measured faster for it.
//
// split (0, 4 or 8): the split form in blocks of that many waves, for a
// launch without a reset mask at K = 16 and N <= 16 (where it is
// instantiated); 0 = the plain form. The caller picks it (split_waves).
template <typename IoT, int K, int NMAX, int STATES, int RESETS, int CW = 0>
hipError_t launch_flags(const ScanParams& p, hipStream_t stream, int split = 0) {
  const bool gate = p.z != nullptr, reset = p.reset != nullptr;
  if constexpr (K == 16 && NMAX <= 16 && STATES == kNoStates && RESETS == 0 && CW == 0) {
    if (split == 4) {
      if (gate) return launch_t<IoT, K, 4, NMAX, true, false, STATES, CW, 2>(p, stream);
      return launch_t<IoT, K, 4, NMAX, false, false, STATES, CW, 2>(p, stream);
    }
    if (split == 8) {
      if (gate) return launch_t<IoT, K, 8, NMAX, true, false, STATES, CW, 2>(p, stream);
      return launch_t<IoT, K, 8, NMAX, false, false, STATES, CW, 2>(p, stream);
    }
  }
  // 8-wave blocks when 4 waves fit per SIMD (two blocks per CU), else 4-wave
  // blocks (three per CU at 3 waves per SIMD)
  // (the every-token states variant stages a 20 KB tile per 16 channels:
  // 4-wave blocks keep three blocks per CU)
  constexpr int W = (min_waves_per_simd<IoT, K, false>() == 4 && STATES != kAllStates) ? 8 : 4;
  constexpr int WR = 4;
  if constexpr (RESETS != 0) {
    if (reset || RESETS == 1) {
      if (gate) return launch_t<IoT, K, WR, NMAX, true, true, STATES, CW>(p, stream);
      return launch_t<IoT, K, WR, NMAX, false, true, STATES, CW>(p, stream);
    }
  }
  if constexpr (RESETS != 1) {
    if (gate) return launch_t<IoT, K, W, NMAX, true, false, STATES, CW>(p, stream);
    return launch_t<IoT, K, W, NMAX, false, false, STATES, CW>(p, stream);
  }
  return hipErrorInvalidValue;
}

// N_max instances: 4, 8, 16, 32, 64 (coordinates past N run as the identity).
// K = 32 is instantiated up to 16 coordinates only; wider states take K = 16.
template <typename IoT, int K, int STATES, int RESETS>
hipError_t launch_n(const ScanParams& p, hipStream_t stream, int split = 0) {
  if (p.N <= 4) return launch_flags<IoT, K, 4, STATES, RESETS>(p, stream, split);
  if (p.N <= 8) return launch_flags<IoT, K, 8, STATES, RESETS>(p, stream, split);
  if (p.N <= 16) return launch_flags<IoT, K, 16, STATES, RESETS>(p, stream, split);
  if constexpr (K == 16) {
    if (p.N <= 32) return launch_flags<IoT, K, 32, STATES, RESETS>(p, stream);
    return launch_flags<IoT, K, 64, STATES, RESETS>(p, stream);
  } else {
    return launch_n<IoT, 16, STATES, RESETS>(p, stream);
  }
}

}  // namespace
}  // namespace ss


