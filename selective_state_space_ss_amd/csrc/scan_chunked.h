// Prompt / prefill selective scan for gfx950: the chunked kernel (included by
// scan_fwd.hip for the plain scan and by scan_states.hip for the variants that
// also write per-token states).
//
// Work decomposition. A channel row (b, c) is owned by one 16-lane DPP row of
// a wavefront: a wave holds 4 channels of one batch row, a block of W waves
// 4W channels of that batch row. (Launches with few rows give a row 32 or 64
// lanes instead: 2 or 1 channels per wave; RL below.) The sequence is walked
// in chunks of 16*K tokens; inside a chunk lane l of a row owns the K
// consecutive tokens [l*K, (l+1)*K). Per chunk:
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

// SS_LDS_POISON=1 builds the race check of the B/C stage (a debug library,
// libssscan_lds_poison.so): before every fill the whole stage is set to NaN
// between two barriers, so an operand read that the fill's barrier did not
// order after the fill returns NaN, and a write racing a previous reader
// poisons that reader's result. The outputs of a correct kernel are bitwise
// those of the normal build.
#ifndef SS_LDS_POISON
#define SS_LDS_POISON 0
#endif

#ifndef SS_SCAN_L2_PREFETCH
#define SS_SCAN_L2_PREFETCH 1
#endif

namespace ss {
namespace {

// What the kernel writes besides y and h_last (ScanParams::states):
// nothing, the state after every token ([batch, channels, N, L], seq fastest
// like x and y) or the state after token ScanParams::time_step
// ([batch, channels, N]).
enum StatesOut { kNoStates = 0, kAllStates = 1, kOneState = 2 };

constexpr int kRowLanes = 16;
constexpr int kRowsPerWave = 4;

// Launch forms for few rows (launch_flags).
enum Form { kPlain = 0, kRows32w4 = 1, kRows32w8 = 2, kRows64w4 = 3 };

// RL: lanes per row (16, 32 or 64): a wave holds 64 / RL rows, and a chunk
// is RL K tokens.
template <int K, int W, int RL = kRowLanes>
struct Shape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kRows = 64 / RL;    // rows per wave
  static constexpr int kChan = kRows * W;  // channels per block
  static constexpr int kT = RL * K;        // tokens per chunk
};

// Waves per SIMD the register budget is set for (launch bound). K = 16 with
// bf16 I/O and no reset mask fits 4 (<= 128 VGPRs); the reset mask and fp32
// z need more registers and run at 3; K = 32 at 2. Rows of 32 or 64 lanes in
// 4-wave blocks run 3 blocks per CU (LDS), so 3 waves per SIMD.
template <typename IoT, int K, bool RESET, int W = 8, int RL = kRowLanes>
constexpr int min_waves_per_simd() {
  return K == 32 ? 2 : ((RESET || sizeof(IoT) == 4 || (RL > kRowLanes && W == 4)) ? 3 : 4);
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
// RL: lanes per row, 16, or 32 / 64 for launches with few rows (a wave or
// two per SIMD at 16): a row's chunk is then spread over 2 or 4 DPP rows,
// the wave holds 2 rows or 1 and the launch twice or four times the waves;
// the chunk scan takes one or two more steps across DPP rows, and B / C are
// staged 8 or 4 coordinates at a time so that the stage stays 40 KB.
template <typename IoT, int K, int W, int NMAX, bool GATE, bool RESET, int STATES, int CW = 0, int RL = kRowLanes>
__global__ __launch_bounds__(64 * W, (min_waves_per_simd<IoT, K, RESET, W, RL>())) void scan_fwd_kernel(
    const ScanParams p) {
  static_assert(CW == 0 || (K == 16 && STATES == kNoStates), "the fused conv runs at 16 tokens per lane");
  static_assert(RL == kRowLanes || STATES == kNoStates, "long rows: y and h_last only");
  using S = Shape<K, W, RL>;
  constexpr int RPW = S::kRows;
  constexpr int T = S::kT;
  constexpr int KP = K + 4;  // LDS stride of one lane's K values (spreads the banks)
  constexpr int VEC = Io<IoT>::kVec;
  static_assert(K % VEC == 0 && K % 16 == 0, "K must hold whole 16-byte vectors");
  // State coordinates go in groups of NG: a group's B and C are staged in LDS
  // at a time (one group when NMAX <= 16 at 16 lanes per row; LDS holds 16
  // coordinates' worth of 256-token chunks, 8 of 512, 4 of 1024).
  constexpr int NGMAX = 16 * kRowLanes / RL;
  constexpr int NG = NMAX < NGMAX ? NMAX : NGMAX;
  constexpr int kGroups = NMAX / NG;
  static_assert(kGroups * NG == NMAX, "NMAX is a multiple of the group size");
  __shared__ float sB[NG][RL][KP];
  __shared__ float sC[NG][RL][KP];
  __shared__ float sA2[S::kChan * NMAX];     // A[c, n] * log2(e) per row of the block
  // sCarry: the state entering the current chunk, per row; then, 8 dwords
  // on, sZero: what the other lanes of a row read in place of the carry.
  // With N_max >= 16 every row's carry sits a multiple of 16 dwords from the
  // first, so a zero row 8 dwords off that grid never shares a bank with
  // the carries that lane 0 of each row reads in the same instruction.
  __shared__ float sCarryZero[S::kChan * NMAX + 8 + NMAX];
  float* const sCarry = sCarryZero;
  float* const sZero = sCarryZero + S::kChan * NMAX + 8;
  static_assert((S::kChan * NMAX) % 16 == 0, "row carries on a 16-dword grid");
  // kAllStates: one coordinate's states of the chunk per row, each lane's K
  // tokens padded to KP, re-read in token order for coalesced stores
  __shared__ __align__(16) float sSt[STATES == kAllStates ? S::kChan : 1][STATES == kAllStates ? kRowLanes * KP : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = lane / RL;
  const int tl = lane % RL;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.chan_blocks;
  const int64_t c_raw = (blk - b * p.chan_blocks) * S::kChan + wave * RPW + row;
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
  const int slot = (wave * RPW + row) * NMAX;
  for (int n = tl; n < NMAX; n += RL) {
    sA2[slot + n] = n < N ? p.A[c * N + n] * kLog2e : 0.0f;
    sCarry[slot + n] = (n < N && p.h0) ? p.h0[(b * p.channels + c) * N + n] : 0.0f;
  }
  for (int n = tid; n < NMAX; n += S::kThreads) sZero[n] = 0.0f;
  // The carried state enters a chunk at lane 0 of each row; the other lanes
  // read zeros in its place, so the first fold step needs no select. sZero is
  // only ever read after the first chunk's staging barrier.
  const float* __restrict__ carry_src = tl == 0 ? &sCarry[slot] : sZero;
  const bool carry_writer = tl == RL - 1;  // the row's last lane ends the chunk
  const float Dc = p.D ? p.D[c] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[c] : 0.0f;

  const int64_t nchunks = (L + T - 1) / T;
  // K = 32 instances (two waves per SIMD, long sequences) bring the next
  // chunk's B and C into L2 while this chunk is computed: every block of a
  // batch row stages the same chunk at about the same time, so on a cold
  // cache each staging would otherwise wait for HBM with little other work
  // to hide it. Thread i reads one dword of line i of the next chunk's B
  // rows then C rows (128-byte lines, N rows of T tokens each); the value is
  // only folded into `touched` after the following staging barrier, whose
  // own loads are waited for anyway (loads complete in order), so nothing
  // waits on it early. (Measured on MI355X, 4 x 2048 channels x 8192 tokens
  // with a reset mask: 308.8 -> 303.6 us warm, 328.2 -> 317.9 us after a
  // cache flush. The K = 16 instances gained nothing: at the 8 x 5120 x 2048
  // shape the two registers spill, 329 -> 336 us; at 4 x 1536 x 2048 the cold
  // launch was no faster.)
  constexpr bool kTouch = SS_SCAN_L2_PREFETCH != 0 && K == 32;
  constexpr int kLineElems = 128 / (int)sizeof(IoT);
  constexpr int kLinesPerRow = T / kLineElems;
  static_assert(T % kLineElems == 0, "a chunk's row is whole 128-byte lines");
  uint32_t touched = 0, pf_val = 0;
  auto touch_next = [&](int64_t chk) {
    if (!kTouch || !p.vec_ok || (chk + 1) * T > L) return;
    // (the line's place is recomputed from an opaque copy of the thread
    // index: hoisted out of the chunk loop, it holds registers the loop needs)
    int ti = tid;
    asm volatile("" : "+v"(ti));
    const int lines = N * kLinesPerRow;  // per tensor
    if (ti < 2 * lines) {
      const int li = ti < lines ? ti : ti - lines;
      const int n = li / kLinesPerRow;
      const int64_t e = (int64_t)n * L + chk * T + (int64_t)(li - n * kLinesPerRow) * kLineElems;
      const IoT* src = (ti < lines ? static_cast<const IoT*>(p.B) : static_cast<const IoT*>(p.C)) + b * N * L + e;
      pf_val = *reinterpret_cast<const uint32_t*>(src);
    }
  };
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * T;
    const int64_t tb = t0 + tl * K;  // this lane's first token
    const bool full = p.vec_ok && (t0 + T <= L);

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
        if constexpr (CW == 0) load_vec16(xg + tb + v * VEC, xv + v * VEC);
        load_vec16(dg + tb + v * VEC, dv + v * VEC);
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
      if constexpr (SS_LDS_POISON != 0) {
        float* sb = &sB[0][0][0];
        float* sc = &sC[0][0][0];
        for (int i = tid; i < NG * RL * KP; i += S::kThreads) {
          sb[i] = __builtin_nanf("");
          sc[i] = __builtin_nanf("");
        }
        __syncthreads();
      }
      {
        constexpr int kSegPerN = T / VEC;
        constexpr int kSeg = NG * kSegPerN;
        // Segment u of a coordinate's chunk (VEC tokens, one 16-byte load)
        // goes to lane row sl at token sj: the 8 threads of a group of 8
        // take the same piece of 8 consecutive lane rows. Their LDS rows
        // are KP / 4 (odd) 16-byte slots apart, so the group's 16-byte
        // stores fall in 8 different groups of 4 banks (the LDS serves such
        // stores 8 lanes at a time over 32 banks). A wave's load still
        // covers whole coordinate rows of the chunk.
        static_assert((KP / 4) % 2 == 1 && RL % 8 == 0 && kSegPerN % 8 == 0, "conflict-free staging order");
        auto place = [](int u, int& sl, int& sj) {
          constexpr int kRowGroups = RL / 8;
          const int gg = u >> 3;
          sl = 8 * (gg % kRowGroups) + (u & 7);
          sj = (gg / kRowGroups) * VEC;
        };
        for (int s = tid; s < kSeg; s += S::kThreads) {
          const int nl = s / kSegPerN;
          const int n = grp * NG + nl;
          int sl, sj;
          place(s - nl * kSegPerN, sl, sj);
          const int tpos = sl * K + sj;
          float vb[VEC], vc[VEC];
          const int64_t g = (int64_t)n * L + t0 + tpos;
          // (each branch stores its own values: with one shared set the
          // compiler zero-fills it on the common path too)
          if (full && n < N) {
            load_vec16(Bg + g, vb);
            load_vec16(Cg + g, vc);
          } else {
            // (offsets recomputed from an opaque copy of s: hoisted out of
            // the chunk loop for this rare path, they were spilled to scratch)
            int so = s;
            asm volatile("" : "+v"(so));
            const int nlo = so / kSegPerN, no = grp * NG + nlo;
            int slo, sjo;
            place(so - nlo * kSegPerN, slo, sjo);
            const int tpo = slo * K + sjo;
            const int64_t go = (int64_t)no * L + t0 + tpo;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const bool in = no < N && t0 + tpo + e < L;
              vb[e] = in ? Io<IoT>::to_f32(Bg[go + e]) : 0.0f;
              vc[e] = in ? Io<IoT>::to_f32(Cg[go + e]) : 0.0f;
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
    if constexpr (kTouch) {
      touched ^= pf_val;
      touch_next(ch + 1);
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
      yv[j] = Dc * xv[j];
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
#pragma unroll
      for (int nl = 0; nl < NG; ++nl) {
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
        row_scan_and_enter<RL>(Al, Bl, h, av[0]);  // Bl: state after this lane's tokens; h: after its first
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

    // 5. gate and store
    if constexpr (GATE) {
      float zv[K];
      if (full) {
#pragma unroll
        for (int v = 0; v < K / VEC; ++v) load_vec16(zg + tb + v * VEC, zv + v * VEC);
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

  if constexpr (kTouch) {
    if (p.N < 0) p.h_last[0] = (float)(touched ^ pf_val);  // never taken (N >= 1): keeps the touches
  }

  // The row's place is recomputed here from an opaque copy of the thread
  // index: kept live from the prologue across the chunk loop, these values
  // were spilled to scratch.
  if (p.h_last) {
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));
    const int wave_e = tid_e >> 6, lane_e = tid_e & 63, row_e = lane_e / RL, tl_e = lane_e % RL;
    const int64_t ce = (blk - b * p.chan_blocks) * S::kChan + wave_e * RPW + row_e;
    if (ce < p.channels) {
      const int slot_e = (wave_e * RPW + row_e) * NMAX;
      for (int n = tl_e; n < N; n += RL) p.h_last[(b * p.channels + ce) * N + n] = sCarry[slot_e + n];
    }
  }
}

template <typename IoT, int K, int W, int NMAX, bool GATE, bool RESET, int STATES, int CW = 0, int RL = kRowLanes>
hipError_t launch_t(const ScanParams& p0, hipStream_t stream) {
  using S = Shape<K, W, RL>;
  ScanParams p = p0;
  p.chan_blocks = (p.channels + S::kChan - 1) / S::kChan;
  const int64_t blocks = p.batch * p.chan_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  return launch_kernel(reinterpret_cast<const void*>(&scan_fwd_kernel<IoT, K, W, NMAX, GATE, RESET, STATES, CW, RL>),
      dim3((unsigned)blocks), dim3(S::kThreads), args, stream);
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
// form: how a launch with few rows spreads them, for a launch without a
// reset mask at K = 16 and N <= 16 (where the forms are instantiated):
// kPlain, or kRows32w4 / kRows32w8 / kRows64w4: rows of 32 or 64 lanes in
// blocks of 4 or 8 waves. The caller picks it.
template <typename IoT, int K, int NMAX, int STATES, int RESETS, int CW = 0>
hipError_t launch_flags(const ScanParams& p, hipStream_t stream, int form = 0) {
  const bool gate = p.z != nullptr, reset = p.reset != nullptr;
  if constexpr (K == 16 && NMAX <= 16 && STATES == kNoStates && RESETS == 0 && CW == 0) {
#define SS_FORM(CODE, WV, RLN)                                                         \
  if (form == CODE) {                                                                  \
    if (gate) return launch_t<IoT, K, WV, NMAX, true, false, STATES, CW, RLN>(p, stream); \
    return launch_t<IoT, K, WV, NMAX, false, false, STATES, CW, RLN>(p, stream);         \
  }
    SS_FORM(kRows32w4, 4, 32)
    SS_FORM(kRows32w8, 8, 32)
    SS_FORM(kRows64w4, 4, 64)
#undef SS_FORM
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
hipError_t launch_n(const ScanParams& p, hipStream_t stream, int form = 0) {
  if (p.N <= 4) return launch_flags<IoT, K, 4, STATES, RESETS>(p, stream, form);
  if (p.N <= 8) return launch_flags<IoT, K, 8, STATES, RESETS>(p, stream, form);
  if (p.N <= 16) return launch_flags<IoT, K, 16, STATES, RESETS>(p, stream, form);
  if constexpr (K == 16) {
    if (p.N <= 32) return launch_flags<IoT, K, 32, STATES, RESETS>(p, stream);
    return launch_flags<IoT, K, 64, STATES, RESETS>(p, stream);
  } else {
    return launch_n<IoT, 16, STATES, RESETS>(p, stream);
  }
}

}  // namespace
}  // namespace ss


