// Scalar-gated state scan for gfx950 ("Mamba 2 Gated State Scan" problem
// page, statement): per batch item a dk x dv state,
//
//   S_t = gamma_t S_{t-1} + k_t v_t^T,   y_t = q_t^T S_t,
//
// from an initial state (zeros by default), in fp32 with fp32 matrix cores.
// s0 and final_state are fp32 or bf16 (StT); q, k, v and y share IoT.
//
// Chunked form. Over a chunk of T = 16 tokens starting from S_prev, with
// P_t = gamma_0 ... gamma_t (products within the chunk) and
// L[t][s] = gamma_{s+1} ... gamma_t for s <= t (0 above the diagonal):
//
//   y_t   = sum_{s<=t} L[t][s] (q_t . k_s) v_s + P_t q_t^T S_prev
//   S_new = P_15 S_prev + sum_s L[15][s] k_s v_s^T
//
// which is the recurrence unrolled over the chunk (the page's S_t written out
// from S_prev). Every product is a 16 x 16 x 4 fp32 MFMA.
//
// Layout. A block is one batch item and 16 columns of dv, 4 waves; wave w
// owns rows [w R, (w + 1) R) of dk (R = dk padded to 64, over 4) and keeps
// its rows of S in registers in the MFMA accumulator layout. Per chunk the
// block stages q, k (also transposed), v^T and gamma in LDS and builds P and
// L; each wave then computes, over its own rows, the partial
//   A^T = K Q^T,  M = A o L,  Y = M V + diag(P) Q S_prev,
//   S  <- P_15 S + (K o L[15])^T V,
// and the block sums the 4 partial Y (A, hence M and Y, are linear in the
// rows of dk they run over). Operands are read from LDS as float4 runs: in
// the MFMA of step g, lane group G of the wave supplies the contraction index
// 4G + g (any bijection of the contraction index serves, if A and B operands
// use the same one), which also makes the accumulator of A^T, register r at
// lane (t, G), exactly the A operand M[t][4G + r] of the next product.
//
// Rows of dk past dk, columns past dv and tokens past L are staged as zeros
// (gamma as 1): they change nothing and are never stored.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kT = 16;     // tokens per chunk
constexpr int kCols = 16;  // columns of dv per block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTS = kT + 4;  // LDS stride of the [row][token] arrays

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename IoT, typename StT, int RT>
__global__ __launch_bounds__(kThreads) void gated_scan_kernel(const GatedParams p) {
  constexpr int R = 16 * RT;        // dk rows per wave
  constexpr int DKP = kWaves * R;   // dk padded
  constexpr int QS = DKP + 4;       // LDS stride of the [token][dk] and [column][dk] arrays
  __shared__ __align__(16) float sQ[kT][QS];         // q[t][i]
  __shared__ __align__(16) float sK[kT][QS];         // k[s][i]
  __shared__ __align__(16) float sKT[DKP][kTS];      // k[s][i] at [i][s]
  __shared__ __align__(16) float sVT[kCols][kTS];    // v[s][j] at [j][s]
  __shared__ __align__(16) float sL[kT][kTS];        // L[t][s]
  __shared__ float sG[kT];                           // gamma of the chunk's tokens
  __shared__ __align__(16) float sP[kT];             // P[t]
  __shared__ __align__(16) float sST[kCols][QS];     // S_prev[i][j] at [j][i]
  __shared__ __align__(16) float sYT[kWaves][kCols][kTS];  // partial y[t][j] at [w][j][t]

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int G = l >> 4;   // lane group: the MFMA's contraction slot
  const int c16 = l & 15;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / p.col_blocks;
  const int64_t j0 = (blk - b * p.col_blocks) * kCols;
  const int64_t L = p.L;
  const int dk = p.dk;
  const int64_t dv = p.dv;
  const int i0w = w * R;  // this wave's first row of dk
  const IoT* __restrict__ qg = static_cast<const IoT*>(p.q) + b * L * dk;
  const IoT* __restrict__ kg = static_cast<const IoT*>(p.k) + b * L * dk;
  const IoT* __restrict__ vg = static_cast<const IoT*>(p.v) + b * L * dv;
  const float* __restrict__ gg = p.gamma + b * L;

  // This wave's rows of the state: S[rt][r] = S[i0w + 16 rt + 4 G + r][j0 + c16].
  v4f S[RT];
  const int64_t jg = j0 + c16;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0w + 16 * rt + 4 * G + r;
      S[rt][r] = (p.s0 && i < dk && jg < dv) ? Io<StT>::to_f32(static_cast<const StT*>(p.s0)[(b * dk + i) * dv + jg])
                                             : 0.0f;
    }
  auto publish_state = [&]() {  // S -> sST (this wave's rows only)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      *reinterpret_cast<v4f*>(&sST[c16][i0w + 16 * rt + 4 * G]) = S[rt];
  };
  publish_state();

  const int64_t nchunks = (L + kT - 1) / kT;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * kT;

    // 1. stage the chunk (the previous chunk's readers are done first)
    __syncthreads();
    for (int e = tid; e < kT * DKP; e += kThreads) {
      const int t = e / DKP, i = e - t * DKP;
      const int64_t tt = t0 + t;
      const bool in = tt < L && i < dk;
      const float qv = in ? Io<IoT>::to_f32(qg[tt * dk + i]) : 0.0f;
      const float kv = in ? Io<IoT>::to_f32(kg[tt * dk + i]) : 0.0f;
      sQ[t][i] = qv;
      sK[t][i] = kv;
      sKT[i][t] = kv;
    }
    {
      const int t = tid / kCols, j = tid - t * kCols;  // kThreads == kT * kCols
      const int64_t tt = t0 + t;
      sVT[j][t] = (tt < L && j0 + j < dv) ? Io<IoT>::to_f32(vg[tt * dv + j0 + j]) : 0.0f;
      if (tid < kT) sG[tid] = t0 + tid < L ? gg[t0 + tid] : 1.0f;
    }
    __syncthreads();
    {
      // L[t][s] = gamma_{s+1} ... gamma_t (s <= t), P[t] = gamma_0 L[t][0]
      const int t = tid / kT, s = tid - t * kT;
      float prod = 1.0f;
      for (int i = s + 1; i <= t; ++i) prod *= sG[i];
      sL[t][s] = s <= t ? prod : 0.0f;
      if (s == 0) sP[t] = sG[0] * prod;
    }
    __syncthreads();

    // 2. A^T[s][t] = sum over this wave's rows i of k[s][i] q[t][i]
    v4f At = {0.0f, 0.0f, 0.0f, 0.0f};
    v4f qa[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int i = i0w + 16 * rt + 4 * G;
      const v4f ka = *reinterpret_cast<const v4f*>(&sK[c16][i]);
      qa[rt] = *reinterpret_cast<const v4f*>(&sQ[c16][i]);
#pragma unroll
      for (int g = 0; g < 4; ++g) At = mfma4(ka[g], qa[rt][g], At);
    }
    // 3. M^T[s][t] = A^T[s][t] L[t][s]; register r holds s = 4G + r, t = c16
    const v4f lt = *reinterpret_cast<const v4f*>(&sL[c16][4 * G]);
    const v4f mt = At * lt;
    // 4. Y[t][j] = sum_s M[t][s] v[s][j]  (contraction slot of step g: s = 4G + g)
    const v4f vb = *reinterpret_cast<const v4f*>(&sVT[c16][4 * G]);
    v4f Y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 4; ++g) Y = mfma4(mt[g], vb[g], Y);
    // 5. Y[t][j] += P[t] sum over this wave's rows i of q[t][i] S_prev[i][j]
    v4f Z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const v4f sa = *reinterpret_cast<const v4f*>(&sST[c16][i0w + 16 * rt + 4 * G]);
#pragma unroll
      for (int g = 0; g < 4; ++g) Z = mfma4(qa[rt][g], sa[g], Z);
    }
    const v4f pt = *reinterpret_cast<const v4f*>(&sP[4 * G]);
    Y += pt * Z;
    // 6. S <- P_15 S + sum_s (k[s][i] L[15][s]) v[s][j]
    const float p15 = sP[kT - 1];
    const v4f l15 = *reinterpret_cast<const v4f*>(&sL[kT - 1][4 * G]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const v4f kt = *reinterpret_cast<const v4f*>(&sKT[i0w + 16 * rt + c16][4 * G]) * l15;
      S[rt] *= p15;
#pragma unroll
      for (int g = 0; g < 4; ++g) S[rt] = mfma4(kt[g], vb[g], S[rt]);
    }
    publish_state();
    // 7. this wave's partial y
    *reinterpret_cast<v4f*>(&sYT[w][c16][4 * G]) = Y;
    __syncthreads();

    // 8. sum the partials and store y (16 threads per token: contiguous columns)
    {
      const int t = tid / kCols, j = tid - t * kCols;
      const int64_t tt = t0 + t;
      float acc = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) acc += sYT[ww][j][t];
      if (tt < L && j0 + j < dv) static_cast<IoT*>(p.y)[(b * L + tt) * dv + j0 + j] = Io<IoT>::from_f32(acc);
    }
  }

  if (p.final_state && jg < dv) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0w + 16 * rt + 4 * G + r;
        if (i < dk) static_cast<StT*>(p.final_state)[(b * dk + i) * dv + jg] = Io<StT>::from_f32(S[rt][r]);
      }
  }
}

template <typename IoT, typename StT, int RT>
hipError_t launch_rt(const GatedParams& p0, hipStream_t stream) {
  GatedParams p = p0;
  p.col_blocks = (p.dv + kCols - 1) / kCols;
  const int64_t blocks = p.batch * p.col_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gated_scan_kernel<IoT, StT, RT>), dim3((unsigned)blocks),
                         dim3(kThreads), args, 0, stream);
}

template <typename IoT, typename StT>
hipError_t launch_io(const GatedParams& p, hipStream_t stream) {
  if (p.dk <= 64) return launch_rt<IoT, StT, 1>(p, stream);
  if (p.dk <= 128) return launch_rt<IoT, StT, 2>(p, stream);
  if (p.dk <= 192) return launch_rt<IoT, StT, 3>(p, stream);
  return launch_rt<IoT, StT, 4>(p, stream);
}

}  // namespace

hipError_t launch_gated_scan(const GatedParams& p, bool io_bf16, bool state_bf16, hipStream_t stream) {
  if (io_bf16) return state_bf16 ? launch_io<bf16_t, bf16_t>(p, stream) : launch_io<bf16_t, float>(p, stream);
  return state_bf16 ? launch_io<float, bf16_t>(p, stream) : launch_io<float, float>(p, stream);
}

int64_t gated_scan_blocks(int64_t batch, int64_t dv) { return batch * ((dv + kCols - 1) / kCols); }

}  // namespace ss
