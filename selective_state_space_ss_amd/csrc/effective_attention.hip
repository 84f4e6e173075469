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
// Two kernels. The summed matrix with N <= 16 and L <= 512 takes the tiled
// form further below: the tiles left of the diagonal as fp32 matrix-core
// contractions of prefix, gap and suffix products of the decay factors. The
// per-coordinate matrix, and larger N or L, take the column walk described
// here. Both are bound by writing M, and M's stores carry the nontemporal
// hint (M is written once and never read back).
//
// Column walk. Every (i, j) element of the lower triangle needs the N
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

#include <type_traits>

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
        if (n < N) stream_store(term[n], q);
        q += plane;
      }
    } else {
      stream_store(m, q);
    }
  };
  auto store_zero = [&](int64_t i) {
    float* q = Mo + i * L + j;
    if constexpr (PER_STATE) {
#pragma unroll
      for (int n = 0; n < NMAX; ++n) {
        if (n < N) stream_store(0.0f, q);
        q += plane;
      }
    } else {
      stream_store(0.0f, q);
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

// ---- Summed over up to 16 coordinates, L <= 512: the tiles below the
// diagonal on the matrix cores.
//
// For a 16 x 16 tile with rows i0 .. i0 + 15 and columns j0 .. j0 + 15 left
// of the row tile (j0 + 16 <= i0), the decay from column j to row i splits at
// the tiles' edges into three products of factors exp(A dt) <= 1:
//
//   prod_{k=j+1}^{i} a_k = Rj[j] * g * Ri[i],
//   Rj[j] = prod_{k=j+1}^{j0+15} a_k,  g = prod_{k=j0+16}^{i0} a_k,  Ri[i] = prod_{k=i0+1}^{i} a_k,
//
// per coordinate n, so the tile is the contraction over n of
// C'[i][n] = C[b, n, i] Ri[i][n] with B'[j][n] g[n], B'[j][n] = B[b, n, j] (dt_j) Rj[j][n]:
// four 16 x 16 x 4 fp32 MFMAs. Every factor is a product of the same
// exp(A dt) the column walk multiplies, grouped differently, and none can
// overflow.
//
// A block is one (b, c), 8 waves. First the block makes B' and each column
// tile's full product T for the whole sequence, in LDS (one exp per column
// and coordinate; suffix products by 16-lane DPP scans). Then each wave
// takes row tiles w and 15 - w of every 16 (equal work): it makes C' (prefix
// products by a DPP scan) and g = a of its first row, walks its diagonal
// tile (lane (l, G) holds column i0 + l's products for coordinates 4 s + G,
// the row's factors reach it as DPP broadcasts from lane (ii, G), and the
// four lane groups' partial sums are added by two cross-lane permutes), then
// runs its column tiles from right to left (g extended by each finished
// tile's T), gathering four tiles' output in LDS so that rows leave in 256-byte
// pieces, and stores zeros right of its diagonal tile.
constexpr int kMT = 16;      // tile edge
constexpr int kTW = 8;       // waves per block
typedef float v4f __attribute__((ext_vector_type(4)));

// f(integral_constant<int, R>) for R = B .. E - 1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// Lane R of the caller's 16-lane DPP row, to every lane of the row.
template <int R>
__device__ __forceinline__ float row_bcast(float v) {
  return dpp_or<kDppRowNewBcast0 + R>(v, v);
}

__device__ __forceinline__ float lane_xor(float v, int lane, int m) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, v)));
}

template <typename IoT, int LMAX>
__global__ __launch_bounds__(64 * kTW) __attribute__((amdgpu_waves_per_eu(4))) void
effective_attention_tiles_kernel(const AttnParams p) {
  __shared__ __align__(16) float sBp[LMAX][16];           // B'[j][G 4 + s], coordinate 4 s + G
  __shared__ __align__(16) float sT[LMAX / kMT][16];      // each column tile's T, same order
  __shared__ __align__(16) float sO[kTW][kMT][64 + 4];    // a wave's 16 x 64 output block
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, G = lane >> 4;
  const int64_t L = p.L;
  const int N = p.N;
  const int64_t ntiles = (L + kMT - 1) / kMT;
  const int64_t bc = blockIdx.x;
  const int64_t b = bc / p.channels;
  const int64_t c = bc - b * p.channels;
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
  float* __restrict__ Mb = p.M + bc * L * L;
  const bool incl = p.include_dt != 0;

  float A2[4];  // coordinates n = 4 s + G of this lane
#pragma unroll
  for (int s = 0; s < 4; ++s) A2[s] = 4 * s + G < N ? Ac[4 * s + G] * kLog2e : 0.0f;

  // B' and T of every column tile (lane (r16, G): column q 16 + r16)
  for (int64_t q = w; q < ntiles; q += kTW) {
    const int64_t jc = q * kMT + r16;
    const bool in = jc < L;
    const float dtc = in ? step_size(jc) : 0.0f;
    float bp[4], T[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int n = 4 * s + G;
      const bool on = in && n < N;
      const float a = on ? fast_exp2(A2[s] * dtc) : 1.0f;
      float x = a;  // suffix products: prod_{k=j}^{j0+15} a_k
      x *= dpp_or<kDppRowShl1>(1.0f, x);
      x *= dpp_or<kDppRowShl1 + 1>(1.0f, x);
      x *= dpp_or<kDppRowShl1 + 3>(1.0f, x);
      x *= dpp_or<kDppRowShl1 + 7>(1.0f, x);
      T[s] = row_bcast<0>(x);
      const float rj = dpp_or<kDppRowShl1>(1.0f, x);  // prod_{k=j+1}^{j0+15} a_k
      const float bv = on ? Io<IoT>::to_f32(Bg[n * L + jc]) : 0.0f;
      bp[s] = bv * (incl ? dtc : 1.0f) * rj;
    }
    *reinterpret_cast<float4*>(&sBp[q * kMT + r16][4 * G]) = make_float4(bp[0], bp[1], bp[2], bp[3]);
    if (r16 == 0) *reinterpret_cast<float4*>(&sT[q][4 * G]) = make_float4(T[0], T[1], T[2], T[3]);
  }
  __syncthreads();

  auto row_tile = [&](int64_t pt) {
    const int64_t i0 = pt * kMT;
    const int64_t ir = i0 + r16;
    const bool row_in = ir < L;
    const float dtr = row_in ? step_size(ir) : 0.0f;
    float ar[4], cr[4], cp[4], g[4], d[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int n = 4 * s + G;
      const bool on = row_in && n < N;
      ar[s] = on ? fast_exp2(A2[s] * dtr) : 1.0f;
      cr[s] = on ? Io<IoT>::to_f32(Cg[n * L + ir]) : 0.0f;
      float x = r16 == 0 ? 1.0f : ar[s];  // prefix products: prod_{k=i0+1}^{i} a_k
      x *= dpp_or<kDppRowShr1>(1.0f, x);
      x *= dpp_or<kDppRowShr1 + 1>(1.0f, x);
      x *= dpp_or<kDppRowShr1 + 3>(1.0f, x);
      x *= dpp_or<kDppRowShr1 + 7>(1.0f, x);
      cp[s] = cr[s] * x;
      g[s] = row_bcast<0>(ar[s]);  // the adjacent column tile's gap: a of row i0
      // the diagonal walk's column i0 + r16 (the same index as the row)
      d[s] = on ? Io<IoT>::to_f32(Bg[n * L + ir]) * (incl ? dtr : 1.0f) : 0.0f;
    }

    // the diagonal tile: row i0 + ii against column i0 + r16
    float m[kMT];
    static_for<0, kMT>([&](auto IIC) {
      constexpr int ii = decltype(IIC)::value;
      const bool extend = ii > r16;
      float part = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float a = row_bcast<ii>(ar[s]), cv = row_bcast<ii>(cr[s]);
        asm volatile("" : "+v"(a), "+v"(cv));  // taken with the whole wave active
        d[s] *= extend ? a : 1.0f;
        part = __builtin_fmaf(cv, d[s], part);
      }
      m[ii] = part;
    });
#pragma unroll
    for (int ii = 0; ii < kMT; ++ii) {
      m[ii] += lane_xor(m[ii], lane, 16);
      m[ii] += lane_xor(m[ii], lane, 32);
    }
#pragma unroll
    for (int ii = 0; ii < kMT; ++ii) {  // every lane holds every sum; lane group ii mod 4 stores row ii
      if ((ii & 3) == G && i0 + ii < L && row_in) stream_store(ii >= r16 ? m[ii] : 0.0f, &Mb[(i0 + ii) * L + ir]);
    }

    // the column tiles left of the diagonal, right to left, in blocks of four
    // tiles (64 columns) gathered in this wave's LDS slot
    for (int64_t q = pt - 1; q >= 0; --q) {
      const float4 b4 = *reinterpret_cast<const float4*>(&sBp[q * kMT + r16][4 * G]);
      const float4 t4 = *reinterpret_cast<const float4*>(&sT[q][4 * G]);
      const float bq[4] = {b4.x, b4.y, b4.z, b4.w}, tq[4] = {t4.x, t4.y, t4.z, t4.w};
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cp[s], bq[s] * g[s], acc, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) g[s] *= tq[s];
      // register r at lane (r16, G): row 4 G + r, column 16 (q mod 4) + r16 of the block
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[w][4 * G + r][16 * (q & 3) + r16] = acc[r];
      if ((q & 3) == 0) {
        // the block's columns q 16 .. min(q 16 + 64, i0) - 1, rows in 16-byte pieces
        const int ncols = static_cast<int>((i0 - q * kMT) < 64 ? (i0 - q * kMT) : 64);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int e = lane + 64 * v;
          const int rr = e >> 4, cc = (e & 15) * 4;
          if (cc < ncols && i0 + rr < L) {
            const float4 o = *reinterpret_cast<const float4*>(&sO[w][rr][cc]);
            float* dst = Mb + (i0 + rr) * L + q * kMT + cc;
            if (p.out_vec) {
              stream_store16(o, dst);
            } else {
              stream_store(o.x, dst); stream_store(o.y, dst + 1); stream_store(o.z, dst + 2); stream_store(o.w, dst + 3);
            }
          }
        }
      }
    }

    // zeros right of the diagonal tile
    const int rows = static_cast<int>(L - i0 < kMT ? L - i0 : kMT);
    const int64_t z0 = i0 + kMT;
    for (int rr = 0; rr < rows; ++rr) {
      float* row = Mb + (i0 + rr) * L;
      if (p.out_vec) {
        for (int64_t jz = z0 + 4 * lane; jz < L; jz += 256)
          stream_store16(make_float4(0.0f, 0.0f, 0.0f, 0.0f), row + jz);
      } else {
        for (int64_t jz = z0 + lane; jz < L; jz += 64) stream_store(0.0f, row + jz);
      }
    }
  };

  // row tiles w and 15 - w of every 16
  for (int64_t k0 = 0; k0 < ntiles; k0 += kMT) {
    if (k0 + w < ntiles) row_tile(k0 + w);
    if (k0 + kMT - 1 - w < ntiles) row_tile(k0 + kMT - 1 - w);
  }
}

template <typename IoT>
hipError_t launch_tiles(AttnParams p, hipStream_t stream) {
  const int64_t blocks = p.batch * p.channels;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  p.out_vec = (p.L % 4 == 0) && reinterpret_cast<uintptr_t>(p.M) % 16 == 0;
  void* args[] = {&p};
  const void* fn = p.L <= 256 ? reinterpret_cast<const void*>(&effective_attention_tiles_kernel<IoT, 256>)
                              : reinterpret_cast<const void*>(&effective_attention_tiles_kernel<IoT, 512>);
  return launch_kernel(fn, dim3((unsigned)blocks), dim3(64 * kTW), args, stream);
}

template <typename IoT, bool PER_STATE>
hipError_t launch_ps(const AttnParams& p0, hipStream_t stream) {
  AttnParams p = p0;
  p.jblocks = (p.L + kCols - 1) / kCols;
  void* args[] = {&p};
  if (!PER_STATE && p.N <= 16 && p.L <= 512) return launch_tiles<IoT>(p, stream);
  const int64_t blocks = p.batch * p.channels * p.jblocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const void* fn;
  if (p.N <= 4) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 4, PER_STATE>);
  else if (p.N <= 8) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 8, PER_STATE>);
  else if (p.N <= 16) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 16, PER_STATE>);
  else if (p.N <= 32) fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 32, PER_STATE>);
  else fn = reinterpret_cast<const void*>(&effective_attention_kernel<IoT, 64, PER_STATE>);
  return launch_kernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, stream);
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
  // the column-walk form's grid (the tiled form's, batch x channels, is smaller)
  return batch * channels * ((L + kCols - 1) / kCols);
}

}  // namespace ss
