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
// from S_prev). With fp32 I/O every product is a 16 x 16 x 4 fp32 MFMA; with
// bf16 I/O the products run on the bf16 matrix cores with fp32 accumulation,
// the fp32 operands split exactly into three bf16 terms (chunk_bf16 below).
//
// Layout. A block is one batch item and 64 columns of dv, 4 waves of 16
// columns each; a wave keeps all dk rows of its columns of S in registers, in
// the MFMA accumulator layout: register r of tile rt at lane (c, G) (c = lane
// mod 16, G = lane / 16) is S[16 rt + 4 G + r][column c]. That is also the B
// operand of q^T S_prev when the contraction slot of step g is row
// 16 rt + 4 G + g, so the state never leaves registers. Each wave forms the
// 16 x 16 token-token product q k^T over all of dk itself (no exchange
// between waves).
//
// Staging. The block stages a chunk in LDS, double buffered with one barrier
// per chunk: q and k row-major (operands of q k^T and q S), v, plus L and P.
// The operands that contract over tokens need 4 consecutive tokens of one
// column of k or v per lane: with bf16 I/O they are read from the row-major
// tiles with the transposing LDS load (ld_col4); with fp32 I/O k and v are
// also staged in 4-token groups [t / 4][row][t % 4]. The next
// chunk's q, k, v are loaded into registers with 16-byte loads, and its gamma
// one token per lane, while the current chunk is computed (no scalar loads in
// the loop: they would share the LDS wait counter). Inputs whose rows are not
// whole 16-byte vectors take a slower element-wise path.
//
// Rows of dk past dk, columns past dv and tokens past L are staged as zeros
// (gamma as 1): they change nothing and are never stored. A chunk's y goes to
// LDS and is stored, as whole 16-byte row segments when rows allow, after the
// next chunk's barrier.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kT = 16;     // tokens per chunk
constexpr int kWaves = 4;
constexpr int kCols = 16 * kWaves;  // columns of dv per block
constexpr int kThreads = 64 * kWaves;
constexpr int kLS = kT + 4;  // LDS stride of L[t][s]

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive staged fp32 elements (the fp32 path).
__device__ __forceinline__ v4f ld4(const float* p) { return *reinterpret_cast<const v4f*>(p); }

template <typename E>
__device__ __forceinline__ E zero_elem() {
  if constexpr (sizeof(E) == 2) return bf16_t{0};
  else return 0.0f;
}

// Element e of a 16-byte vector of E held as raw words. The element is
// copied to a scalar before any bit cast: hipcc's __builtin_bit_cast of a
// vector-element lvalue reads element 0 whatever the index.
template <typename E>
__device__ __forceinline__ E elem(const u32x4 v, int e) {
  if constexpr (sizeof(E) == 2) {
    const uint32_t w = v[e >> 1];
    return bf16_t{static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu))};
  } else {
    const uint32_t w = v[e];
    return __builtin_bit_cast(float, w);
  }
}


// ---- bf16 I/O: products on the bf16 matrix cores
//
// q, k and v are exact bf16 values, so their products are exact in fp32 and
// the bf16 MFMAs (fp32 accumulation) compute q k^T as exactly as the fp32
// ones. The operands that are fp32 (the state for q S, the weighted M for
// M v, and L[15] v for the state update) are split into three bf16 terms by
// truncation: hi keeps the top 8 significant bits, mid the next 8 of the
// exact remainder, lo the rest (at most 8 bits, so exact), and
// hi + mid + lo is the fp32 value exactly; each term's products with a bf16
// operand are exact, so the split adds no rounding of its own.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct Split4 {
  u32x2 hi, mid, lo;  // four bf16 values each, two per dword (element 0 low)
};

// The high halves of two words as one word (a's in the low half): one
// v_perm_b32, so the low halves need not be cleared first.
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ Split4 split4(const v4f x) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xe = x[e];
    const uint32_t hb = __builtin_bit_cast(uint32_t, xe) & 0xffff0000u;
    const float r = xe - __builtin_bit_cast(float, hb);
    const uint32_t mb = __builtin_bit_cast(uint32_t, r) & 0xffff0000u;
    // r has at most 16 significant bits and mid holds its top 8, so the rest
    // has at most 8: a bf16 value as it stands (its low half is zero)
    const float r2 = r - __builtin_bit_cast(float, mb);
    h[e] = hb;
    m[e] = mb;
    l[e] = __builtin_bit_cast(uint32_t, r2);
  }
  Split4 o;
  o.hi = u32x2{pack_hi(h[0], h[1]), pack_hi(h[2], h[3])};
  o.mid = u32x2{pack_hi(m[0], m[1]), pack_hi(m[2], m[3])};
  o.lo = u32x2{pack_hi(l[0], l[1]), pack_hi(l[2], l[3])};
  return o;
}

__device__ __forceinline__ v4f mfma16(const u32x2 a, const u32x2 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), c, 0, 0,
                                                   0);
}
__device__ __forceinline__ v4f mfma32(const u32x4 a, const u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}
__device__ __forceinline__ u32x2 ld2w(const bf16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// Four rows of one column of a row-major bf16 tile, through the gfx950
// transposing LDS read: in each 16-lane group, lane 4 r + q names 4
// consecutive elements (q-th group of 4 columns) of the group's row r, and
// lane c receives column c of those 4 x 16 elements, rows 0..3 (element 0 in
// the low half of the first dword). The caller passes, for lane c16, the
// address of element 4 (c16 mod 4) of row c16 / 4.
__device__ __forceinline__ u32x2 ld_col4(const bf16_t* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4* lds_s4;
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(p));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x4 cat(const u32x2 a, const u32x2 b) { return u32x4{a.x, a.y, b.x, b.y}; }

template <typename E, int RT>
struct Stage;

// One chunk of one wave with bf16 I/O (see the chunked form above): returns
// the wave's 16 columns of y for the chunk's 16 tokens (register r at lane
// (column, G) is token 4 G + r) and updates S in place. In every MFMA, the A
// and B operands of lane group G carry the same contraction indices in the
// same element order, which is all the product needs.
template <typename St, int RT>
__device__ __forceinline__ v4f chunk_bf16(const St& s, v4f (&S)[RT], int w, int G, int c16) {
  // the lane's swizzled offsets within its rows of q and k (St::sw): the
  // pieces' bit is below the multiples of 16 and 32 added to them
  const int o8 = St::sw(c16, 8 * G), o4 = St::sw(c16, 4 * G);
  const int oc = St::sw(4 * G + (c16 >> 2), 4 * (c16 & 3));
  // A^T[s][t] = k_s . q_t over dk: 32 indices per MFMA, 16 for an odd tile
  v4f At = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ch = 0; ch < RT / 2; ++ch) {
    const u32x4 ka = *reinterpret_cast<const u32x4*>(&s.k[c16][32 * ch + o8]);
    const u32x4 qa = *reinterpret_cast<const u32x4*>(&s.q[c16][32 * ch + o8]);
    At = mfma32(ka, qa, At);
  }
  if constexpr (RT % 2 == 1) {
    const int i = 16 * (RT - 1) + o4;
    At = mfma16(ld2w(&s.k[c16][i]), ld2w(&s.q[c16][i]), At);
  }
  // Y = (A o L) V: M[t][4 G + r] in register r is the A operand of token
  // slots 4 G .. 4 G + 3; v of those tokens for this column from the grouped v
  const v4f mt = At * *reinterpret_cast<const v4f*>(&s.L[c16][4 * G]);
  // v of tokens 4 G .. 4 G + 3 for this lane's column (the B operand)
  const u32x2 vraw = ld_col4(&s.v[4 * G + (c16 >> 2)][16 * w + 4 * (c16 & 3)]);
  const Split4 ms = split4(mt);
  v4f Y = {0.0f, 0.0f, 0.0f, 0.0f};
  Y = mfma16(ms.hi, vraw, Y);
  Y = mfma16(ms.mid, vraw, Y);
  Y = mfma16(ms.lo, vraw, Y);
  // Z = Q S_prev: rows 16 rt + 4 G + r of S are the B operand of index slots
  // 4 G + r of tile rt; two tiles per 32-index MFMA
  v4f Z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int pr = 0; pr < RT / 2; ++pr) {
    const u32x4 qa = cat(ld2w(&s.q[c16][32 * pr + o4]), ld2w(&s.q[c16][32 * pr + 16 + o4]));
    const Split4 s0 = split4(S[2 * pr]), s1 = split4(S[2 * pr + 1]);
    Z = mfma32(qa, cat(s0.hi, s1.hi), Z);
    Z = mfma32(qa, cat(s0.mid, s1.mid), Z);
    Z = mfma32(qa, cat(s0.lo, s1.lo), Z);
  }
  if constexpr (RT % 2 == 1) {
    const u32x2 qa = ld2w(&s.q[c16][16 * (RT - 1) + o4]);
    const Split4 sl = split4(S[RT - 1]);
    Z = mfma16(qa, sl.hi, Z);
    Z = mfma16(qa, sl.mid, Z);
    Z = mfma16(qa, sl.lo, Z);
  }
  Y += *reinterpret_cast<const v4f*>(&s.P[4 * G]) * Z;
  // S <- P_15 S + K^T (L[15] o V): the weighted v of token slots 4 G .. 4 G + 3
  // (the same for every row tile), k of those tokens for row 16 rt + c16
  const v4f wv = v4f{__builtin_bit_cast(float, vraw.x << 16), __builtin_bit_cast(float, vraw.x & 0xffff0000u),
                     __builtin_bit_cast(float, vraw.y << 16), __builtin_bit_cast(float, vraw.y & 0xffff0000u)} *
                 *reinterpret_cast<const v4f*>(&s.L[kT - 1][4 * G]);
  const Split4 ws = split4(wv);
  const float p15 = s.P[kT - 1];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // k of tokens 4 G .. 4 G + 3 for row 16 rt + c16 (the A operand)
    const u32x2 kt = ld_col4(&s.k[4 * G + (c16 >> 2)][16 * rt + oc]);
    S[rt] *= p15;
    S[rt] = mfma16(kt, ws.hi, S[rt]);
    S[rt] = mfma16(kt, ws.mid, S[rt]);
    S[rt] = mfma16(kt, ws.lo, S[rt]);
  }
  return Y;
}

template <typename E, int RT>
struct Stage {
  static constexpr int DKP = 16 * RT;                     // dk padded
  static constexpr int QS = DKP + 32 / (int)sizeof(E);    // row stride of q, k
  static constexpr int KGS = 4 * DKP + 64;                // group stride of the grouped k
  static constexpr int VGS = 4 * kCols + 64;              // group stride of the grouped v
  static constexpr bool kGrouped = sizeof(E) == 4;      // fp32: token-grouped copies of k and v
  static constexpr int VS = kCols + 16 / (int)sizeof(E);  // row stride of the row-major v (bf16)
  // Element e of row t of q or k sits at sw(t, e): rows 8..15 swap the
  // 16-byte pieces of each pair. A row of q or k is twice an odd number of
  // 16-byte slots long (mod the 16 slots that span the 64 banks; for bf16
  // when dk is a multiple of 32), so rows 0..7 of one piece land in 8
  // different even slot groups, and with the swap rows 8..15 in the 8 odd
  // ones: the 16 lanes of a quarter wave reading one piece of 16 rows hit 16
  // different groups of 4 banks (without the swap, rows r and r + 8 share).
  static constexpr int PE = 16 / (int)sizeof(E);  // elements per 16-byte piece
  static __device__ __forceinline__ int sw(int t, int e) { return e ^ (((t >> 3) & 1) * PE); }
  static_assert(DKP % (2 * PE) == 0, "pieces swapped in pairs");
  E q[kT][QS];
  E k[kT][QS];
  E kg[kGrouped ? 4 * KGS : 1];  // fp32: k[t][i] at [t / 4][i][t % 4]
  E vg[kGrouped ? 4 * VGS : 1];  // fp32: v[t][j] at [t / 4][j][t % 4]
  alignas(16) E v[kGrouped ? 1 : kT][VS];  // bf16: v row-major (read by columns with the transposing load)
  float L[kT][kLS];
  float P[kT];
  E y[kT][kCols + 16 / sizeof(E)];  // the chunk's y, stored one chunk later as whole rows
};

template <typename IoT, typename StT, int RT, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RT <= 8 ? 3 : 1))) void gated_scan_kernel(
    const GatedParams p) {
  using St = Stage<IoT, RT>;
  constexpr int DKP = St::DKP;
  constexpr int VEC_E = 16 / sizeof(IoT);            // elements per 16-byte vector
  constexpr int QV = kT * DKP / VEC_E;               // vectors per chunk of q (and of k)
  constexpr int NQV = (QV + kThreads - 1) / kThreads;
  constexpr int VV = kT * kCols / VEC_E;             // vectors per chunk of v
  static_assert(VV <= kThreads, "one v vector per thread");
  static_assert(DKP % VEC_E == 0, "whole vectors per staged row");
  __shared__ __align__(16) St stage[2];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int G = l >> 4;
  const int c16 = l & 15;
  const int64_t col_blocks = p.col_blocks;
  const int64_t b = blockIdx.x / col_blocks;
  const int64_t jb = (blockIdx.x - b * col_blocks) * kCols;  // block's first column
  const int64_t L = p.L;
  const int dk = p.dk;
  const int64_t dv = p.dv;
  const IoT* __restrict__ qg = static_cast<const IoT*>(p.q) + b * L * dk;
  const IoT* __restrict__ kgp = static_cast<const IoT*>(p.k) + b * L * dk;
  const IoT* __restrict__ vgp = static_cast<const IoT*>(p.v) + b * L * dv;
  const float* __restrict__ gg = p.gamma + b * L;
  const int64_t jw = jb + 16 * w;       // this wave's first column
  const int64_t jc = jw + c16;          // this lane's column
  const bool wave_live = jw < dv;

  v4f S[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * rt + 4 * G + r;
      S[rt][r] = (p.s0 && i < dk && jc < dv)
                     ? Io<StT>::to_f32(static_cast<const StT*>(p.s0)[(b * dk + i) * dv + jc])
                     : 0.0f;
    }

  // ---- the next chunk, in registers (q, k, v: vector path only)
  u32x4 qr[NQV], kr[NQV], vr;
  float gam;
  auto prefetch = [&](int64_t t0) {
    if constexpr (VEC) {
#pragma unroll
      for (int n = 0; n < NQV; ++n) {
        const int e = tid + n * kThreads;
        const int t = e / (DKP / VEC_E);
        const int i = (e - t * (DKP / VEC_E)) * VEC_E;
        const bool in = e < QV && t0 + t < L && i < dk;
        // a block-uniform base and a small lane offset (no per-lane 64-bit
        // addresses to keep live across the loop)
        const int off = t * dk + i;
        qr[n] = in ? *reinterpret_cast<const u32x4*>(qg + t0 * dk + off) : u32x4{0, 0, 0, 0};
        kr[n] = in ? *reinterpret_cast<const u32x4*>(kgp + t0 * dk + off) : u32x4{0, 0, 0, 0};
      }
      {
        const int t = tid / (kCols / VEC_E);
        const int j = (tid - t * (kCols / VEC_E)) * VEC_E;
        const bool in = tid < VV && t0 + t < L && jb + j < dv;
        vr = in ? *reinterpret_cast<const u32x4*>(vgp + (t0 * dv + jb) + (static_cast<int64_t>(t) * dv + j))
                : u32x4{0, 0, 0, 0};
      }
    }
    // gamma of token t0 + (tid mod 16), 1 past L
    gam = t0 + (tid & 15) < L ? gg[t0 + (tid & 15)] : 1.0f;
  };

  // y of the chunk starting at t0, from s.y: 16 rows of 64 columns, whole
  // 16-byte row segments when rows allow
  IoT* __restrict__ yg = static_cast<IoT*>(p.y) + b * L * dv;
  auto store_y = [&](const St& s, int64_t t0) {
    IoT* yt = yg + t0 * dv + jb;  // block-uniform
    if constexpr (VEC) {
      constexpr int RV = kCols / VEC_E;  // vectors per row
      for (int e = tid; e < kT * RV; e += kThreads) {
        const int t = e / RV, j = (e - t * RV) * VEC_E;
        if (t0 + t < L && jb + j < dv)
          *reinterpret_cast<u32x4*>(yt + static_cast<int64_t>(t) * dv + j) =
              *reinterpret_cast<const u32x4*>(&s.y[t][j]);
      }
    } else {
      for (int e = tid; e < kT * kCols; e += kThreads) {
        const int t = e / kCols, j = e - t * kCols;
        if (t0 + t < L && jb + j < dv) yt[static_cast<int64_t>(t) * dv + j] = s.y[t][j];
      }
    }
  };

  auto write_stage = [&](St& s, int64_t t0) {
    if constexpr (VEC) {
#pragma unroll
      for (int n = 0; n < NQV; ++n) {
        const int e = tid + n * kThreads;
        if (e < QV) {
          const int t = e / (DKP / VEC_E);
          const int i = (e - t * (DKP / VEC_E)) * VEC_E;
          *reinterpret_cast<u32x4*>(&s.q[t][St::sw(t, i)]) = qr[n];
          *reinterpret_cast<u32x4*>(&s.k[t][St::sw(t, i)]) = kr[n];
          if constexpr (St::kGrouped) {
#pragma unroll
            for (int x = 0; x < VEC_E; ++x) s.kg[(t >> 2) * St::KGS + (i + x) * 4 + (t & 3)] = elem<IoT>(kr[n], x);
          }
        }
      }
      if (tid < VV) {
        const int t = tid / (kCols / VEC_E);
        const int j = (tid - t * (kCols / VEC_E)) * VEC_E;
        if constexpr (St::kGrouped) {
#pragma unroll
          for (int x = 0; x < VEC_E; ++x) s.vg[(t >> 2) * St::VGS + (j + x) * 4 + (t & 3)] = elem<IoT>(vr, x);
        } else {
          *reinterpret_cast<u32x4*>(&s.v[t][j]) = vr;
        }
      }
    } else {
      for (int e = tid; e < kT * DKP; e += kThreads) {
        const int t = e / DKP, i = e - t * DKP;
        const bool in = t0 + t < L && i < dk;
        const IoT qv = in ? qg[(t0 + t) * dk + i] : zero_elem<IoT>();
        const IoT kv = in ? kgp[(t0 + t) * dk + i] : zero_elem<IoT>();
        s.q[t][St::sw(t, i)] = qv;
        s.k[t][St::sw(t, i)] = kv;
        if constexpr (St::kGrouped) s.kg[(t >> 2) * St::KGS + i * 4 + (t & 3)] = kv;
      }
      for (int e = tid; e < kT * kCols; e += kThreads) {
        const int t = e / kCols, j = e - t * kCols;
        const bool in = t0 + t < L && jb + j < dv;
        const IoT vv = in ? vgp[(t0 + t) * dv + jb + j] : zero_elem<IoT>();
        if constexpr (St::kGrouped) s.vg[(t >> 2) * St::VGS + j * 4 + (t & 3)] = vv;
        else s.v[t][j] = vv;
      }
    }
    // Thread 16 t + u holds gamma_u. Over each 16-lane row (one t), the
    // suffix products of a_u = (u <= t ? gamma_u : 1) give
    // L[t][s] = a_{s+1} ... a_15 = gamma_{s+1} ... gamma_t and
    // P[t] = a_0 ... a_15 = gamma_0 ... gamma_t.
    {
      const int t = tid >> 4, u = tid & 15;
      float x = u <= t ? gam : 1.0f;
      x *= dpp_or<kDppRowShl1>(1.0f, x);
      x *= dpp_or<kDppRowShl1 + 1>(1.0f, x);
      x *= dpp_or<kDppRowShl1 + 3>(1.0f, x);
      x *= dpp_or<kDppRowShl1 + 7>(1.0f, x);
      const float after = dpp_or<kDppRowShl1>(1.0f, x);  // a_{u+1} ... a_15
      s.L[t][u] = u <= t ? after : 0.0f;
      if (u == 0) s.P[t] = x;
    }
  };

  const int64_t nchunks = (L + kT - 1) / kT;
  if (nchunks > 0) prefetch(0);
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * kT;
    St& s = stage[ch & 1];
    write_stage(s, t0);
    __syncthreads();
    if (ch + 1 < nchunks) prefetch(t0 + kT);
    if (ch > 0) store_y(stage[(ch - 1) & 1], t0 - kT);
    if (!wave_live) continue;

    v4f Y;
    if constexpr (sizeof(IoT) == 2) {
      Y = chunk_bf16<St, RT>(s, S, w, G, c16);
    } else {
      // A^T[s][t] = k_s . q_t: register r at lane (t, G) is s = 4 G + r
      v4f A0 = {0.0f, 0.0f, 0.0f, 0.0f}, A1 = A0;
      const int o4 = St::sw(c16, 4 * G);  // the lane's swizzled offset in its rows of q and k
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const v4f ka = ld4(&s.k[c16][16 * rt + o4]);
        const v4f qa = ld4(&s.q[c16][16 * rt + o4]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (rt & 1) A1 = mfma4(ka[g], qa[g], A1);
          else A0 = mfma4(ka[g], qa[g], A0);
        }
      }
      // M[t][s] = A[t][s] L[t][s]: the A operand of M V with slot s = 4 G + g
      const v4f mt = (A0 + A1) * *reinterpret_cast<const v4f*>(&s.L[c16][4 * G]);
      const v4f vb = ld4(&s.vg[G * St::VGS + (16 * w + c16) * 4]);  // v[4 G + g][column]
      Y = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < 4; ++g) Y = mfma4(mt[g], vb[g], Y);
      // Z[t][j] = q_t . S_prev[:, j]
      asm volatile("" ::: "memory");  // q is read again below rather than held
      v4f Z0 = {0.0f, 0.0f, 0.0f, 0.0f}, Z1 = Z0;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const v4f qa = ld4(&s.q[c16][16 * rt + o4]);  // read again: fewer live registers
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (rt & 1) Z1 = mfma4(qa[g], S[rt][g], Z1);
          else Z0 = mfma4(qa[g], S[rt][g], Z0);
        }
      }
      Y += *reinterpret_cast<const v4f*>(&s.P[4 * G]) * (Z0 + Z1);
      // S <- P_15 S + sum_s (L[15][s] k_s) v_s^T
      const float p15 = s.P[kT - 1];
      const v4f l15 = *reinterpret_cast<const v4f*>(&s.L[kT - 1][4 * G]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const v4f kt = ld4(&s.kg[G * St::KGS + (16 * rt + c16) * 4]) * l15;
        S[rt] *= p15;
#pragma unroll
        for (int g = 0; g < 4; ++g) S[rt] = mfma4(kt[g], vb[g], S[rt]);
      }
    }
    // y: register r at lane (column, G) is token 4 G + r; to LDS, stored
    // with the next chunk (after its barrier)
#pragma unroll
    for (int r = 0; r < 4; ++r) s.y[4 * G + r][16 * w + c16] = Io<IoT>::from_f32(Y[r]);
  }
  if (nchunks > 0) {
    __syncthreads();
    store_y(stage[(nchunks - 1) & 1], (nchunks - 1) * kT);
  }

  // The lane's column and lane group go through opaque copies here, so that
  // the compiler does not keep the prologue's per-element s0 offsets (the
  // same expressions) live across the whole chunk loop.
  int c16e = c16, Ge = G;
  asm volatile("" : "+v"(c16e), "+v"(Ge));
  const int64_t jce = jw + c16e;
  if (p.final_state && jce < dv) {
    StT* fs = static_cast<StT*>(p.final_state) + b * dk * dv + jce;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * rt + 4 * Ge + r;
        if (i < dk) fs[static_cast<int64_t>(i) * dv] = Io<StT>::from_f32(S[rt][r]);
      }
  }
}

template <typename IoT, typename StT, int RT>
hipError_t launch_rt(const GatedParams& p0, hipStream_t stream) {
  GatedParams p = p0;
  p.col_blocks = (p.dv + kCols - 1) / kCols;
  const int64_t blocks = p.batch * p.col_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // 16-byte vectors: whole vectors per row and 16-byte aligned bases
  constexpr int VEC_E = 16 / sizeof(IoT);
  const bool vec = p.dk % VEC_E == 0 && p.dv % VEC_E == 0 && reinterpret_cast<uintptr_t>(p.q) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.k) % 16 == 0 && reinterpret_cast<uintptr_t>(p.v) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.y) % 16 == 0;
  void* args[] = {&p};
  const void* fn = vec ? reinterpret_cast<const void*>(&gated_scan_kernel<IoT, StT, RT, true>)
                       : reinterpret_cast<const void*>(&gated_scan_kernel<IoT, StT, RT, false>);
  return launch_kernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, stream);
}

template <typename IoT, typename StT>
hipError_t launch_io(const GatedParams& p, hipStream_t stream) {
  if (p.dk <= 16) return launch_rt<IoT, StT, 1>(p, stream);
  if (p.dk <= 32) return launch_rt<IoT, StT, 2>(p, stream);
  if (p.dk <= 64) return launch_rt<IoT, StT, 4>(p, stream);
  if (p.dk <= 128) return launch_rt<IoT, StT, 8>(p, stream);
  if (p.dk <= 192) return launch_rt<IoT, StT, 12>(p, stream);
  return launch_rt<IoT, StT, 16>(p, stream);
}

}  // namespace

hipError_t launch_gated_scan(const GatedParams& p, bool io_bf16, bool state_bf16, hipStream_t stream) {
  if (io_bf16) return state_bf16 ? launch_io<bf16_t, bf16_t>(p, stream) : launch_io<bf16_t, float>(p, stream);
  return state_bf16 ? launch_io<float, bf16_t>(p, stream) : launch_io<float, float>(p, stream);
}

int64_t gated_scan_blocks(int64_t batch, int64_t dv) { return batch * ((dv + kCols - 1) / kCols); }

}  // namespace ss
