// Device-side helpers of the gfx950 selective-scan kernels: fp32 numerics,
// bf16 load/store, and the 16-lane DPP scan of the associative pair (a, b).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- I/O types
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Io;

template <>
struct Io<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};

template <>
struct Io<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static float to_f32(bf16_t v) { return __builtin_bit_cast(float, uint32_t(v.bits) << 16); }
  __device__ static bf16_t from_f32(float v) {
    __bf16 h = (__bf16)v;  // round to nearest even (v_cvt_pk_bf16_f32)
    return bf16_t{__builtin_bit_cast(uint16_t, h)};
  }
};

// Two fp32 values rounded to nearest even as bf16 and packed (lo in the low
// half): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Load kVec consecutive elements (16 bytes) and widen to fp32.
__device__ __forceinline__ void load_vec16(const float* p, float* out) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
__device__ __forceinline__ void load_vec16(const bf16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

// Widen 16 bytes already loaded as raw words.
template <typename IoT>
__device__ __forceinline__ void unpack_vec16(const uint4 v, float* out);
template <>
__device__ __forceinline__ void unpack_vec16<float>(const uint4 v, float* out) {
  out[0] = __builtin_bit_cast(float, v.x); out[1] = __builtin_bit_cast(float, v.y);
  out[2] = __builtin_bit_cast(float, v.z); out[3] = __builtin_bit_cast(float, v.w);
}
template <>
__device__ __forceinline__ void unpack_vec16<bf16_t>(const uint4 v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

// Stores of outputs that the writing kernel never reads back carry the
// nontemporal hint: they stream to memory instead of settling in the caches
// (conv1d + SiLU output at 8 x 5120 x 2048 bf16: 64 -> 53 us; M of the
// effective attention: 103 -> 86 us; the scan's y: no change).
__device__ __forceinline__ void stream_store(float v, float* p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stream_store16(uint4 v, void* p) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u4{v.x, v.y, v.z, v.w}, reinterpret_cast<u4*>(p));
}
__device__ __forceinline__ void stream_store16(float4 v, void* p) {
  stream_store16(make_uint4(__builtin_bit_cast(uint32_t, v.x), __builtin_bit_cast(uint32_t, v.y),
                            __builtin_bit_cast(uint32_t, v.z), __builtin_bit_cast(uint32_t, v.w)),
                 p);
}

// Narrow and store kVec consecutive elements (16 bytes, streaming).
__device__ __forceinline__ void store_vec16(float* p, const float* v) {
  stream_store16(make_float4(v[0], v[1], v[2], v[3]), p);
}
__device__ __forceinline__ void store_vec16(bf16_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  }
  stream_store16(make_uint4(w[0], w[1], w[2], w[3]), p);
}

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(u), u = e^{-|v|} in (0, 1].
// log1p(u) is log(w) for w = fl(1 + u) plus the rounding error of that sum,
// delta = u - (w - 1) (exact by Sterbenz), since log(1 + u) = log(w) +
// log(1 + delta / w) and |delta| <= 2^-24 makes the second term delta to
// within 2^-24 relative (the compensated log1p of Goldberg, 1991).
//
// max(v, 0) + l is formed as 0.5 (v + |v|) + l: v + |v| is exactly 2 max(v, 0),
// so the result is the same number, in one add and one FMA (fmaxf would cost
// an extra canonicalising max on its input).
__device__ __forceinline__ float softplus_f32(float v) {
  const float u = fast_exp2(-__builtin_fabsf(v) * kLog2e);
  const float w = 1.0f + u;
  const float delta = u - (w - 1.0f);
  const float l = __builtin_fmaf(fast_log2(w), kLn2, delta);
  return __builtin_fmaf(0.5f, v + __builtin_fabsf(v), l);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^{-z}); e^{-z} = inf gives -0.
__device__ __forceinline__ float silu_f32(float z) {
  return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// ---------------------------------------------------------------- DPP
// DPP control words (gfx9 encoding).
constexpr int kDppRowShl1 = 0x101;  // row_shl:k is kDppRowShl1 + k - 1: lane i reads lane i + k
constexpr int kDppRowShr1 = 0x111;  // row_shr:1: lane i reads lane i - 1
constexpr int kDppRowNewBcast0 = 0x150;   // lane 0 of each row to its whole row
constexpr int kDppRowNewBcast15 = 0x15F;  // lane 15 of each row to its whole row
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm:[2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float dpp_or(float old, float v) {
  // Lanes whose source is outside the row keep `old`.
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                               false));
}

// Inclusive scan over each 16-lane row of the affine pair (A, B), lane i
// combining the elements of lanes 0..i of its row in order:
//   (A1, B1) then (A2, B2)  ->  (A2 * A1, A2 * B1 + B2)
// (the composition h -> A2 (A1 h + B1) + B2; "s6_reset" post, Associative
// Boundary Resetting, binop). Hillis-Steele steps of 1, 2, 4, 8 lanes; a lane
// whose partner falls outside the row has its DPP write disabled and keeps its
// value, which is combining with the identity (1, 0). In each step the B
// update reads the lane's A before the A update overwrites it; the last step
// needs no A update, so A is left holding the products over 8-lane windows.
//
// Then the entry into the lane's own tokens: lanes 1..15 take the state that
// lane l-1 ends with, h <- a0 * B[l-1] + h (h holds the first token's b0 on
// entry), in one DPP FMA; lane 0's DPP write is disabled, so it keeps h
// (which must already hold its first token's state, from the carry).
//
// The leading s_nops cover the VALU-write -> DPP-read wait states (2 on gfx9);
// inside the block each DPP read is at least 3 instructions after the write.
__device__ __forceinline__ void row16_scan_and_enter(float A, float& B, float& h, float a0) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %2, %1, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(A), "+v"(B), "+v"(h)
      : "v"(a0));
}

// The same over 32-lane segments (lanes 0..31 and 32..63): the 16-lane scan
// with the A products completed, then one step in which rows 1 and 3 combine
// with lane 15 of the row before (row_bcast:15, rows 0 and 2 masked off).
// The entry: lanes 1..31 of the first segment and 16..31 of the second take
// lane l-1 through a wave-wide shift (wave_shr:1, row 2 masked off: its first
// lane starts the second segment), lanes 33..47 through row_shr:1 on row 2
// alone; lanes 0 and 32 keep h.
__device__ __forceinline__ void row32_scan_and_enter(float A, float& B, float& h, float a0) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %2, %1, %3 wave_shr:1 row_mask:0xb bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %1, %3 row_shr:1 row_mask:0x4 bank_mask:0xf\n\t"
      : "+v"(A), "+v"(B), "+v"(h)
      : "v"(a0));
}

// Over the whole wave (64 lanes): the 32-lane steps with the A products of
// rows 1 and 3 completed, then rows 2 and 3 combine with lane 31
// (row_bcast:31); the entry shifts across the wave (lane 0 keeps h).
__device__ __forceinline__ void row64_scan_and_enter(float A, float& B, float& h, float a0) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %2, %1, %3 wave_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(A), "+v"(B), "+v"(h)
      : "v"(a0));
}

template <int RL>
__device__ __forceinline__ void row_scan_and_enter(float A, float& B, float& h, float a0) {
  static_assert(RL == 16 || RL == 32 || RL == 64, "segments of 16, 32 or 64 lanes");
  if constexpr (RL == 16) row16_scan_and_enter(A, B, h, a0);
  else if constexpr (RL == 32) row32_scan_and_enter(A, B, h, a0);
  else row64_scan_and_enter(A, B, h, a0);
}

}  // namespace ss
