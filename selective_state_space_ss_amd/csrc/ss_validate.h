// Host-only argument checks of the C ABI. No HIP dependency: the same code is
// compiled into the library and into a plain g++ test.
#pragma once

#include <stdint.h>

#include "ss_scan.h"

namespace ss {

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
  Span() = default;
  Span(const void* p, int64_t bytes) {
    if (p && bytes > 0) {
      lo = reinterpret_cast<uintptr_t>(p);
      hi = lo + static_cast<uintptr_t>(bytes);
    }
  }
  bool empty() const { return lo == hi; }
  bool overlaps(const Span& o) const { return !empty() && !o.empty() && lo < o.hi && o.lo < hi; }
};

inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

inline bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

// The prompt scan's arguments are the public struct (ss_scan_fwd in ss_scan.h).
using ScanArgs = ss_scan_args;

// SS_OK means "launch"; *noop set means "valid and nothing to do".
inline ss_status validate_scan(const ScanArgs& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != SS_F32 && a.io_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.batch < 0 || a.channels < 0 || a.seqlen < 0 || a.state_dim < 0) return SS_ERR_SHAPE;
  if (a.state_dim < 1 || a.state_dim > SS_MAX_STATE_DIM) return SS_ERR_UNSUPPORTED;
  if (a.batch == 0 || a.channels == 0) {
    *noop = true;
    return SS_OK;
  }
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t rows, tok, tok_bytes, bcn, bc_bytes, st, st_bytes, cn, a_bytes, rs_bytes;
  if (!mul_ok(a.batch, a.channels, &rows) || !mul_ok(rows, a.seqlen, &tok) || !mul_ok(tok, es, &tok_bytes) ||
      !mul_ok(a.batch, a.state_dim, &bcn) || !mul_ok(bcn, a.seqlen, &bcn) || !mul_ok(bcn, es, &bc_bytes) ||
      !mul_ok(rows, a.state_dim, &st) || !mul_ok(st, 4, &st_bytes) || !mul_ok(a.channels, a.state_dim, &cn) ||
      !mul_ok(cn, 4, &a_bytes) || !mul_ok(a.batch, a.seqlen, &rs_bytes))
    return SS_ERR_SHAPE;
  if (tok_bytes > (INT64_MAX >> 2)) return SS_ERR_SHAPE;
  const bool has_tokens = a.seqlen > 0;
  if (!a.A) return SS_ERR_NULL;
  if (has_tokens && (!a.x || !a.dt || !a.B || !a.C || !a.y)) return SS_ERR_NULL;
  const void* io_ptrs[] = {a.x, a.dt, a.z, a.B, a.C, a.y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SS_ERR_ALIGN;
  const void* f32_ptrs[] = {a.A, a.D, a.dt_bias, a.h0, a.h_last};
  for (const void* p : f32_ptrs)
    if (p && !aligned(p, 4)) return SS_ERR_ALIGN;

  const Span x(a.x, has_tokens ? tok_bytes : 0), dt(a.dt, has_tokens ? tok_bytes : 0),
      z(a.z, has_tokens ? tok_bytes : 0), B(a.B, has_tokens ? bc_bytes : 0), C(a.C, has_tokens ? bc_bytes : 0),
      A(a.A, a_bytes), D(a.D, a.channels * 4), bias(a.dt_bias, a.channels * 4), h0(a.h0, st_bytes),
      reset(a.reset, has_tokens ? rs_bytes : 0), y(a.y, has_tokens ? tok_bytes : 0), hl(a.h_last, st_bytes);
  const Span inputs[] = {x, dt, z, B, C, A, D, bias, h0, reset};
  for (const Span& in : inputs) {
    if (y.overlaps(in)) return SS_ERR_ALIAS;
    if (&in != &inputs[8] && hl.overlaps(in)) return SS_ERR_ALIAS;
  }
  if (hl.overlaps(h0) && a.h_last != a.h0) return SS_ERR_ALIAS;
  if (y.overlaps(hl)) return SS_ERR_ALIAS;
  return SS_OK;
}

// The per-token states output of ss_scan_fwd_states (after validate_scan has
// accepted the rest): states must be given, time_step below seqlen, and the
// buffer must not overlap any input or the other outputs.
inline ss_status validate_scan_states(const ScanArgs& a, const float* states, int64_t time_step) {
  if (!states) return SS_ERR_NULL;
  if (time_step >= a.seqlen) return SS_ERR_SHAPE;
  if (!aligned(states, 4)) return SS_ERR_ALIGN;
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t rows, st, st_bytes, tok, tok_bytes, bn, bc_bytes, cn, a_bytes, rs_bytes, s_bytes;
  if (!mul_ok(a.batch, a.channels, &rows) || !mul_ok(rows, a.state_dim, &st) || !mul_ok(st, 4, &st_bytes) ||
      !mul_ok(st, time_step < 0 ? a.seqlen : 1, &s_bytes) || !mul_ok(s_bytes, 4, &s_bytes) ||
      !mul_ok(rows, a.seqlen, &tok) || !mul_ok(tok, es, &tok_bytes) || !mul_ok(a.batch, a.state_dim, &bn) ||
      !mul_ok(bn, a.seqlen, &bc_bytes) || !mul_ok(bc_bytes, es, &bc_bytes) ||
      !mul_ok(a.channels, a.state_dim, &cn) || !mul_ok(cn, 4, &a_bytes) || !mul_ok(a.batch, a.seqlen, &rs_bytes))
    return SS_ERR_SHAPE;
  const Span s(states, s_bytes);
  const Span others[] = {Span(a.x, tok_bytes),      Span(a.dt, tok_bytes),           Span(a.z, tok_bytes),
                         Span(a.B, bc_bytes),       Span(a.C, bc_bytes),             Span(a.A, a_bytes),
                         Span(a.D, a.channels * 4), Span(a.dt_bias, a.channels * 4), Span(a.h0, st_bytes),
                         Span(a.reset, rs_bytes),   Span(a.y, tok_bytes),            Span(a.h_last, st_bytes)};
  for (const Span& o : others)
    if (s.overlaps(o)) return SS_ERR_ALIAS;
  return SS_OK;
}

// The fused conv's extra arguments of ss_scan_fwd_conv (after validate_scan
// has accepted the scan's): the width, the weights, and no overlap of the
// weights with the outputs.
inline ss_status validate_scan_conv(const ScanArgs& a, const float* conv_w, const float* conv_b, int64_t width) {
  if (width < 1 || width > SS_MAX_CONV_WIDTH) return SS_ERR_UNSUPPORTED;
  if (!conv_w) return SS_ERR_NULL;
  if (!aligned(conv_w, 4) || (conv_b && !aligned(conv_b, 4))) return SS_ERR_ALIGN;
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t rows, tok, tok_bytes, st, st_bytes, wn, w_bytes, b_bytes;
  if (!mul_ok(a.batch, a.channels, &rows) || !mul_ok(rows, a.seqlen, &tok) || !mul_ok(tok, es, &tok_bytes) ||
      !mul_ok(rows, a.state_dim, &st) || !mul_ok(st, 4, &st_bytes) || !mul_ok(a.channels, width, &wn) ||
      !mul_ok(wn, 4, &w_bytes) || !mul_ok(a.channels, 4, &b_bytes))
    return SS_ERR_SHAPE;
  const Span w(conv_w, w_bytes), cb(conv_b, b_bytes), y(a.y, a.seqlen > 0 ? tok_bytes : 0), hl(a.h_last, st_bytes);
  if (w.overlaps(y) || w.overlaps(hl) || cb.overlaps(y) || cb.overlaps(hl)) return SS_ERR_ALIAS;
  return SS_OK;
}

// Inputs of the scalar-gated state scan, in ABI order; see ss_gated_scan.
struct GatedArgs {
  int64_t batch, seqlen, dk, dv;
  int io_dtype, state_dtype;
  const void *q, *k, *v;
  const float* gamma;
  const void* s0;
  void* y;
  void* final_state;
};

inline ss_status validate_gated(const GatedArgs& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != SS_F32 && a.io_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.state_dtype != SS_F32 && a.state_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.batch < 0 || a.seqlen < 0 || a.dk < 0 || a.dv < 0) return SS_ERR_SHAPE;
  if (a.dk < 1 || a.dk > SS_MAX_GATED_DK || a.dv < 1) return SS_ERR_UNSUPPORTED;
  if (a.batch == 0) {
    *noop = true;
    return SS_OK;
  }
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  const int64_t ses = a.state_dtype == SS_BF16 ? 2 : 4;
  int64_t bl, qk, qk_bytes, vy, vy_bytes, g_bytes, st, st_bytes;
  if (!mul_ok(a.batch, a.seqlen, &bl) || !mul_ok(bl, a.dk, &qk) || !mul_ok(qk, es, &qk_bytes) ||
      !mul_ok(bl, a.dv, &vy) || !mul_ok(vy, es, &vy_bytes) || !mul_ok(bl, 4, &g_bytes) ||
      !mul_ok(a.batch, a.dk, &st) || !mul_ok(st, a.dv, &st) || !mul_ok(st, ses, &st_bytes))
    return SS_ERR_SHAPE;
  if (qk_bytes > (INT64_MAX >> 2) || vy_bytes > (INT64_MAX >> 2) || st_bytes > (INT64_MAX >> 2)) return SS_ERR_SHAPE;
  const bool has_tokens = a.seqlen > 0;
  if (has_tokens && (!a.q || !a.k || !a.v || !a.gamma || !a.y)) return SS_ERR_NULL;
  const void* io_ptrs[] = {a.q, a.k, a.v, a.y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SS_ERR_ALIGN;
  if (a.gamma && !aligned(a.gamma, 4)) return SS_ERR_ALIGN;
  const void* st_ptrs[] = {a.s0, a.final_state};
  for (const void* p : st_ptrs)
    if (p && !aligned(p, ses)) return SS_ERR_ALIGN;
  const Span q(a.q, has_tokens ? qk_bytes : 0), k(a.k, has_tokens ? qk_bytes : 0), v(a.v, has_tokens ? vy_bytes : 0),
      g(a.gamma, has_tokens ? g_bytes : 0), s0(a.s0, st_bytes), y(a.y, has_tokens ? vy_bytes : 0),
      fs(a.final_state, st_bytes);
  const Span inputs[] = {q, k, v, g, s0};
  for (const Span& in : inputs) {
    if (y.overlaps(in)) return SS_ERR_ALIAS;
    if (&in != &inputs[4] && fs.overlaps(in)) return SS_ERR_ALIAS;
  }
  if (fs.overlaps(s0) && a.final_state != a.s0) return SS_ERR_ALIAS;
  if (y.overlaps(fs)) return SS_ERR_ALIAS;
  return SS_OK;
}

// Inputs of the effective attention, in ABI order; see ss_effective_attention.
struct AttnArgs {
  int64_t batch, channels, state_dim, seqlen;
  int io_dtype;
  const void* dt;
  const float* A;
  const void *B, *C;
  const float* dt_bias;
  int dt_softplus, include_dt_scaling, per_state_coord;
  float* M;
};

inline ss_status validate_attention(const AttnArgs& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != SS_F32 && a.io_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.batch < 0 || a.channels < 0 || a.state_dim < 0 || a.seqlen < 0) return SS_ERR_SHAPE;
  if (a.state_dim < 1 || a.state_dim > SS_MAX_STATE_DIM) return SS_ERR_UNSUPPORTED;
  if (a.batch == 0 || a.channels == 0 || a.seqlen == 0) {
    *noop = true;
    return SS_OK;
  }
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t bc, bcl, x_bytes, bn, bnl, bc_bytes, a_elems, a_bytes, ll, m, m_bytes;
  if (!mul_ok(a.batch, a.channels, &bc) || !mul_ok(bc, a.seqlen, &bcl) || !mul_ok(bcl, es, &x_bytes) ||
      !mul_ok(a.batch, a.state_dim, &bn) || !mul_ok(bn, a.seqlen, &bnl) || !mul_ok(bnl, es, &bc_bytes) ||
      !mul_ok(a.channels, a.state_dim, &a_elems) || !mul_ok(a_elems, 4, &a_bytes) ||
      !mul_ok(a.seqlen, a.seqlen, &ll) || !mul_ok(bc, ll, &m) ||
      !mul_ok(m, a.per_state_coord ? a.state_dim : 1, &m) || !mul_ok(m, 4, &m_bytes))
    return SS_ERR_SHAPE;
  if (x_bytes > (INT64_MAX >> 2) || m_bytes > (INT64_MAX >> 2)) return SS_ERR_SHAPE;
  if (!a.dt || !a.A || !a.B || !a.C || !a.M) return SS_ERR_NULL;
  const void* io_ptrs[] = {a.dt, a.B, a.C};
  for (const void* p : io_ptrs)
    if (!aligned(p, es)) return SS_ERR_ALIGN;
  const void* f32_ptrs[] = {a.A, a.dt_bias, a.M};
  for (const void* p : f32_ptrs)
    if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
  const Span out(a.M, m_bytes);
  const Span inputs[] = {Span(a.dt, x_bytes), Span(a.A, a_bytes), Span(a.B, bc_bytes), Span(a.C, bc_bytes),
                         Span(a.dt_bias, a.channels * 4)};
  for (const Span& in : inputs)
    if (out.overlaps(in)) return SS_ERR_ALIAS;
  return SS_OK;
}

// Inputs of the input-side producers; see ss_conv1d_silu and ss_dt_proj.
struct ConvArgs {
  int64_t batch, channels, seqlen, width;
  int io_dtype;
  const void* x_pre;
  const float *conv_w, *conv_b;
  const uint8_t* reset;
  void* x;
};

inline ss_status validate_conv(const ConvArgs& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != SS_F32 && a.io_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.batch < 0 || a.channels < 0 || a.seqlen < 0 || a.width < 0) return SS_ERR_SHAPE;
  if (a.width < 1 || a.width > SS_MAX_CONV_WIDTH) return SS_ERR_UNSUPPORTED;
  if (a.batch == 0 || a.channels == 0 || a.seqlen == 0) {
    *noop = true;
    return SS_OK;
  }
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t bc, n, bytes, wn, w_bytes, r_bytes;
  if (!mul_ok(a.batch, a.channels, &bc) || !mul_ok(bc, a.seqlen, &n) || !mul_ok(n, es, &bytes) ||
      !mul_ok(a.channels, a.width, &wn) || !mul_ok(wn, 4, &w_bytes) || !mul_ok(a.batch, a.seqlen, &r_bytes))
    return SS_ERR_SHAPE;
  if (bytes > (INT64_MAX >> 2)) return SS_ERR_SHAPE;
  if (!a.x_pre || !a.conv_w || !a.x) return SS_ERR_NULL;
  if (!aligned(a.x_pre, es) || !aligned(a.x, es)) return SS_ERR_ALIGN;
  if (!aligned(a.conv_w, 4) || (a.conv_b && !aligned(a.conv_b, 4))) return SS_ERR_ALIGN;
  const Span out(a.x, bytes);
  const Span inputs[] = {Span(a.x_pre, bytes), Span(a.conv_w, w_bytes), Span(a.conv_b, a.channels * 4),
                         Span(a.reset, r_bytes)};
  for (const Span& in : inputs)
    if (out.overlaps(in)) return SS_ERR_ALIAS;
  return SS_OK;
}

struct ProjArgs {
  int64_t batch, channels, seqlen, rank;
  int io_dtype;
  const void *w_dt, *delta;
  const float* dt_bias;
  int apply_softplus;
  void* dt;
};

inline ss_status validate_proj(const ProjArgs& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != SS_F32 && a.io_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.batch < 0 || a.channels < 0 || a.seqlen < 0 || a.rank < 0) return SS_ERR_SHAPE;
  if (a.rank < 1) return SS_ERR_UNSUPPORTED;
  if (a.batch == 0 || a.channels == 0 || a.seqlen == 0) {
    *noop = true;
    return SS_OK;
  }
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t bc, n, out_bytes, wn, w_bytes, bl, dn, d_bytes;
  if (!mul_ok(a.batch, a.channels, &bc) || !mul_ok(bc, a.seqlen, &n) || !mul_ok(n, es, &out_bytes) ||
      !mul_ok(a.channels, a.rank, &wn) || !mul_ok(wn, es, &w_bytes) || !mul_ok(a.batch, a.seqlen, &bl) ||
      !mul_ok(bl, a.rank, &dn) || !mul_ok(dn, es, &d_bytes))
    return SS_ERR_SHAPE;
  if (out_bytes > (INT64_MAX >> 2) || d_bytes > (INT64_MAX >> 2)) return SS_ERR_SHAPE;
  if (!a.w_dt || !a.delta || !a.dt) return SS_ERR_NULL;
  if (!aligned(a.w_dt, es) || !aligned(a.delta, es) || !aligned(a.dt, es)) return SS_ERR_ALIGN;
  if (a.dt_bias && !aligned(a.dt_bias, 4)) return SS_ERR_ALIGN;
  const Span out(a.dt, out_bytes);
  const Span inputs[] = {Span(a.w_dt, w_bytes), Span(a.delta, d_bytes), Span(a.dt_bias, a.channels * 4)};
  for (const Span& in : inputs)
    if (out.overlaps(in)) return SS_ERR_ALIAS;
  return SS_OK;
}

// The decode step's arguments are the public struct (ss_state_update in ss_scan.h).
using UpdateArgs = ss_update_args;

inline ss_status validate_update(const UpdateArgs& a, bool* noop) {
  *noop = false;
  if (a.io_dtype != SS_F32 && a.io_dtype != SS_BF16) return SS_ERR_DTYPE;
  if (a.batch < 0 || a.channels < 0 || a.state_dim < 0) return SS_ERR_SHAPE;
  if (a.state_dim < 1 || a.state_dim > SS_MAX_STATE_DIM) return SS_ERR_UNSUPPORTED;
  if (a.batch == 0 || a.channels == 0) {
    *noop = true;
    return SS_OK;
  }
  const int64_t es = a.io_dtype == SS_BF16 ? 2 : 4;
  int64_t rows, tok_bytes, st, st_bytes, bcn, bc_bytes, cn, a_bytes;
  if (!mul_ok(a.batch, a.channels, &rows) || !mul_ok(rows, es, &tok_bytes) || !mul_ok(rows, a.state_dim, &st) ||
      !mul_ok(st, 4, &st_bytes) || !mul_ok(a.batch, a.state_dim, &bcn) || !mul_ok(bcn, es, &bc_bytes) ||
      !mul_ok(a.channels, a.state_dim, &cn) || !mul_ok(cn, 4, &a_bytes))
    return SS_ERR_SHAPE;
  if (st_bytes > (INT64_MAX >> 2)) return SS_ERR_SHAPE;
  if (!a.state || !a.x || !a.dt || !a.A || !a.B || !a.C || !a.y) return SS_ERR_NULL;
  const void* io_ptrs[] = {a.x, a.dt, a.z, a.B, a.C, a.y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SS_ERR_ALIGN;
  const void* f32_ptrs[] = {a.state, a.A, a.D, a.dt_bias};
  for (const void* p : f32_ptrs)
    if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
  const Span state(a.state, st_bytes), x(a.x, tok_bytes), dt(a.dt, tok_bytes), z(a.z, tok_bytes),
      B(a.B, bc_bytes), C(a.C, bc_bytes), A(a.A, a_bytes), D(a.D, a.channels * 4), bias(a.dt_bias, a.channels * 4),
      y(a.y, tok_bytes);
  const Span inputs[] = {x, dt, z, B, C, A, D, bias};
  for (const Span& in : inputs)
    if (y.overlaps(in) || state.overlaps(in)) return SS_ERR_ALIAS;
  if (y.overlaps(state)) return SS_ERR_ALIAS;
  return SS_OK;
}

}  // namespace ss
