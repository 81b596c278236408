// Device helpers shared by the LM-head kernels (up to 16 hidden rows per launch, and the
// wide variant for up to 128): MFMA operand views, bounded buffer loads, the 4-bit
// expansion, the weight layouts, coherent partial hand-off and the final row statistics.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mtp {
namespace lm {

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Raw buffer loads: a load whose byte offset lies at or beyond the record count returns
// zeros without touching memory, so masked tiles and rows past the vocabulary need no
// branch (a branch around a load keeps the compiler from counting outstanding loads).
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
// tiled heads are read once, front to back, in whole KiB: non-temporal (streaming) hint
constexpr int kStream = 2;   // cache-policy bits: nt
__device__ __forceinline__ uint4 bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream));
}

template <int WT> struct Layout {
  static constexpr bool q4 = WT == MTP_W_Q4A32 || WT == MTP_W_Q4A32_TILED;
  static constexpr bool tiled = WT == MTP_W_BF16_TILED || WT == MTP_W_Q4A32_TILED;
  static constexpr bool f32 = WT == MTP_W_F32;
};

// eight 4-bit codes (element 2m in the low nibble of byte m) -> bf16 values 128 + q, in
// the lane order [q0, q2, q1, q3, q4, q6, q5, q7]
// (bf16 128 + q is 0x4300 | q).  The low and high nibbles of the four bytes are masked
// out, then each byte permute puts two of them under the exponent byte 0x43: 7 operations.
__device__ __forceinline__ uint4 q4_expand(uint32_t w) {
  const uint32_t x0 = w & 0x0F0F0F0Fu, x1 = (w >> 4) & 0x0F0F0F0Fu, e = 0x43434343u;
  // selector bytes 0-3 pick bytes of the second operand, 4-7 bytes of the first
  return uint4{__builtin_amdgcn_perm(e, x0, 0x04010400u), __builtin_amdgcn_perm(e, x1, 0x04010400u),
               __builtin_amdgcn_perm(e, x0, 0x04030402u), __builtin_amdgcn_perm(e, x1, 0x04030402u)};
}

// the same lane order applied to eight bf16 hidden values
__device__ __forceinline__ uint4 q4_order(uint4 v) {
  return uint4{(v.x & 0xFFFFu) | (v.y << 16), (v.x >> 16) | (v.y & 0xFFFF0000u),
               (v.z & 0xFFFFu) | (v.w << 16), (v.z >> 16) | (v.w & 0xFFFF0000u)};
}

// Sum of one 32-value group of bf16 hidden values in one fixed order that every kernel
// uses: each quarter of 8 values left to right, then (q0 + q1) + (q2 + q3).
__device__ __forceinline__ float quarter_sum8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float a = __uint_as_float(w[0] << 16);
  a += __uint_as_float(w[0] & 0xFFFF0000u);
#pragma unroll
  for (int e = 1; e < 4; ++e) {
    a += __uint_as_float(w[e] << 16);
    a += __uint_as_float(w[e] & 0xFFFF0000u);
  }
  return a;
}
// the group from its four quarters (raw memory order, 8 values each)
__device__ __forceinline__ float group_sum_quarters(const uint4 (&v)[4]) {
  return (quarter_sum8(v[0]) + quarter_sum8(v[1])) + (quarter_sum8(v[2]) + quarter_sum8(v[3]));
}
// the group from memory (64 contiguous, 16-byte aligned bytes)
__device__ __forceinline__ float group_sum32(const uint16_t* h) {
  uint4 v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = *reinterpret_cast<const uint4*>(h + 8 * c);
  return group_sum_quarters(v);
}

template <int WT>
__device__ __forceinline__ size_t row_bytes(int d) {
  return WT == MTP_W_F32 ? (size_t)d * 4 : (Layout<WT>::q4 ? (size_t)d / 2 : (size_t)d * 2);
}

// partials are handed between blocks as 16-byte device-scope buffer stores/loads (NP of
// the RowAcc's three pieces; a piece not loaded keeps its initial values)
constexpr int kCoherent = 16;   // cache-policy bits: device scope (sc1)
// field-major partials: 16-byte piece i of (row j, block b) at ((i * M + j) * G + b) * 16,
// so that lanes reading consecutive blocks of one row read contiguous bytes
__device__ __forceinline__ uint32_t partial_piece_off(int i, int j, int b, int M, int G) {
  return (uint32_t)((((size_t)i * M + j) * G + b) * 16);
}
template <int NP>
__device__ __forceinline__ void store_partial_fm(__amdgpu_buffer_rsrc_t r, int j, int b, int M, int G, const RowAcc& a) {
  const u32x4* v = reinterpret_cast<const u32x4*>(&a);
#pragma unroll
  for (int i = 0; i < NP; ++i) __builtin_amdgcn_raw_buffer_store_b128(v[i], r, (int)partial_piece_off(i, j, b, M, G), 0, kCoherent);
}
template <int NP>
__device__ __forceinline__ RowAcc load_partial_fm(__amdgpu_buffer_rsrc_t r, int j, int b, int M, int G) {
  RowAcc a;
  rowacc_init(a);
  u32x4* v = reinterpret_cast<u32x4*>(&a);
#pragma unroll
  for (int i = 0; i < NP; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)partial_piece_off(i, j, b, M, G), 0, kCoherent);
  return a;
}

// Row statistics of a fully merged row (z_tok is filled in by the caller).
__device__ __forceinline__ mtp_row_stats finalize_row(const RowAcc& a, bool sampled) {
  mtp_row_stats st;
  uint32_t fl = a.nonfinite ? MTP_ROW_NONFINITE : 0u;
  st.n_posinf = a.nposinf;
  st.reserved = 0;
  st.z_tok = kNegInf;
  if (a.nposinf > 0) {
    fl |= MTP_ROW_POSINF;
    st.max = 0.0f;
    st.lse = logf((float)a.nposinf);
    st.argmax = a.pinf_min;
    st.sample = sampled ? a.pgidx : a.pinf_min;
  } else if (a.imax == kNoIndex) {
    fl |= MTP_ROW_INVALID;
    st.max = kNegInf;
    st.lse = kNegInf;
    st.argmax = -1;
    st.sample = -1;
  } else {
    st.max = a.zmax;
    st.lse = a.m + logf(a.s);
    st.argmax = a.imax;
    st.sample = sampled ? a.gidx : a.imax;
  }
  st.flags = fl;
  return st;
}

}  // namespace lm
}  // namespace mtp
