// Device-side building blocks shared by the LM-head, acceptance and commit kernels:
// MFMA operand types, Philox4x32-10, Gumbel / uniform maps, and the running row
// statistics merged by the fused LM-head epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mtp.h"

namespace mtp {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();
constexpr int kNoIndex = 0x7fffffff;

// Philox stream ids (the counter's second word is stream << 8 | row).
constexpr uint32_t kStreamDraft = 0;
constexpr uint32_t kStreamAccept = 1;
constexpr uint32_t kStreamResample = 2;
constexpr uint32_t kStreamTrunk = 3;   // the trunk's own sample, keyed by position

// ---------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies on counter words 0 and 2, whose high halves are crossed with words 1 and 3
// and the round key; the key is bumped by the two Weyl increments between rounds.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c.x;
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// word x & 3 of counter (x >> 2, stream << 8 | row, request, cycle)
__device__ __forceinline__ uint32_t philox_word(uint32_t k0, uint32_t k1, uint32_t stream,
                                                uint32_t row, uint32_t request, uint32_t cycle,
                                                uint32_t x) {
  const u32x4 w = philox4x32_10(u32x4{x >> 2, (stream << 8) | row, request, cycle}, k0, k1);
  const uint32_t s = x & 3u;
  return s == 0 ? w.x : (s == 1 ? w.y : (s == 2 ? w.z : w.w));
}

// Standard Gumbel noise -ln(-ln u), u = (2 (w >> 9) + 1) 2^-24.  -ln u is taken as
// -log1p(-(1 - u)) with 1 - u formed exactly from the integer, so draws near u = 1
// (the ones that win an argmax over many ids) keep full relative precision.
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const uint32_t m = w >> 9;
  const float one_minus_u = static_cast<float>(16777215u - 2u * m) * 5.9604644775390625e-8f;
  const float neg_ln_u = -log1pf(-one_minus_u);
  return -logf(neg_ln_u);
}

// acceptance uniform u = ((w >> 8) + 1) 2^-24 in (0, 1]
__device__ __forceinline__ float uniform_accept(uint32_t w) {
  return static_cast<float>((w >> 8) + 1u) * 5.9604644775390625e-8f;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Sanitised logit given the row's flags: NaN -> -inf; in a row holding +inf, +inf -> 0
// and everything else -> -inf.
__device__ __forceinline__ float sanitize(float z, uint32_t row_flags) {
  if (row_flags & MTP_ROW_POSINF) return z == kPosInf ? 0.0f : kNegInf;
  return (z != z) ? kNegInf : z;
}

// ---------------------------------------------------------------------------------
// Running statistics of one hidden row over a set of vocabulary rows.  Within one
// lane ids are pushed in increasing order, so a strict '>' keeps the lowest id on ties;
// merges compare ids explicitly.  48 bytes; the first 32 hold every field a row scored
// without sampling changes (the rest keep their initial values there).
// ---------------------------------------------------------------------------------
struct RowAcc {
  float m;        // max of finite z / T_eff (-inf if none yet)
  float s;        // sum of exp(z / T_eff - m) over finite z
  float zmax;     // max finite z
  int imax;       // its lowest id (kNoIndex if none)
  int nonfinite;  // count of NaN / +-inf
  int nposinf;    // count of +inf
  int pinf_min;   // lowest +inf id
  int pgidx;      // id of the best Gumbel among +inf ids
  float gbest;    // best z / T + Gumbel over finite z
  int gidx;       // its id
  float gz;       // z at gidx
  float pg;       // best Gumbel among +inf ids (their sanitised logit is 0)
};
// 16-byte pieces of a RowAcc that a merge needs: all three under sampling, the first two
// otherwise
template <bool SAMPLED>
constexpr int rowacc_pieces() { return SAMPLED ? 3 : 2; }

__device__ __forceinline__ void rowacc_init(RowAcc& a) {
  a.m = kNegInf; a.s = 0.0f; a.zmax = kNegInf; a.imax = kNoIndex;
  a.gbest = kNegInf; a.gidx = kNoIndex; a.gz = kNegInf;
  a.nonfinite = 0; a.nposinf = 0; a.pinf_min = kNoIndex; a.pg = kNegInf; a.pgidx = kNoIndex;
}

// z / T_eff and z / T_eff + G, each rounded on its own (never fused into one multiply-add),
// so that every kernel scoring a logit produces the same bits
__device__ __forceinline__ float score_scaled(float z, float inv_t) {
#pragma clang fp contract(off)
  return z * inv_t;
}
__device__ __forceinline__ float score_gumbel(float sv, float gumbel) {
#pragma clang fp contract(off)
  return sv + gumbel;
}

template <bool SAMPLED>
__device__ __forceinline__ void rowacc_push(RowAcc& a, float z, int x, float inv_t, float gumbel) {
  if (__builtin_isfinite(z)) {
    if (z > a.zmax) { a.zmax = z; a.imax = x; }
    const float sv = score_scaled(z, inv_t);
    if (sv > a.m) {
      a.s = a.s * __expf(a.m - sv) + 1.0f;
      a.m = sv;
    } else {
      a.s += __expf(sv - a.m);
    }
    if (SAMPLED) {
      const float sc = score_gumbel(sv, gumbel);
      if (sc > a.gbest) { a.gbest = sc; a.gidx = x; a.gz = z; }
    }
  } else {
    a.nonfinite += 1;
    if (z > 0.0f) {
      a.nposinf += 1;
      a.pinf_min = min(a.pinf_min, x);
      if (SAMPLED && gumbel > a.pg) { a.pg = gumbel; a.pgidx = x; }
    }
  }
}

// (va, ia) ranks above (vb, ib): larger value, then lower id (bitwise, branch-free)
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

// Sum-exp of two parts with maxima ma, mb: the larger part's sum stays as it is and the
// other is scaled by exp(-|ma - mb|) (one exponential).  Commutative bit for bit.
__device__ __forceinline__ float sumexp_merge(float ma, float sa, float mb, float sb) {
  const bool ge = ma >= mb;
  const float e = (ma == kNegInf || mb == kNegInf) ? 0.0f : __expf(ge ? mb - ma : ma - mb);
  return ge ? sa + sb * e : sb + sa * e;
}

// a <- merge(a, b).  Commutative: merge(a, b) and merge(b, a) give the same bits.
__device__ __forceinline__ void rowacc_merge(RowAcc& a, const RowAcc& b) {
  a.s = sumexp_merge(a.m, a.s, b.m, b.s);
  a.m = fmaxf(a.m, b.m);
  if (better(b.zmax, b.imax, a.zmax, a.imax)) { a.zmax = b.zmax; a.imax = b.imax; }
  if (better(b.gbest, b.gidx, a.gbest, a.gidx)) { a.gbest = b.gbest; a.gidx = b.gidx; a.gz = b.gz; }
  a.nonfinite += b.nonfinite;
  a.nposinf += b.nposinf;
  a.pinf_min = min(a.pinf_min, b.pinf_min);
  if (better(b.pg, b.pgidx, a.pg, a.pgidx)) { a.pg = b.pg; a.pgidx = b.pgidx; }
}

// ---------------------------------------------------------------------------------
// Data handed from one block to another inside a launch (per-block partials, the
// drafted-token logit) is written and read with relaxed device-scope atomics: on gfx950
// they are ordinary stores and loads carrying the device scope bits, written through to
// and read from the point of coherence shared by all XCDs.  A device-scope fence would
// instead write back and invalidate the whole L2 of the XCD under every other wave's
// weight stream.  Ordering: each wave waits for its stores to be acknowledged
// (wait_stores) before the block barrier that precedes the completion ticket.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void store_coherent_obj(T* dst, const T& v) {
  static_assert(sizeof(T) % 4 == 0, "word-sized objects only");
  const uint32_t* s = reinterpret_cast<const uint32_t*>(&v);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) store_coherent(d + i, s[i]);
}
template <class T>
__device__ __forceinline__ T load_coherent_obj(const T* src) {
  static_assert(sizeof(T) % 4 == 0, "word-sized objects only");
  T v;
  uint32_t* d = reinterpret_cast<uint32_t*>(&v);
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) d[i] = load_coherent(s + i);
  return v;
}
// wait until this wave's memory operations (the coherent stores above) are acknowledged
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
// completion ticket: returns the number of blocks that arrived before this one
__device__ __forceinline__ unsigned int take_ticket(unsigned int* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exchange between the lanes l and l ^ MASK (MASK = 1, 2, 4, 8, inside each row of 16
// lanes) on the DPP network: VALU moves with no LDS round trip.  xor 1 and xor 2 are quad
// permutations; xor 4 is the half-row mirror (l -> 7 - l in each 8) followed by the quad
// reversal (l -> 3 - l in each 4); xor 8 is a rotation of the 16-lane row by 8.
template <int MASK>
__device__ __forceinline__ int xor16(int v) {
  static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8, "lanes of one 16-lane row");
  if constexpr (MASK == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad [1,0,3,2]
  if constexpr (MASK == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad [2,3,0,1]
  if constexpr (MASK == 4) {
    const int h = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);                  // row half-mirror
    return __builtin_amdgcn_update_dpp(0, h, 0x1B, 0xF, 0xF, false);                          // quad [3,2,1,0]
  }
  return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);                           // row rotate by 8
}
template <int MASK>
__device__ __forceinline__ float xor16(float v) {
  return __int_as_float(xor16<MASK>(__float_as_int(v)));
}

template <int MASK>
__device__ __forceinline__ RowAcc rowacc_xor16(const RowAcc& a) {
  RowAcc b;
  b.m = xor16<MASK>(a.m);
  b.s = xor16<MASK>(a.s);
  b.zmax = xor16<MASK>(a.zmax);
  b.imax = xor16<MASK>(a.imax);
  b.gbest = xor16<MASK>(a.gbest);
  b.gidx = xor16<MASK>(a.gidx);
  b.gz = xor16<MASK>(a.gz);
  b.nonfinite = xor16<MASK>(a.nonfinite);
  b.nposinf = xor16<MASK>(a.nposinf);
  b.pinf_min = xor16<MASK>(a.pinf_min);
  b.pg = xor16<MASK>(a.pg);
  b.pgidx = xor16<MASK>(a.pgidx);
  return b;
}

__device__ __forceinline__ RowAcc rowacc_shfl_xor(const RowAcc& a, int mask) {
  RowAcc b;
  b.m = __shfl_xor(a.m, mask);
  b.s = __shfl_xor(a.s, mask);
  b.zmax = __shfl_xor(a.zmax, mask);
  b.imax = __shfl_xor(a.imax, mask);
  b.gbest = __shfl_xor(a.gbest, mask);
  b.gidx = __shfl_xor(a.gidx, mask);
  b.gz = __shfl_xor(a.gz, mask);
  b.nonfinite = __shfl_xor(a.nonfinite, mask);
  b.nposinf = __shfl_xor(a.nposinf, mask);
  b.pinf_min = __shfl_xor(a.pinf_min, mask);
  b.pg = __shfl_xor(a.pg, mask);
  b.pgidx = __shfl_xor(a.pgidx, mask);
  return b;
}

}  // namespace mtp
