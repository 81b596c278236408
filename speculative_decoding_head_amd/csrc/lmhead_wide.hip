// Verify pass for 17..128 hidden rows (several requests' k+1 verify rows in one launch):
// the verify of lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", section "What"
// (every draft of a request checked by one batched forward of the full head), batched over
// requests.
//
// The mapping is the one of the kernel for up to 16 rows (weights are the MFMA B operand,
// streamed once, tile by tile; every logit is one accumulator chain over K in a fixed
// order), with three changes that 128 hidden rows force:
//   * each wave keeps the accumulators of all 8 column blocks (16 hidden rows each) of the
//     tiles it is working on, and the hidden rows (640 KB at d = 2560) are staged through
//     LDS one K-chunk at a time, double buffered, with one block barrier per chunk;
//   * after a tile, the 16 lanes that hold its 16 vocabulary rows reduce each hidden row's
//     logits with a transposed butterfly that halves the rows a lane carries at every
//     level, so a lane ends up owning 2 hidden rows and keeps only their running state;
//   * the block partials are merged by a second kernel, one block per hidden row.
// Logits, the argmax, the Gumbel-max sample and the drafted-id logit are bit-identical to
// those of the 16-row kernel; max and log-sum-exp of a row do not depend on how many rows
// (17..128) share the launch or where the row sits, and agree with the 16-row kernel's
// up to the order of the fp32 summation.
#include "kernels.hpp"
#include "lmhead_common.hpp"

namespace mtp {

namespace {

using namespace lm;

constexpr int kWaves = kLmheadThreads / 64;   // 8
constexpr int WTV = 2;                        // tiles a wave works on at once
constexpr int WU = 4;                         // K steps per staged chunk
constexpr int NCB = 8;                        // column blocks of 16 hidden rows
constexpr int kRows = NCB * 16;               // 128
constexpr int kFragsPerChunk = WU * NCB * 64; // 16-byte A fragments per chunk
constexpr int kMergeThreads = 256;
static_assert(kRows == kLmheadMaxWideRows, "one column block per 16 rows of the widest launch");
static_assert(kFragsPerChunk == WU * kLmheadThreads, "staging: one fragment per thread and K step");
static_assert(WU * kRows == kLmheadThreads, "staging: one group sum per thread and chunk");
// LDS layout (bytes).  The per-step tables come first, so that every compute-loop access is
// a lane base address plus an offset that fits the 16-bit offset field of an LDS read.
constexpr int kOffHtab = 0;
constexpr int kOffHbuf = kOffHtab + 2 * WU * kRows * 4;
constexpr int kOffTok = kOffHbuf + 2 * kFragsPerChunk * 16;
constexpr int kOffRow = kOffTok + kRows * 4;
constexpr int kOffReq = kOffRow + kRows * 4;
constexpr int kOffRun = kOffReq + kRows * 4;
constexpr int kOffGum = kOffRun + kWaves * kRows * (int)sizeof(RowAcc);
constexpr int kLdsBytes = kOffGum + kWaves * 4 * 16 * 16 * 4;

// running max / sum-exp / argmax and Gumbel best of a set of finite logits of one row (the
// verify pass reports the sampled id, not its logit)
struct Tuple {
  float zmax;
  int imax;
  float s;   // sum of exp(z / T - zmax / T)
  float gbest;
  int gidx;
};

// commutative: merge(a, b) and merge(b, a) give the same bits
__device__ __forceinline__ void tuple_merge(Tuple& a, const Tuple& b, float inv_t) {
  const float ma = score_scaled(a.zmax, inv_t), mb = score_scaled(b.zmax, inv_t);
  const float m = fmaxf(ma, mb);
  const float sa = (a.zmax == kNegInf) ? 0.0f : a.s * __expf(ma - m);
  const float sb = (b.zmax == kNegInf) ? 0.0f : b.s * __expf(mb - m);
  a.s = sa + sb;
  if (better(b.zmax, b.imax, a.zmax, a.imax)) { a.zmax = b.zmax; a.imax = b.imax; }
  if (better(b.gbest, b.gidx, a.gbest, a.gidx)) { a.gbest = b.gbest; a.gidx = b.gidx; }
}

__device__ __forceinline__ Tuple tuple_shfl_xor(const Tuple& a, int mask) {
  Tuple b;
  b.zmax = __shfl_xor(a.zmax, mask);
  b.imax = __shfl_xor(a.imax, mask);
  b.s = __shfl_xor(a.s, mask);
  b.gbest = __shfl_xor(a.gbest, mask);
  b.gidx = __shfl_xor(a.gidx, mask);
  return b;
}

__device__ __forceinline__ RowAcc tuple_to_rowacc(const Tuple& t, float inv_t) {
  RowAcc a;
  rowacc_init(a);
  if (t.zmax != kNegInf) {
    a.m = score_scaled(t.zmax, inv_t);
    a.s = t.s;
    a.zmax = t.zmax;
    a.imax = t.imax;
    a.gbest = t.gbest;
    a.gidx = t.gidx;
  }
  return a;
}

template <int WT, bool SAMPLED>
__device__ __forceinline__ void wide_body(const LmheadLaunch& p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  using L = Layout<WT>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xi = lane & 15, g = lane >> 4;
  const int M = p.M, d = p.d;
  const int nsteps = L::f32 ? d / 16 : d / 32;
  const int nch = ((nsteps + WU - 1) / WU + 1) & ~1;   // chunks per pass, even

  float* htab = reinterpret_cast<float*>(smem + kOffHtab);       // [2][WU][128] group sums of h
  uint4* hbuf = reinterpret_cast<uint4*>(smem + kOffHbuf);      // [2][WU][NCB][4][16] A fragments
  int* ltok = reinterpret_cast<int*>(smem + kOffTok);            // [128] drafted id per row
  uint32_t* lrow = reinterpret_cast<uint32_t*>(smem + kOffRow);  // [128] Philox row word
  uint32_t* lreq = reinterpret_cast<uint32_t*>(smem + kOffReq);  // [128] Philox request word
  RowAcc* lrun = reinterpret_cast<RowAcc*>(smem + kOffRun);      // [8 waves][128] running state
  float* gum = reinterpret_cast<float*>(smem + kOffGum) + wave * 1024;   // this wave's [4 g][16 n][16 xi] noise

  // ---- tiles of this wave; every wave of the block runs the same number of passes --
  const int tiles = (p.n_rows + 15) >> 4;
  const long long nw = (long long)gridDim.x * kWaves;
  auto range = [&](int w, int& b0, int& b1) {
    const long long gw = (long long)blockIdx.x * kWaves + w;
    b0 = (int)(gw * tiles / nw);
    b1 = (int)((gw + 1) * tiles / nw);
  };
  int t_begin, t_end;
  range(wave, t_begin, t_end);
  int npass = 0;
  for (int w = 0; w < kWaves; ++w) {
    int b0, b1;
    range(w, b0, b1);
    npass = max(npass, (b1 - b0 + WTV - 1) / WTV);
  }

  const size_t rb = row_bytes<WT>(d);
  const int G32 = d / 32;
  const size_t rows_cov = L::tiled ? (size_t)tiles * 16 : (size_t)p.n_rows;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, (uint32_t)(rows_cov * rb));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.scale, (uint32_t)(rows_cov * G32 * 2));
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(p.minv, (uint32_t)(rows_cov * G32 * 2));
  const uint32_t tile_bytes = (uint32_t)(16 * rb);

  if (tid < kRows) {
    const int b = tid / p.rows_per_req, i = tid % p.rows_per_req;
    ltok[tid] = (tid < M && i < p.k) ? p.drafts[(size_t)b * p.k_max + i] : -1;
    lrow[tid] = (uint32_t)(p.stream_id << 8) | (uint32_t)(i + p.row_base);
    lreq[tid] = p.request_base + (uint32_t)b;
  }
  for (int e = tid; e < kWaves * kRows; e += kLmheadThreads) rowacc_init(lrun[e]);

  // ---- weight chunks: iteration it covers K-chunk it % nch of pass it / nch ----------
  typedef typename std::conditional<L::q4, uint32_t, uint4>::type WFrag;
  struct Chunk {
    WFrag w[WTV][WU];
    uint2 sc[WTV], mn[WTV];   // 4-bit heads: scales / mins of the chunk's 4 groups
  };
  auto load = [&](Chunk& ck, int it) {
    const int tb = t_begin + (it / nch) * WTV;
    const int s0 = (it % nch) * WU;
#pragma unroll
    for (int t = 0; t < WTV; ++t) {
      const int x = (tb + t) * 16 + xi;
      uint32_t roff;
      if constexpr (L::tiled)
        roff = (tb + t) < t_end ? (uint32_t)(tb + t) * tile_bytes + (uint32_t)(lane * 16) : kOOB;
      else
        roff = ((tb + t) < t_end && x < p.n_rows) ? (uint32_t)((size_t)x * rb) : kOOB;
      if constexpr (WT == MTP_W_Q4A32_TILED) {
        // one KiB block per group quad: the chunk's four groups in one load
        const uint32_t oob = s0 < nsteps ? 0u : kOOB;
        const uint4 v = bload16_stream(wr, (roff | oob) + (uint32_t)(s0 / 4) * 1024u);
        ck.w[t][0] = v.x; ck.w[t][1] = v.y; ck.w[t][2] = v.z; ck.w[t][3] = v.w;
      } else {
#pragma unroll
        for (int u = 0; u < WU; ++u) {
          const int s = s0 + u;
          const uint32_t oob = s < nsteps ? 0u : kOOB;
          if constexpr (WT == MTP_W_Q4A32)
            ck.w[t][u] = bload4(wr, (roff | oob) + (uint32_t)((4 * s + g) * 4));
          else if constexpr (WT == MTP_W_BF16_TILED)
            ck.w[t][u] = bload16_stream(wr, (roff | oob) + (uint32_t)s * 1024u);
          else
            ck.w[t][u] = bload16(wr, (roff | oob) + (uint32_t)((4 * s + g) * 16));
        }
      }
      if constexpr (L::q4) {
        const uint32_t oob = s0 < nsteps ? 0u : kOOB;
        uint32_t so;
        if constexpr (L::tiled)   // block (tile, octet) of 256 B, 16 B per row
          so = roff == kOOB ? kOOB : (roff - (uint32_t)(lane * 16)) / 8u + (uint32_t)(xi * 16);
        else
          so = roff == kOOB ? kOOB : (roff / (uint32_t)rb) * (uint32_t)(G32 * 2);
        // the chunk's 4 groups are one half of an octet of groups
        const uint32_t step = L::tiled ? (uint32_t)(s0 / 8) * 256u + (uint32_t)(s0 & 4) * 2u : (uint32_t)(s0 * 2);
        ck.sc[t] = bload8(sr, (so | oob) + step);
        ck.mn[t] = bload8(mr, (so | oob) + step);
      }
    }
  };

  // ---- hidden staging: registers <- chunk c (global), then registers -> LDS buffer --
  struct Staged {
    uint4 v[WU];
    float hs;   // 4-bit heads: one (row, group) sum of the hidden values
  };
  auto stage_load = [&](Staged& st, int c) {
    // fragment f = u * 512 + tid = ((u * NCB + cb) * 4 + gg) * 16 + i
    const int cb = tid >> 6, gg = (tid >> 4) & 3, i = tid & 15, j = cb * 16 + i;
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int s = c * WU + u;
      uint4 v = uint4{0u, 0u, 0u, 0u};
      if (j < M && s < nsteps) {
        if (L::f32) {
          v = *reinterpret_cast<const uint4*>(static_cast<const float*>(p.hidden) + (size_t)j * d + 16 * s + 4 * gg);
        } else {
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.hidden) + (size_t)j * d + 32 * s + 8 * gg);
          if (L::q4) v = q4_order(v);
        }
      }
      st.v[u] = v;
    }
    if constexpr (L::q4) {
      // entry u * 128 + j: sum of row j's 32 values of group c * WU + u
      const int u = tid / kRows, jj = tid % kRows, s = c * WU + u;
      st.hs = (jj < M && s < nsteps) ? group_sum32(static_cast<const uint16_t*>(p.hidden) + (size_t)jj * d + 32 * s)
                                     : 0.0f;
    }
  };
  auto stage_store = [&](const Staged& st, int buf) {
#pragma unroll
    for (int u = 0; u < WU; ++u) hbuf[buf * kFragsPerChunk + u * kLmheadThreads + tid] = st.v[u];
    if constexpr (L::q4) htab[buf * WU * kRows + tid] = st.hs;
  };

  f32x4 c[WTV][NCB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int t = 0; t < WTV; ++t)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) c[t][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };
  // chunk ch of the current pass, hidden fragments from LDS buffer buf.  Steps past the
  // end (padding of the last chunk) multiply zero weights by zero hidden values.
  auto comp = [&](const Chunk& ck, int ch, int buf) {
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int s = ch * WU + u;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint4 a = hbuf[buf * kFragsPerChunk + ((u * NCB + cb) * 4 + g) * 16 + xi];
        if constexpr (WT == MTP_W_BF16 || WT == MTP_W_BF16_TILED) {
#pragma unroll
          for (int t = 0; t < WTV; ++t)
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(ck.w[t][u]), c[t][cb], 0, 0, 0);
        } else if constexpr (L::f32) {
          const float a0 = __uint_as_float(a.x), a1 = __uint_as_float(a.y);
          const float a2 = __uint_as_float(a.z), a3 = __uint_as_float(a.w);
#pragma unroll
          for (int t = 0; t < WTV; ++t) {
            const uint4 w = ck.w[t][u];
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, __uint_as_float(w.x), c[t][cb], 0, 0, 0);
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, __uint_as_float(w.y), c[t][cb], 0, 0, 0);
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, __uint_as_float(w.z), c[t][cb], 0, 0, 0);
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, __uint_as_float(w.w), c[t][cb], 0, 0, 0);
          }
        } else {
          // 4-bit affine: D = sum (128 + q) h over the group, then z += s D + (min - 128 s) sum(h)
          const f32x4 hs = *reinterpret_cast<const f32x4*>(htab + buf * WU * kRows + u * kRows + cb * 16 + 4 * g);
#pragma unroll
          for (int t = 0; t < WTV; ++t) {
            const f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(a), as_bf16x8(q4_expand(ck.w[t][u])), f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const uint32_t sw = (u < 2) ? ck.sc[t].x : ck.sc[t].y;
            const uint32_t mw = (u < 2) ? ck.mn[t].x : ck.mn[t].y;
            const float sv = bf16_to_f32((uint16_t)((u & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
            const float mv = bf16_to_f32((uint16_t)((u & 1) ? (mw >> 16) : (mw & 0xFFFFu)));
            const float off = mv - 128.0f * sv;
#pragma unroll
            for (int r = 0; r < 4; ++r) c[t][cb][r] = fmaf(off, hs[r], fmaf(sv, D[r], c[t][cb][r]));
          }
        }
      }
    }
    if constexpr (L::q4) {
      // the scaling of this chunk's products must happen here: left to itself the
      // optimiser sinks it past the block barrier into the next chunk, holding 64 products
      // (256 registers) across the barrier
#pragma unroll
      for (int t = 0; t < WTV; ++t)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) asm volatile("" : "+v"(c[t][cb]));
    }
  };

  // ---- per-tile epilogue --------------------------------------------------------------
  // Lane (xi, g) holds, for column block cb, the logits of hidden rows cb*16 + 4g + r at
  // vocabulary row x = 16 tile + xi.  Half h of the column blocks (cb = 4h .. 4h+3) gives
  // 16 rows per lane, indexed n = 4 (cb - 4h) + r.  A transposed butterfly over the 16
  // lanes of the row group halves the rows a lane carries at every level (lanes with bit m
  // of xi set keep the upper half), so that lane xi ends up with row n = xi of the tile.
  // Its running state lives in LDS (one slot per wave and row) between tiles.
  float* ztok = reinterpret_cast<float*>(static_cast<unsigned char*>(p.ws) + 256);
  auto epilogue = [&](int pass) {
    // the lane coordinates again, opaque to the optimiser: otherwise per-row addresses and
    // indices of this code are hoisted out of the pass loop and held across the whole
    // compute loop
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int xi = lane_o & 15, g = lane_o >> 4;
    // Gumbel noise of the 16 rows of half h at the tile's 16 vocabulary rows.  One Philox
    // block covers 4 consecutive ids of one row, so the 16 lanes of a row group compute the
    // 64 blocks of their rows once (lane 4m + a: rows n = 4a .. 4a+3, ids 16 tile + 4m ..
    // 4m+3) and hand the values over through this wave's LDS slice; lane xi then reads the
    // noise of row n at gum[(16 g + n) * 16 + xi].
    auto make_noise = [&](int tile, int h) {
      const int m = xi >> 2, a = xi & 3;
#pragma unroll 1
      for (int q = 0; q < 4; ++q) {
        const int j = (4 * h + a) * 16 + 4 * g + q;
        const u32x4 wd = philox4x32_10(u32x4{(uint32_t)(4 * tile + m), lrow[j], lreq[j], p.cycle}, p.key0, p.key1);
        const f32x4 gv = f32x4{gumbel_from_word(wd.x), gumbel_from_word(wd.y), gumbel_from_word(wd.z),
                               gumbel_from_word(wd.w)};
        *reinterpret_cast<f32x4*>(gum + (16 * g + 4 * a + q) * 16 + 4 * m) = gv;
      }
      // lanes of this wave read what other lanes wrote: LDS requests of a wave complete in order
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto noise = [&](int n) -> float { return gum[(16 * g + n) * 16 + xi]; };
    auto make_tuple = [&](float z, int n, int x, bool inc) -> Tuple {
      Tuple v;
      v.zmax = inc ? z : kNegInf;
      v.imax = inc ? x : kNoIndex;
      v.s = inc ? 1.0f : 0.0f;
      v.gbest = kNegInf;
      v.gidx = kNoIndex;
      if (SAMPLED && inc) {
        v.gbest = score_gumbel(score_scaled(z, p.inv_t), noise(n));
        v.gidx = x;
      }
      return v;
    };
    const int tb = t_begin + pass * WTV;
#pragma unroll
    for (int t = 0; t < WTV; ++t) {
      if (tb + t >= t_end) continue;   // wave-uniform
      const int x = (tb + t) * 16 + xi;
      const bool xin = x < p.n_rows;
      bool fin = true;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int4 tk = *reinterpret_cast<const int4*>(ltok + cb * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = cb * 16 + 4 * g + r;
          const float z = c[t][cb][r];
          fin = fin && (!xin || __builtin_isfinite(z));
          if (!xin || j >= M) continue;
          if (p.logits) p.logits[(long long)j * p.logits_stride + x] = z;
          const int tok = r == 0 ? tk.x : (r == 1 ? tk.y : (r == 2 ? tk.z : tk.w));
          if (x == tok) ztok[j] = z;
        }
      }
      const bool all_fin = __all(fin);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int jo = (4 * h + xi / 4) * 16 + 4 * g + xi % 4;   // the row this lane ends up with
        RowAcc tile_acc;
        if (SAMPLED) make_noise(tb + t, h);
        if (all_fin) {
          // first level (mask 8) straight from the accumulators: rows n and n + 8 are column
          // blocks 4h + n/4 and 4h + n/4 + 2
          const bool hi8 = (xi & 8) != 0;
          Tuple v[8];
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const int cb = 4 * h + n / 4, r = n % 4;
            const float zl = c[t][cb][r], zh = c[t][cb + 2][r];
            const int jl = cb * 16 + 4 * g + r, jh = jl + 32;
            const float zk = hi8 ? zh : zl, zs = hi8 ? zl : zh;
            const int jk = hi8 ? jh : jl, js = hi8 ? jl : jh;
            Tuple mine = make_tuple(zk, hi8 ? n + 8 : n, x, xin && jk < M);
            const Tuple recv = tuple_shfl_xor(make_tuple(zs, hi8 ? n : n + 8, x, xin && js < M), 8);
            tuple_merge(mine, recv, p.inv_t);
            v[n] = mine;
          }
#pragma unroll
          for (int lvl = 1; lvl < 4; ++lvl) {
            const int mask = 8 >> lvl, half = 8 >> lvl;
            const bool hi = (xi & mask) != 0;
#pragma unroll
            for (int n = 0; n < half; ++n) {
              Tuple mine = hi ? v[n + half] : v[n];
              const Tuple send = hi ? v[n] : v[n + half];
              const Tuple recv = tuple_shfl_xor(send, mask);
              tuple_merge(mine, recv, p.inv_t);
              v[n] = mine;
            }
          }
          tile_acc = tuple_to_rowacc(v[0], p.inv_t);
        } else {
          // a NaN or infinity in the tile (rare): full row statistics, one row at a time, with
          // the same pairing of lanes as the butterfly above
          rowacc_init(tile_acc);
#pragma unroll 1
          for (int n = 0; n < 16; ++n) {
            float z = c[t][4 * h][0];
#pragma unroll
            for (int q = 1; q < 16; ++q) z = (n == q) ? c[t][4 * h + q / 4][q % 4] : z;
            const int j = (4 * h + n / 4) * 16 + 4 * g + n % 4;
            RowAcc a;
            rowacc_init(a);
            if (xin && j < M) rowacc_push<SAMPLED>(a, z, x, p.inv_t, SAMPLED ? noise(n) : 0.0f);
#pragma unroll
            for (int mask = 8; mask >= 1; mask >>= 1) {
              const RowAcc o = rowacc_shfl_xor(a, mask);
              rowacc_merge(a, o);
            }
            if (xi == n) tile_acc = a;
          }
        }
        RowAcc run = lrun[wave * kRows + jo];
        rowacc_merge(run, tile_acc);
        lrun[wave * kRows + jo] = run;
      }
    }
  };

  // ---- pipeline: while chunk it computes, hidden chunk it+1 and the weights of chunk
  //      it+1 (the next pass's first chunk at the end of a pass) are in flight; hidden
  //      loads are issued first so that waiting for them does not also wait for the
  //      weights.  One barrier per chunk; the epilogue of a pass overlaps the next pass's
  //      first loads. --------------------------------------------------------------------
  Chunk A, B;
  Staged S;
  stage_load(S, 0);
  load(A, 0);
  stage_store(S, 0);
  __syncthreads();
  int it = 0;
  for (int pass = 0; pass < npass; ++pass) {
    zero_acc();
    for (int ch = 0; ch < nch; ch += 2, it += 2) {
      stage_load(S, ch + 1);
      load(B, it + 1);
      comp(A, ch, 0);
      stage_store(S, 1);
      __syncthreads();
      stage_load(S, ch + 2 < nch ? ch + 2 : 0);
      load(A, it + 2);
      comp(B, ch + 1, 1);
      stage_store(S, 0);
      __syncthreads();
    }
    epilogue(pass);
  }

  // ---- block partial per row: the waves' states merged in wave order, after every
  //      wave's last epilogue ----------------------------------------------------------
  __syncthreads();
  if (tid < M) {
    RowAcc a = lrun[tid];
    for (int w = 1; w < kWaves; ++w) rowacc_merge(a, lrun[w * kRows + tid]);
    RowAcc* partials = reinterpret_cast<RowAcc*>(static_cast<unsigned char*>(p.ws) + lmhead_partials_offset(M));
    partials[(size_t)blockIdx.x * M + tid] = a;
  }
}

// one block per hidden row: the G block partials merged in a fixed tree, then the row's
// statistics and the drafted-id logit
template <bool SAMPLED>
__device__ __forceinline__ void wide_merge_body(const LmheadLaunch& p, int G) {
  __shared__ RowAcc wred[kMergeThreads / 64];
  const int j = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M;
  const unsigned char* ws = static_cast<const unsigned char*>(p.ws);
  const RowAcc* partials = reinterpret_cast<const RowAcc*>(ws + lmhead_partials_offset(M));
  RowAcc a;
  rowacc_init(a);
  for (int blk = tid; blk < G; blk += kMergeThreads) rowacc_merge(a, partials[(size_t)blk * M + j]);
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) {
    const RowAcc o = rowacc_shfl_xor(a, mask);
    rowacc_merge(a, o);
  }
  if (lane == 0) wred[wave] = a;
  __syncthreads();
  if (tid != 0) return;
  a = wred[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) rowacc_merge(a, wred[w]);
  mtp_row_stats st = finalize_row(a, SAMPLED);
  const int b = j / p.rows_per_req, i = j % p.rows_per_req;
  const int t = (i < p.k) ? p.drafts[(size_t)b * p.k_max + i] : -1;
  const float* ztok = reinterpret_cast<const float*>(ws + 256);
  st.z_tok = (t >= 0 && t < p.n_rows && !(st.flags & MTP_ROW_INVALID)) ? sanitize(ztok[j], st.flags) : kNegInf;
  p.stats[(size_t)j * p.out_stride + p.out_offset] = st;
}

}  // namespace

template <int WT, bool SAMPLED>
__global__ __launch_bounds__(kLmheadThreads) __attribute__((amdgpu_waves_per_eu(1)))
void mtp_verify_wide_kernel(LmheadLaunch p) {
  wide_body<WT, SAMPLED>(p);
}

template <bool SAMPLED>
__global__ __launch_bounds__(kMergeThreads) void mtp_verify_wide_merge_kernel(LmheadLaunch p, int G) {
  wide_merge_body<SAMPLED>(p, G);
}

size_t lmhead_wide_lds_bytes() { return kLdsBytes; }

template <int WT, bool SAMPLED>
static hipError_t launch_wide_t(const LmheadLaunch& p, hipStream_t stream) {
  const int G = lmhead_grid(p.n_rows);
  const size_t lds = lmhead_wide_lds_bytes();
  auto kern = mtp_verify_wide_kernel<WT, SAMPLED>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(G), dim3(kLmheadThreads), lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mtp_verify_wide_merge_kernel<SAMPLED>, dim3(p.M), dim3(kMergeThreads), 0, stream, p, G);
  return hipGetLastError();
}

hipError_t launch_lmhead_wide(const LmheadLaunch& p, hipStream_t stream) {
  if (p.M <= kLmheadMaxRows || p.M > kLmheadMaxWideRows || !p.verify) return hipErrorInvalidValue;
  switch (p.wtype) {
    case MTP_W_F32: return p.sampled ? launch_wide_t<MTP_W_F32, true>(p, stream) : launch_wide_t<MTP_W_F32, false>(p, stream);
    case MTP_W_BF16: return p.sampled ? launch_wide_t<MTP_W_BF16, true>(p, stream) : launch_wide_t<MTP_W_BF16, false>(p, stream);
    case MTP_W_Q4A32: return p.sampled ? launch_wide_t<MTP_W_Q4A32, true>(p, stream) : launch_wide_t<MTP_W_Q4A32, false>(p, stream);
    case MTP_W_BF16_TILED:
      return p.sampled ? launch_wide_t<MTP_W_BF16_TILED, true>(p, stream) : launch_wide_t<MTP_W_BF16_TILED, false>(p, stream);
    case MTP_W_Q4A32_TILED:
      return p.sampled ? launch_wide_t<MTP_W_Q4A32_TILED, true>(p, stream) : launch_wide_t<MTP_W_Q4A32_TILED, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
