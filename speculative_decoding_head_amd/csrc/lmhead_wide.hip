// Verify pass for 17..128 hidden rows (several requests' k+1 verify rows in one launch):
// the verify of lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", section "What"
// (every draft of a request checked by one batched forward of the full head), batched over
// requests.  It also takes every verify of a head whose hidden size is too large for the
// other kernel to stage 16 hidden rows in LDS (its own LDS use does not depend on d).
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
constexpr int NB = 2;                         // weight chunks in registers (NB-1 in flight)
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
constexpr int kOffCyc = kOffReq + kRows * 4;
constexpr int kOffRun = kOffCyc + kRows * 4;
constexpr int kOffGum = kOffRun + kWaves * kRows * (int)sizeof(RowAcc);
constexpr int kLdsBytes = kOffGum + kWaves * 4 * 16 * 16 * 4;

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled by construction
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

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
  a.s = sumexp_merge(score_scaled(a.zmax, inv_t), a.s, score_scaled(b.zmax, inv_t), b.s);
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

template <int MASK>
__device__ __forceinline__ Tuple tuple_xor16(const Tuple& a) {
  Tuple b;
  b.zmax = xor16<MASK>(a.zmax);
  b.imax = xor16<MASK>(a.imax);
  b.s = xor16<MASK>(a.s);
  b.gbest = xor16<MASK>(a.gbest);
  b.gidx = xor16<MASK>(a.gidx);
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
  const int nch = ((nsteps + WU - 1) / WU + NB - 1) / NB * NB;   // chunks per pass, a multiple of NB

  float* htab = reinterpret_cast<float*>(smem + kOffHtab);       // [2][WU][128] group sums of h
  uint4* hbuf = reinterpret_cast<uint4*>(smem + kOffHbuf);      // [2][WU][NCB][4][16] A fragments
  int* ltok = reinterpret_cast<int*>(smem + kOffTok);            // [128] drafted id per row
  uint32_t* lrow = reinterpret_cast<uint32_t*>(smem + kOffRow);  // [128] Philox row word
  uint32_t* lreq = reinterpret_cast<uint32_t*>(smem + kOffReq);  // [128] Philox request word
  uint32_t* lcyc = reinterpret_cast<uint32_t*>(smem + kOffCyc);  // [128] Philox cycle / position word
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
    // exact-match acceptance at T > 0: the trunk's own sample, stream 3 keyed by position
    const bool bypos = p.positions != nullptr;
    lrow[tid] = bypos ? (uint32_t)(kStreamTrunk << 8) : (uint32_t)(p.stream_id << 8) | (uint32_t)(i + p.row_base);
    lreq[tid] = p.request_base + (uint32_t)b;
    lcyc[tid] = (bypos && tid < M) ? (uint32_t)(p.positions[b] + i) : p.cycle;
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
    uint32_t roff[WTV];
#pragma unroll
    for (int t = 0; t < WTV; ++t) {
      const int x = (tb + t) * 16 + xi;
      if constexpr (L::tiled)
        roff[t] = (tb + t) < t_end ? (uint32_t)(tb + t) * tile_bytes + (uint32_t)(lane * 16) : kOOB;
      else
        roff[t] = ((tb + t) < t_end && x < p.n_rows) ? (uint32_t)((size_t)x * rb) : kOOB;
    }
    if constexpr (WT == MTP_W_Q4A32_TILED) {
      // one KiB block per group quad: the chunk's four groups in one load
      const uint32_t oob = s0 < nsteps ? 0u : kOOB;
#pragma unroll
      for (int t = 0; t < WTV; ++t) {
        const uint4 v = bload16_stream(wr, (roff[t] | oob) + (uint32_t)(s0 / 4) * 1024u);
        ck.w[t][0] = v.x; ck.w[t][1] = v.y; ck.w[t][2] = v.z; ck.w[t][3] = v.w;
      }
    } else {
      // K step outer: the chunk's first MFMAs need only the first WTV loads to have landed
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        const int s = s0 + u;
        const uint32_t oob = s < nsteps ? 0u : kOOB;
#pragma unroll
        for (int t = 0; t < WTV; ++t) {
          if constexpr (WT == MTP_W_Q4A32)
            ck.w[t][u] = bload4(wr, (roff[t] | oob) + (uint32_t)((4 * s + g) * 4));
          else if constexpr (WT == MTP_W_BF16_TILED)
            ck.w[t][u] = bload16_stream(wr, (roff[t] | oob) + (uint32_t)s * 1024u);
          else
            ck.w[t][u] = bload16(wr, (roff[t] | oob) + (uint32_t)((4 * s + g) * 16));
        }
      }
    }
    if constexpr (L::q4) {
      const uint32_t oob = s0 < nsteps ? 0u : kOOB;
      // the chunk's 4 groups are one half of an octet of groups
      const uint32_t step = L::tiled ? (uint32_t)(s0 / 8) * 256u + (uint32_t)(s0 & 4) * 2u : (uint32_t)(s0 * 2);
#pragma unroll
      for (int t = 0; t < WTV; ++t) {
        uint32_t so;
        if constexpr (L::tiled)   // block (tile, octet) of 256 B, 16 B per row
          so = roff[t] == kOOB ? kOOB : (roff[t] - (uint32_t)(lane * 16)) / 8u + (uint32_t)(xi * 16);
        else
          so = roff[t] == kOOB ? kOOB : (roff[t] / (uint32_t)rb) * (uint32_t)(G32 * 2);
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
  auto comp = [&](const Chunk& ck, int ch, int buf, auto u0_c, auto u1_c) {
#pragma unroll
    for (int u = decltype(u0_c)::value; u < decltype(u1_c)::value; ++u) {
      const int s = ch * WU + u;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint4 a = hbuf[buf * kFragsPerChunk + ((u * NCB + cb) * 4 + g) * 16 + xi];
        if constexpr (WT == MTP_W_BF16 || WT == MTP_W_BF16_TILED) {
#pragma unroll
          for (int t = 0; t < WTV; ++t)   // weights as A: D[vocab row][hidden row]
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ck.w[t][u]), as_bf16x8(a), c[t][cb], 0, 0, 0);
        } else if constexpr (L::f32) {
          const float a0 = __uint_as_float(a.x), a1 = __uint_as_float(a.y);
          const float a2 = __uint_as_float(a.z), a3 = __uint_as_float(a.w);
#pragma unroll
          for (int t = 0; t < WTV; ++t) {
            const uint4 w = ck.w[t][u];
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), a0, c[t][cb], 0, 0, 0);
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), a1, c[t][cb], 0, 0, 0);
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), a2, c[t][cb], 0, 0, 0);
            c[t][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), a3, c[t][cb], 0, 0, 0);
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

  // ---- epilogue of a pass, bf16 and fp32 heads ------------------------------------------
  // With the weights as the MFMA A operand, lane (i, q) holds for tile t and column block
  // cb the logits of hidden row j = cb*16 + i at the four consecutive vocabulary rows
  // x = 16 tile + 4q + r.  Each lane keeps, for its 8 hidden rows, a running max, argmax,
  // sum-exp (and Gumbel best) over its own vocabulary rows: no lane exchange until the end
  // of the kernel.  A pass that holds a NaN or an infinity goes through full row statistics
  // instead, merged into this wave's LDS slot for the row.
  float* ztok = reinterpret_cast<float*>(static_cast<unsigned char*>(p.ws) + 256);   // drafted-id logits
  float fz[NCB], fm[NCB], fs[NCB], fg[NCB];
  int fi[NCB], fgi[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    fz[cb] = kNegInf; fm[cb] = kNegInf; fs[cb] = 0.0f; fg[cb] = kNegInf;
    fi[cb] = kNoIndex; fgi[cb] = kNoIndex;
  }
  auto epilogue_t = [&](int pass) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));   // keeps per-row addresses out of the compute loop
    const int li = lane_o & 15, q = lane_o >> 4;
    const int tb = t_begin + pass * WTV;
    if (tb >= t_end) return;   // wave-uniform
    bool tval[WTV];
    int x4[WTV];
#pragma unroll
    for (int t = 0; t < WTV; ++t) {
      tval[t] = tb + t < t_end;
      x4[t] = (tb + t) * 16 + 4 * q;
    }
    // bitwise, not short-circuit: 64 branches otherwise
    uint32_t bad = 0;
#pragma unroll
    for (int t = 0; t < WTV; ++t)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bad |= (uint32_t)(tval[t] & (x4[t] + r < p.n_rows)) & (uint32_t)!__builtin_isfinite(c[t][cb][r]);
    const bool all_fin = __all(bad == 0);

    if (p.logits) {   // raw logits: four consecutive ids per lane and row
      const bool vec = (p.logits_stride & 3) == 0;   // rows 16-byte aligned (wave-uniform)
#pragma unroll
      for (int t = 0; t < WTV; ++t) {
        if (!tval[t]) continue;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int j = cb * 16 + li;
          if (j >= M) continue;
          float* dst = p.logits + (long long)j * p.logits_stride + x4[t];
          if (vec && x4[t] + 3 < p.n_rows) {
            *reinterpret_cast<f32x4*>(dst) = c[t][cb];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (x4[t] + r < p.n_rows) dst[r] = c[t][cb][r];
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < WTV; ++t) {   // the drafted-id logits
      if (!tval[t]) continue;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int j = cb * 16 + li, tok = ltok[j];
        if ((tok >= 0) & ((tok & ~3) == x4[t]) & (j < M)) {
          const int r = tok & 3;
          ztok[j] = r == 0 ? c[t][cb][0] : (r == 1 ? c[t][cb][1] : (r == 2 ? c[t][cb][2] : c[t][cb][3]));
        }
      }
    }

    if (all_fin) {
      constexpr float kLog2e = 1.4426950408889634f;
      const float c1 = p.inv_t * kLog2e;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int j = cb * 16 + li;
        const bool rowok = j < M;
        // the pass's logits of row j at this lane; -inf where there is none
        float zv[WTV * 4];
        int xv[WTV * 4];
#pragma unroll
        for (int t = 0; t < WTV; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            xv[4 * t + r] = x4[t] + r;
            zv[4 * t + r] = (rowok & tval[t] & (x4[t] + r < p.n_rows)) ? c[t][cb][r] : kNegInf;
          }
        // max and its lowest id (ids increase with k)
        float zm = zv[0];
        int im = (zv[0] > kNegInf) ? xv[0] : kNoIndex;
#pragma unroll
        for (int k = 1; k < WTV * 4; ++k) {
          const bool up = zv[k] > zm;
          zm = up ? zv[k] : zm;
          im = up ? xv[k] : im;
        }
        if (zm > kNegInf) {
          const bool up = zm > fz[cb];   // a tie keeps the earlier (lower) id
          const float zn = up ? zm : fz[cb];
          fi[cb] = up ? im : fi[cb];
          fz[cb] = zn;
          // sum of exp(z/T - max/T): the old sum rescaled, the new terms added
          const float mn = score_scaled(zn, p.inv_t);
          const float c0 = -mn * kLog2e;
          float acc = fs[cb] * __builtin_amdgcn_exp2f((fm[cb] - mn) * kLog2e);   // 0 while fm = -inf
          if (fm[cb] == kNegInf) acc = 0.0f;
#pragma unroll
          for (int k = 0; k < WTV * 4; ++k) acc += __builtin_amdgcn_exp2f(fmaf(zv[k], c1, c0));
          fs[cb] = acc;
          fm[cb] = mn;
        }
        if (SAMPLED) {
#pragma unroll
          for (int t = 0; t < WTV; ++t) {
            if (!tval[t]) continue;
            // one Philox block = the Gumbel noise of these four ids
            const u32x4 wd = philox4x32_10(u32x4{(uint32_t)x4[t] >> 2, lrow[j], lreq[j], lcyc[j]}, p.key0, p.key1);
            const float gn[4] = {gumbel_from_word(wd.x), gumbel_from_word(wd.y), gumbel_from_word(wd.z),
                                 gumbel_from_word(wd.w)};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float zr = zv[4 * t + r];
              const float sc = score_gumbel(score_scaled(zr, p.inv_t), gn[r]);
              const bool gup = (zr > kNegInf) & better(sc, xv[4 * t + r], fg[cb], fgi[cb]);
              fg[cb] = gup ? sc : fg[cb];
              fgi[cb] = gup ? xv[4 * t + r] : fgi[cb];
            }
          }
        }
      }
    } else {
      // a NaN or infinity in the pass (rare): full statistics per row, merged over the
      // four lanes of the row, then into the wave's LDS slot
      static_for<NCB>([&](auto cb_c) {   // compile-time column blocks: the accumulators stay in registers
        constexpr int cb = decltype(cb_c)::value;
        const int j = cb * 16 + li;
        RowAcc a;
        rowacc_init(a);
#pragma unroll
        for (int t = 0; t < WTV; ++t) {
          if (!tval[t]) continue;
          const f32x4 zz = c[t][cb];
          u32x4 wd = u32x4{0u, 0u, 0u, 0u};
          if (SAMPLED) wd = philox4x32_10(u32x4{(uint32_t)x4[t] >> 2, lrow[j], lreq[j], lcyc[j]}, p.key0, p.key1);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int x = x4[t] + r;
            const float gnr = SAMPLED ? gumbel_from_word(r == 0 ? wd.x : (r == 1 ? wd.y : (r == 2 ? wd.z : wd.w))) : 0.0f;
            if (j < M && x < p.n_rows) rowacc_push<SAMPLED>(a, zz[r], x, p.inv_t, gnr);
          }
        }
        rowacc_merge(a, rowacc_shfl_xor(a, 16));
        rowacc_merge(a, rowacc_shfl_xor(a, 32));
        if (q == 0 && j < M) {
          RowAcc run = lrun[wave * kRows + j];
          rowacc_merge(run, a);
          lrun[wave * kRows + j] = run;
        }
      });
    }
  };
  // end of the kernel: each row's lane states merged over the four lanes that hold it,
  // then with the wave's LDS slot (passes that went the slow way)
  auto finish_t = [&]() {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      Tuple v{fz[cb], fi[cb], fs[cb], fg[cb], fgi[cb]};
      tuple_merge(v, tuple_shfl_xor(v, 16), p.inv_t);
      tuple_merge(v, tuple_shfl_xor(v, 32), p.inv_t);
      const int j = cb * 16 + xi;
      if (g == 0 && j < M) {
        RowAcc run = lrun[wave * kRows + j];
        rowacc_merge(run, tuple_to_rowacc(v, p.inv_t));
        lrun[wave * kRows + j] = run;
      }
    }
  };

  // ---- epilogue of a pass, 4-bit heads --------------------------------------------------
  // (The scales are per vocabulary row, so the weights stay the MFMA B operand.)
  // Lane (xi, g) holds, for tile t of the pass and column block cb, the logits of hidden
  // rows cb*16 + 4g + r at vocabulary row x_t = 16 (tile) + xi.  The lane first merges its
  // WTV logits of each row (one exponential per extra tile).  Half h of the column blocks
  // (cb = 4h .. 4h+3) then gives 16 rows per lane, indexed n = 4 (cb - 4h) + r; a
  // transposed butterfly over the 16 lanes of the row group halves the rows a lane carries
  // at every level (lanes with bit m of xi set keep the upper half), so that lane xi ends
  // up with row n = xi.  Its running state lives in LDS (one slot per wave and row).
  auto epilogue_q = [&](int pass) {
    // the lane coordinates again, opaque to the optimiser: otherwise per-row addresses and
    // indices of this code are hoisted out of the pass loop and held across the whole
    // compute loop
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int xi = lane_o & 15, g = lane_o >> 4;
    const int tb = t_begin + pass * WTV;
    bool tval[WTV], xin[WTV];
    int xs[WTV];
#pragma unroll
    for (int t = 0; t < WTV; ++t) {
      tval[t] = tb + t < t_end;   // wave-uniform
      xs[t] = (tb + t) * 16 + xi;
      xin[t] = tval[t] && xs[t] < p.n_rows;
    }
    if (!tval[0]) return;   // no tile in this pass (wave-uniform)

    // raw logits (sampling needs them) and the drafted-id logits
    if (p.logits) {
#pragma unroll
      for (int t = 0; t < WTV; ++t) {
        float* lrow0 = p.logits + (long long)(4 * g) * p.logits_stride + xs[t];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (xin[t] && cb * 16 + 4 * g + r < M) lrow0[(long long)(cb * 16 + r) * p.logits_stride] = c[t][cb][r];
      }
    }
    bool fin = true;
#pragma unroll
    for (int t = 0; t < WTV; ++t) {
      uint32_t hit = 0;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int4 tk = *reinterpret_cast<const int4*>(ltok + cb * 16 + 4 * g);
        hit |= (uint32_t)(xs[t] == tk.x) << (4 * cb) | (uint32_t)(xs[t] == tk.y) << (4 * cb + 1) |
               (uint32_t)(xs[t] == tk.z) << (4 * cb + 2) | (uint32_t)(xs[t] == tk.w) << (4 * cb + 3);
#pragma unroll
        for (int r = 0; r < 4; ++r) fin = fin & (!xin[t] | (bool)__builtin_isfinite(c[t][cb][r]));   // bitwise
      }
      if (!xin[t]) hit = 0;
      if (hit) {   // rare: a drafted id inside this tile
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((hit >> (4 * cb + r)) & 1u) ztok[cb * 16 + 4 * g + r] = c[t][cb][r];
      }
    }
    const bool all_fin = __all(fin);

    // Gumbel noise of the 16 rows of half h at tile t's 16 vocabulary rows.  One Philox
    // block covers 4 consecutive ids of one row, so the 16 lanes of a row group compute the
    // 64 blocks of their rows once (lane 4m + a: rows n = 4a .. 4a+3, ids 16 tile + 4m ..
    // 4m+3) and hand the values over through this wave's LDS slice; lane xi then reads the
    // noise of row n at gum[(16 g + n) * 16 + xi].
    auto make_noise = [&](int tile, int h) {
      const int m = xi >> 2, a = xi & 3;
#pragma unroll 1
      for (int q = 0; q < 4; ++q) {
        const int j = (4 * h + a) * 16 + 4 * g + q;
        const u32x4 wd = philox4x32_10(u32x4{(uint32_t)(4 * tile + m), lrow[j], lreq[j], lcyc[j]}, p.key0, p.key1);
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

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jo = (4 * h + xi / 4) * 16 + 4 * g + xi % 4;   // the row this lane ends up with
      RowAcc pass_acc;
      // sampled: best z/T + G over the pass's tiles for each of the half's 16 rows
      float gsc[16];
      int gix[16];
      if (SAMPLED) {
#pragma unroll
        for (int n = 0; n < 16; ++n) { gsc[n] = kNegInf; gix[n] = kNoIndex; }
#pragma unroll
        for (int t = 0; t < WTV; ++t) {
          if (!tval[t]) continue;   // wave-uniform
          make_noise(tb + t, h);
#pragma unroll
          for (int n = 0; n < 16; ++n) {
            const int cb = 4 * h + n / 4, r = n % 4;
            const bool ok = xin[t] & (cb * 16 + 4 * g + r < M) & all_fin;
            const float sc = ok ? score_gumbel(score_scaled(c[t][cb][r], p.inv_t), noise(n)) : kNegInf;
            if (better(sc, ok ? xs[t] : kNoIndex, gsc[n], gix[n])) { gsc[n] = sc; gix[n] = xs[t]; }
          }
        }
      }
      // the lane's merged tuple of row n (both tiles)
      auto row_tuple = [&](int n, int cb, int r) -> Tuple {
        Tuple v{kNegInf, kNoIndex, 0.0f, kNegInf, kNoIndex};
#pragma unroll
        for (int t = 0; t < WTV; ++t) {
          const bool ok = xin[t] & (cb * 16 + 4 * g + r < M);
          const Tuple e{ok ? c[t][cb][r] : kNegInf, ok ? xs[t] : kNoIndex, ok ? 1.0f : 0.0f, kNegInf, kNoIndex};
          if (t == 0) v = e; else tuple_merge(v, e, p.inv_t);
        }
        if (SAMPLED) { v.gbest = gsc[n]; v.gidx = gix[n]; }
        return v;
      };
      if (all_fin) {
        // first level (mask 8) straight from the accumulators: rows n and n + 8 are column
        // blocks 4h + n/4 and 4h + n/4 + 2
        const bool hi8 = (xi & 8) != 0;
        Tuple v[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int cb = 4 * h + n / 4, r = n % 4;
          const Tuple lo = row_tuple(n, cb, r), hi = row_tuple(n + 8, cb + 2, r);
          Tuple mine = hi8 ? hi : lo;
          const Tuple recv = tuple_xor16<8>(hi8 ? lo : hi);
          tuple_merge(mine, recv, p.inv_t);
          v[n] = mine;
        }
        auto level = [&](auto mask_c) {
          constexpr int mask = decltype(mask_c)::value, half = mask;
          const bool hi = (xi & mask) != 0;
#pragma unroll
          for (int n = 0; n < half; ++n) {
            Tuple mine = hi ? v[n + half] : v[n];
            const Tuple send = hi ? v[n] : v[n + half];
            const Tuple recv = tuple_xor16<mask>(send);
            tuple_merge(mine, recv, p.inv_t);
            v[n] = mine;
          }
        };
        level(std::integral_constant<int, 4>{});
        level(std::integral_constant<int, 2>{});
        level(std::integral_constant<int, 1>{});
        pass_acc = tuple_to_rowacc(v[0], p.inv_t);
      } else {
        // a NaN or infinity in the pass (rare): full row statistics, one row at a time,
        // with the same pairing of lanes as the butterfly above
        rowacc_init(pass_acc);
#pragma unroll 1
        for (int n = 0; n < 16; ++n) {
          RowAcc a;
          rowacc_init(a);
          const int j = (4 * h + n / 4) * 16 + 4 * g + n % 4;
#pragma unroll
          for (int t = 0; t < WTV; ++t) {
            if (!tval[t]) continue;   // wave-uniform
            if (SAMPLED) make_noise(tb + t, h);
            float z = c[t][4 * h][0];
#pragma unroll
            for (int q = 1; q < 16; ++q) z = (n == q) ? c[t][4 * h + q / 4][q % 4] : z;
            if (xin[t] && j < M) rowacc_push<SAMPLED>(a, z, xs[t], p.inv_t, SAMPLED ? noise(n) : 0.0f);
          }
          rowacc_merge(a, rowacc_xor16<8>(a));
          rowacc_merge(a, rowacc_xor16<4>(a));
          rowacc_merge(a, rowacc_xor16<2>(a));
          rowacc_merge(a, rowacc_xor16<1>(a));
          if (xi == n) pass_acc = a;
        }
      }
      RowAcc run = lrun[wave * kRows + jo];
      rowacc_merge(run, pass_acc);
      lrun[wave * kRows + jo] = run;
    }
  };

  // ---- pipeline.  Chunk it's weights are issued NB-1 chunks ahead (NB register
  //      buffers); its hidden fragments are loaded into registers at the end of chunk
  //      it-2 and written to LDS (double buffer) at the end of chunk it-1.  Loads retire
  //      in issue order, so the hidden loads are issued last in each chunk: waiting for
  //      them never waits for weights issued after them.  One barrier per chunk; the
  //      epilogue of a pass runs with the next pass's first chunks in flight.  A pass has
  //      a multiple of NB chunks; chunks past the end of K only keep the pipeline in step.
  Chunk Wb[NB];
  Staged S;
  stage_load(S, 0);
  stage_store(S, 0);
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k) load(Wb[k], k);
  stage_load(S, 1 % nch);
  __syncthreads();
  int it = 0;
  auto step = [&](Chunk& cur, Chunk& ahead, int ch) {
    load(ahead, it + NB - 1);
    // the next chunk's hidden fragments go to LDS between the two halves of this chunk's
    // MFMAs, so that the LDS writes overlap the second half
    const bool act = ch * WU < nsteps;
    if (act) comp(cur, ch, it & 1, std::integral_constant<int, 0>{}, std::integral_constant<int, WU / 2>{});
    stage_store(S, (it + 1) & 1);
    if (act) comp(cur, ch, it & 1, std::integral_constant<int, WU / 2>{}, std::integral_constant<int, WU>{});
    stage_load(S, (ch + 2) % nch);
    __syncthreads();
    ++it;
  };
  for (int pass = 0; pass < npass; ++pass) {
    zero_acc();
    for (int ch = 0; ch < nch; ch += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) step(Wb[k], Wb[(k + NB - 1) % NB], ch + k);
    }
    if constexpr (L::q4) epilogue_q(pass); else epilogue_t(pass);
  }
  if constexpr (!L::q4) finish_t();

  // ---- block partial per row: the waves' states merged in wave order, after every
  //      wave's last epilogue ----------------------------------------------------------
  __syncthreads();
  if (tid < M) {
    RowAcc a = lrun[tid];
    for (int w = 1; w < kWaves; ++w) rowacc_merge(a, lrun[w * kRows + tid]);
    // field-major: 16-byte piece i of (row, block) at [i][row][block], so the merge's
    // lanes (consecutive blocks of one row) read contiguous bytes
    u32x4* pf = reinterpret_cast<u32x4*>(static_cast<unsigned char*>(p.ws) + lmhead_partials_offset(M));
    const u32x4* av = reinterpret_cast<const u32x4*>(&a);
#pragma unroll
    for (int i = 0; i < rowacc_pieces<SAMPLED>(); ++i) pf[((size_t)i * M + tid) * gridDim.x + blockIdx.x] = av[i];
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
  const u32x4* pf = reinterpret_cast<const u32x4*>(ws + lmhead_partials_offset(M));
  RowAcc a;
  rowacc_init(a);
  for (int blk = tid; blk < G; blk += kMergeThreads) {
    RowAcc b;
    rowacc_init(b);
    u32x4* bv = reinterpret_cast<u32x4*>(&b);
#pragma unroll
    for (int i = 0; i < rowacc_pieces<SAMPLED>(); ++i) bv[i] = pf[((size_t)i * M + j) * G + blk];
    rowacc_merge(a, b);
  }
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

// Blocks of the wide kernel for a head of n_rows vocabulary rows (a function of n_rows
// only).  Every wave of a block runs the same number of passes, so the kernel takes about
// passes x blocks pass-times of streaming; this picks the block count in
// [lmhead_grid / 2, lmhead_grid] that minimises that product (fewest idle tile slots),
// preferring more blocks on ties.  152,064 rows: 9,504 tiles = 198 blocks x 8 waves x 3
// passes x 2 tiles exactly.
static int wide_grid(int n_rows) {
  const int tiles = (n_rows + 15) / 16;
  const int gmax = lmhead_grid(n_rows);   // the workspace holds this many partials per row
  int best = gmax;
  long long best_cost = -1;
  for (int G = gmax; G >= (gmax + 1) / 2; --G) {
    const long long waves = (long long)G * kWaves;
    const long long per_wave = (tiles + waves - 1) / waves;
    const long long passes = (per_wave + WTV - 1) / WTV;
    const long long cost = passes * G;
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = G; }
  }
  return best;
}

template <int WT, bool SAMPLED>
static hipError_t launch_wide_t(const LmheadLaunch& p, hipStream_t stream) {
  const int G = wide_grid(p.n_rows);
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
  if (p.M < 1 || p.M > kLmheadMaxWideRows || !p.verify) return hipErrorInvalidValue;
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
