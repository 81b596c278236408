// Draft head and verify pass: a skinny LM-head GEMM with a fused softmax / argmax /
// Gumbel-max epilogue.
//
// What it computes (lucebox-hub PR "feat(qwen4exp): MTP speculative decoding",
// section "What"): logits z[j][x] = sum_k W[x][k] h[j][k] for M <= 16 hidden rows j and
// the first n_rows vocabulary rows x of the shared head, then per hidden row the lowest-id
// argmax, max and log-sum-exp of z / T, a Gumbel-max sample at T, and (verify) the logit
// at the drafted id.  The draft head runs it over the first n_draft rows with one hidden
// row per request; the verify pass over all rows with the k+1 rows of every request.
//
// Mapping on gfx950 (wave64, MFMA):
//   * W is the B operand of v_mfma_f32_16x16x32_bf16 (fp32 heads: 16x16x4f32): lane l
//     streams vocabulary row x0 + l%16, 16 bytes of K-slice l/16 per step, so one load
//     instruction reads 16 rows x 64 contiguous bytes; weights are read exactly once.
//   * the hidden rows are the A operand, staged once per block in LDS in fragment order
//     (lane l's 16 bytes of step s at [s][l/16][l%16]), zero for rows >= M;
//   * every logit is one accumulator chain over K in a fixed order that does not depend
//     on M, the grid, or the row's position in the batch;
//   * 4-bit affine heads: nibbles become the bf16 values 128 + q by byte permutes and an
//     and-or with the exponent pattern; one MFMA per 32-value group gives
//     D = sum (128 + q) h, and the group's scale and min are applied after it:
//     z += s * D + (min - 128 s) * sum(h).  Products stay exact in fp32.
//   * epilogue per lane over its vocabulary rows: online max / sum-exp, argmax, Gumbel
//     argmax; then a 16-lane butterfly, a cross-wave merge through LDS, one partial per
//     block, and the last block to finish (atomic ticket) merges the partials in block
//     order.  No floating-point atomics: results are deterministic.
#include "kernels.hpp"
#include "lmhead_common.hpp"

namespace mtp {

namespace {

using namespace lm;

// Launch shape (measured choices): 8 waves per block, one block per CU at most; tiles per
// wave pass and K steps per prefetch chunk per head format.
constexpr int kWaves = 8;            // waves per block (4, one per SIMD, was slower everywhere)
constexpr int kThreads = 64 * kWaves;
constexpr int kTV = 1;               // 16-row vocabulary tiles per wave per pass
constexpr int kU = 8;                // K steps per prefetch chunk
constexpr int kTVQ4 = 2;             // the same for 4-bit heads, whose K steps carry a
constexpr int kUQ4 = 8;              // quarter of the bytes
// 4-bit heads under sampling keep the Gumbel state of four hidden rows live through the K
// loop: one tile per pass keeps them out of scratch (two spilled 128-180 bytes per lane and
// ran 9-11% slower); the one-row draft head holds two without spilling
constexpr int kTVQ4S = 1;

// tiles per wave pass of a launch (RL: accumulator rows a lane holds live)
template <int WT, bool SAMPLED, int RL = 4>
constexpr int tiles_per_pass() {
  return Layout<WT>::q4 ? ((SAMPLED && RL != 1) ? kTVQ4S : kTVQ4) : kTV;
}
constexpr int kMaxGrid = 256;        // blocks per launch (partials per row in the workspace)

// Quad broadcast on the DPP network: every lane of each group of 4 reads lane R's value.
template <int R>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, R * 0x55, 0xF, 0xF, false);
}

// RL: accumulator rows a lane can hold live (row 4g + r exists only if r < M).  4-bit heads
// apply each group's scale and min per accumulator row on the VALU, so a launch of one
// hidden row (the draft head of one request) skips the three rows no lane holds.
template <int WT, bool SAMPLED, bool VERIFY, int RL>
__device__ __forceinline__ void lmhead_body(const LmheadLaunch& p) {
  static_assert(RL == 1 || RL == 4, "one live row or all four");
  static_assert(sizeof(RowAcc) == 48, "partials are three 16-byte vectors");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xi = lane & 15, g = lane >> 4;
  const int M = p.M, d = p.d;
  using L = Layout<WT>;
  constexpr int TV = tiles_per_pass<WT, SAMPLED, RL>();
  constexpr int U = L::q4 ? kUQ4 : kU;
  static_assert(!L::q4 || U % 8 == 0, "4-bit chunks cover whole octets of groups (one scale vector each)");
  const int nsteps = L::f32 ? d / 16 : d / 32;
  // chunks per tile group, rounded up to even for the two-buffer pipeline (a chunk past
  // the end reads out of range, i.e. zeros, and its MFMAs add +0)
  const int nchunks = ((nsteps + U - 1) / U + 1) & ~1;

  uint4* frag = reinterpret_cast<uint4*>(smem);
  const size_t frag_bytes = (size_t)nsteps * 4 * M * 16;
  float* htab = reinterpret_cast<float*>(smem + frag_bytes);
  const size_t htab_bytes = L::q4 ? (size_t)nsteps * 16 * 4 : 0;
  RowAcc* red = reinterpret_cast<RowAcc*>(smem + frag_bytes + htab_bytes);
  int* last_flag = reinterpret_cast<int*>(red + kWaves * 16);

  // ---- this wave's contiguous range of 16-row tiles ------------------------------
  const int tiles = (p.n_rows + 15) >> 4;
  const long long nw = (long long)gridDim.x * kWaves;
  const long long gw = (long long)blockIdx.x * kWaves + wave;
  const int t_begin = (int)(gw * tiles / nw), t_end = (int)((gw + 1) * tiles / nw);

  const unsigned char* wbase = static_cast<const unsigned char*>(p.w);
  const size_t rb = row_bytes<WT>(d);
  const int G32 = d / 32;
  // row-major heads cover n_rows rows; tiled heads whole tiles (rows past vocab are zero)
  const size_t rows_cov = L::tiled ? (size_t)tiles * 16 : (size_t)p.n_rows;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)(rows_cov * rb));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.scale, (uint32_t)(rows_cov * G32 * 2));
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(p.minv, (uint32_t)(rows_cov * G32 * 2));
  const uint32_t tile_bytes = (uint32_t)(16 * rb);

  // per-lane base offsets in tile group tb (kOOB: reads zeros):
  //   row-major: the lane's weight row; tiled: the tile's first block plus the lane's 16 B
  auto row_offsets = [&](int tb, uint32_t (&roff)[TV]) {
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      const int x = (tb + t) * 16 + xi;
      if constexpr (L::tiled)
        roff[t] = (tb + t) < t_end ? (uint32_t)(tb + t) * tile_bytes + (uint32_t)(lane * 16) : kOOB;
      else
        roff[t] = ((tb + t) < t_end && x < p.n_rows) ? (uint32_t)((size_t)x * rb) : kOOB;
    }
  };

  // ---- loads and MFMA steps of one chunk (U K-steps of TV tiles) -----------------
  // valid offsets are < 2^31 (the host caps a head at 2 GiB): OR-ing in the top bit moves a
  // step past the end out of range without a branch, so the compiler counts loads exactly
  typedef typename std::conditional<L::q4, uint32_t, uint4>::type WFrag;
  struct Chunk {
    WFrag w[TV][U];
    uint4 sc[TV][(U + 7) / 8], mn[TV][(U + 7) / 8];   // 4-bit heads: scales and mins, 8 groups each
  };
  auto load = [&](Chunk& ck, const uint32_t (&roff)[TV], int s0) {
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      if constexpr (WT == MTP_W_Q4A32_TILED) {
        // one KiB block per group quad: four groups' nibble words per lane
#pragma unroll
        for (int u = 0; u < U; u += 4) {
          const uint32_t oob = s0 + u < nsteps ? 0u : kOOB;
          const uint4 v = bload16_stream(wr, (roff[t] | oob) + (uint32_t)((s0 + u) / 4) * 1024u);
          ck.w[t][u] = v.x; ck.w[t][u + 1] = v.y; ck.w[t][u + 2] = v.z; ck.w[t][u + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int s = s0 + u;
          const uint32_t oob = s < nsteps ? 0u : kOOB;
          if constexpr (WT == MTP_W_Q4A32)
            ck.w[t][u] = bload4(wr, (roff[t] | oob) + (uint32_t)((4 * s + g) * 4));
          else if constexpr (WT == MTP_W_BF16_TILED)
            ck.w[t][u] = bload16_stream(wr, (roff[t] | oob) + (uint32_t)s * 1024u);
          else
            ck.w[t][u] = bload16(wr, (roff[t] | oob) + (uint32_t)((4 * s + g) * 16));
        }
      }
      if constexpr (L::q4) {
        uint32_t so;
        if constexpr (L::tiled)   // block (tile, octet) of 256 B, 16 B per row
          so = roff[t] == kOOB ? kOOB : (roff[t] - (uint32_t)(lane * 16)) / 8u + (uint32_t)(xi * 16);
        else
          so = roff[t] == kOOB ? kOOB : (roff[t] / (uint32_t)rb) * (uint32_t)(G32 * 2);
#pragma unroll
        for (int o = 0; o < (U + 7) / 8; ++o) {
          const int s = s0 + 8 * o;
          const uint32_t oob = s < nsteps ? 0u : kOOB;
          const uint32_t step = L::tiled ? (uint32_t)(s / 8) * 256u : (uint32_t)(s * 2);
          ck.sc[t][o] = bload16(sr, (so | oob) + step);
          ck.mn[t][o] = bload16(mr, (so | oob) + step);
        }
      }
    }
  };
  f32x4 c[TV];
  auto comp = [&](const Chunk& ck, int s0) {
    // 4-bit heads: d is a multiple of 256 and a chunk a multiple of 8 K steps, so a chunk
    // is either inside K or wholly past it (wave-uniform)
    if (L::q4 && s0 >= nsteps) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      const uint4 a = (xi < M && s < nsteps) ? frag[(s * 4 + g) * M + xi] : uint4{0u, 0u, 0u, 0u};
      if constexpr (WT == MTP_W_BF16 || WT == MTP_W_BF16_TILED) {
#pragma unroll
        for (int t = 0; t < TV; ++t)
          c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(ck.w[t][u]), c[t], 0, 0, 0);
      } else if constexpr (L::f32) {
        const float a0 = __uint_as_float(a.x), a1 = __uint_as_float(a.y);
        const float a2 = __uint_as_float(a.z), a3 = __uint_as_float(a.w);
#pragma unroll
        for (int t = 0; t < TV; ++t) {
          const uint4 w = ck.w[t][u];
          c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, __uint_as_float(w.x), c[t], 0, 0, 0);
          c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, __uint_as_float(w.y), c[t], 0, 0, 0);
          c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, __uint_as_float(w.z), c[t], 0, 0, 0);
          c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, __uint_as_float(w.w), c[t], 0, 0, 0);
        }
      } else {
        // 4-bit affine: D = sum (128 + q) h over the group, then z += s D + (min - 128 s) sum(h)
        const f32x4 hs = *reinterpret_cast<const f32x4*>(htab + s * 16 + 4 * g);
#pragma unroll
        for (int t = 0; t < TV; ++t) {
          const f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(a), as_bf16x8(q4_expand(ck.w[t][u])), f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          const uint4 sq = ck.sc[t][u / 8], mq = ck.mn[t][u / 8];
          const int uo = u % 8;
          const uint32_t sw = (uo < 2) ? sq.x : (uo < 4) ? sq.y : (uo < 6) ? sq.z : sq.w;
          const uint32_t mw = (uo < 2) ? mq.x : (uo < 4) ? mq.y : (uo < 6) ? mq.z : mq.w;
          const float sv = bf16_to_f32((uint16_t)((u & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
          const float mv = bf16_to_f32((uint16_t)((u & 1) ? (mw >> 16) : (mw & 0xFFFFu)));
          const float off = mv - 128.0f * sv;
#pragma unroll
          for (int r = 0; r < RL; ++r) c[t][r] = fmaf(off, hs[r], fmaf(sv, D[r], c[t][r]));
        }
      }
    }
  };

  // ---- stage the hidden rows as A-operand fragments, with the first weight chunk in
  //      flight.  Loads retire in issue order: the hidden loads go out first and all
  //      together (up to kPreFrags per thread, which covers d = 2560 at 16 rows), so
  //      writing them to LDS waits for neither the weights nor a chain of round trips.
  const int nfrag = nsteps * 4 * M;
  auto hfrag = [&](int f) {
    const int i = f % M, sg = f / M, gg = sg & 3, s = sg >> 2;
    uint4 v;
    if (L::f32) {
      v = *reinterpret_cast<const uint4*>(static_cast<const float*>(p.hidden) + (size_t)i * d + 16 * s + 4 * gg);
    } else {
      v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.hidden) + (size_t)i * d + 32 * s + 8 * gg);
      if (L::q4) v = q4_order(v);
    }
    return v;
  };
  Chunk A, B;
  uint32_t roff_cur[TV], roff_nxt[TV];
  if constexpr (!L::q4) {
    constexpr int kPreFrags = 80 / kWaves;   // d = 2560 at 16 rows: 5,120 fragments per block
    uint4 hv[kPreFrags];
#pragma unroll
    for (int q = 0; q < kPreFrags; ++q)
      if (tid + q * kThreads < nfrag) hv[q] = hfrag(tid + q * kThreads);
    row_offsets(t_begin, roff_cur);
    load(A, roff_cur, 0);
#pragma unroll
    for (int q = 0; q < kPreFrags; ++q)
      if (tid + q * kThreads < nfrag) frag[tid + q * kThreads] = hv[q];
    for (int f = tid + kPreFrags * kThreads; f < nfrag; f += kThreads) frag[f] = hfrag(f);
  } else {
    // 4-bit heads: a thread stages the four quarters of one (step, row) unit and their group
    // sum (the factor of the group's min), so the sums cost no extra round trip to memory
    const int nunit = nsteps * M;
    const uint16_t* hid = static_cast<const uint16_t*>(p.hidden);
    auto unit_load = [&](int unit, uint4 (&v)[4]) {
      const int s = unit / M, i = unit % M;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) v[gg] = *reinterpret_cast<const uint4*>(hid + (size_t)i * d + 32 * s + 8 * gg);
    };
    auto unit_store = [&](int unit, const uint4 (&v)[4]) {
      const int s = unit / M, i = unit % M;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) frag[(s * 4 + gg) * M + i] = q4_order(v[gg]);
      htab[s * 16 + i] = group_sum_quarters(v);
    };
    constexpr int kPreUnits = 3;   // d = 2560 at 16 rows: 1,280 units per block
    uint4 hv[kPreUnits][4];
#pragma unroll
    for (int q = 0; q < kPreUnits; ++q)
      if (tid + q * kThreads < nunit) unit_load(tid + q * kThreads, hv[q]);
    row_offsets(t_begin, roff_cur);
    load(A, roff_cur, 0);
#pragma unroll
    for (int q = 0; q < kPreUnits; ++q)
      if (tid + q * kThreads < nunit) unit_store(tid + q * kThreads, hv[q]);
    for (int unit = tid + kPreUnits * kThreads; unit < nunit; unit += kThreads) {
      uint4 v[4];
      unit_load(unit, v);
      unit_store(unit, v);
    }
    // rows no launch row occupies
    for (int e = tid; e < nsteps * 16; e += kThreads)
      if ((e & 15) >= M) htab[e] = 0.0f;
  }
  __syncthreads();

  // ---- per-lane hidden rows: j = 4g + r -----------------------------------------
  int tok[4];
  uint32_t prow[4], preq[4], pcyc[4];
  bool rvalid[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * g + r;
    rvalid[r] = j < M;
    const int b = j / p.rows_per_req, i = j % p.rows_per_req;
    // counter words 1 and 3 of the row's draws: (stream, row) and the cycle, or for the
    // trunk's own sample under exact-match acceptance (stream 3) the absolute position
    const bool bypos = VERIFY && p.positions != nullptr;
    prow[r] = bypos ? (uint32_t)(kStreamTrunk << 8) : (uint32_t)(p.stream_id << 8) | (uint32_t)(i + p.row_base);
    preq[r] = p.request_base + (uint32_t)b;
    pcyc[r] = (bypos && rvalid[r]) ? (uint32_t)(p.positions[b] + i) : p.cycle;
    tok[r] = (VERIFY && rvalid[r] && i < p.k) ? p.drafts[(size_t)b * p.k_max + i] : -1;
  }
  // Gumbel draws of ids x = 4m..4m+3 for one hidden row are the four words of one Philox
  // block, and lanes 4m..4m+3 of a 16-lane row hold those ids for the same four hidden
  // rows: lane 4m+e computes the block of row 4g+e and the quad exchanges the words (the
  // same draws at a quarter of the Philox work).  Used when the ids are the rows (verify,
  // or a draft head without an id list) and there is more than one hidden row.
  const bool quad_draws = SAMPLED && (VERIFY || p.ids == nullptr) && M > 1;
  const int qe = xi & 3;
  uint32_t prow_q = prow[0], preq_q = preq[0], pcyc_q = pcyc[0];
#pragma unroll
  for (int r = 1; r < 4; ++r)
    if (qe == r) { prow_q = prow[r]; preq_q = preq[r]; pcyc_q = pcyc[r]; }

  RowAcc acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rowacc_init(acc[r]);

  // ---- stream the tile groups; the next group's first chunk overlaps the epilogue --
  for (int tb = t_begin; tb < t_end; tb += TV) {
    row_offsets(tb + TV, roff_nxt);
#pragma unroll
    for (int t = 0; t < TV; ++t) c[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int ch = 0; ch < nchunks; ch += 2) {
      load(B, roff_cur, (ch + 1) * U);
      comp(A, ch * U);
      const bool more = ch + 2 < nchunks;
      uint32_t ro[TV];
#pragma unroll
      for (int t = 0; t < TV; ++t) ro[t] = more ? roff_cur[t] : roff_nxt[t];
      load(A, ro, more ? (ch + 2) * U : 0);
      comp(B, (ch + 1) * U);
    }

    // epilogue: this tile group's logits for the lane's four hidden rows
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      const int x = (tb + t) * 16 + xi;
      if ((tb + t) >= t_end) continue;   // wave-uniform: every lane takes part in the exchange
      float gq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (SAMPLED && quad_draws) {
        const u32x4 wd = philox4x32_10(u32x4{(uint32_t)x >> 2, prow_q, preq_q, pcyc_q}, p.key0, p.key1);
        auto word_of = [&](auto rc) {   // word qe of row rc's block, from lane rc of the quad
          constexpr int R = decltype(rc)::value;
          const uint32_t w0 = quad_bcast<R>(wd.x), w1 = quad_bcast<R>(wd.y);
          const uint32_t w2 = quad_bcast<R>(wd.z), w3 = quad_bcast<R>(wd.w);
          return qe == 0 ? w0 : (qe == 1 ? w1 : (qe == 2 ? w2 : w3));
        };
        const uint32_t wq[4] = {word_of(std::integral_constant<int, 0>{}), word_of(std::integral_constant<int, 1>{}),
                                word_of(std::integral_constant<int, 2>{}), word_of(std::integral_constant<int, 3>{})};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (rvalid[r]) gq[r] = gumbel_from_word(wq[r]);
      }
      if (x >= p.n_rows) continue;
      // a draft head gathered from a set of ids: its row x stands for vocabulary id
      // ids[x]; ids and draws refer to the vocabulary, the stored logits to the row
      const int xv = (!VERIFY && p.ids) ? p.ids[x] : x;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!rvalid[r]) continue;
        const int j = 4 * g + r;
        const float z = c[t][r];
        float gn = gq[r];
        if (SAMPLED && !quad_draws) {
          const u32x4 wd = philox4x32_10(u32x4{(uint32_t)xv >> 2, prow[r], preq[r], pcyc[r]}, p.key0, p.key1);
          const int sel = xv & 3;
          gn = gumbel_from_word(sel == 0 ? wd.x : (sel == 1 ? wd.y : (sel == 2 ? wd.z : wd.w)));
        }
        rowacc_push<SAMPLED>(acc[r], z, xv, p.inv_t, gn);
        if (p.logits) p.logits[(long long)j * p.logits_stride + x] = z;
        if (VERIFY && x == tok[r])
          store_coherent(reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(p.ws) + 256) + j, __float_as_uint(z));
      }
    }
#pragma unroll
    for (int t = 0; t < TV; ++t) roff_cur[t] = roff_nxt[t];
  }

  // ---- reduce: 16 lanes of a row group, then the block's waves -------------------
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!rvalid[r]) continue;   // uniform over the 16 lanes the butterfly reads
    rowacc_merge(acc[r], rowacc_xor16<1>(acc[r]));
    rowacc_merge(acc[r], rowacc_xor16<2>(acc[r]));
    rowacc_merge(acc[r], rowacc_xor16<4>(acc[r]));
    rowacc_merge(acc[r], rowacc_xor16<8>(acc[r]));
  }
  if (xi == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (rvalid[r]) red[wave * 16 + 4 * g + r] = acc[r];
  }
  __syncthreads();

  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  unsigned int* counter = reinterpret_cast<unsigned int*>(ws);
  float* ztok = reinterpret_cast<float*>(ws + 256);
  const size_t part_off = lmhead_partials_offset(M);
  const int G = gridDim.x;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(ws + part_off, (uint32_t)((size_t)G * M * sizeof(RowAcc)));
  if (tid < M) {
    RowAcc a = red[tid];
    for (int w = 1; w < kWaves; ++w) rowacc_merge(a, red[w * 16 + tid]);
    store_partial_fm<rowacc_pieces<SAMPLED>()>(pr, tid, blockIdx.x, M, G, a);
  }
  wait_stores();
  __syncthreads();
  if (tid == 0) *last_flag = (take_ticket(counter) == (unsigned)G - 1);
  __syncthreads();
  if (!*last_flag) return;

  // ---- last block: wave w merges rows w, w + kWaves, ... (M <= 16): 4 partials per lane
  //      in block order, then a butterfly over the 64 lanes (DPP inside rows of 16,
  //      exchanges across them).  One fixed tree for every row and every M, so a row's
  //      statistics do not depend on the launch size.  The rows' chains are interleaved
  //      step by step, and every partial load (and the drafted-id logit) goes out before the
  //      first merge: these loads bypass the caches and each round trip is long.
  constexpr int RPW = kLmheadMaxRows / kWaves;   // rows per wave
  static_assert(RPW * kWaves == kLmheadMaxRows && kMaxGrid <= 4 * 64, "whole rows per wave, 4 partials per lane");
  {
    constexpr int NP = kMaxGrid / 64;
    int jr[RPW];
    bool live[RPW];   // wave-uniform: a chain runs only when it has a row (chain 0 always)
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      jr[r] = wave + kWaves * r;
      live[r] = r == 0 || jr[r] < M;
    }
    RowAcc part[RPW][NP];
    uint32_t zbits[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int blk = lane + 64 * q;
        if (jr[r] < M && blk < G) part[r][q] = load_partial_fm<rowacc_pieces<SAMPLED>()>(pr, jr[r], blk, M, G);
        else rowacc_init(part[r][q]);
      }
      zbits[r] = (VERIFY && jr[r] < M) ? load_coherent(reinterpret_cast<const uint32_t*>(ztok) + jr[r]) : 0u;
    }
    RowAcc a[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) a[r] = part[r][0];
#pragma unroll
    for (int q = 1; q < NP; ++q)
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        if (live[r]) rowacc_merge(a[r], part[r][q]);
    // one butterfly step on every chain; the exchange reads a lane's partner before the
    // merge writes
    auto bfly = [&](auto xchg) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        if (live[r]) {
          const RowAcc o = xchg(a[r]);
          rowacc_merge(a[r], o);
        }
    };
    bfly([](const RowAcc& x) { return rowacc_xor16<1>(x); });
    bfly([](const RowAcc& x) { return rowacc_xor16<2>(x); });
    bfly([](const RowAcc& x) { return rowacc_xor16<4>(x); });
    bfly([](const RowAcc& x) { return rowacc_xor16<8>(x); });
    bfly([](const RowAcc& x) { return rowacc_shfl_xor(x, 16); });
    bfly([](const RowAcc& x) { return rowacc_shfl_xor(x, 32); });
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int j = jr[r];
      if (j >= M || lane != 0) continue;
      mtp_row_stats st = finalize_row(a[r], SAMPLED);
      const uint32_t fl = st.flags;
      if (VERIFY) {
        const int b = j / p.rows_per_req, i = j % p.rows_per_req;
        const int t = (i < p.k) ? p.drafts[(size_t)b * p.k_max + i] : -1;
        st.z_tok = (t >= 0 && t < p.n_rows && !(fl & MTP_ROW_INVALID)) ? sanitize(__uint_as_float(zbits[r]), fl)
                                                                         : kNegInf;
      } else {
        st.z_tok = (fl & MTP_ROW_POSINF) ? 0.0f : ((fl & MTP_ROW_INVALID) ? kNegInf : (SAMPLED ? a[r].gz : a[r].zmax));
        p.tokens[(size_t)j * p.k_max + p.row_base] = st.sample;
      }
      p.stats[(size_t)j * p.out_stride + p.out_offset] = st;
    }
  }
  if (tid == 0) store_coherent(counter, 0u);
}

}  // namespace

template <int WT, bool SAMPLED, int RL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void mtp_draft_head_kernel(LmheadLaunch p) {
  lmhead_body<WT, SAMPLED, false, RL>(p);
}

template <int WT, bool SAMPLED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void mtp_verify_logits_kernel(LmheadLaunch p) {
  lmhead_body<WT, SAMPLED, true, 4>(p);
}

int lmhead_grid(int n_rows) {
  const int tiles = (n_rows + 15) / 16;
  const int g = (tiles + 7) / 8;   // the workspace's partials per row: one per 8 tiles, at most 256
  return g < 1 ? 1 : (g > kMaxGrid ? kMaxGrid : g);
}

size_t lmhead_ws_bytes(int M, int n_rows) {
  return lmhead_partials_offset(M) + (size_t)lmhead_grid(n_rows) * M * kPartialBytes;
}

static size_t lmhead_lds_bytes(int wtype, int d, int M) {
  const int nsteps = wtype == MTP_W_F32 ? d / 16 : d / 32;
  size_t b = (size_t)nsteps * 4 * M * 16;
  if (wtype == MTP_W_Q4A32 || wtype == MTP_W_Q4A32_TILED) b += (size_t)nsteps * 16 * 4;
  return b + kWaves * 16 * sizeof(RowAcc) + 16;
}

// Blocks of one launch (a function of the vocabulary rows only, so a row's merge order never
// depends on the launch size).  A wave takes its tiles TV at a time, so the launch lasts
// about (passes of its busiest wave) x blocks pass-times of streaming: pick the block count
// in [lmhead_grid / 2, lmhead_grid] that minimises that product, preferring more blocks on
// ties.  152,064 rows: 9,504 tiles = 198 blocks x 8 waves x 6 tiles exactly (256 blocks
// would give some waves 5 tiles and others 4).
static int lmhead_launch_grid(int n_rows, int tv) {
  const int tiles = (n_rows + 15) / 16;
  const int gmax = lmhead_grid(n_rows);   // the workspace holds this many partials per row
  int best = gmax;
  long long best_cost = -1;
  for (int G = gmax; G >= (gmax + 1) / 2; --G) {
    const long long waves = (long long)G * kWaves;
    const long long passes = ((tiles + waves - 1) / waves + tv - 1) / tv;
    const long long cost = passes * G;
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = G; }
  }
  return best;
}

template <int WT, bool SAMPLED>
static hipError_t launch_t(const LmheadLaunch& p, hipStream_t stream) {
  // the one-row specialisation only changes 4-bit heads' code
  const bool one_row = Layout<WT>::q4 && !p.verify && p.M == 1;
  const int G = lmhead_launch_grid(p.n_rows, one_row ? tiles_per_pass<WT, SAMPLED, 1>() : tiles_per_pass<WT, SAMPLED, 4>());
  const size_t lds = lmhead_lds_bytes(WT, p.d, p.M);
  auto kern = p.verify ? mtp_verify_logits_kernel<WT, SAMPLED> : mtp_draft_head_kernel<WT, SAMPLED, 4>;
  if constexpr (Layout<WT>::q4)
    if (one_row) kern = mtp_draft_head_kernel<WT, SAMPLED, 1>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(G), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_lmhead(const LmheadLaunch& p, hipStream_t stream) {
  switch (p.wtype) {
    case MTP_W_F32: return p.sampled ? launch_t<MTP_W_F32, true>(p, stream) : launch_t<MTP_W_F32, false>(p, stream);
    case MTP_W_BF16: return p.sampled ? launch_t<MTP_W_BF16, true>(p, stream) : launch_t<MTP_W_BF16, false>(p, stream);
    case MTP_W_Q4A32: return p.sampled ? launch_t<MTP_W_Q4A32, true>(p, stream) : launch_t<MTP_W_Q4A32, false>(p, stream);
    case MTP_W_BF16_TILED:
      return p.sampled ? launch_t<MTP_W_BF16_TILED, true>(p, stream) : launch_t<MTP_W_BF16_TILED, false>(p, stream);
    case MTP_W_Q4A32_TILED:
      return p.sampled ? launch_t<MTP_W_Q4A32_TILED, true>(p, stream) : launch_t<MTP_W_Q4A32_TILED, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t lmhead_lds_bytes_for(int wtype, int d, int M) { return lmhead_lds_bytes(wtype, d, M); }

}  // namespace mtp
