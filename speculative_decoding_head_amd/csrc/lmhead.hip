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
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {

constexpr int kWaves = kLmheadThreads / 64;
constexpr int TV = 2;   // 16-row vocabulary tiles per wave per pass
constexpr int U = 8;    // K steps per prefetch chunk
constexpr int kMaxGrid = 512;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// eight 4-bit codes (element 2m in the low nibble of byte m) -> bf16 values 128 + q, in
// the lane order [q0, q2, q1, q3, q4, q6, q5, q7]
__device__ __forceinline__ uint4 q4_expand(uint32_t w) {
  const uint32_t lo = __builtin_amdgcn_perm(0u, w, 0x0c010c00u);   // bytes 0,1 -> 16-bit lanes
  const uint32_t hi = __builtin_amdgcn_perm(0u, w, 0x0c030c02u);   // bytes 2,3
  const uint32_t m = 0x000F000Fu, e = 0x43004300u;
  return uint4{(lo & m) | e, ((lo >> 4) & m) | e, (hi & m) | e, ((hi >> 4) & m) | e};
}

// the same lane order applied to eight bf16 hidden values
__device__ __forceinline__ uint4 q4_order(uint4 v) {
  return uint4{(v.x & 0xFFFFu) | (v.y << 16), (v.x >> 16) | (v.y & 0xFFFF0000u),
               (v.z & 0xFFFFu) | (v.w << 16), (v.z >> 16) | (v.w & 0xFFFF0000u)};
}

template <int WT>
__device__ __forceinline__ size_t row_bytes(int d) {
  return WT == MTP_W_F32 ? (size_t)d * 4 : (WT == MTP_W_BF16 ? (size_t)d * 2 : (size_t)d / 2);
}

template <int WT, bool SAMPLED, bool VERIFY>
__device__ __forceinline__ void lmhead_body(const LmheadLaunch& p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xi = lane & 15, g = lane >> 4;
  const int M = p.M, d = p.d;
  const int nsteps = (WT == MTP_W_F32) ? d / 16 : d / 32;

  uint4* frag = reinterpret_cast<uint4*>(smem);
  const size_t frag_bytes = (size_t)nsteps * 4 * M * 16;
  float* htab = reinterpret_cast<float*>(smem + frag_bytes);
  const size_t htab_bytes = (WT == MTP_W_Q4A32) ? (size_t)nsteps * 16 * 4 : 0;
  RowAcc* red = reinterpret_cast<RowAcc*>(smem + frag_bytes + htab_bytes);
  int* last_flag = reinterpret_cast<int*>(red + kWaves * 16);

  // ---- stage the hidden rows as A-operand fragments -------------------------------
  const int nfrag = nsteps * 4 * M;
  for (int f = tid; f < nfrag; f += kLmheadThreads) {
    const int i = f % M, sg = f / M, gg = sg & 3, s = sg >> 2;
    uint4 v;
    if (WT == MTP_W_F32) {
      v = *reinterpret_cast<const uint4*>(static_cast<const float*>(p.hidden) + (size_t)i * d + 16 * s + 4 * gg);
    } else {
      v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.hidden) + (size_t)i * d + 32 * s + 8 * gg);
      if (WT == MTP_W_Q4A32) v = q4_order(v);
    }
    frag[f] = v;
  }
  if (WT == MTP_W_Q4A32) {
    // per 32-value group and hidden row: sum of the hidden values, in k order
    for (int e = tid; e < nsteps * 16; e += kLmheadThreads) {
      const int s = e >> 4, i = e & 15;
      float acc = 0.0f;
      if (i < M) {
        const uint16_t* h = static_cast<const uint16_t*>(p.hidden) + (size_t)i * d + 32 * s;
        for (int kk = 0; kk < 32; ++kk) acc += bf16_to_f32(h[kk]);
      }
      htab[e] = acc;
    }
  }
  __syncthreads();

  // ---- per-lane hidden rows: j = 4g + r -----------------------------------------
  int tok[4];
  uint32_t prow[4], preq[4];
  bool rvalid[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * g + r;
    rvalid[r] = j < M;
    const int b = j / p.rows_per_req, i = j % p.rows_per_req;
    prow[r] = (uint32_t)(p.stream_id << 8) | (uint32_t)(i + p.row_base);
    preq[r] = p.request_base + (uint32_t)b;
    tok[r] = (VERIFY && rvalid[r] && i < p.k) ? p.drafts[(size_t)b * p.k_max + i] : -1;
  }

  // ---- this wave's contiguous range of 16-row tiles ------------------------------
  const int tiles = (p.n_rows + 15) >> 4;
  const long long nw = (long long)gridDim.x * kWaves;
  const long long gw = (long long)blockIdx.x * kWaves + wave;
  const int t_begin = (int)(gw * tiles / nw), t_end = (int)((gw + 1) * tiles / nw);

  const unsigned char* wbase = static_cast<const unsigned char*>(p.w);
  const size_t rb = row_bytes<WT>(d);
  const int G32 = d / 32;

  RowAcc acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rowacc_init(acc[r]);

  for (int tb = t_begin; tb < t_end; tb += TV) {
    const unsigned char* rowp[TV];
    bool tv[TV];
    int xr[TV];
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      tv[t] = (tb + t) < t_end;
      xr[t] = (tb + t) * 16 + xi;
      const int xc = min(xr[t], p.n_rows - 1);
      rowp[t] = wbase + (size_t)xc * rb;
    }
    f32x4 c[TV];
#pragma unroll
    for (int t = 0; t < TV; ++t) c[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if constexpr (WT == MTP_W_BF16 || WT == MTP_W_F32) {
      uint4 bufA[TV][U], bufB[TV][U];
      auto load = [&](uint4 (&buf)[TV][U], int s0) {
#pragma unroll
        for (int t = 0; t < TV; ++t)
          if (tv[t]) {
            const uint4* row = reinterpret_cast<const uint4*>(rowp[t]);
#pragma unroll
            for (int u = 0; u < U; ++u) buf[t][u] = row[4 * (s0 + u) + g];
          }
      };
      auto step = [&](const uint4 (&wv)[TV], int s) {
        const uint4 a = (xi < M) ? frag[(s * 4 + g) * M + xi] : uint4{0u, 0u, 0u, 0u};
        if constexpr (WT == MTP_W_BF16) {
#pragma unroll
          for (int t = 0; t < TV; ++t)
            c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(wv[t]), c[t], 0, 0, 0);
        } else {
          const float a0 = __uint_as_float(a.x), a1 = __uint_as_float(a.y);
          const float a2 = __uint_as_float(a.z), a3 = __uint_as_float(a.w);
#pragma unroll
          for (int t = 0; t < TV; ++t) {
            c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, __uint_as_float(wv[t].x), c[t], 0, 0, 0);
            c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, __uint_as_float(wv[t].y), c[t], 0, 0, 0);
            c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, __uint_as_float(wv[t].z), c[t], 0, 0, 0);
            c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, __uint_as_float(wv[t].w), c[t], 0, 0, 0);
          }
        }
      };
      auto comp = [&](const uint4 (&buf)[TV][U], int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint4 wv[TV];
#pragma unroll
          for (int t = 0; t < TV; ++t) wv[t] = buf[t][u];
          step(wv, s0 + u);
        }
      };
      const int nchunks = nsteps / U;
      if (nchunks > 0) load(bufA, 0);
      for (int ch = 0; ch < nchunks; ch += 2) {
        if (ch + 1 < nchunks) load(bufB, (ch + 1) * U);
        comp(bufA, ch * U);
        if (ch + 2 < nchunks) load(bufA, (ch + 2) * U);
        if (ch + 1 < nchunks) comp(bufB, (ch + 1) * U);
      }
      for (int s = nchunks * U; s < nsteps; ++s) {
        uint4 wv[TV];
#pragma unroll
        for (int t = 0; t < TV; ++t)
          wv[t] = tv[t] ? reinterpret_cast<const uint4*>(rowp[t])[4 * s + g] : uint4{0u, 0u, 0u, 0u};
        step(wv, s);
      }
    } else {
      // 4-bit affine: U groups per chunk; scales and mins of U groups are one 16-byte load
      uint32_t nibA[TV][U], nibB[TV][U];
      uint4 scA[TV], mnA[TV], scB[TV], mnB[TV];
      const uint16_t* scale_rows[TV];
      const uint16_t* min_rows[TV];
#pragma unroll
      for (int t = 0; t < TV; ++t) {
        const int xc = min(xr[t], p.n_rows - 1);
        scale_rows[t] = p.scale + (size_t)xc * G32;
        min_rows[t] = p.minv + (size_t)xc * G32;
      }
      auto load = [&](uint32_t (&nib)[TV][U], uint4 (&sc)[TV], uint4 (&mn)[TV], int s0) {
#pragma unroll
        for (int t = 0; t < TV; ++t)
          if (tv[t]) {
            const uint32_t* row = reinterpret_cast<const uint32_t*>(rowp[t]);
#pragma unroll
            for (int u = 0; u < U; ++u) nib[t][u] = row[4 * (s0 + u) + g];
            sc[t] = *reinterpret_cast<const uint4*>(scale_rows[t] + s0);
            mn[t] = *reinterpret_cast<const uint4*>(min_rows[t] + s0);
          }
      };
      auto comp = [&](const uint32_t (&nib)[TV][U], const uint4 (&sc)[TV], const uint4 (&mn)[TV], int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int s = s0 + u;
          const uint4 a = (xi < M) ? frag[(s * 4 + g) * M + xi] : uint4{0u, 0u, 0u, 0u};
          const f32x4 hs = *reinterpret_cast<const f32x4*>(htab + s * 16 + 4 * g);
#pragma unroll
          for (int t = 0; t < TV; ++t) {
            const f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(a), as_bf16x8(q4_expand(nib[t][u])), f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const uint32_t sw = (u < 2) ? sc[t].x : (u < 4) ? sc[t].y : (u < 6) ? sc[t].z : sc[t].w;
            const uint32_t mw = (u < 2) ? mn[t].x : (u < 4) ? mn[t].y : (u < 6) ? mn[t].z : mn[t].w;
            const float sv = bf16_to_f32((uint16_t)((u & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
            const float mv = bf16_to_f32((uint16_t)((u & 1) ? (mw >> 16) : (mw & 0xFFFFu)));
            const float off = mv - 128.0f * sv;
#pragma unroll
            for (int r = 0; r < 4; ++r) c[t][r] = fmaf(off, hs[r], fmaf(sv, D[r], c[t][r]));
          }
        }
      };
      const int nchunks = nsteps / U;   // the host requires d % 256 == 0 for this format
      load(nibA, scA, mnA, 0);
      for (int ch = 0; ch < nchunks; ch += 2) {
        if (ch + 1 < nchunks) load(nibB, scB, mnB, (ch + 1) * U);
        comp(nibA, scA, mnA, ch * U);
        if (ch + 2 < nchunks) load(nibA, scA, mnA, (ch + 2) * U);
        if (ch + 1 < nchunks) comp(nibB, scB, mnB, (ch + 1) * U);
      }
    }

    // ---- epilogue: this tile's logits for the lane's four hidden rows -----------
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      const int x = xr[t];
      if (!tv[t] || x >= p.n_rows) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!rvalid[r]) continue;
        const int j = 4 * g + r;
        const float z = c[t][r];
        float gn = 0.0f;
        if (SAMPLED) {
          const u32x4 wd = philox4x32_10(u32x4{(uint32_t)x >> 2, prow[r], preq[r], p.cycle}, p.key0, p.key1);
          const int sel = x & 3;
          gn = gumbel_from_word(sel == 0 ? wd.x : (sel == 1 ? wd.y : (sel == 2 ? wd.z : wd.w)));
        }
        rowacc_push<SAMPLED>(acc[r], z, x, p.inv_t, gn);
        if (p.logits) p.logits[(long long)j * p.logits_stride + x] = z;
        if (VERIFY && x == tok[r]) reinterpret_cast<float*>(static_cast<unsigned char*>(p.ws) + 256)[j] = z;
      }
    }
  }

  // ---- reduce: 16 lanes of a row group, then the block's waves -------------------
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int mask = 1; mask < 16; mask <<= 1) {
      const RowAcc o = rowacc_shfl_xor(acc[r], mask);
      rowacc_merge(acc[r], o);
    }
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
  RowAcc* partials = reinterpret_cast<RowAcc*>(ws + 256 + ((M * 4 + 255) / 256) * 256);
  if (tid < M) {
    RowAcc a = red[tid];
    for (int w = 1; w < kWaves; ++w) rowacc_merge(a, red[w * 16 + tid]);
    partials[(size_t)blockIdx.x * M + tid] = a;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) *last_flag = (atomicAdd(counter, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!*last_flag) return;
  __threadfence();

  // ---- last block: merge the per-block partials in block order, write results -----
  const int G = gridDim.x;
  for (int j = wave; j < M; j += kWaves) {
    RowAcc a;
    rowacc_init(a);
    for (int blk = lane; blk < G; blk += 64) rowacc_merge(a, partials[(size_t)blk * M + j]);
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) {
      const RowAcc o = rowacc_shfl_xor(a, mask);
      rowacc_merge(a, o);
    }
    if (lane == 0) {
      mtp_row_stats st;
      uint32_t fl = a.nonfinite ? MTP_ROW_NONFINITE : 0u;
      st.n_posinf = a.nposinf;
      st.reserved = 0;
      if (a.nposinf > 0) {
        fl |= MTP_ROW_POSINF;
        st.max = 0.0f;
        st.lse = logf((float)a.nposinf);
        st.argmax = a.pinf_min;
        st.sample = SAMPLED ? a.pgidx : a.pinf_min;
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
        st.sample = SAMPLED ? a.gidx : a.imax;
      }
      st.flags = fl;
      if (VERIFY) {
        const int b = j / p.rows_per_req, i = j % p.rows_per_req;
        const int t = (i < p.k) ? p.drafts[(size_t)b * p.k_max + i] : -1;
        st.z_tok = (t >= 0 && t < p.n_rows && !(fl & MTP_ROW_INVALID)) ? sanitize(ztok[j], fl) : kNegInf;
      } else {
        st.z_tok = (fl & MTP_ROW_POSINF) ? 0.0f : ((fl & MTP_ROW_INVALID) ? kNegInf : (SAMPLED ? a.gz : a.zmax));
        p.tokens[(size_t)j * p.k_max + p.row_base] = st.sample;
      }
      p.stats[(size_t)j * p.out_stride + p.out_offset] = st;
    }
  }
  if (tid == 0) *counter = 0u;
}

}  // namespace

template <int WT, bool SAMPLED>
__global__ __launch_bounds__(kLmheadThreads) void mtp_draft_head_kernel(LmheadLaunch p) {
  lmhead_body<WT, SAMPLED, false>(p);
}

template <int WT, bool SAMPLED>
__global__ __launch_bounds__(kLmheadThreads) void mtp_verify_logits_kernel(LmheadLaunch p) {
  lmhead_body<WT, SAMPLED, true>(p);
}

int lmhead_grid(int n_rows) {
  const int tiles = (n_rows + 15) / 16;
  const int g = (tiles + 2 * kWaves - 1) / (2 * kWaves);
  return g < 1 ? 1 : (g > kMaxGrid ? kMaxGrid : g);
}

size_t lmhead_ws_bytes(int M, int n_rows) {
  return 256 + ((size_t)(M * 4 + 255) / 256) * 256 + (size_t)lmhead_grid(n_rows) * M * kPartialBytes;
}

static size_t lmhead_lds_bytes(int wtype, int d, int M) {
  const int nsteps = wtype == MTP_W_F32 ? d / 16 : d / 32;
  size_t b = (size_t)nsteps * 4 * M * 16;
  if (wtype == MTP_W_Q4A32) b += (size_t)nsteps * 16 * 4;
  return b + kWaves * 16 * sizeof(RowAcc) + 16;
}

template <int WT, bool SAMPLED>
static hipError_t launch_t(const LmheadLaunch& p, hipStream_t stream) {
  const int G = lmhead_grid(p.n_rows);
  const size_t lds = lmhead_lds_bytes(WT, p.d, p.M);
  auto kern = p.verify ? mtp_verify_logits_kernel<WT, SAMPLED> : mtp_draft_head_kernel<WT, SAMPLED>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(G), dim3(kLmheadThreads), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_lmhead(const LmheadLaunch& p, hipStream_t stream) {
  switch (p.wtype) {
    case MTP_W_F32: return p.sampled ? launch_t<MTP_W_F32, true>(p, stream) : launch_t<MTP_W_F32, false>(p, stream);
    case MTP_W_BF16: return p.sampled ? launch_t<MTP_W_BF16, true>(p, stream) : launch_t<MTP_W_BF16, false>(p, stream);
    case MTP_W_Q4A32: return p.sampled ? launch_t<MTP_W_Q4A32, true>(p, stream) : launch_t<MTP_W_Q4A32, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t lmhead_lds_bytes_for(int wtype, int d, int M) { return lmhead_lds_bytes(wtype, d, M); }

}  // namespace mtp
