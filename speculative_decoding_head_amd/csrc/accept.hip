// Acceptance, first rejection, residual resample and EOS truncation for B requests.
//
// Greedy (T = 0): a draft is accepted only if it equals the verify row's argmax
// (lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", section "Exactness"); with
// exact-match acceptance at T > 0 (same PR, "Exactness" and "Notes") it must equal the
// verify row's sample, the trunk's own position-keyed draw, which is also the token
// emitted at the first rejection and after the last draft.
// Sampled (T > 0): draft t is accepted iff p(t) > 0 and u * q(t) <= p(t); at the first
// rejection the next token is drawn from max(0, p - q) renormalised (DS4Server issue
// "Add Qwen3.8 Flash Next native MTP speculation", section "Implementation" and closing
// comment "Review"); EOS inside the block ends it with nothing kept beyond EOS (same
// issue, "Implementation").
//
// Grid (B, S): every block walks the request's acceptance chain (at most 7 rows of
// per-row statistics), then, if the request stopped at a rejection with T > 0, scores
// its 1/S slice of the vocabulary for the residual draw: ln r(x) + Gumbel(x) with
// ln r = ln p + log1p(-exp(ln q - ln p)) where p > q.  Each block writes its best
// (score, id) and whether it saw residual mass; the last of the S blocks to finish
// (atomic ticket per request) merges the slices in order and writes the request's
// tokens, counts and flags.  At T = 0, S = 1 and no workspace is used.
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {

constexpr int kSliceElems = 4096;
constexpr int kMaxSlices = 64;

struct SlicePartial {
  float score;
  int idx;
  int has_mass;
  int pad;
};

enum StopKind { kRejected = 0, kEosDraft = 1, kAllAccepted = 2, kInvalidRow = 3 };

struct Chain {
  int a;         // accepted drafts kept in the block (= committed snapshot index)
  int kind;      // StopKind
  int last;      // token after the accepted drafts (kInvalidRow: none)
  uint32_t flags;
};

// draft row of vocabulary id x (-1: outside the draft vocabulary)
__device__ __forceinline__ int draft_row(const AcceptLaunch& p, int x) {
  if (p.draft_row_of) return p.draft_row_of[x];
  return x < p.n_draft ? x : -1;
}

__device__ __forceinline__ float draft_logq(const AcceptLaunch& p, int b, int i, int t, float inv_t,
                                            const mtp_row_stats& ds) {
  if (t < 0 || t >= p.vocab || (ds.flags & MTP_ROW_INVALID)) return kNegInf;
  const int r = draft_row(p, t);
  if (r < 0 || r >= p.n_draft) return kNegInf;
  const float z = sanitize(p.dlogits[((size_t)b * p.k_max + i) * p.n_draft + r], ds.flags);
  return z * inv_t - ds.lse;
}

__device__ Chain walk_chain(const AcceptLaunch& p, int b, float inv_t) {
  Chain c{p.k, kAllAccepted, -1, 0u};
  const bool sampled = p.temperature > 0.0f;
  const int K1 = p.k + 1;
  for (int i = 0; i < p.k; ++i) {
    const mtp_row_stats vs = p.vstats[(size_t)b * K1 + i];
    if (vs.flags & MTP_ROW_INVALID) {
      c.a = i;
      c.kind = kInvalidRow;
      return c;
    }
    if (vs.flags & MTP_ROW_NONFINITE) c.flags |= MTP_ACC_NONFINITE_TARGET;
    const mtp_row_stats ds = p.dstats[(size_t)b * p.k_max + i];
    if (ds.flags & MTP_ROW_NONFINITE) c.flags |= MTP_ACC_NONFINITE_DRAFT;
    const int t = p.drafts[(size_t)b * p.k_max + i];
    const bool t_ok = t >= 0 && t < p.vocab;
    if (!t_ok) c.flags |= MTP_ACC_DRAFT_INVALID;
    bool ok;
    if (!sampled || p.exact) {
      ok = t_ok && t == (sampled ? vs.sample : vs.argmax);
    } else if (!t_ok) {
      ok = false;
    } else {
      const float zt = sanitize(p.vlogits[((size_t)b * K1 + i) * p.vocab + t], vs.flags);
      const float lp = zt * inv_t - vs.lse;
      const float lq = draft_logq(p, b, i, t, inv_t, ds);
      const uint32_t w = philox_word(p.key0, p.key1, kStreamAccept, (uint32_t)i,
                                     p.request_base + (uint32_t)b, p.cycle, 0u);
      const float lu = logf(uniform_accept(w));
      ok = lp > kNegInf && (lu + lq) <= lp;
    }
    if (!ok) {
      c.a = i;
      c.kind = kRejected;
      return c;
    }
    if (p.eos >= 0 && t == p.eos) {
      c.a = i;
      c.kind = kEosDraft;
      c.last = p.eos;
      return c;
    }
  }
  const mtp_row_stats vk = p.vstats[(size_t)b * K1 + p.k];
  if (vk.flags & MTP_ROW_INVALID) {
    c.a = p.k;
    c.kind = kInvalidRow;
    return c;
  }
  if (vk.flags & MTP_ROW_NONFINITE) c.flags |= MTP_ACC_NONFINITE_TARGET;
  c.last = sampled ? vk.sample : vk.argmax;
  return c;
}

__global__ __launch_bounds__(kAcceptThreads) void mtp_accept_sample_kernel(AcceptLaunch p) {
  __shared__ float s_score[kAcceptThreads / 64];
  __shared__ int s_idx[kAcceptThreads / 64];
  __shared__ int s_mass[kAcceptThreads / 64];
  __shared__ int s_last;

  const int b = blockIdx.x, slice = blockIdx.y, S = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool sampled = p.temperature > 0.0f;
  const float inv_t = sampled ? 1.0f / p.temperature : 1.0f;
  const int K1 = p.k + 1;

  Chain c = walk_chain(p, b, inv_t);
  const bool resample = sampled && !p.exact && c.kind == kRejected;

  // ---- residual slice: best ln r(x) + Gumbel(x) over x in this block's range ------
  float best = kNegInf;
  int best_idx = kNoIndex;
  int mass = 0;
  if (resample) {
    const int i = c.a;
    const mtp_row_stats vs = p.vstats[(size_t)b * K1 + i];
    const mtp_row_stats ds = p.dstats[(size_t)b * p.k_max + i];
    const float* zrow = p.vlogits + ((size_t)b * K1 + i) * p.vocab;
    const float* qrow = p.dlogits + ((size_t)b * p.k_max + i) * p.n_draft;
    const bool q_valid = !(ds.flags & MTP_ROW_INVALID);
    const int per = (p.vocab + S - 1) / S;
    const int x0 = slice * per, x1 = min(p.vocab, x0 + per);
    const uint32_t prow = (kStreamResample << 8) | (uint32_t)i;
    const uint32_t preq = p.request_base + (uint32_t)b;
    // each thread takes groups of 4 consecutive ids: one Philox call per group
    for (int xg = (x0 & ~3) + 4 * tid; xg < x1; xg += 4 * kAcceptThreads) {
      const u32x4 wd = philox4x32_10(u32x4{(uint32_t)xg >> 2, prow, preq, p.cycle}, p.key0, p.key1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = xg + e;
        if (x < x0 || x >= x1) continue;
        const float lp = sanitize(zrow[x], vs.flags) * inv_t - vs.lse;
        const int dr = q_valid ? draft_row(p, x) : -1;
        const float lq = (dr >= 0 && dr < p.n_draft) ? sanitize(qrow[dr], ds.flags) * inv_t - ds.lse : kNegInf;
        if (lp > lq) {
          const float lr = lp + log1pf(-__expf(lq - lp));
          if (lr > kNegInf) {
            mass = 1;
            const uint32_t w = e == 0 ? wd.x : (e == 1 ? wd.y : (e == 2 ? wd.z : wd.w));
            const float sc = lr + gumbel_from_word(w);
            if (sc > best) { best = sc; best_idx = x; }
          }
        }
      }
    }
  }
  // block reduction (lowest id on equal scores)
  for (int m = 1; m < 64; m <<= 1) {
    const float ob = __shfl_xor(best, m);
    const int oi = __shfl_xor(best_idx, m);
    const int om = __shfl_xor(mass, m);
    if (better(ob, oi, best, best_idx)) { best = ob; best_idx = oi; }
    mass |= om;
  }
  if (lane == 0) { s_score[wave] = best; s_idx[wave] = best_idx; s_mass[wave] = mass; }
  __syncthreads();

  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  if (S > 1) {
    SlicePartial* part = reinterpret_cast<SlicePartial*>(ws + (((size_t)p.B * 4 + 255) / 256) * 256);
    unsigned int* counters = reinterpret_cast<unsigned int*>(ws);
    if (tid == 0) {
      float bs = s_score[0];
      int bi = s_idx[0], bm = s_mass[0];
      for (int w = 1; w < kAcceptThreads / 64; ++w) {
        if (better(s_score[w], s_idx[w], bs, bi)) { bs = s_score[w]; bi = s_idx[w]; }
        bm |= s_mass[w];
      }
      store_coherent_obj(&part[(size_t)b * S + slice], SlicePartial{bs, bi, bm, 0});
      wait_stores();
      s_last = (take_ticket(&counters[b]) == (unsigned)S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (tid != 0) return;
    float bs = kNegInf;
    int bi = kNoIndex, bm = 0;
    for (int sl = 0; sl < S; ++sl) {
      const SlicePartial q = load_coherent_obj(&part[(size_t)b * S + sl]);
      if (better(q.score, q.idx, bs, bi)) { bs = q.score; bi = q.idx; }
      bm |= q.has_mass;
    }
    store_coherent(&counters[b], 0u);
    best = bs; best_idx = bi; mass = bm;
  } else {
    if (tid != 0) return;
    best = s_score[0]; best_idx = s_idx[0]; mass = s_mass[0];
    for (int w = 1; w < kAcceptThreads / 64; ++w) {
      if (better(s_score[w], s_idx[w], best, best_idx)) { best = s_score[w]; best_idx = s_idx[w]; }
      mass |= s_mass[w];
    }
  }

  // ---- one thread writes the request's result ------------------------------------
  if (c.kind == kRejected) {
    const mtp_row_stats vs = p.vstats[(size_t)b * K1 + c.a];
    if (!sampled) {
      c.last = vs.argmax;
    } else if (p.exact) {
      c.last = vs.sample;   // the trunk's own sample at this position
    } else if (mass) {
      c.last = best_idx;
    } else {
      c.flags |= MTP_ACC_RESID_FALLBACK;
      c.last = vs.sample;   // argmax(z/T + Gumbel) on the same stream-2 draws = a draw from p
    }
  }
  if (c.kind == kAllAccepted) c.flags |= MTP_ACC_ALL_ACCEPTED;
  if (c.kind == kInvalidRow) c.flags |= MTP_ACC_ROW_INVALID;
  const bool has_last = c.kind != kInvalidRow;
  if (has_last && p.eos >= 0 && c.last == p.eos) c.flags |= MTP_ACC_EOS;
  int32_t* out = p.out_tokens + (size_t)b * K1;
  for (int i = 0; i < K1; ++i) {
    int v = -1;
    if (i < c.a) v = p.drafts[(size_t)b * p.k_max + i];
    else if (i == c.a && has_last) v = c.last;
    out[i] = v;
  }
  p.n_accept[b] = c.a;
  p.n_emit[b] = c.a + (has_last ? 1 : 0);
  p.flags[b] = c.flags;
}

}  // namespace

int accept_slices(int vocab, bool residual) {
  if (!residual) return 1;
  int s = (vocab + kSliceElems - 1) / kSliceElems;
  return s < 1 ? 1 : (s > kMaxSlices ? kMaxSlices : s);
}

size_t accept_ws_bytes(int B, int vocab, bool residual) {
  const int S = accept_slices(vocab, residual);
  if (S <= 1) return 0;
  return (((size_t)B * 4 + 255) / 256) * 256 + (size_t)B * S * sizeof(SlicePartial);
}

hipError_t launch_accept(const AcceptLaunch& p, hipStream_t stream) {
  const int S = accept_slices(p.vocab, p.temperature > 0.0f && !p.exact);
  hipLaunchKernelGGL(mtp_accept_sample_kernel, dim3(p.B, S), dim3(kAcceptThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mtp
