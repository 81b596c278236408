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
// Grid (B, S), one wave per 64 threads.  Every wave evaluates the request's acceptance
// chain in parallel, lane i for draft row i and lane k for the bonus row, and finds the
// first row that stops the block with a ballot: all rows' statistics (and under the ratio
// rule their drafted-id logits and acceptance draws) are fetched at once, not one
// dependent round trip per row.  If the request stopped at a rejection with T > 0, each
// block then scores its 1/S slice of the vocabulary (about 1,024 ids, one pass per thread)
// for the residual draw: ln r(x) + Gumbel(x) with ln r = ln p + log1p(-exp(ln q - ln p))
// where p > q.  Each block writes its best (score, id) and whether it saw residual mass;
// the last of the S blocks to finish (atomic ticket per request) loads all slice results
// at once and reduces them (the comparison is a total order: higher score, then lower id,
// so the result does not depend on the reduction order) and writes the request's tokens,
// counts and flags.  At T = 0, S = 1 and no workspace is used.
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {

constexpr int kSliceElems = 1024;
constexpr int kMaxSlices = 256;   // 4 slice results per lane of one wave in the final merge

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
  // statistics of the verify row and draft row at index a
  uint32_t vflags, dflags;
  float vlse, dlse;
  int vsample, vargmax;
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

// The acceptance chain of request b, evaluated by one wave: lane i < k takes draft row i,
// lane k the bonus row.  A row stops the block if its target row is unusable, its draft is
// rejected or its accepted draft is EOS; the bonus row always stops it.  Flags come from
// every row before the stopping one and from the stopping row itself unless its target row
// is unusable (the block ends before that row).  Every lane returns the same chain.
__device__ Chain walk_chain(const AcceptLaunch& p, int b, float inv_t, int lane) {
  const bool sampled = p.temperature > 0.0f;
  const int K1 = p.k + 1;
  const int i = lane;
  mtp_row_stats vs{}, ds{};
  int t = -1;
  if (i < K1) vs = p.vstats[(size_t)b * K1 + i];
  if (i < p.k) {
    ds = p.dstats[(size_t)b * p.k_max + i];
    t = p.drafts[(size_t)b * p.k_max + i];
  }
  const bool invalid = i < K1 && (vs.flags & MTP_ROW_INVALID);
  uint32_t rf = (i < K1 && (vs.flags & MTP_ROW_NONFINITE)) ? MTP_ACC_NONFINITE_TARGET : 0u;
  bool ok = false, eos = false;
  if (i < p.k) {
    if (ds.flags & MTP_ROW_NONFINITE) rf |= MTP_ACC_NONFINITE_DRAFT;
    const bool t_ok = t >= 0 && t < p.vocab;
    if (!t_ok) rf |= MTP_ACC_DRAFT_INVALID;
    if (!sampled || p.exact) {
      ok = t_ok && t == (sampled ? vs.sample : vs.argmax);
    } else if (t_ok) {
      const float zt = sanitize(p.vlogits[((size_t)b * K1 + i) * p.vocab + t], vs.flags);
      const float lp = zt * inv_t - vs.lse;
      const float lq = draft_logq(p, b, i, t, inv_t, ds);
      const uint32_t w = philox_word(p.key0, p.key1, kStreamAccept, (uint32_t)i,
                                     p.request_base + (uint32_t)b, p.cycle, 0u);
      const float lu = logf(uniform_accept(w));
      ok = lp > kNegInf && (lu + lq) <= lp;
    }
    eos = p.eos >= 0 && t == p.eos;
  }
  const bool stop = i == p.k || (i < p.k && (invalid || !ok || eos));
  const int s = __ffsll((unsigned long long)__ballot(stop)) - 1;   // lane k always stops: k <= 7
  uint32_t fl = (i < s || (i == s && !invalid)) ? rf : 0u;
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) fl |= __shfl_xor(fl, m);   // rows 0..7 live in lanes 0..7

  Chain c;
  c.a = s;
  c.flags = __shfl(fl, 0);
  const bool inv_s = __shfl(invalid ? 1 : 0, s) != 0;
  const bool ok_s = __shfl(ok ? 1 : 0, s) != 0;
  c.vflags = __shfl(vs.flags, s);
  c.vlse = __shfl(vs.lse, s);
  c.vsample = __shfl(vs.sample, s);
  c.vargmax = __shfl(vs.argmax, s);
  c.dflags = __shfl(ds.flags, s);
  c.dlse = __shfl(ds.lse, s);
  if (inv_s) {
    c.kind = kInvalidRow;
    c.last = -1;
  } else if (s == p.k) {
    c.kind = kAllAccepted;
    c.last = sampled ? c.vsample : c.vargmax;
  } else if (!ok_s) {
    c.kind = kRejected;
    c.last = -1;
  } else {
    c.kind = kEosDraft;
    c.last = p.eos;
  }
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

  Chain c = walk_chain(p, b, inv_t, lane);
  const bool resample = sampled && !p.exact && c.kind == kRejected;

  // ---- residual slice: best ln r(x) + Gumbel(x) over x in this block's range ------
  float best = kNegInf;
  int best_idx = kNoIndex;
  int mass = 0;
  if (resample) {
    const int i = c.a;
    const float* zrow = p.vlogits + ((size_t)b * K1 + i) * p.vocab;
    const float* qrow = p.dlogits + ((size_t)b * p.k_max + i) * p.n_draft;
    const bool q_valid = !(c.dflags & MTP_ROW_INVALID);
    const int per = ((p.vocab + S - 1) / S + 3) & ~3;   // slices start on groups of 4 ids
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
        const float lp = sanitize(zrow[x], c.vflags) * inv_t - c.vlse;
        const int dr = q_valid ? draft_row(p, x) : -1;
        const float lq = (dr >= 0 && dr < p.n_draft) ? sanitize(qrow[dr], c.dflags) * inv_t - c.dlse : kNegInf;
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
    if (!s_last || wave != 0) return;
    // wave 0: every slice result is loaded at once (up to 4 per lane), then reduced
    SlicePartial q[kMaxSlices / 64];
#pragma unroll
    for (int u = 0; u < kMaxSlices / 64; ++u) {
      const int sl = lane + 64 * u;
      q[u] = sl < S ? load_coherent_obj(&part[(size_t)b * S + sl]) : SlicePartial{kNegInf, kNoIndex, 0, 0};
    }
    best = kNegInf; best_idx = kNoIndex; mass = 0;
#pragma unroll
    for (int u = 0; u < kMaxSlices / 64; ++u) {
      if (better(q[u].score, q[u].idx, best, best_idx)) { best = q[u].score; best_idx = q[u].idx; }
      mass |= q[u].has_mass;
    }
    for (int m = 1; m < 64; m <<= 1) {
      const float ob = __shfl_xor(best, m);
      const int oi = __shfl_xor(best_idx, m);
      const int om = __shfl_xor(mass, m);
      if (better(ob, oi, best, best_idx)) { best = ob; best_idx = oi; }
      mass |= om;
    }
    if (lane != 0) return;
    store_coherent(&counters[b], 0u);
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
    if (!sampled) {
      c.last = c.vargmax;
    } else if (p.exact) {
      c.last = c.vsample;   // the trunk's own sample at this position
    } else if (mass) {
      c.last = best_idx;
    } else {
      c.flags |= MTP_ACC_RESID_FALLBACK;
      c.last = c.vsample;   // argmax(z/T + Gumbel) on the same stream-2 draws = a draw from p
    }
  }
  if (c.kind == kAllAccepted) c.flags |= MTP_ACC_ALL_ACCEPTED;
  if (c.kind == kInvalidRow) c.flags |= MTP_ACC_ROW_INVALID;
  if (c.kind == kEosDraft) c.flags |= MTP_ACC_EOS_DRAFT;
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
