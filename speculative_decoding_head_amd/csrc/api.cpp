// C ABI entry points: argument validation, workspace sizing and kernel launches.
// Nothing here allocates, frees or synchronises; every call enqueues on the caller's
// stream.  A validation failure returns a negative status and enqueues nothing.
#include <math.h>
#include <stdint.h>

#include "../../include/mtp.h"
#include "kernels.hpp"

using namespace mtp;

namespace {

constexpr int kMaxK = 7;
constexpr size_t kMaxLds = 160 * 1024 - 4096;   // gfx950: 160 KiB of LDS per CU

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

bool is_q4(int wtype) { return wtype == MTP_W_Q4A32 || wtype == MTP_W_Q4A32_TILED; }
bool is_tiled(int wtype) { return wtype == MTP_W_BF16_TILED || wtype == MTP_W_Q4A32_TILED; }

int check_head(const mtp_head* h, int htype) {
  if (!h || !h->w) return MTP_ERR_NULL;
  if (h->reserved != 0) return MTP_ERR_RANGE;
  if (h->wtype < MTP_W_F32 || h->wtype > MTP_W_Q4A32_TILED) return MTP_ERR_DTYPE;
  if (htype != MTP_H_F32 && htype != MTP_H_BF16) return MTP_ERR_DTYPE;
  // pairings: f32 x f32; bf16, q4a32 and their tiled forms x bf16
  if ((h->wtype == MTP_W_F32) != (htype == MTP_H_F32)) return MTP_ERR_DTYPE;
  if (h->d <= 0 || h->d % 32 != 0 || h->vocab <= 0) return MTP_ERR_SHAPE;
  if (is_q4(h->wtype)) {
    if (!h->scale || !h->minv) return MTP_ERR_NULL;
    if (h->d % 256 != 0) return MTP_ERR_SHAPE;
    if (!aligned16(h->scale) || !aligned16(h->minv)) return MTP_ERR_ALIGN;
  }
  if (!aligned16(h->w)) return MTP_ERR_ALIGN;
  if (h->row_ids && !aligned16(h->row_ids)) return MTP_ERR_ALIGN;
  // weights are addressed with 32-bit buffer offsets: at most 2 GiB per head
  const size_t row = h->wtype == MTP_W_F32 ? (size_t)h->d * 4 : (is_q4(h->wtype) ? (size_t)h->d / 2 : (size_t)h->d * 2);
  const size_t rows = is_tiled(h->wtype) ? (size_t)(h->vocab + 15) / 16 * 16 : (size_t)h->vocab;
  if (rows * row >= ((size_t)1 << 31)) return MTP_ERR_SHAPE;
  return MTP_OK;
}

int check_sampling(const mtp_sampling* s) {
  if (!s) return MTP_ERR_NULL;
  if (!(s->temperature >= 0.0f) || !isfinite(s->temperature)) return MTP_ERR_RANGE;
  if (s->eos_id < -1) return MTP_ERR_RANGE;
  if (s->accept_rule != MTP_ACCEPT_RATIO && s->accept_rule != MTP_ACCEPT_EXACT) return MTP_ERR_RANGE;
  if (s->reserved != 0) return MTP_ERR_RANGE;
  return MTP_OK;
}

// T > 0 with the ratio test: draws from q and p (draft logits, residual)
bool ratio_sampling(const mtp_sampling* s) { return s->temperature > 0.0f && s->accept_rule == MTP_ACCEPT_RATIO; }

float inv_t_eff(float t) { return t > 0.0f ? 1.0f / t : 1.0f; }

}  // namespace

extern "C" {

int mtp_abi_version(void) { return MTP_ABI_VERSION; }

const char* mtp_status_str(int status) {
  switch (status) {
    case MTP_OK: return "ok";
    case MTP_ERR_NULL: return "a required pointer is NULL";
    case MTP_ERR_SHAPE: return "a size is out of range";
    case MTP_ERR_DTYPE: return "unsupported weight or hidden type";
    case MTP_ERR_RANGE: return "a parameter is out of range";
    case MTP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MTP_ERR_WORKSPACE: return "workspace missing or too small";
    case MTP_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

size_t mtp_workspace_bytes(int32_t op, int32_t rows, int32_t n_vocab_rows, int32_t B) {
  switch (op) {
    case MTP_OP_DRAFT:
    case MTP_OP_VERIFY:
      if (rows < 1 || n_vocab_rows < 1) return 0;
      if (rows > (op == MTP_OP_VERIFY ? kLmheadMaxWideRows : kLmheadMaxRows)) return 0;
      return lmhead_ws_bytes(rows, n_vocab_rows);
    case MTP_OP_ACCEPT:
      if (B < 1 || n_vocab_rows < 1) return 0;
      // sized for sampled acceptance (greedy needs none)
      return accept_ws_bytes(B, n_vocab_rows, true) + 256;
    default:
      return 0;
  }
}

size_t mtp_tiled_bytes(int32_t wtype, int32_t d, int32_t vocab, int32_t part) {
  if ((wtype != MTP_W_BF16 && wtype != MTP_W_Q4A32) || d <= 0 || d % 32 != 0 || vocab <= 0) return 0;
  if (wtype == MTP_W_Q4A32 && d % 256 != 0) return 0;
  if (part < 0 || part > 2) return 0;
  return tiled_bytes(wtype, d, vocab, part);
}

int mtp_pack_head(const mtp_head* src, void* dst_w, void* dst_scale, void* dst_minv, void* stream) {
  if (!src) return MTP_ERR_NULL;
  if (src->wtype != MTP_W_BF16 && src->wtype != MTP_W_Q4A32) return MTP_ERR_DTYPE;
  int st = check_head(src, MTP_H_BF16);
  if (st != MTP_OK) return st;
  if (!dst_w) return MTP_ERR_NULL;
  if (!aligned16(dst_w)) return MTP_ERR_ALIGN;
  if (tiled_bytes(src->wtype, src->d, src->vocab, 0) >= ((size_t)1 << 31)) return MTP_ERR_SHAPE;
  if (src->wtype == MTP_W_Q4A32) {
    if (!dst_scale || !dst_minv) return MTP_ERR_NULL;
    if (!aligned16(dst_scale) || !aligned16(dst_minv)) return MTP_ERR_ALIGN;
  }
  return launch_pack(src->wtype, src->w, src->scale, src->minv, src->d, src->vocab, dst_w, dst_scale, dst_minv,
                     static_cast<hipStream_t>(stream)) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

int mtp_gather_rows(const mtp_head* src, const int32_t* ids, int32_t n, void* dst_w, void* dst_scale,
                    void* dst_minv, void* stream) {
  int st = check_head(src, src && src->wtype == MTP_W_F32 ? MTP_H_F32 : MTP_H_BF16);
  if (st != MTP_OK) return st;
  if (src->wtype != MTP_W_F32 && src->wtype != MTP_W_BF16 && src->wtype != MTP_W_Q4A32) return MTP_ERR_DTYPE;
  if (src->row_ids) return MTP_ERR_SHAPE;
  if (!ids || !dst_w) return MTP_ERR_NULL;
  if (n < 1 || n > src->vocab) return MTP_ERR_SHAPE;
  if (!aligned16(ids) || !aligned16(dst_w)) return MTP_ERR_ALIGN;
  if (src->wtype == MTP_W_Q4A32) {
    if (!dst_scale || !dst_minv) return MTP_ERR_NULL;
    if (!aligned16(dst_scale) || !aligned16(dst_minv)) return MTP_ERR_ALIGN;
  }
  return launch_gather(src->wtype, src->w, src->scale, src->minv, src->d, src->vocab, ids, n, dst_w, dst_scale,
                       dst_minv, static_cast<hipStream_t>(stream)) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

int mtp_draft_head(const mtp_head* head, int32_t n_draft, const void* hidden, int32_t htype,
                   int32_t B, int32_t slot, int32_t k_max, const mtp_sampling* smp,
                   int32_t* draft_tokens, mtp_row_stats* draft_stats, float* draft_logits,
                   void* ws, size_t ws_bytes, void* stream) {
  int st = check_head(head, htype);
  if (st != MTP_OK) return st;
  if ((st = check_sampling(smp)) != MTP_OK) return st;
  if (!hidden || !draft_tokens || !draft_stats) return MTP_ERR_NULL;
  if (n_draft < 1 || n_draft > head->vocab) return MTP_ERR_SHAPE;
  if (B < 1 || B > kLmheadMaxRows) return MTP_ERR_SHAPE;
  if (k_max < 1 || k_max > kMaxK) return MTP_ERR_SHAPE;
  if (slot < 0 || slot >= k_max) return MTP_ERR_RANGE;
  const bool sampled = ratio_sampling(smp);   // exact-match acceptance drafts the argmax
  if (sampled && !draft_logits) return MTP_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(draft_stats) || (draft_logits && !aligned16(draft_logits)))
    return MTP_ERR_ALIGN;
  if (lmhead_lds_bytes_for(head->wtype, head->d, B) > kMaxLds) return MTP_ERR_SHAPE;
  if (!ws || !aligned256(ws)) return ws ? MTP_ERR_ALIGN : MTP_ERR_WORKSPACE;
  if (ws_bytes < lmhead_ws_bytes(B, n_draft)) return MTP_ERR_WORKSPACE;

  LmheadLaunch p{};
  p.wtype = head->wtype;
  p.w = head->w;
  p.scale = static_cast<const uint16_t*>(head->scale);
  p.minv = static_cast<const uint16_t*>(head->minv);
  p.d = head->d;
  p.n_rows = n_draft;
  p.hidden = hidden;
  p.htype = htype;
  p.M = B;
  p.rows_per_req = 1;
  p.row_base = slot;
  p.stream_id = 0;
  p.key0 = (uint32_t)(smp->seed & 0xFFFFFFFFu);
  p.key1 = (uint32_t)(smp->seed >> 32);
  p.cycle = smp->cycle;
  p.request_base = smp->request_base;
  p.positions = nullptr;
  p.ids = head->row_ids;
  p.inv_t = inv_t_eff(sampled ? smp->temperature : 0.0f);
  p.sampled = sampled;
  p.verify = 0;
  p.drafts = nullptr;
  p.k_max = k_max;
  p.k = 0;
  p.tokens = draft_tokens;
  p.stats = draft_stats;
  p.out_stride = k_max;
  p.out_offset = slot;
  p.logits = draft_logits ? draft_logits + (size_t)slot * n_draft : nullptr;
  p.logits_stride = (long long)k_max * n_draft;
  p.ws = ws;
  return launch_lmhead(p, static_cast<hipStream_t>(stream)) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

int mtp_verify_logits(const mtp_head* head, const void* hidden, int32_t htype, int32_t B,
                      int32_t k, const int32_t* draft_tokens, int32_t k_max,
                      const mtp_sampling* smp, mtp_row_stats* row_stats, float* logits,
                      void* ws, size_t ws_bytes, void* stream) {
  VerifyPlan plan;
  const int st = verify_logits_prepare(head, hidden, htype, B, k, draft_tokens, k_max, smp, row_stats, logits, &plan);
  return st != MTP_OK ? st : verify_logits_run(plan, ws, ws_bytes, stream);
}

}  // extern "C"

namespace mtp {

int verify_logits_prepare(const mtp_head* head, const void* hidden, int32_t htype, int32_t B, int32_t k,
                          const int32_t* draft_tokens, int32_t k_max, const mtp_sampling* smp,
                          mtp_row_stats* row_stats, float* logits, VerifyPlan* plan) {
  int st = check_head(head, htype);
  if (st != MTP_OK) return st;
  if ((st = check_sampling(smp)) != MTP_OK) return st;
  if (head->row_ids) return MTP_ERR_SHAPE;   // the verify scores the whole vocabulary
  if (!hidden || !draft_tokens || !row_stats) return MTP_ERR_NULL;
  if (k < 1 || k > kMaxK || k_max < k || k_max > kMaxK) return MTP_ERR_SHAPE;
  if (B < 1) return MTP_ERR_SHAPE;
  const int M = B * (k + 1);
  if (M > kLmheadMaxWideRows) return MTP_ERR_SHAPE;
  // the wide kernel above 16 rows, and for every row count of a head whose 16 hidden rows
  // do not fit the other kernel's LDS (a property of the head alone, so a row's results
  // still do not depend on how many rows share the launch)
  const bool wide = M > kLmheadMaxRows || lmhead_lds_bytes_for(head->wtype, head->d, kLmheadMaxRows) > kMaxLds;
  const bool sampled = smp->temperature > 0.0f;
  const bool exact = sampled && smp->accept_rule == MTP_ACCEPT_EXACT;
  if (sampled && !exact && !logits) return MTP_ERR_NULL;
  if (exact && !smp->positions) return MTP_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(row_stats) || (logits && !aligned16(logits))) return MTP_ERR_ALIGN;
  if (exact && !aligned16(smp->positions)) return MTP_ERR_ALIGN;
  if (wide && lmhead_wide_lds_bytes() > kMaxLds) return MTP_ERR_SHAPE;

  LmheadLaunch& p = plan->p;
  p = LmheadLaunch{};
  p.wtype = head->wtype;
  p.w = head->w;
  p.scale = static_cast<const uint16_t*>(head->scale);
  p.minv = static_cast<const uint16_t*>(head->minv);
  p.d = head->d;
  p.n_rows = head->vocab;
  p.hidden = hidden;
  p.htype = htype;
  p.M = M;
  p.rows_per_req = k + 1;
  p.row_base = 0;
  p.stream_id = 2;
  p.key0 = (uint32_t)(smp->seed & 0xFFFFFFFFu);
  p.key1 = (uint32_t)(smp->seed >> 32);
  p.cycle = smp->cycle;
  p.request_base = smp->request_base;
  p.positions = exact ? smp->positions : nullptr;
  p.ids = nullptr;
  p.inv_t = inv_t_eff(smp->temperature);
  p.sampled = sampled;
  p.verify = 1;
  p.drafts = draft_tokens;
  p.k_max = k_max;
  p.k = k;
  p.tokens = nullptr;
  p.stats = row_stats;
  p.out_stride = 1;
  p.out_offset = 0;
  p.logits = logits;
  p.logits_stride = head->vocab;
  p.ws = nullptr;
  plan->wide = wide;
  plan->ws_need = lmhead_ws_bytes(M, head->vocab);
  return MTP_OK;
}

int verify_logits_run(VerifyPlan& plan, void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned256(ws)) return ws ? MTP_ERR_ALIGN : MTP_ERR_WORKSPACE;
  if (ws_bytes < plan.ws_need) return MTP_ERR_WORKSPACE;
  plan.p.ws = ws;
  const hipError_t e = plan.wide ? launch_lmhead_wide(plan.p, static_cast<hipStream_t>(stream))
                                 : launch_lmhead(plan.p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

}  // namespace mtp

extern "C" {

int mtp_accept_sample(int32_t B, int32_t k, int32_t k_max, int32_t vocab, int32_t n_draft,
                      const mtp_sampling* smp, const int32_t* draft_tokens,
                      const mtp_row_stats* draft_stats, const float* draft_logits,
                      const mtp_row_stats* row_stats, const float* logits, const int32_t* draft_row_of,
                      int32_t* out_tokens, int32_t* n_accept, int32_t* n_emit, uint32_t* flags,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = check_sampling(smp);
  if (st != MTP_OK) return st;
  if (B < 1 || B > 65535 * 64) return MTP_ERR_SHAPE;
  if (k < 1 || k > kMaxK || k_max < k || k_max > kMaxK) return MTP_ERR_SHAPE;
  if (vocab < 1 || n_draft < 1 || n_draft > vocab) return MTP_ERR_SHAPE;
  if (!draft_tokens || !draft_stats || !row_stats || !out_tokens || !n_accept || !n_emit || !flags)
    return MTP_ERR_NULL;
  const bool ratio = ratio_sampling(smp);
  if (ratio && (!draft_logits || !logits)) return MTP_ERR_NULL;
  if (!aligned16(draft_stats) || !aligned16(row_stats)) return MTP_ERR_ALIGN;
  if (draft_row_of && !aligned16(draft_row_of)) return MTP_ERR_ALIGN;
  const size_t need = accept_ws_bytes(B, vocab, ratio);
  if (need > 0) {
    if (!ws) return MTP_ERR_WORKSPACE;
    if (!aligned256(ws)) return MTP_ERR_ALIGN;
    if (ws_bytes < need) return MTP_ERR_WORKSPACE;
  }
  AcceptLaunch p{};
  p.B = B;
  p.k = k;
  p.k_max = k_max;
  p.vocab = vocab;
  p.n_draft = n_draft;
  p.temperature = smp->temperature;
  p.exact = smp->accept_rule == MTP_ACCEPT_EXACT;
  p.eos = smp->eos_id;
  p.key0 = (uint32_t)(smp->seed & 0xFFFFFFFFu);
  p.key1 = (uint32_t)(smp->seed >> 32);
  p.cycle = smp->cycle;
  p.request_base = smp->request_base;
  p.drafts = draft_tokens;
  p.dstats = draft_stats;
  p.dlogits = draft_logits;
  p.vstats = row_stats;
  p.vlogits = logits;
  p.draft_row_of = draft_row_of;
  p.out_tokens = out_tokens;
  p.n_accept = n_accept;
  p.n_emit = n_emit;
  p.flags = flags;
  p.ws = ws;
  return launch_accept(p, static_cast<hipStream_t>(stream)) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

int mtp_commit_state(int32_t B, int32_t k, const int32_t* n_accept, const void* snapshots,
                     void* live, size_t state_bytes, void* kv, int32_t n_layers,
                     int32_t max_rows, size_t kv_row_bytes, int32_t* kv_len, void* stream) {
  if (B < 1 || B > 65535) return MTP_ERR_SHAPE;
  if (k < 1 || k > kMaxK) return MTP_ERR_SHAPE;
  if (!n_accept || !kv_len) return MTP_ERR_NULL;
  if (state_bytes % 16 != 0) return MTP_ERR_SHAPE;
  if (state_bytes > 0 && (!snapshots || !live)) return MTP_ERR_NULL;
  if (n_layers < 0 || max_rows < 0) return MTP_ERR_SHAPE;
  if (n_layers > 0) {
    if (!kv) return MTP_ERR_NULL;
    if (kv_row_bytes == 0 || kv_row_bytes % 16 != 0 || max_rows < 1) return MTP_ERR_SHAPE;
    if (!aligned16(kv)) return MTP_ERR_ALIGN;
  }
  if ((snapshots && !aligned16(snapshots)) || (live && !aligned16(live))) return MTP_ERR_ALIGN;
  if (state_bytes / (16 * 1024) >= 0x7fffffff) return MTP_ERR_SHAPE;   // grid.x of the commit
  CommitLaunch p{};
  p.B = B;
  p.k = k;
  p.n_accept = n_accept;
  p.snapshots = snapshots;
  p.live = live;
  p.state_bytes = state_bytes;
  p.kv = kv;
  p.n_layers = n_layers;
  p.max_rows = max_rows;
  p.kv_row_bytes = kv_row_bytes;
  p.kv_len = kv_len;
  return launch_commit(p, static_cast<hipStream_t>(stream)) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

}  // extern "C"
