// Host-side launch interface of the kernels behind the C ABI.  Validation happens in
// api.cpp before any of these is called; the launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mtp.h"

namespace mtp {

// Blocks of the LM-head kernels for a head of n_rows vocabulary rows.  A function of
// n_rows only, so that a row's statistics never depend on how many hidden rows share
// the launch (batch invariance).
int lmhead_grid(int n_rows);
constexpr int kLmheadThreads = 512;
constexpr int kLmheadMaxRows = 16;        // hidden rows per launch of the LM-head kernels
constexpr int kLmheadMaxWideRows = 128;   // hidden rows per launch of the wide verify kernel
constexpr size_t kPartialBytes = 48;      // sizeof(RowAcc)
constexpr int kAcceptThreads = 256;
int accept_slices(int vocab, bool residual);   // vocabulary slices of the residual draw

struct LmheadLaunch {
  int wtype;
  const void* w;
  const uint16_t* scale;
  const uint16_t* minv;
  int d;
  int n_rows;             // vocabulary rows scored (n_draft or vocab)
  const void* hidden;     // [M][d]
  int htype;
  int M;                  // hidden rows
  int rows_per_req;       // hidden rows per request (1 for the draft head, k+1 for verify)
  int row_base;           // Philox row of hidden row 0 of a request (draft slot, or 0)
  int stream_id;          // Philox stream (0 draft, 2 verify)
  uint32_t key0, key1, cycle, request_base;
  const int32_t* positions;   // verify with exact-match acceptance at T > 0: [B] position of
                              // row 0; the sample then comes from the position-keyed stream 3
  const int32_t* ids;         // draft head gathered from a set of ids: vocabulary id of each row
  float inv_t;            // 1 / T_eff
  int sampled;            // T > 0
  int verify;             // 1: verify pass, 0: draft head
  const int32_t* drafts;  // verify: [B][k_max]
  int k_max, k;
  int32_t* tokens;        // draft: [B][k_max], column row_base
  mtp_row_stats* stats;   // row j -> stats[j * out_stride + out_offset]
  int out_stride, out_offset;
  float* logits;          // row j -> logits + j * logits_stride (NULL: not stored)
  long long logits_stride;
  void* ws;               // partials, drafted-logit slots, completion counter
};

// LM-head workspace: completion counter at 0, drafted-id logits at 256 (one float per
// hidden row), then the [grid][M] block partials
__host__ __device__ inline size_t lmhead_partials_offset(int M) { return 256 + ((size_t)(M * 4 + 255) / 256) * 256; }
size_t lmhead_ws_bytes(int M, int n_rows);
size_t lmhead_lds_bytes_for(int wtype, int d, int M);   // LDS a launch needs
hipError_t launch_lmhead(const LmheadLaunch& p, hipStream_t stream);
// verify pass with the wide kernel, then one merge block per hidden row: for
// kLmheadMaxRows < M <= kLmheadMaxWideRows, and for any M when the head's hidden size leaves
// no room for 16 staged hidden rows in the other kernel's LDS
size_t lmhead_wide_lds_bytes();
hipError_t launch_lmhead_wide(const LmheadLaunch& p, hipStream_t stream);

struct AcceptLaunch {
  int B, k, k_max, vocab, n_draft;
  float temperature;
  int exact;              // T > 0: exact-match acceptance against the verify row's sample
  int eos;
  uint32_t key0, key1, cycle, request_base;
  const int32_t* drafts;
  const mtp_row_stats* dstats;
  const float* dlogits;
  const mtp_row_stats* vstats;
  const float* vlogits;
  const int32_t* draft_row_of;   // [vocab] draft row of each id, or -1; NULL: rows are ids 0..n_draft-1
  int32_t* out_tokens;
  int32_t* n_accept;
  int32_t* n_emit;
  uint32_t* flags;
  void* ws;
};

size_t accept_ws_bytes(int B, int vocab, bool residual);
hipError_t launch_accept(const AcceptLaunch& p, hipStream_t stream);

struct CommitLaunch {
  int B, k;
  const int32_t* n_accept;
  const void* snapshots;
  void* live;
  size_t state_bytes;
  void* kv;
  int n_layers, max_rows;
  size_t kv_row_bytes;
  int32_t* kv_len;
};

hipError_t launch_commit(const CommitLaunch& p, hipStream_t stream);

// mtp_verify_logits in two steps, shared by the entry point that takes a caller's workspace
// and the one that uses the library's own scratch: prepare validates every argument but the
// workspace and fills the launch (no device call); run checks the workspace and launches.
struct VerifyPlan {
  LmheadLaunch p;
  bool wide;
  size_t ws_need;   // workspace bytes the launch needs
};
int verify_logits_prepare(const mtp_head* head, const void* hidden, int32_t htype, int32_t B, int32_t k,
                          const int32_t* draft_tokens, int32_t k_max, const mtp_sampling* smp,
                          mtp_row_stats* row_stats, float* logits, VerifyPlan* plan);
int verify_logits_run(VerifyPlan& plan, void* ws, size_t ws_bytes, void* stream);

size_t tiled_bytes(int wtype, int d, int vocab, int part);   // source wtype BF16 or Q4A32
hipError_t launch_gather(int wtype, const void* w, const void* scale, const void* minv, int d, int vocab,
                         const int32_t* ids, int n, void* dst_w, void* dst_scale, void* dst_minv, hipStream_t stream);
hipError_t launch_pack(int wtype, const void* w, const void* scale, const void* minv, int d, int vocab,
                       void* dst_w, void* dst_scale, void* dst_minv, hipStream_t stream);

}  // namespace mtp
