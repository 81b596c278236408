/*
 * mtp.h - C ABI of one native-MTP speculative decoding cycle on an MI355X (gfx950).
 *
 * One cycle, as the pages describe it:
 *   draft   k times: the truncated-vocabulary draft head (the first n_draft rows of
 *           the shared LM head) scores one hidden row per request and picks the next
 *           draft token on the GPU; the token stays in device memory and feeds the
 *           next draft (lucebox-hub PR "feat(qwen4exp): MTP speculative decoding",
 *           section "What");
 *   verify  the trunk's k+1 verify rows get full-vocabulary logits in one batched
 *           pass, with softmax statistics at temperature T (same section);
 *   accept  exact match at T = 0 (same PR, section "Exactness"), or probability-ratio
 *           acceptance u*q <= p with a max(0, p - q) residual resample at the first
 *           rejection, zero/non-finite probabilities handled and EOS inside the block
 *           truncating (DS4Server issue "Add Qwen3.8 Flash Next native MTP
 *           speculation", section "Implementation" and closing comment "Review");
 *   commit  the accepted row's recurrent-state snapshot becomes live and the
 *           rejected KV rows are trimmed (same issue, "Implementation"; llama.cpp PR
 *           "qwen4exp : port NextN/MTP speculative decoding to master", commit "keep
 *           speculative checkpoints on device").
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises; each call only enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns.  Inputs and outputs must
 *     stay alive until the stream has run the work.
 *   - Host structs (mtp_head, mtp_sampling) are read during the call only.
 *   - Return value: MTP_OK, or a negative mtp_status from argument validation or from
 *     the kernel launch.  Validation failures enqueue nothing.  Outcomes that depend on
 *     device data (non-finite logits, EOS, residual fallback, out-of-range n_accept) are
 *     reported through device-side flags, never by the return value.
 *   - No global mutable state: calls are thread-safe.  Calls that share a workspace
 *     must be ordered on one stream.
 *   - Row-major layouts throughout; all tensors contiguous; every pointer 16-byte
 *     aligned.
 */
#ifndef MTP_H_
#define MTP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_ABI_VERSION 3

/* ---------------------------------------------------------------------------------- */
/* status codes                                                                        */
/* ---------------------------------------------------------------------------------- */
/* Invalid input is reported, never crashed on: the loader commit of llama.cpp PR
 * "qwen4exp : port NextN/MTP speculative decoding to master" (the PR body) makes a bad
 * drafter load stop with a clear message where it used to segfault.  Every call here
 * checks its arguments first and returns one of these codes; it never aborts, throws or
 * touches memory it was not given. */
typedef enum mtp_status {
  MTP_OK = 0,
  MTP_ERR_NULL = -1,      /* a required pointer is NULL                                 */
  MTP_ERR_SHAPE = -2,     /* a size is out of range (k, B, d, vocab, n_draft, rows...)  */
  MTP_ERR_DTYPE = -3,     /* unknown weight or hidden type, or an unsupported pairing   */
  MTP_ERR_RANGE = -4,     /* temperature negative or not finite; slot >= k_max; ...     */
  MTP_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned                           */
  MTP_ERR_WORKSPACE = -6, /* workspace missing or smaller than mtp_workspace_bytes()    */
  MTP_ERR_HIP = -7        /* the HIP runtime reported an error at launch                */
} mtp_status;

/* ---------------------------------------------------------------------------------- */
/* shared LM head                                                                      */
/* ---------------------------------------------------------------------------------- */
typedef enum mtp_wtype {
  MTP_W_F32 = 0,   /* w: float [vocab][d]                                              */
  MTP_W_BF16 = 1,  /* w: bf16 bit patterns, uint16 [vocab][d]                          */
  MTP_W_Q4A32 = 2, /* 4-bit affine, 32-value groups along d (DS4Server issue above,
                      closing comment "Implementation"):  w[x][32g+j] = scale*q + min,
                      q = unsigned nibble j of group g;
                        w:     uint8 [vocab][d/2], element 2m in the low nibble of byte m,
                               element 2m+1 in the high nibble;
                        scale: bf16 [vocab][d/32];  minv: bf16 [vocab][d/32]            */
  /* Tiled layouts: the same numbers as BF16 / Q4A32, rearranged so that the LM-head
   * kernels read 1024 contiguous bytes per wave per load.  Rows come in tiles of 16
   * (tile t = rows 16t..16t+15; rows past vocab are zero).  Made by mtp_pack_head.   */
  MTP_W_BF16_TILED = 3,  /* w: block (t, s) of 1024 bytes at ((t*(d/32) + s) * 1024),
                            s = 32-value step; bytes 16l..16l+15 of the block (l = 0..63)
                            hold W[16t + l%16][32s + 8(l/16) + e], e = 0..7 (bf16)       */
  MTP_W_Q4A32_TILED = 4  /* w: block (t, q) of 1024 bytes at ((t*(d/128) + q) * 1024),
                            q = group quad (groups 4q..4q+3); bytes 16l..16l+15 are four
                            little-endian words, word u = the 4 row-major nibble bytes
                            [16(4q+u) + 4(l/16), +4) of row 16t + l%16;
                            scale, minv: block (t, c) of 256 bytes at ((t*(d/256) + c) * 256),
                            c = group octet; bytes 16r..16r+15 = the 8 bf16 values of
                            row 16t + r for groups 8c..8c+7                              */
} mtp_wtype;

typedef enum mtp_htype {
  MTP_H_F32 = 0,   /* hidden rows: float [rows][d]                                     */
  MTP_H_BF16 = 1   /* hidden rows: bf16 bit patterns, uint16 [rows][d]                 */
} mtp_htype;

/* Supported pairings: F32 weights with F32 hiddens; BF16, Q4A32 and their tiled forms
 * with BF16 hiddens.  d must be a positive multiple of 32 (of 256 for the 4-bit
 * formats); vocab >= 1; the weight array of one head must be smaller than 2 GiB. */
typedef struct mtp_head {
  int32_t wtype;       /* mtp_wtype                                                    */
  int32_t d;           /* hidden size                                                  */
  int32_t vocab;       /* V, rows of the shared head                                   */
  int32_t reserved;    /* must be 0                                                    */
  const void* w;       /* device, layout per wtype                                     */
  const void* scale;   /* device, Q4A32 only (else NULL)                               */
  const void* minv;    /* device, Q4A32 only (else NULL)                               */
  const int32_t* row_ids; /* device int32 [vocab] or NULL: the vocabulary id of each row,
                           * strictly ascending (a draft head gathered from a set of ids,
                           * see mtp_gather_rows); NULL = row r is id r.  Only the draft
                           * head takes a head with row ids.                          */
} mtp_head;

/* ---------------------------------------------------------------------------------- */
/* sampling parameters                                                                 */
/* ---------------------------------------------------------------------------------- */
/* Random draws use Philox4x32-10 (Salmon et al., SC'11): key = (seed lo32, seed hi32),
 * counter = (x >> 2, stream << 8 | row, request_base + b, cycle), word x & 3, where x is
 * the vocabulary id (0 for the acceptance uniform).  Streams: 0 draft sample, 1
 * acceptance uniform, 2 correction/bonus sample, 3 the trunk's own sample under
 * exact-match acceptance, whose counter is (x >> 2, 3 << 8, request_base + b, position):
 * keyed by the absolute position of the token, not by the cycle or the row.  Uniforms:
 * acceptance u = ((w >> 8) + 1) * 2^-24 in (0, 1]; Gumbel u = (2 (w >> 9) + 1) * 2^-24
 * in (0, 1), noise -ln(-ln u).  Every categorical draw is argmax(z/T + noise), lowest id
 * on ties. */
typedef enum mtp_accept_rule {
  /* T > 0: u*q <= p with the residual resample (DS4Server issue above, closing comment
   * "Review"): the output follows p, but it is not the token sequence of decoding
   * without speculation */
  MTP_ACCEPT_RATIO = 0,
  /* T > 0: a draft is accepted only if it equals the token the trunk samples at that
   * position (lucebox-hub PR above, sections "Exactness" and "Notes"): with the trunk's
   * draws keyed by position (stream 3), the output is the token sequence of decoding
   * without speculation under the same seed.  Drafts are the draft head's argmax. */
  MTP_ACCEPT_EXACT = 1
} mtp_accept_rule;

typedef struct mtp_sampling {
  float temperature;     /* T >= 0; 0 = greedy (argmax drafts, exact-match acceptance) */
  int32_t eos_id;        /* end-of-sequence id, or -1 for none                          */
  uint64_t seed;         /* Philox key                                                  */
  uint32_t cycle;        /* cycle counter; a new value gives fresh draws                */
  uint32_t request_base; /* counter index of request 0 of this call                     */
  int32_t accept_rule;   /* mtp_accept_rule; no effect at T = 0                          */
  int32_t reserved;      /* must be 0                                                   */
  const int32_t* positions; /* device int32 [B], read by mtp_verify_logits under
                             * MTP_ACCEPT_EXACT at T > 0 (else may be NULL): absolute
                             * position of the token verify row 0 of request b predicts;
                             * row i samples position positions[b] + i                  */
} mtp_sampling;

/* ---------------------------------------------------------------------------------- */
/* per-row results of the draft head and the verify pass (32 bytes)                    */
/* ---------------------------------------------------------------------------------- */
/* Logits are sanitised before any statistic: NaN -> -inf; a row holding +inf becomes
 * 0 at its +inf ids and -inf elsewhere (uniform over them).  T_eff = T, or 1 when T = 0. */
typedef struct mtp_row_stats {
  float max;         /* max of the sanitised logits (-inf if every one is -inf)         */
  float lse;         /* log sum exp(z / T_eff) of the sanitised logits                  */
  float z_tok;       /* sanitised logit of this row's token of interest:
                        draft rows - the picked draft token;
                        verify row i < k - the drafted token d_{i+1}; row k - -inf      */
  int32_t argmax;    /* lowest-id argmax; -1 if the row is invalid                      */
  int32_t sample;    /* argmax(z/T + Gumbel) at T > 0, = argmax at T = 0; -1 if invalid  */
  uint32_t flags;    /* MTP_ROW_* bits                                                 */
  int32_t n_posinf;  /* number of +inf logits in the row                                */
  int32_t reserved;
} mtp_row_stats;

#define MTP_ROW_NONFINITE 0x1u   /* the row held NaN or +-inf                           */
#define MTP_ROW_POSINF 0x2u      /* the row held +inf and was made uniform over those ids */
#define MTP_ROW_INVALID 0x4u     /* every sanitised logit is -inf                       */

/* per-request acceptance flags */
#define MTP_ACC_ALL_ACCEPTED 0x01u     /* all k drafts accepted; a bonus token emitted  */
#define MTP_ACC_EOS 0x02u              /* the block ends with eos_id                     */
#define MTP_ACC_RESID_FALLBACK 0x04u   /* empty residual; the correction was drawn from p */
#define MTP_ACC_ROW_INVALID 0x08u      /* a target row was all -inf: no token after it   */
#define MTP_ACC_NONFINITE_TARGET 0x10u /* a target row examined held NaN/+-inf           */
#define MTP_ACC_NONFINITE_DRAFT 0x20u  /* a draft row examined held NaN/+-inf            */
#define MTP_ACC_DRAFT_INVALID 0x40u    /* a draft token was -1 (all -inf draft row)      */
#define MTP_ACC_EOS_DRAFT 0x80u        /* the block ended on an accepted EOS draft: draft
                                          n_accept+1 was EOS and was accepted (with EOS
                                          alone, the EOS may be a correction or bonus)   */

/* ---------------------------------------------------------------------------------- */
/* workspace                                                                           */
/* ---------------------------------------------------------------------------------- */
typedef enum mtp_op { MTP_OP_DRAFT = 0, MTP_OP_VERIFY = 1, MTP_OP_ACCEPT = 2 } mtp_op;

/* Bytes of device workspace an op needs (DS4Server issue "Add Qwen3.8 Flash Next native
 * MTP speculation", section "Implementation": draft history, verify width, allocator
 * caches and temporary buffers are bounded and counted in memory admission; this is that
 * bound for the temporaries, so a caller can admit a request before running it).
 * rows = hidden rows of the call (draft: B,
 * verify: B*(k+1)); n_vocab_rows = rows of the head it scores (draft: n_draft, verify
 * and accept: vocab); B = requests.  The workspace holds per-block partial results and
 * completion counters.  It must be 256-byte aligned and zero-filled once after it is
 * allocated; every call leaves its counters at zero again, so one workspace of the
 * largest size can serve every call on a stream.  Returns 0 for invalid arguments. */
size_t mtp_workspace_bytes(int32_t op, int32_t rows, int32_t n_vocab_rows, int32_t B);

/* ---------------------------------------------------------------------------------- */
/* the four calls                                                                      */
/* ---------------------------------------------------------------------------------- */

/* Draft head, one draft slot for B requests (lucebox-hub PR above, section "What":
 * a 64,000-row draft head, token picked on the GPU and fed from device memory).
 *   z[b][x] = sum_j W[x][j] * hidden[b][j]   for x < n_draft   (fp32 accumulation)
 *   T = 0: token = lowest-id argmax of z;  T > 0: token = argmax(z/T + Gumbel(stream 0,
 *   row = slot)), a sample of q = softmax(z/T) over the first n_draft ids.  Under
 *   MTP_ACCEPT_EXACT the draft head works as at T = 0 (argmax, statistics at T_eff = 1).
 *   A head with row_ids (the same PR, "What": control/special tokens plus the lowest
 *   ids) scores its n_draft rows and reports vocabulary ids: the token, the argmax and
 *   the Gumbel draws (keyed by the vocabulary id) refer to row_ids[r]; draft_logits stay
 *   indexed by row.
 * hidden:        [B][d] in htype.
 * draft_tokens:  int32 [B][k_max]; writes column `slot`; -1 for an all -inf row.
 * draft_stats:   mtp_row_stats [B][k_max]; writes column `slot`.
 * draft_logits:  float [B][k_max][n_draft] raw (unsanitised) logits, writes slot `slot`;
 *                required when T > 0 under MTP_ACCEPT_RATIO (the residual needs q), else
 *                may be NULL.
 * 1 <= n_draft <= vocab; 1 <= B <= 16; 0 <= slot < k_max <= 7.                        */
int mtp_draft_head(const mtp_head* head, int32_t n_draft, const void* hidden, int32_t htype,
                   int32_t B, int32_t slot, int32_t k_max, const mtp_sampling* smp,
                   int32_t* draft_tokens, mtp_row_stats* draft_stats, float* draft_logits,
                   void* ws, size_t ws_bytes, void* stream);

/* Verify pass: full-vocabulary logits of the k+1 verify rows of B requests in one
 * batched pass (lucebox-hub PR above, section "What"; its "Exactness" section requires
 * the verify to be batch-invariant: a row's logits and statistics here do not depend on
 * B, k or the row's position in the batch).
 * hidden:        [B][k+1][d] in htype; row 0 = the last committed token, row i = draft d_i.
 * draft_tokens:  int32 [B][k_max]; row i < k records z at draft_tokens[b][i].
 * row_stats:     mtp_row_stats [B][k+1].  At T > 0 `sample` is argmax(z/T + Gumbel) on
 *                stream 2, row i, or under MTP_ACCEPT_EXACT on stream 3 at position
 *                smp->positions[b] + i (the trunk's own sample, the same draw whatever the
 *                cycle, row or batch the position is verified in).
 * logits:        float [B][k+1][vocab] raw logits; required when T > 0 under
 *                MTP_ACCEPT_RATIO, else may be NULL.
 * 1 <= k <= k_max <= 7; 1 <= B*(k+1) <= 128.                                           */
int mtp_verify_logits(const mtp_head* head, const void* hidden, int32_t htype, int32_t B,
                      int32_t k, const int32_t* draft_tokens, int32_t k_max,
                      const mtp_sampling* smp, mtp_row_stats* row_stats, float* logits,
                      void* ws, size_t ws_bytes, void* stream);

/* Acceptance for B requests (one block per request).  For i = 0..k-1, draft t = d_{i+1}:
 *   a target row i that is all -inf stops the block before it (MTP_ACC_ROW_INVALID,
 *   n_emit = n_accept = i, no further token);
 *   T = 0: accepted iff t == argmax of verify row i (lucebox-hub PR, "Exactness");
 *   T > 0, MTP_ACCEPT_RATIO: accepted iff p_i(t) > 0 and u*q_i(t) <= p_i(t), u from
 *          stream 1 (DS4Server issue, closing comment "Review"); q is 0 outside the draft
 *          vocabulary;
 *   T > 0, MTP_ACCEPT_EXACT: accepted iff t == the sample of verify row i (lucebox-hub
 *          PR, "Exactness");
 *   at the first rejection the next token is y_i (T = 0), the sample of row i
 *   (MTP_ACCEPT_EXACT), or a draw from max(0, p_i - q_i) renormalised (Gumbel-max on
 *   stream 2, row i); an empty residual draws from p_i instead (MTP_ACC_RESID_FALLBACK);
 *   an accepted t == eos_id ends the block with EOS as its last token (DS4Server issue,
 *   "Implementation": nothing is kept beyond EOS); n_accept = i;
 *   all k accepted: a bonus token from row k (argmax, or the stream-2 sample).
 * Inputs are the outputs of the draft and verify calls of the same cycle (draft_logits
 * and logits are read only when T > 0 under MTP_ACCEPT_RATIO).  vocab and n_draft must
 * match those calls.  draft_row_of: device int32 [vocab], the draft row of vocabulary id
 * x or -1 (the inverse of the draft head's row_ids; q is 0 off its rows), or NULL when
 * the draft rows are ids 0..n_draft-1; read only when T > 0 under MTP_ACCEPT_RATIO.
 * out_tokens: int32 [B][k+1] = d_1..d_a, last, then -1;  n_accept, n_emit: int32 [B]
 * (n_emit = n_accept + 1 except with MTP_ACC_ROW_INVALID);  flags: uint32 [B].        */
int mtp_accept_sample(int32_t B, int32_t k, int32_t k_max, int32_t vocab, int32_t n_draft,
                      const mtp_sampling* smp, const int32_t* draft_tokens,
                      const mtp_row_stats* draft_stats, const float* draft_logits,
                      const mtp_row_stats* row_stats, const float* logits, const int32_t* draft_row_of,
                      int32_t* out_tokens, int32_t* n_accept, int32_t* n_emit, uint32_t* flags,
                      void* ws, size_t ws_bytes, void* stream);

/* Commit (DS4Server issue, "Implementation": commit only accepted rows, trim rejected
 * rows; lucebox-hub PR, "Exactness": state restored bit-exactly).  Per request b with
 * a = clamp(n_accept[b], 0, k) and L = clamp(kv_len[b], 0, max_rows):
 *   live[b] <- snapshots[b][a]                        (state_bytes bytes, a byte copy)
 *   rows L+a+1 .. L+k of every layer's K and V in kv  are zero-filled (clipped to max_rows)
 *   kv_len[b] <- min(L + a + 1, max_rows)
 * snapshots: [B][k+1][state_bytes], snapshot r = recurrent state after verify row r.
 * live:      [B][state_bytes].
 * kv:        [B][n_layers][2][max_rows][kv_row_bytes] (may be NULL when n_layers = 0).
 * state_bytes and kv_row_bytes must be multiples of 16.                               */
int mtp_commit_state(int32_t B, int32_t k, const int32_t* n_accept, const void* snapshots,
                     void* live, size_t state_bytes, void* kv, int32_t n_layers,
                     int32_t max_rows, size_t kv_row_bytes, int32_t* kv_len, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops or harnesses that forbid hipMalloc): mtp_verify_logits without a workspace.  The
 * scratch the verify kernels need lives in a device array inside the library, 1,573,632
 * bytes per GPU (enough for any valid call: up to 128 rows, any vocabulary), held until
 * the process ends; the array used is that of the device the stream runs on (the current
 * device for the null stream), and its address is resolved, and its completion ticket
 * cleared, on the first call on each device.  The call allocates nothing.  Results are those of
 * mtp_verify_logits, bit for bit.  All calls on one GPU share the array and each leaves
 * it ready for the next: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  MTP_ERR_WORKSPACE if a call would
 * need more scratch than the array holds; otherwise the same status codes as
 * mtp_verify_logits. */
int mtp_verify_logits_noalloc(const mtp_head* head, const void* hidden, int32_t htype, int32_t B,
                              int32_t k, const int32_t* draft_tokens, int32_t k_max,
                              const mtp_sampling* smp, mtp_row_stats* row_stats, float* logits,
                              void* stream);

/* ---------------------------------------------------------------------------------- */
/* adaptive verify width (host side)                                                   */
/* ---------------------------------------------------------------------------------- */
/* lucebox-hub PR above, section "What": by default the verify width adapts, up to seven
 * drafts, from the acceptance seen at each draft depth and a per-request fit of the
 * cycle's cost.  One controller per request stream, owned by the caller; host memory
 * only, no device work.  The metrics the PR reports (drafted and accepted tokens,
 * verifier passes, acceptance depths) are its counters.
 *   alpha[j]  exponential moving average (weight `decay` per observation) of "draft j+1
 *             was accepted", over cycles that decided draft j+1: accepted (an accepted EOS
 *             draft, MTP_ACC_EOS_DRAFT, included) or rejected (an EOS correction
 *             included); a block that ended at an unusable target row leaves its stopping
 *             depth untouched;
 *   weight[j] recency of depth j: each request-cycle multiplies every weight by
 *             (1 - decay) and adds 1 at each depth it decided;
 *   a[j]      = alpha[j] where weight[j] >= 1/2, else a[j-1] (a[0] = alpha[0]): a depth
 *             not decided recently is estimated by the depth before it, an optimistic
 *             estimate that makes the controller explore deeper drafts when acceptance
 *             rises;
 *   E(k)      = 1 + sum_{i=1..k} prod_{j<i} a[j]   (expected tokens of a k-draft cycle);
 *   c(k)      = c0 + c1 k, least squares over the observed (k, seconds) pairs with weights
 *             decaying by (1 - decay) per observation; fewer than two distinct widths:
 *             c1 = slope_prior * c0; a negative fitted slope is taken as 0; no timing
 *             yet: c0 = 1, c1 = slope_prior;
 *   choose    = argmax over 1 <= k <= k_max of E(k) / c(k) (smallest k on ties; widths
 *             priced at <= 0 are skipped; 1 if all are). */
typedef struct mtp_width_ctl {
  int32_t k_max;                 /* 1..7                                                  */
  int32_t reserved;
  double decay;                  /* (0, 1]                                                */
  double slope_prior;            /* >= 0: c1 / c0 until two widths have been timed         */
  double alpha[7];
  double weight[7];              /* recency of each depth's estimate                        */
  double sw, sk, skk, st, skt;   /* decayed sums of 1, k, k^2, t, k t                       */
  uint64_t verifier_passes;      /* mtp_width_observe calls                                */
  uint64_t cycles;               /* request-cycles observed                                */
  uint64_t drafted, accepted;    /* drafts made / drafts kept                              */
  uint64_t depth_hist[8];        /* request-cycles that kept a = 0..7 drafts               */
} mtp_width_ctl;

/* A new controller (lucebox-hub PR above, "What": the adaptive width): alpha[*] = alpha0
 * in [0, 1]; counters and sums zero.  MTP_ERR_RANGE / _SHAPE on bad arguments. */
int mtp_width_init(mtp_width_ctl* c, int32_t k_max, double decay, double alpha0, double slope_prior);
/* The per-depth acceptance and the cost fit (lucebox-hub PR above, "What"), fed by one
 * verify pass of B requests with k drafts each: n_accept and flags are HOST copies
 * of mtp_accept_sample's outputs; seconds = the pass's measured cycle time (<= 0: not
 * timed).  MTP_ERR_RANGE if some n_accept is outside [0, k]; nothing is updated then. */
int mtp_width_observe(mtp_width_ctl* c, int32_t k, int32_t B, const int32_t* n_accept, const uint32_t* flags,
                      double seconds);
/* E(k), 0 <= k <= 7: expected tokens of a k-draft cycle from the per-depth acceptance
 * (lucebox-hub PR above, "What"). */
double mtp_width_expected_tokens(const mtp_width_ctl* c, int32_t k);
/* c(k): the fitted cycle cost (lucebox-hub PR above, "What": a per-request cost fit). */
double mtp_width_cost(const mtp_width_ctl* c, int32_t k);
/* k*, in 1..k_max: the width for the next cycle (lucebox-hub PR above, "What": up to seven
 * drafts by default). */
int32_t mtp_width_choose(const mtp_width_ctl* c);

/* ---------------------------------------------------------------------------------- */
/* weight preparation                                                                  */
/* ---------------------------------------------------------------------------------- */
/* Build infrastructure, no passage (the pages fix the weights' arithmetic, not their
 * layout in memory): the tiled layouts above are this library's own.
 * Bytes of one array of a tiled head for a source of type wtype (MTP_W_BF16 or
 * MTP_W_Q4A32): part 0 = w, 1 = scale, 2 = minv (0 for a part the format lacks, or for
 * invalid arguments). */
size_t mtp_tiled_bytes(int32_t wtype, int32_t d, int32_t vocab, int32_t part);

/* Gather rows of a row-major head (F32, BF16 or Q4A32) into a new row-major head, once,
 * at load time: row r of dst = row ids[r] of src, with its scales and mins
 * (lucebox-hub PR above, "What": the draft head is a subset of the vocabulary).
 * ids: device int32 [n],
 * strictly ascending ids in [0, src->vocab) (an id outside gives a zero row); dst_* hold
 * n rows of src's formats (dst_scale and dst_minv for Q4A32 only), 16-byte aligned, not
 * overlapping src.  The result is used with row_ids = ids, directly or after
 * mtp_pack_head. */
int mtp_gather_rows(const mtp_head* src, const int32_t* ids, int32_t n, void* dst_w, void* dst_scale,
                    void* dst_minv, void* stream);

/* Build infrastructure, no passage (see mtp_tiled_bytes).
 * Repack a row-major BF16 or Q4A32 head into the tiled layout (MTP_W_BF16_TILED /
 * MTP_W_Q4A32_TILED) on the device, once, at load time.  dst_* are device buffers of
 * mtp_tiled_bytes(src->wtype, ...) bytes (dst_scale and dst_minv only for Q4A32), 16-byte
 * aligned, not overlapping the source.  The tiled head gives the LM-head kernels the
 * same logits, bit for bit, as the row-major head it came from. */
int mtp_pack_head(const mtp_head* src, void* dst_w, void* dst_scale, void* dst_minv, void* stream);

/* ---------------------------------------------------------------------------------- */
/* misc                                                                                */
/* ---------------------------------------------------------------------------------- */
/* The clear message for a status code (llama.cpp PR above, loader commit): a static
 * string, never NULL, "unknown status" for a code not listed. */
const char* mtp_status_str(int status);
/* Build infrastructure, no passage: MTP_ABI_VERSION, for a caller to check at load time
 * that its copy of this header matches the library. */
int mtp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTP_H_ */
