"""Plain CPU oracle of one native-MTP speculative cycle, in fp64.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the CPU-baseline leg
of the bench may import, call or run this module.  It shares no code, header, table or
constant generator with the HIP library and imports nothing from it; the only thing the
two sides share is the input bytes made by the seeded generator package ``synth``.

What it computes, step by step, in the order the method runs.  Sources are the three
pages the method is described on, cited by title and section:
  [MTP-PR]   lucebox-hub PR "feat(qwen4exp): MTP speculative decoding"
             (sections "What", "Exactness", "Notes");
  [PORT-PR]  llama.cpp PR "qwen4exp : port NextN/MTP speculative decoding to master"
             (commit messages "full checkpoints for MTP rollback", "replay livelock fix",
             "keep speculative checkpoints on device"; PR body "Result");
  [DS4-98]   DS4Server issue "Add Qwen3.8 Flash Next native MTP speculation"
             (sections "Implementation", "Verification", "Completion requirements",
             and the closing comment's "Implementation", "Review", "Verification").

  O0  weights to fp64 (fp32 and bf16 convert exactly; 4-bit affine: scale*q + min)
  O1  draft logits over the first n_draft rows of the shared head   [MTP-PR "What"]
  O2  sanitise non-finite logits          [DS4-98 closing comment "Review": zero/non-finite]
  O3  draft token: argmax (T=0) or a sample from q = softmax(z/T)   [MTP-PR "What"]
  O4  verify logits over the full vocabulary for the k+1 rows        [MTP-PR "What"]
  O5  acceptance: exact match (T=0) [MTP-PR "Exactness"]; u*q <= p with a max(0, p-q)
      residual at the first rejection (T>0) [DS4-98 "Implementation", closing "Review"];
      EOS inside the block truncates [DS4-98 "Implementation"]
  O6  commit: the accepted row's recurrent snapshot becomes live, rejected KV rows are
      trimmed [DS4-98 "Implementation"; MTP-PR "Exactness"; PORT-PR on-device checkpoints]

Readings where the pages are silent (each is a stated choice, listed with the design):
  * draft vocabulary = the first n_draft ids of the shared head, or a strictly ascending
    id list (control/special tokens plus the lowest ids [MTP-PR "What"]); draws for a
    draft row are keyed by its vocabulary id;
  * argmax ties go to the lowest id;
  * NaN -> -inf; a row holding +inf becomes uniform over its +inf ids; an all -inf
    target row stops the block before that row (flag ROW_INVALID, no correction token);
    an all -inf draft row gives draft -1, which is rejected with q = 0;
  * u in (0, 1], accept iff p(t) > 0 and u*q(t) <= p(t) (compared in log space);
  * empty residual (p <= q everywhere): sample from p instead, flag RESID_FALLBACK;
  * drafts at T > 0 are samples from q at the same T (Gumbel-max);
  * every categorical draw is Gumbel-max on Philox4x32-10 words; counter =
    (x >> 2, stream << 8 | row, request, cycle), key = (seed lo32, seed hi32), word x & 3;
    streams: 0 draft, 1 acceptance uniform, 2 correction/bonus, 3 the trunk's own sample
    under exact-match acceptance, whose counter is (x >> 2, 3 << 8, request, position):
    the same draw for a position in whatever cycle or row it is verified;
  * exact-match acceptance at T > 0 takes the drafts as the draft head's argmax;
  * all k drafts accepted -> one bonus token from row k;
  * an accepted EOS draft ends the block: n_accept = its row, the EOS is the last token
    and is never consumed, so snapshot n_accept is committed;
  * snapshot r = state after consuming verify row r; commit keeps kv rows up to
    kv_len + n_accept and zeroes the rejected ones.

Where floating point decides an integer (an argmax, the ratio test), the decision is
taken in fp32, the kernel's precision, on the fp64 quantities rounded once to fp32.

Near ties.  A GPU logit may differ from the oracle's by up to the logit tolerance delta
(the comparison's hard check on every materialised logit).  A decision is flagged -- the
GPU may take it either way -- when its margin, measured in fp64 in the units of its own
score, is within what that tolerance moves the score:
  * an argmax of logits z: top-1 minus top-2 <= delta;
  * an argmax of z/T + Gumbel (draft sample, bonus, the trunk's own sample): top-1 minus
    top-2 <= delta/T;
  * the ratio test: |ln u + ln q(t) - ln p(t)| <= delta/T;
  * the residual pick argmax(ln max(0, p - q) + Gumbel): every ln p(x) and ln q(x) may
    move by eps = 2 delta/T (delta/T from the logit, delta/T from the row's log-sum-exp);
    under such moves max(0, p - q) ranges over an interval per id, and the pick is
    flagged when the least score of the picked id does not exceed the greatest score of
    some other id.  An empty residual is flagged when such moves can give it mass.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------
# flags
# ----------------------------------------------------------------------------------
ROW_NONFINITE = 1 << 0   # the row held NaN or +-inf before sanitising
ROW_POSINF = 1 << 1      # the row held +inf and became uniform over those ids
ROW_INVALID = 1 << 2     # every sanitised logit is -inf

ACC_ALL_ACCEPTED = 1 << 0
ACC_EOS = 1 << 1
ACC_RESID_FALLBACK = 1 << 2
ACC_ROW_INVALID = 1 << 3
ACC_NONFINITE_TARGET = 1 << 4
ACC_NONFINITE_DRAFT = 1 << 5
ACC_DRAFT_INVALID = 1 << 6
ACC_EOS_DRAFT = 1 << 7   # the block ended on an accepted EOS draft (not a correction/bonus EOS)

STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESAMPLE, STREAM_TRUNK = 0, 1, 2, 3
RULE_RATIO, RULE_EXACT = "ratio", "exact"

NEG_INF = -np.inf
F32 = np.float32

# ----------------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
# 1, 2, 3", SC'11).  Each round multiplies counter words 0 and 2 by the two round
# multipliers, forms the next counter from the high/low halves crossed with words 1
# and 3 and the round key, then bumps the key by the two Weyl constants.
# ----------------------------------------------------------------------------------
_PHILOX_MUL = (0xD2511F53, 0xCD9E8D57)
_PHILOX_WEYL = (0x9E3779B9, 0xBB67AE85)
_LO32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Ten Philox4x32 rounds on uint32-valued counters (arrays broadcast); returns 4 uint32 arrays."""
    c = [np.asarray(v, dtype=np.uint64) & _LO32 for v in (c0, c1, c2, c3)]
    c = list(np.broadcast_arrays(*c))
    m0, m1 = np.uint64(_PHILOX_MUL[0]), np.uint64(_PHILOX_MUL[1])
    key0, key1 = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for _ in range(10):
        prod0 = c[0] * m0          # both factors < 2^32: the 64-bit product is exact
        prod1 = c[2] * m1
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & _LO32
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & _LO32
        c = [hi1 ^ c[1] ^ np.uint64(key0), lo1, hi0 ^ c[3] ^ np.uint64(key1), lo0]
        key0 = (key0 + _PHILOX_WEYL[0]) & 0xFFFFFFFF
        key1 = (key1 + _PHILOX_WEYL[1]) & 0xFFFFFFFF
    return [v.astype(np.uint32) for v in c]


def philox_words(seed: int, stream: int, row, b, cycle: int, x) -> np.ndarray:
    """The uint32 word for element x of (stream, row, request b, cycle) under ``seed``."""
    x = np.asarray(x, dtype=np.uint64)
    row = np.asarray(row, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    ctr1 = (np.uint64(stream) << np.uint64(8)) | row
    out = philox4x32_10(x >> np.uint64(2), ctr1, b, np.uint64(cycle & 0xFFFFFFFF),
                        seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (x & np.uint64(3)).astype(np.int64)
    stacked = np.stack(np.broadcast_arrays(*out), axis=0)
    sel = np.broadcast_to(sel, stacked.shape[1:])
    return np.take_along_axis(stacked, sel[None], axis=0)[0]


def uniform_accept(w) -> np.ndarray:
    """u = ((w >> 8) + 1) * 2^-24, in (0, 1]: exactly representable in fp32."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(8)) + np.uint64(1)).astype(np.float64) * 2.0 ** -24


def uniform_gumbel(w) -> np.ndarray:
    """u = (2 * (w >> 9) + 1) * 2^-24, in (0, 1): exactly representable in fp32."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)) * np.uint64(2) + np.uint64(1)).astype(np.float64) * 2.0 ** -24


def gumbel_noise(seed: int, stream: int, row, b, cycle: int, n: int, ids=None) -> np.ndarray:
    """Standard Gumbel noise -ln(-ln u) for ids 0..n-1 (or for the given ids); shape
    broadcast(b, row) + (n,)."""
    b = np.asarray(b)[..., None]
    row = np.asarray(row)[..., None]
    xs = np.arange(n) if ids is None else np.asarray(ids)
    u = uniform_gumbel(philox_words(seed, stream, row, b, cycle, xs))
    return -np.log(-np.log(u))


def trunk_noise(seed: int, b: int, position: int, n: int) -> np.ndarray:
    """Gumbel noise of the trunk's own draw for request b at an absolute position.

    Exact-match acceptance [MTP-PR "Exactness", "Notes"] keeps a draft only if it equals
    the token the trunk samples, so that the output is the token sequence of decoding
    without speculation: that draw must depend on the position alone, never on the cycle
    or the verify row.  Stream 3, counter (x >> 2, 3 << 8, b, position).
    """
    return gumbel_noise(seed, STREAM_TRUNK, 0, b, int(position) & 0xFFFFFFFF, n)


def trunk_sample(z_row: np.ndarray, T: float, seed: int, b: int, position: int):
    """The trunk's token at one position: argmax(z/T + trunk noise), lowest id on ties,
    decided in fp32; also the fp64 top-2 gap of the scores.  z_row is sanitised."""
    G = trunk_noise(seed, b, position, z_row.shape[-1])
    return int(argmax_lowest_f32(_f32_add(z_row / T, G))), float(top2_gap(z_row / T + G))


# ----------------------------------------------------------------------------------
# O0  weights and hidden rows to fp64
# ----------------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact): the bf16 bits are the top half of an fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def head_weights_f64(head) -> np.ndarray:
    """O0: the shared LM head W[V][d] in fp64.

    4-bit affine with 32-value groups [DS4-98 closing comment "Implementation"]:
    w[x][32g + j] = scale[x][g] * q + min[x][g], q = nibble j of group g (element 2m
    in the low nibble of byte m).  Every term is exact in fp64.
    """
    if head.wtype == "f32":
        return np.asarray(head.w, dtype=np.float64)
    if head.wtype == "bf16":
        return bf16_to_f64(head.w)
    if head.wtype == "q4a32":
        nib = np.asarray(head.w, dtype=np.uint8)
        V, half = nib.shape
        q = np.empty((V, 2 * half), dtype=np.float64)
        q[:, 0::2] = nib & 0x0F
        q[:, 1::2] = nib >> 4
        scale = np.repeat(bf16_to_f64(head.scale), 32, axis=1)
        minv = np.repeat(bf16_to_f64(head.minv), 32, axis=1)
        return scale * q + minv
    raise ValueError(head.wtype)


def hidden_f64(h: np.ndarray, htype: str) -> np.ndarray:
    if htype == "f32":
        return np.asarray(h, dtype=np.float64)
    if htype == "bf16":
        return bf16_to_f64(h)
    raise ValueError(htype)


# ----------------------------------------------------------------------------------
# O1/O4  logits, O2 sanitising, row statistics
# ----------------------------------------------------------------------------------
def logits_f64(W64: np.ndarray, H64: np.ndarray) -> np.ndarray:
    """z = W h for every hidden row: [..., d] -> [..., V] (a plain fp64 matmul)."""
    return H64 @ W64.T


def sanitize(z: np.ndarray):
    """O2: NaN -> -inf; a row with any +inf becomes {+inf -> 0, all else -> -inf}.

    Returns (sanitised logits, per-row ROW_* flags).
    """
    z = np.asarray(z, dtype=np.float64)
    posinf = np.isposinf(z)
    any_pos = posinf.any(axis=-1)
    nonfinite = ~np.isfinite(z).all(axis=-1)
    out = np.where(np.isnan(z), NEG_INF, z)
    out = np.where(any_pos[..., None], np.where(posinf, 0.0, NEG_INF), out)
    invalid = ~(out > NEG_INF).any(axis=-1)
    flags = (nonfinite * ROW_NONFINITE) | (any_pos * ROW_POSINF) | (invalid * ROW_INVALID)
    return out, flags.astype(np.uint32)


def logsumexp_rows(s: np.ndarray) -> np.ndarray:
    """log sum_x exp(s[..., x]); -inf for an all -inf row."""
    m = s.max(axis=-1)
    safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return safe + np.log(np.exp(s - safe[..., None]).sum(axis=-1))


def argmax_lowest_f32(scores: np.ndarray) -> np.ndarray:
    """Lowest-id argmax of the scores rounded to fp32; -1 where every score is -inf."""
    s = np.asarray(scores, dtype=np.float64).astype(F32)
    idx = np.argmax(s, axis=-1)          # first occurrence = lowest id
    valid = (s > NEG_INF).any(axis=-1)
    return np.where(valid, idx, -1).astype(np.int64)


def top2_gap(scores: np.ndarray) -> np.ndarray:
    """fp64 gap between the best and second-best score (inf with < 2 finite scores)."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[-1]
    if n < 2:
        return np.full(s.shape[:-1], np.inf)
    part = -np.partition(-s, 1, axis=-1)[..., :2]
    gap = part[..., 0] - part[..., 1]
    return np.where(np.isfinite(part[..., 1]), gap, np.inf)


def argmax_margin(zs: np.ndarray, rflags: np.ndarray) -> np.ndarray:
    """Top-2 gap of sanitised logits for the argmax; infinite for a row that held +inf,
    whose argmax is its lowest +inf id by an exact rule on exact values (the sanitised +inf
    ids are all exactly 0), which no logit tolerance can turn."""
    gap = top2_gap(zs)
    return np.where((np.asarray(rflags) & ROW_POSINF) != 0, np.inf, gap)


def _f32_add(a, b):
    return np.asarray(a, dtype=np.float64).astype(F32) + np.asarray(b, dtype=np.float64).astype(F32)


def _teff(T: float) -> float:
    return T if T > 0 else 1.0


# ----------------------------------------------------------------------------------
# near-tie flags (decisions the logit tolerance delta can turn either way)
# ----------------------------------------------------------------------------------
def score_tolerance(delta: float, T: float) -> float:
    """What a logit tolerance delta moves a score z/T + Gumbel by: delta/T (delta at T = 0,
    where the score is the logit itself)."""
    return delta / T if T > 0 else delta


def gap_near_tie(gap, tol: float) -> np.ndarray:
    """An argmax whose top-1 minus top-2 score is within the score's tolerance."""
    return np.asarray(gap, dtype=np.float64) <= tol


def ratio_near_tie(margin, delta: float, T: float) -> np.ndarray:
    """The ratio test u*q(t) <= p(t) with |ln u + ln q(t) - ln p(t)| <= delta/T."""
    m = np.asarray(margin, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        return np.isfinite(m) & (np.abs(m) <= delta / T)


def residual_logprob_shift(delta: float, T: float) -> float:
    """How far a logit tolerance delta can move ln p(x) = z_x/T - lse(z/T): delta/T through
    z_x and delta/T through the log-sum-exp (which moves by at most the largest logit
    move)."""
    return 2.0 * delta / T


def residual_bounds(lp, lq, eps: float):
    """Least and greatest ln max(0, p' - q') over ln p' in [lp - eps, lp + eps] and
    ln q' in [lq - eps, lq + eps] (-inf where the residual can vanish / is always 0)."""
    lp = np.asarray(lp, dtype=np.float64)
    lq = np.asarray(lq, dtype=np.float64)
    lo_p, hi_q = lp - eps, lq + eps          # smallest p' - q'
    hi_p, lo_q = lp + eps, lq - eps          # largest p' - q'
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        lo = np.where(hi_q < lo_p, lo_p + np.log1p(-np.exp(hi_q - lo_p)), NEG_INF)
        hi = np.where(lo_q < hi_p, hi_p + np.log1p(-np.exp(lo_q - hi_p)), NEG_INF)
    return lo, hi


def residual_near_tie(lp, lq, G, pick, delta: float, T: float) -> np.ndarray:
    """Residual picks [n] (argmax of ln max(0, p - q) + G over rows [n][V]) that moves of
    ln p and ln q within residual_logprob_shift could change: the picked id's least score
    is not above the greatest score of some other id."""
    lo, hi = residual_bounds(lp, lq, residual_logprob_shift(delta, T))
    G = np.asarray(G, dtype=np.float64)
    rows = np.arange(G.shape[0])
    pick = np.asarray(pick, dtype=np.int64)
    s_lo = lo[rows, pick] + G[rows, pick]
    s_hi = hi + G
    s_hi[rows, pick] = NEG_INF
    return s_lo <= s_hi.max(axis=-1)


def empty_residual_near_tie(lp, lq, delta: float, T: float) -> np.ndarray:
    """Rows [n][V] with an empty residual (p <= q everywhere) that moves within
    residual_logprob_shift could give mass."""
    _, hi = residual_bounds(lp, lq, residual_logprob_shift(delta, T))
    return (hi > NEG_INF).any(axis=-1)


# ----------------------------------------------------------------------------------
# O1-O3  draft head
# ----------------------------------------------------------------------------------
def draft_rows(W64: np.ndarray, n_draft: int, h: np.ndarray, T: float, seed: int,
               slot: int, cycle: int, delta: float, b_ids=None, ids=None) -> dict:
    """One draft-head call for B requests (one hidden row each) [MTP-PR "What"].

    The head is the first n_draft rows of the shared LM head, or its rows ``ids`` (the
    draft vocabulary as an ascending id list, n_draft = len(ids)).  T == 0: the draft is
    the lowest-id argmax.  T > 0: the draft is argmax(z/T + Gumbel) over the draft
    vocabulary (noise keyed by the vocabulary id), i.e. a sample from q = softmax(z/T)
    restricted to it.  Also returns the row statistics (max, lse of z/T) and the raw
    logits (indexed by draft row), which the acceptance step needs.
    """
    B = h.shape[0]
    b_ids = np.arange(B) if b_ids is None else np.asarray(b_ids)
    rows = np.arange(n_draft) if ids is None else np.asarray(ids, dtype=np.int64)
    z = logits_f64(W64[rows], h)
    zs, rflags = sanitize(z)
    if T > 0:
        G = gumbel_noise(seed, STREAM_DRAFT, slot, b_ids, cycle, rows.size, ids=rows)
        local = argmax_lowest_f32(_f32_add(zs / T, G))
        margin = top2_gap(zs / T + G)
    else:
        local = argmax_lowest_f32(zs)
        margin = argmax_margin(zs, rflags)
    token = np.where(local >= 0, rows[np.maximum(local, 0)], -1)
    z_tok = np.where(local >= 0, np.take_along_axis(zs, np.maximum(local, 0)[:, None], 1)[:, 0], NEG_INF)
    return dict(token=token, max=zs.max(axis=-1), lse=logsumexp_rows(zs / _teff(T)), z_tok=z_tok,
                flags=rflags, logits=z, margin=margin, near_tie=gap_near_tie(margin, score_tolerance(delta, T)))


# ----------------------------------------------------------------------------------
# O4  verify rows
# ----------------------------------------------------------------------------------
def verify_rows(W64: np.ndarray, h_v: np.ndarray, drafts, T: float, seed: int, cycle: int,
                delta: float, b_ids=None, positions=None) -> dict:
    """Full-vocabulary logits of the k+1 verify rows of every request [MTP-PR "What"].

    h_v [B][k+1][d]; drafts [B][k] (row i is checked against drafts[:, i]).  Per row:
    lowest-id argmax y, the Gumbel-max sample at T from stream 2 (the bonus token at row
    k) -- or, when ``positions`` [B] is given (exact-match acceptance), the trunk's own
    sample at position positions[b] + i --, max and lse of the sanitised z/T, and the
    sanitised logit at the drafted id.
    """
    B, K1, _ = h_v.shape
    b_ids = np.arange(B) if b_ids is None else np.asarray(b_ids)
    z = logits_f64(W64, h_v)
    V = z.shape[-1]
    zs, rflags = sanitize(z)
    y = argmax_lowest_f32(zs)
    y_margin = argmax_margin(zs, rflags)
    if T > 0 and positions is not None:
        sample = np.empty((B, K1), dtype=np.int64)
        s_margin = np.empty((B, K1))
        for bi in range(B):
            for i in range(K1):
                sample[bi, i], s_margin[bi, i] = trunk_sample(zs[bi, i], T, seed, int(b_ids[bi]),
                                                              int(positions[bi]) + i)
        sample = np.where((rflags & ROW_INVALID) != 0, -1, sample)
    elif T > 0:
        G = gumbel_noise(seed, STREAM_RESAMPLE, np.arange(K1)[None, :], b_ids[:, None], cycle, V)
        sample = argmax_lowest_f32(_f32_add(zs / T, G))
        s_margin = top2_gap(zs / T + G)
    else:
        sample, s_margin = y.copy(), y_margin.copy()
    z_tok = np.full((B, K1), NEG_INF)
    if drafts is not None:
        drafts = np.asarray(drafts)
        for i in range(min(K1 - 1, drafts.shape[1])):
            t = drafts[:, i]
            ok = (t >= 0) & (t < V)
            z_tok[:, i] = np.where(ok, zs[np.arange(B), i, np.clip(t, 0, V - 1)], NEG_INF)
    return dict(argmax=y, sample=sample, max=zs.max(axis=-1), lse=logsumexp_rows(zs / _teff(T)),
                z_tok=z_tok, flags=rflags, logits=z, y_margin=y_margin, s_margin=s_margin,
                y_near_tie=gap_near_tie(y_margin, delta),
                s_near_tie=gap_near_tie(s_margin, score_tolerance(delta, T)))


# ----------------------------------------------------------------------------------
# O5  acceptance, first rejection, residual resample, EOS
# ----------------------------------------------------------------------------------
def accept_test(lp_t, lq_t, u):
    """Ratio test u*q(t) <= p(t) in log space [DS4-98 closing comment "Review"].

    Rejects when p(t) = 0; accepts when q(t) = 0 < p(t).  Decided in fp32.
    """
    lp_t = np.asarray(lp_t, dtype=np.float64)
    lhs = _f32_add(np.log(u), lq_t)
    return (lp_t > NEG_INF) & (lhs <= lp_t.astype(F32))


def residual_log_weights(lp: np.ndarray, lq: np.ndarray) -> np.ndarray:
    """ln max(0, p - q), elementwise; -inf where p <= q [DS4-98 "Implementation"].

    ln(p - q) = ln p + ln(1 - q/p) = lp + log1p(-exp(lq - lp)) where lp > lq.
    """
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        val = lp + np.log1p(-np.exp(lq - lp))
    return np.where(lp > lq, val, NEG_INF)


def accept(drafts, zd_raw, zv_raw, n_draft: int, T: float, seed: int, cycle: int, eos: int,
           delta: float, b_ids=None, draft_near_tie=None, rule: str = RULE_RATIO, target=None,
           draft_ids=None) -> dict:
    """O5 for B requests: scan the drafts, stop at the first rejection, emit one more token.

    drafts [B][k]; zd_raw [B][k][n_draft] raw draft logits (needed when T > 0);
    zv_raw [B][k+1][V] raw verify logits.
      T == 0: draft d_{i+1} is accepted iff it equals y_i, the lowest-id argmax of row i
              [MTP-PR "Exactness"]; the token after the last accepted draft is y at the
              stopping row (correction or bonus).
      T >  0: accepted iff p_i(t) > 0 and u*q_i(t) <= p_i(t), u from stream 1; at the first
              rejection the token is drawn from max(0, p_i - q_i) renormalised (Gumbel-max on
              stream 2) [DS4-98 "Implementation", closing comment "Review"]; the residual is
              empty only when p = q, then it is drawn from p (flag RESID_FALLBACK).
      T >  0, rule "exact": accepted iff it equals the trunk's own sample at row i, and
              that sample is also the token after the last accepted draft [MTP-PR
              "Exactness", "Notes"]; ``target`` is verify_rows' output with positions.
      An accepted EOS draft ends the block [DS4-98 "Implementation"]; an all -inf target
      row stops the block before it with no extra token.
    Returns tokens [B][k+1] (-1 padded), n_accept, n_emit, flags, and the first row whose
    decision margin is inside the tolerance (-1 if none).
    """
    drafts = np.asarray(drafts, dtype=np.int64)
    B, k = drafts.shape
    b_ids = np.arange(B) if b_ids is None else np.asarray(b_ids)
    zv, vflags = sanitize(zv_raw)
    V = zv.shape[-1]
    # draft row of each vocabulary id (-1 outside the draft vocabulary)
    row_of = np.full(V, -1, dtype=np.int64)
    d_ids = np.arange(n_draft) if draft_ids is None else np.asarray(draft_ids, dtype=np.int64)
    row_of[d_ids] = np.arange(d_ids.size)
    Te = _teff(T)
    lse_v = logsumexp_rows(zv / Te)
    y = argmax_lowest_f32(zv)
    y_margin = argmax_margin(zv, vflags)
    exact = T > 0 and rule == RULE_EXACT
    if exact:
        ys, ys_margin = np.asarray(target["sample"]), np.asarray(target["s_margin"])
    if zd_raw is not None:
        # draft-row flags are reported at any temperature; q itself is used only when T > 0
        zd, dflags = sanitize(zd_raw)
        lse_d = logsumexp_rows(zd / Te)
    elif T > 0 and not exact:
        raise ValueError("the ratio test needs the draft logits")
    else:
        dflags = np.zeros((B, k), dtype=np.uint32)

    n_accept = np.full(B, k, dtype=np.int64)
    last = np.full(B, -1, dtype=np.int64)
    flags = np.zeros(B, dtype=np.uint32)
    stop_kind = np.full(B, -1)          # 0 rejected, 1 eos draft, 2 all accepted, 3 invalid row
    tie_row = np.full(B, -1, dtype=np.int64)
    active = np.ones(B, dtype=bool)
    rows = np.arange(B)

    def mark_tie(mask, i):
        hit = mask & (tie_row < 0)
        tie_row[hit] = i

    if draft_near_tie is not None:
        dnt = np.asarray(draft_near_tie, dtype=bool)
    else:
        dnt = np.zeros((B, k), dtype=bool)

    for i in range(k):
        # target row i must be usable before its draft is judged
        inv = active & ((vflags[:, i] & ROW_INVALID) != 0)
        n_accept[inv] = i
        stop_kind[inv] = 3
        active &= ~inv
        flags[active & ((vflags[:, i] & ROW_NONFINITE) != 0)] |= ACC_NONFINITE_TARGET
        flags[active & ((dflags[:, i] & ROW_NONFINITE) != 0)] |= ACC_NONFINITE_DRAFT
        mark_tie(active & dnt[:, i], i)
        t = drafts[:, i]
        t_ok = (t >= 0) & (t < V)
        flags[active & ~t_ok] |= ACC_DRAFT_INVALID
        tc = np.clip(t, 0, V - 1)
        if exact:
            ok = t_ok & (t == ys[:, i])
            mark_tie(active & gap_near_tie(ys_margin[:, i], score_tolerance(delta, T)), i)
        elif T > 0:
            with np.errstate(invalid="ignore"):   # a non-finite target row gives NaN here, flagged above
                lp_t = np.where(t_ok, zv[rows, i, tc] / T - lse_v[:, i], NEG_INF)
            tr = row_of[tc]
            in_draft = t_ok & (tr >= 0) & ((dflags[:, i] & ROW_INVALID) == 0)
            with np.errstate(invalid="ignore"):
                lq_t = np.where(in_draft, zd[rows, i, np.maximum(tr, 0)] / T - lse_d[:, i], NEG_INF)
            u = uniform_accept(philox_words(seed, STREAM_ACCEPT, i, b_ids, cycle, 0))
            ok = t_ok & accept_test(lp_t, lq_t, u)
            with np.errstate(invalid="ignore"):
                m = np.log(u) + lq_t - lp_t
            mark_tie(active & t_ok & ratio_near_tie(m, delta, T), i)
        else:
            ok = t_ok & (t == y[:, i])
            mark_tie(active & gap_near_tie(y_margin[:, i], delta), i)
        rej = active & ~ok
        n_accept[rej] = i
        stop_kind[rej] = 0
        active &= ~rej
        hit_eos = active & (t == eos) & (eos >= 0)
        n_accept[hit_eos] = i
        stop_kind[hit_eos] = 1
        last[hit_eos] = eos
        active &= ~hit_eos
    # all k drafts accepted: bonus from row k (if row k is usable)
    inv = active & ((vflags[:, k] & ROW_INVALID) != 0)
    stop_kind[inv] = 3
    n_accept[inv] = k
    active &= ~inv
    stop_kind[active] = 2
    flags[active & ((vflags[:, k] & ROW_NONFINITE) != 0)] |= ACC_NONFINITE_TARGET

    # corrections (first rejection) and bonus tokens, grouped by the stopping row
    def gumbel_pick(scores64, G):
        pick = argmax_lowest_f32(_f32_add(scores64, G))
        return pick, top2_gap(scores64 + G)

    for a in range(k):
        sel = np.nonzero((stop_kind == 0) & (n_accept == a))[0]
        if sel.size == 0:
            continue
        if T <= 0:
            last[sel] = y[sel, a]
            continue
        if exact:
            last[sel] = ys[sel, a]
            continue
        lp = zv[sel, a] / T - lse_v[sel, a][:, None]
        lq = np.full((sel.size, V), NEG_INF)
        dval = (dflags[sel, a] & ROW_INVALID) == 0
        lq[np.ix_(np.nonzero(dval)[0], d_ids)] = zd[sel[dval], a] / T - lse_d[sel[dval], a][:, None]
        ln_r = residual_log_weights(lp, lq)
        G = gumbel_noise(seed, STREAM_RESAMPLE, a, b_ids[sel], cycle, V)
        has_mass = (ln_r > NEG_INF).any(axis=-1)
        pick_r = argmax_lowest_f32(_f32_add(ln_r, G))
        pick_p, gap_p = gumbel_pick(zv[sel, a] / T, G)
        last[sel] = np.where(has_mass, pick_r, pick_p)
        flags[sel[~has_mass]] |= ACC_RESID_FALLBACK
        tie_r = residual_near_tie(lp, lq, G, np.maximum(pick_r, 0), delta, T)
        tie_p = empty_residual_near_tie(lp, lq, delta, T) | gap_near_tie(gap_p, score_tolerance(delta, T))
        tie = np.where(has_mass, tie_r, tie_p)
        mark_tie(np.isin(rows, sel[tie]), a)

    sel = np.nonzero(stop_kind == 2)[0]
    flags[sel] |= ACC_ALL_ACCEPTED
    if sel.size:
        if exact:
            last[sel] = ys[sel, k]
            mark_tie(np.isin(rows, sel[gap_near_tie(ys_margin[sel, k], score_tolerance(delta, T))]), k)
        elif T > 0:
            G = gumbel_noise(seed, STREAM_RESAMPLE, k, b_ids[sel], cycle, V)
            last[sel], gap = gumbel_pick(zv[sel, k] / T, G)
            mark_tie(np.isin(rows, sel[gap_near_tie(gap, score_tolerance(delta, T))]), k)
        else:
            last[sel] = y[sel, k]
            mark_tie(np.isin(rows, sel[gap_near_tie(y_margin[sel, k], delta)]), k)
    flags[stop_kind == 3] |= ACC_ROW_INVALID
    flags[stop_kind == 1] |= ACC_EOS_DRAFT

    # emitted block: the accepted drafts, then the correction / bonus / EOS token
    col = np.arange(k + 1)[None, :]
    padded = np.concatenate([drafts, np.full((B, 1), -1, dtype=np.int64)], axis=1)
    tokens = np.where(col < n_accept[:, None], padded, -1)
    has_last = stop_kind != 3
    tokens[rows[has_last], n_accept[has_last]] = last[has_last]
    n_emit = n_accept + has_last.astype(np.int64)
    if eos >= 0:
        flags[has_last & (last == eos)] |= ACC_EOS
    return dict(tokens=tokens, n_accept=n_accept, n_emit=n_emit, flags=flags,
                tie_row=tie_row, stop_kind=stop_kind)


# ----------------------------------------------------------------------------------
# O6  commit
# ----------------------------------------------------------------------------------
def commit(snapshots: np.ndarray, live: np.ndarray, kv: np.ndarray, kv_len: np.ndarray,
           n_accept: np.ndarray, k: int):
    """Keep exactly the accepted rows [DS4-98 "Implementation"; MTP-PR "Exactness"].

    snapshots [B][k+1][S] bytes, snapshot r = recurrent state after verify row r;
    kv [B][L][2][max_rows][row_bytes]; kv_len [B].  With a = clamp(n_accept, 0, k):
    live[b] <- snapshots[b][a]; rows kv_len+a+1 .. kv_len+k of every layer's K and V
    are zeroed (clipped to the cache); kv_len <- min(kv_len + a + 1, max_rows).
    Returns new (live, kv, kv_len); the inputs are not modified.
    """
    live = live.copy()
    kv = kv.copy()
    max_rows = kv.shape[3] if kv.ndim == 5 else 0
    new_len = np.asarray(kv_len, dtype=np.int64).copy()
    for b in range(live.shape[0]):
        a = int(min(max(int(n_accept[b]), 0), k))
        live[b] = snapshots[b, a]
        if kv.ndim == 5:
            base = min(max(int(kv_len[b]), 0), max_rows)
            lo, hi = min(base + a + 1, max_rows), min(base + k + 1, max_rows)
            kv[b, :, :, lo:hi, :] = 0
            new_len[b] = min(base + a + 1, max_rows)
    return live, kv, new_len.astype(np.int32)


# ----------------------------------------------------------------------------------
# one whole cycle
# ----------------------------------------------------------------------------------
def cycle(W64: np.ndarray, n_draft: int, h_d: np.ndarray, h_v: np.ndarray, T: float,
          seed: int, cycle_id: int, eos: int, delta: float, drafts=None, rule: str = RULE_RATIO,
          positions=None, draft_ids=None) -> dict:
    """k draft-head calls, one verify over k+1 rows, acceptance [MTP-PR "What"].

    h_d [B][k][d], h_v [B][k+1][d] in fp64.  ``drafts`` overrides the draft head's picks
    (the draft logits are still computed, since q is needed for the ratio test).  Rule
    "exact" (T > 0) takes argmax drafts and needs ``positions`` [B], the absolute position
    verify row 0 of each request predicts.
    """
    B, k, _ = h_d.shape
    exact = T > 0 and rule == RULE_EXACT
    Td = 0.0 if exact else T
    dr = [draft_rows(W64, n_draft, h_d[:, i], Td, seed, i, cycle_id, delta, ids=draft_ids) for i in range(k)]
    picked = np.stack([r["token"] for r in dr], axis=1)
    use = picked if drafts is None else np.asarray(drafts, dtype=np.int64)
    dnt = np.stack([r["near_tie"] for r in dr], axis=1)
    if drafts is not None:
        dnt[:] = False
    vr = verify_rows(W64, h_v, use, T, seed, cycle_id, delta, positions=positions if exact else None)
    zd = np.stack([r["logits"] for r in dr], axis=1)
    acc = accept(use, zd, vr["logits"], n_draft, T, seed, cycle_id, eos, delta, draft_near_tie=dnt,
                 rule=rule, target=vr, draft_ids=draft_ids)
    return dict(drafts=use, draft=dr, verify=vr, accept=acc)
