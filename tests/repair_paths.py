"""Decode loops on the toy trunk with short-convolution state: ordinary decoding, and
speculative decoding that restores state after each cycle either by capture-commit
(snapshot of every verify row, keep the accepted one, trim rejected KV rows) or by an
ordinary-forward repair (restore the pre-cycle state and replay the accepted tokens).
Test infrastructure; the acceptance decisions come from the oracle."""
from __future__ import annotations

import numpy as np

from oracle import mtp_oracle as O
from toy_trunk import ToyTrunkConv

MAX_ROWS = 512


def kv_bytes(tt, tok) -> np.ndarray:
    return np.frombuffer(tt.kv_row(tok).tobytes(), dtype=np.uint8)


def ordinary(tt: ToyTrunkConv, t0: int, n: int, T: float = 0.0, seed: int = 0):
    """Tokens, the state after each token, and the logits each token was chosen from."""
    st, t = tt.zero_state(), t0
    toks, states, logits = [], [], []
    for pos in range(n):
        st = tt.step(st, t)
        z = tt.W @ tt.hidden(st, t)
        y = int(np.argmax(z)) if T <= 0 else O.trunk_sample(z, T, seed, 0, pos)[0]
        toks.append(y)
        states.append(tt.state_bytes(st))
        logits.append(z)
        t = y
    return toks, states, logits


def speculative(tt: ToyTrunkConv, t0: int, n: int, k: int, mode: str, T: float = 0.0, seed: int = 0,
                commit=None, perturb=None, reverify: bool = False, max_cycles: int = 10_000):
    """mode "capture": snapshots of every verify row, commit = ``commit`` (default the
    oracle's); mode "repair": restore the pre-cycle state and replay the accepted tokens
    through ordinary forward steps.  ``perturb(z, width)`` models logits that change with
    the verify batch shape; ``reverify`` re-checks the replayed tokens against the replay's
    own logits (the livelock the llama.cpp PR's "store" commit removed).  Returns tokens,
    per-cycle records (state bytes, kv, kv_len, the logits of the next position), and the
    number of cycles."""
    commit = commit or O.commit
    W = tt.W
    st = tt.zero_state()
    row_bytes = tt.kv_dim * 8
    kv = np.zeros((1, 1, 2, MAX_ROWS, row_bytes), dtype=np.uint8)
    kv_len = np.zeros(1, dtype=np.int32)
    emitted, cycles = [], []
    c = 0
    while len(emitted) < n and c < max_cycles:
        # drafts from the drafter's own copy of the state
        sd, tok, drafts = st, t0, []
        for i in range(k):
            sd = tt.step(sd, tok)
            d = int(O.draft_rows(W, tt.V, tt.hidden(sd, tok, drafter=True)[None], 0.0, 0, i, c, 1e-9)["token"][0])
            drafts.append(d)
            tok = d
        # verify the k+1 rows in one batch of width k+1, snapshots after each row
        sv, toks, snaps, hv = st, [t0] + drafts, [], []
        for i, tk in enumerate(toks):
            sv = tt.step(sv, tk)
            snaps.append(tt.state_bytes(sv))
            hv.append(tt.hidden(sv, tk))
            r = kv_bytes(tt, tk)
            kv[0, 0, 0, kv_len[0] + i] = r
            kv[0, 0, 1, kv_len[0] + i] = r[::-1]
        zv = (np.array(hv) @ W.T)
        if perturb is not None:
            zv = np.stack([perturb(z, k + 1) for z in zv])
        if T > 0:
            vr = O.verify_rows(W, np.array(hv)[None], np.array([drafts]), T, seed, c, 1e-12, positions=[len(emitted)])
            vr["logits"] = zv[None]
            acc = O.accept(np.array([drafts]), None, zv[None], tt.V, T, seed, c, -1, 1e-12, rule=O.RULE_EXACT,
                           target=vr)
        else:
            acc = O.accept(np.array([drafts]), None, zv[None], tt.V, 0.0, 0, c, -1, 1e-12)
        a, m = int(acc["n_accept"][0]), int(acc["n_emit"][0])
        block = [int(v) for v in acc["tokens"][0, :m]]
        if mode == "capture":
            live, kv, kv_len = commit(np.array([snaps]), np.zeros((1, snaps[0].size), np.uint8), kv, kv_len,
                                      acc["n_accept"], k)
            st = tt.from_bytes(live[0])
        else:
            # repair: back to the pre-cycle state and KV, replay t0, d_1..d_a one token at a
            # time (width 1), then take the continuation at the final position
            kv[0, :, :, kv_len[0]:] = 0
            sr, ok = tt.from_bytes(tt.state_bytes(st)), True
            for i, tk in enumerate(toks[:a + 1]):
                sr = tt.step(sr, tk)
                r = kv_bytes(tt, tk)
                kv[0, 0, 0, kv_len[0] + i] = r
                kv[0, 0, 1, kv_len[0] + i] = r[::-1]
                if reverify and i < a:
                    z = tt.W @ tt.hidden(sr, tk)
                    if perturb is not None:
                        z = perturb(z, 1)
                    if int(np.argmax(z)) != drafts[i]:
                        ok = False             # the replay disagrees: restore again, emit nothing
                        break
            if not ok:
                kv[0, :, :, kv_len[0]:] = 0
                cycles.append(dict(n_accept=-1, live=tt.state_bytes(st), kv=kv.copy(), kv_len=int(kv_len[0]),
                                   n_emitted=len(emitted), next_logits=None))
                c += 1
                continue
            st = sr
            kv_len = kv_len + a + 1
        emitted += block
        t0 = emitted[-1]
        nxt = tt.W @ tt.hidden(tt.step(st, t0), t0)          # the logits of the next position
        cycles.append(dict(n_accept=a, live=tt.state_bytes(st), kv=kv.copy(), kv_len=int(kv_len[0]),
                           n_emitted=len(emitted), next_logits=nxt))
        c += 1
    return emitted[:n], cycles, c
