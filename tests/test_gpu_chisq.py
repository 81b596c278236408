"""Distribution of the GPU path's emitted tokens under sampled speculation.

DS4Server issue "Add Qwen3.8 Flash Next native MTP speculation", section "Completion
requirements": speculation preserves the target distribution.  A tiny head whose logits
equal the hidden rows (W = [I | 0]) fixes p_i and q_i per row; 40,000 independent
requests (distinct Philox request ids) run draft -> verify -> accept on the GPU; at every
position the emitted token, given that the block reached it, must follow p_i (Pearson
chi-square, Bonferroni over positions), and the acceptance rate at row i must match
sum_x min(p_i, q_i).  The same statistics from the oracle are checked in the CPU suite.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import speculative_decoding_head_amd as mtp

pytestmark = pytest.mark.gpu

V, D, ND, K = 16, 32, 8, 3
N = 40_000


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def test_emitted_positions_follow_p_on_gpu():
    rng = np.random.default_rng(21)
    h_v = rng.standard_normal((K + 1, V)) * 1.2
    h_d = rng.standard_normal((K, V)) * 1.2
    h_d[:, :ND] += 0.6 * h_v[:K, :ND]
    W = np.zeros((V, D), np.float32)
    W[:, :V] = np.eye(V, dtype=np.float32)
    pad = lambda h: np.concatenate([h, np.zeros(h.shape[:-1] + (D - V,))], -1).astype(np.float32)
    dev = "cuda"
    head = mtp.Head(mtp.W_F32, D, V, torch.from_numpy(W).to(dev))
    seed, cyc = 99, 5
    dtok = torch.zeros(N, K, dtype=torch.int32, device=dev)
    dst = mtp.row_stats_empty(N, K)
    dlg = torch.zeros(N, K, ND, dtype=torch.float32, device=dev)
    vst = mtp.row_stats_empty(N, K + 1)
    vlg = torch.zeros(N, K + 1, V, dtype=torch.float32, device=dev)
    ws = mtp.workspace(max(mtp.workspace_bytes(mtp.OP_DRAFT, 16, ND, 16), mtp.workspace_bytes(mtp.OP_VERIFY, 16, V, 4),
                           mtp.workspace_bytes(mtp.OP_ACCEPT, 0, V, N)))
    # draft slots: 16 requests per call, each with its own request id
    for i in range(K):
        hd = torch.from_numpy(np.repeat(pad(h_d[i])[None], 16, 0)).to(dev)
        for c in range(N // 16):
            smp = mtp.sampling(1.0, -1, seed, cyc, 16 * c)
            mtp.mtp_draft_head(head, ND, hd, i, K, smp, dtok[16 * c:16 * (c + 1)], dst[16 * c:16 * (c + 1)],
                               dlg[16 * c:16 * (c + 1)], ws)
    hv = torch.from_numpy(np.repeat(pad(h_v)[None], 4, 0)).to(dev)
    for c in range(N // 4):
        smp = mtp.sampling(1.0, -1, seed, cyc, 4 * c)
        sl = slice(4 * c, 4 * (c + 1))
        mtp.mtp_verify_logits(head, hv, K, dtok[sl], K, smp, vst[sl], vlg[sl], ws)
    out = torch.zeros(N, K + 1, dtype=torch.int32, device=dev)
    nacc = torch.zeros(N, dtype=torch.int32, device=dev)
    nemit = torch.zeros(N, dtype=torch.int32, device=dev)
    flg = torch.zeros(N, dtype=torch.int32, device=dev)
    mtp.mtp_accept_sample(N, K, K, V, ND, mtp.sampling(1.0, -1, seed, cyc, 0), dtok, dst, dlg, vst, vlg, out, nacc,
                          nemit, flg, ws)
    torch.cuda.synchronize()
    tokens, n_acc = out.cpu().numpy(), nacc.cpu().numpy()
    drafts = dtok.cpu().numpy()
    assert np.all((n_acc >= 0) & (n_acc <= K)) and np.array_equal(nemit.cpu().numpy(), n_acc + 1)
    for i in range(K):
        m = n_acc > i
        assert np.array_equal(tokens[m, i], drafts[m, i])
    # drafts are samples of q at every slot
    for i in range(K):
        q = _softmax(h_d[i][:ND])
        c = np.bincount(drafts[:, i], minlength=ND)
        assert c[ND:].sum() == 0
        assert stats.chisquare(c[:ND], N * q).pvalue > 1e-4 / K
    pv = []
    for i in range(K + 1):
        reach = n_acc >= i
        p = _softmax(h_v[i])
        c = np.bincount(tokens[reach, i], minlength=V)
        pv.append(stats.chisquare(c, c.sum() * p).pvalue)
    assert min(pv) >= 1e-4 / (K + 1), pv
    for i in range(K):
        p = _softmax(h_v[i])
        q = np.zeros(V)
        q[:ND] = _softmax(h_d[i][:ND])
        reach = n_acc >= i
        rate = np.mean(n_acc[reach] > i)
        want = np.minimum(p, q).sum()
        assert abs(rate - want) < 5 * np.sqrt(want * (1 - want) / reach.sum()) + 1e-3
