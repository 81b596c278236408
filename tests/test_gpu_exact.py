"""Exact-match acceptance under sampling on the GPU, against the oracle.

lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", sections "Exactness" and
"Notes": at T > 0 a draft is kept only if it equals the token the trunk samples; the
trunk's draws are keyed by the absolute position (stream 3), so the emitted tokens are
those of decoding without speculation under the same seed (pinned on the CPU with the
toy trunk).  Here: the verify's sample is that draw in both LM-head kernels, whatever row,
request batch or launch size the position is verified in, and whole cycles with planted
acceptance depths match the oracle.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
import synth
from gpu_cycle import GpuCycle, dev_head, dev_hidden
from oracle import mtp_oracle as O
from parity import add_results, check_cycle, check_excluded, check_verify

pytestmark = pytest.mark.gpu

V, D, ND = 4096, 256, 1024


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _verify(dh, hv: np.ndarray, k: int, drafts: np.ndarray, T: float, seed: int, positions, request_base=0):
    B = hv.shape[0]
    pos = torch.from_numpy(np.asarray(positions, dtype=np.int32)).cuda()
    smp = mtp.sampling(T, -1, seed, 3, request_base, mtp.ACCEPT_EXACT, pos)
    vst = mtp.row_stats_empty(B, k + 1)
    ws = mtp.workspace(mtp.workspace_bytes(mtp.OP_VERIFY, B * (k + 1), V, B))
    mtp.mtp_verify_logits(dh, dev_hidden(hv), k, torch.from_numpy(np.ascontiguousarray(drafts)).cuda(), k, smp,
                          vst, None, ws)   # the exact rule needs no logits
    torch.cuda.synchronize()
    return {kk: v.cpu().numpy() for kk, v in mtp.row_stats_fields(vst).items()}


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
@pytest.mark.parametrize("B,k", [(1, 3), (2, 7), (5, 3), (16, 7)])   # 4 and 16 rows: 16-row kernel; 20, 128: wide
def test_verify_sample_is_the_position_keyed_draw(wtype, B, k):
    T, seed = 0.9, 321
    rng = np.random.default_rng(7 + B)
    head = synth.make_head(rng, V, D, wtype)
    htype = "f32" if wtype == "f32" else "bf16"
    delta = 1e-4 if wtype == "f32" else 2e-2
    h_v, _ = synth.make_hidden(rng, B, k, D)
    hv = synth.encode_hidden(h_v, htype)
    positions = rng.integers(0, 1 << 20, size=B)
    drafts = rng.integers(0, V, size=(B, k)).astype(np.int32)
    vr = O.verify_rows(O.head_weights_f64(head), O.hidden_f64(hv, htype), drafts, T, seed, 3, delta,
                       positions=positions)
    g = {"vstats": _verify(dev_head(head), hv, k, drafts, T, seed, positions)}
    check_verify(g, vr, np.ones((B, k + 1), bool), T, delta, tag=f"{wtype} B{B} k{k}")
    # samples the oracle does not flag as near ties are compared exactly inside check_verify;
    # most rows are not near ties
    assert (vr["s_margin"] > delta / T).mean() > 0.75


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
def test_a_position_draws_the_same_token_in_any_row_and_launch(wtype):
    T, seed = 1.0, 99
    rng = np.random.default_rng(11)
    head = synth.make_head(rng, V, D, wtype)
    htype = "f32" if wtype == "f32" else "bf16"
    dh = dev_head(head)
    h_v, _ = synth.make_hidden(rng, 6, 3, D)
    hv = synth.encode_hidden(h_v, htype)
    P = 5000
    drafts = np.zeros((6, 3), np.int32)
    a = _verify(dh, hv[:1], 3, drafts[:1], T, seed, [P])                       # rows at P..P+3
    b = _verify(dh, np.ascontiguousarray(hv[:1, 2:4]), 1, drafts[:1, :1], T, seed, [P + 2])  # rows 2, 3 as 0, 1
    pos = rng.integers(0, 1 << 20, size=6)
    pos[0] = P
    c = _verify(dh, hv, 3, drafts, T, seed, pos)                                # 24 rows: the wide kernel
    assert np.array_equal(b["sample"][0], a["sample"][0, 2:4])
    assert np.array_equal(c["sample"][0], a["sample"][0])
    # the same rows at other positions or as another request draw differently somewhere
    d = _verify(dh, hv[:1], 3, drafts[:1], T, seed, [P + 1])
    e = _verify(dh, hv[:1], 3, drafts[:1], T, seed, [P], request_base=1)
    assert not np.array_equal(d["sample"][0], a["sample"][0]) or not np.array_equal(e["sample"][0], a["sample"][0])


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
@pytest.mark.parametrize("B", [2, 6])   # 16 and 48 verify rows
def test_exact_rule_cycles_with_planted_depths(wtype, B):
    T, seed, k, eos = 1.0, 1234, 7, 2
    rng = np.random.default_rng(5)
    head = synth.make_head(rng, V, D, wtype, keep_source=True)
    W = O.head_weights_f64(head)
    htype = "f32" if wtype == "f32" else "bf16"
    delta = 1e-4 if wtype == "f32" else 2e-2
    gc = GpuCycle(dev_head(head), ND, B, k, T, seed=seed, eos=eos, rule=mtp.ACCEPT_EXACT)
    positions = rng.integers(0, 1 << 16, size=B)
    seen, total = set(), None
    for cyc in range(8):
        h_v, h_d = synth.make_hidden(rng, B, k, D)
        depths = [(cyc + 3 * b) % (k + 1) for b in range(B)]
        targets = rng.integers(3, ND, size=(B, k + 1))
        alts = (targets + 17) % ND
        if cyc % 3 == 2:
            targets[0, min(depths[0], k - 1)] = eos
        synth.plant_rows(head, h_v, h_d, depths, targets, alts, margin=12.0)
        hv, hd = synth.encode_hidden(h_v, htype), synth.encode_hidden(h_d, htype)
        o = O.cycle(W, ND, O.hidden_f64(hd, htype), O.hidden_f64(hv, htype), T, seed, cyc, eos, delta,
                    rule=O.RULE_EXACT, positions=positions)
        gc.set_positions(positions)
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cyc)
        total = add_results(total, check_cycle(g, o, T, delta, tag=f"{wtype} B{B} cycle {cyc}", rule="exact",
                                               bound=False))
        seen.update(int(a) for a in g["n_accept"])
        # the emitted tokens are the trunk's draws: drafts up to the first mismatch, then the draw
        vs = g["vstats"]
        for b in range(B):
            a, n = int(g["n_accept"][b]), int(g["n_emit"][b])
            assert list(g["tokens"][b, :a]) == list(vs["sample"][b, :a])
            if n == a + 1 and g["tokens"][b, a] != eos:
                assert g["tokens"][b, a] == vs["sample"][b, a]
        positions = positions + g["n_emit"]
    assert len(seen) >= 4
    check_excluded(total, f"{wtype} B{B}")
