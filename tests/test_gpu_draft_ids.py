"""The draft vocabulary as an id list on the GPU (lucebox-hub PR "feat(qwen4exp): MTP
speculative decoding", section "What": the draft head covers control/special tokens plus
the lowest ids).  The draft rows are gathered once into their own head (mtp_gather_rows,
optionally tiled); the draft head reports vocabulary ids through the head's row ids and
acceptance looks q up through the inverse map.  Compared with the oracle's id-list path."""
import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
import synth
from gpu_cycle import GpuCycle, dev_head, dev_hidden
from oracle import mtp_oracle as O
from parity import add_results, check_cycle, check_excluded

pytestmark = pytest.mark.gpu

V, D = 4096, 256


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _ids(rng, n_low=900, n_special=37):
    special = rng.choice(np.arange(n_low, V), size=n_special, replace=False)
    return np.sort(np.concatenate([np.arange(n_low), special])).astype(np.int32)


def _draft_head(head_dev: mtp.Head, ids: np.ndarray, tiled: bool):
    g = mtp.gather_rows(head_dev, torch.from_numpy(ids).cuda())
    if tiled:
        g = mtp.tiled_head(g)
    torch.cuda.synchronize()
    return g


def _row_of(ids):
    r = np.full(V, -1, np.int32)
    r[ids] = np.arange(ids.size, dtype=np.int32)
    return torch.from_numpy(r).cuda()


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
def test_gather_rows_copies_the_rows(wtype):
    rng = np.random.default_rng(1)
    head = synth.make_head(rng, V, D, wtype)
    ids = _ids(rng)
    g = _draft_head(dev_head(head), ids, tiled=False)
    w = g.w.cpu().numpy()
    if wtype == "q4a32":
        assert np.array_equal(w, head.w[ids])
        assert np.array_equal(g.scale.cpu().numpy().view(np.uint16), head.scale[ids])
        assert np.array_equal(g.minv.cpu().numpy().view(np.uint16), head.minv[ids])
    elif wtype == "bf16":
        assert np.array_equal(w.view(np.uint16), head.w[ids])
    else:
        assert np.array_equal(w, head.w[ids])
    assert np.array_equal(g.row_ids.cpu().numpy(), ids)


@pytest.mark.parametrize("wtype,tiled", [("f32", False), ("bf16", False), ("bf16", True), ("q4a32", True)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_id_list_draft_head_against_oracle(wtype, tiled, T):
    rng = np.random.default_rng(2)
    head = synth.make_head(rng, V, D, wtype)
    htype = "f32" if wtype == "f32" else "bf16"
    delta = 1e-4 if wtype == "f32" else 2e-2
    ids = _ids(rng)
    dh = _draft_head(dev_head(head), ids, tiled)
    B, k = 16, 3
    h = synth.encode_hidden(rng.standard_normal((B, D)).astype(np.float32), htype)
    smp = mtp.sampling(T, -1, 77, 4, 0)
    tok = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    st = mtp.row_stats_empty(B, k)
    lg = torch.zeros(B, k, ids.size, dtype=torch.float32, device="cuda") if T > 0 else None
    ws = mtp.workspace(mtp.workspace_bytes(mtp.OP_DRAFT, B, ids.size, B))
    mtp.mtp_draft_head(dh, ids.size, dev_hidden(h), 1, k, smp, tok, st, lg, ws)
    torch.cuda.synchronize()
    o = O.draft_rows(O.head_weights_f64(head), ids.size, O.hidden_f64(h, htype), T, 77, 1, 4, delta, ids=ids)
    got = tok.cpu().numpy()[:, 1]
    clear = ~o["near_tie"]
    assert np.array_equal(got[clear], o["token"][clear])
    assert np.all(np.isin(got, ids))
    f = {kk: v.cpu().numpy()[:, 1] for kk, v in mtp.row_stats_fields(st).items()}
    assert np.allclose(f["max"], o["max"], atol=delta)
    assert np.allclose(f["lse"], o["lse"], atol=delta / (T if T > 0 else 1.0))
    if T > 0:
        assert np.allclose(lg.cpu().numpy()[:, 1], o["logits"], atol=delta)


@pytest.mark.parametrize("wtype", ["bf16", "q4a32"])
@pytest.mark.parametrize("T,rule", [(0.0, mtp.ACCEPT_RATIO), (1.0, mtp.ACCEPT_RATIO), (1.0, mtp.ACCEPT_EXACT)])
def test_id_list_cycles_with_planted_depths(wtype, T, rule):
    rng = np.random.default_rng(5)
    head = synth.make_head(rng, V, D, wtype, keep_source=True)
    W = O.head_weights_f64(head)
    delta = 2e-2
    ids = _ids(rng)
    hd_dev = dev_head(head, tiled=True)
    dh = _draft_head(dev_head(head), ids, tiled=True)
    B, k, eos, seed = 4, 7, 2, 1234
    gc = GpuCycle(hd_dev, ids.size, B, k, T, seed=seed, eos=eos, rule=rule, draft_head=dh,
                  draft_row_of=_row_of(ids))
    positions = rng.integers(0, 1 << 16, size=B)
    orule = O.RULE_EXACT if rule == mtp.ACCEPT_EXACT else O.RULE_RATIO
    total = None
    for cyc in range(6):
        h_v, h_d = synth.make_hidden(rng, B, k, D)
        depths = [(cyc + 2 * b) % (k + 1) for b in range(B)]
        targets = ids[rng.integers(3, ids.size, size=(B, k + 1))]      # drafts must be in the list
        alts = ids[(np.searchsorted(ids, targets) + 17) % ids.size]
        synth.plant_rows(head, h_v, h_d, depths, targets, alts, margin=12.0)
        hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
        o = O.cycle(W, ids.size, O.hidden_f64(hd, "bf16"), O.hidden_f64(hv, "bf16"), T, seed, cyc, eos, delta,
                    rule=orule, positions=positions, draft_ids=ids)
        gc.set_positions(positions)
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cyc)
        total = add_results(total, check_cycle(g, o, T, delta, tag=f"{wtype} T{T} rule{rule} cycle {cyc}",
                                               rule=orule, bound=False))
        assert np.all(np.isin(g["drafts"][g["drafts"] >= 0], ids))
        positions = positions + g["n_emit"]
    check_excluded(total, f"id list {wtype} T{T} rule{rule}")
