"""GPU parity at model scale, in the launch configuration the bench times.

  * greedy cycle at d=2560, V=152,064, 64,000 draft rows, k=7, bf16 head N(0, 0.02):
    drafts, verify statistics and acceptance against the fp64 oracle (which finishes the
    whole vocabulary in seconds), raw and with planted acceptance depths;
  * every verify logit at T=1 within 2e-2 of the oracle;
  * the same for the 4-bit affine head, greedy and sampled;
  * the commit at the model's state size (36 MiB snapshots, 12-layer KV), checked on
    sampled chunks plus the KV rows and kv_len.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
import synth
from gpu_cycle import GpuCycle, dev_head, dev_hidden
from oracle import mtp_oracle as O
from parity import add_results, check_cycle, check_excluded, close

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DELTA = 2e-2


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _model(name):
    """The workload's head, then its hidden rows, in the generator's draw order."""
    wl = synth.WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    head = synth.make_head(rng, wl.V, wl.d, wl.wtype, keep_source=(wl.wtype == "q4a32"))
    h_v, h_d = synth.make_hidden(rng, wl.B, wl.k, wl.d)
    return wl, (synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")), head


@pytest.fixture(scope="module")
def bf16_model():
    wl, rng, head = _model("model_greedy")
    W = O.head_weights_f64(head)
    return wl, rng, head, W, dev_head(head)


@pytest.fixture(scope="module")
def bf16_tiled(bf16_model):
    wl, hs, head, W, dh = bf16_model
    return wl, hs, head, W, mtp.tiled_head(dh)


@pytest.fixture(scope="module")
def q4_model():
    wl, rng, head = _model("q4_greedy")
    W = O.head_weights_f64(head)
    return wl, rng, head, W, dev_head(head)


def _run(wl, W, dh, hv, hd, T, seed, cycle, planted=None):
    o = O.cycle(W, wl.n_draft, O.hidden_f64(hd, "bf16"), O.hidden_f64(hv, "bf16"), T, seed, cycle, -1, DELTA)
    gc = GpuCycle(dh, wl.n_draft, hv.shape[0], wl.k, T, seed=seed)
    g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cycle)
    return g, o


def _raw_requests(wl, hv, hd, n=16):
    """The bench's own request (raw hidden rows of the model-scale workload) and n - 1 more
    raw requests of the same distribution: [n][k+1][d], [n][k][d] bf16 bits."""
    rng = np.random.default_rng(wl.seed + 1000)
    h_v, h_d = synth.make_hidden(rng, n - 1, wl.k, wl.d)
    return (np.concatenate([hv, synth.encode_hidden(h_v, "bf16")]),
            np.concatenate([hd, synth.encode_hidden(h_d, "bf16")]))


def _raw_cycles(wl, W, dh, hv, hd, T, seed, cycle, tag):
    """One cycle per request in the bench's launch configuration (one request per call,
    request b drawing as request b), all requests through the oracle at once; the near-tie
    budget is checked over all of them."""
    HV, HD = _raw_requests(wl, hv, hd)
    n = HV.shape[0]
    o = O.cycle(W, wl.n_draft, O.hidden_f64(HD, "bf16"), O.hidden_f64(HV, "bf16"), T, seed, cycle, -1, DELTA)
    gc = GpuCycle(dh, wl.n_draft, 1, wl.k, T, seed=seed)
    gs = [gc.run(dev_hidden(HD[b:b + 1]), dev_hidden(HV[b:b + 1]), cycle=cycle, request_base=b) for b in range(n)]
    g = {key: np.concatenate([x[key] for x in gs]) for key in ("drafts", "tokens", "n_accept", "n_emit", "flags")}
    for key in ("dstats", "vstats"):
        g[key] = {f: np.concatenate([x[key][f] for x in gs]) for f in gs[0][key]}
    if T > 0:
        g["logits"] = np.concatenate([x["logits"] for x in gs])
        g["draft_logits"] = np.concatenate([x["draft_logits"] for x in gs])
    r = check_cycle(g, o, T, DELTA, tag=tag)
    return g, o, r


def test_model_greedy_cycle(bf16_model):
    # the bench's exact inputs (request 0) and 15 more raw requests: independent hidden rows
    # reject at row 0, the decisions are the first draft and the verify argmax of row 0
    wl, (hv, hd), head, W, dh = bf16_model
    g, o, r = _raw_cycles(wl, W, dh, hv, hd, 0.0, 0, 0, "model greedy raw")
    assert r["requests"] == 16


@pytest.mark.parametrize("depth", [0, 3, 7])
def test_model_greedy_planted_depths(bf16_model, depth):
    wl, _, head, W, dh = bf16_model
    rng = np.random.default_rng(100 + depth)
    head.source = None
    h_v, h_d = synth.make_hidden(rng, 2, wl.k, wl.d)
    targets = rng.integers(3, wl.n_draft, size=(2, wl.k + 1))
    synth.plant_rows(head, h_v, h_d, [depth, (depth + 4) % 8], targets, (targets + 11) % wl.n_draft, margin=10.0)
    hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
    g, o = _run(wl, W, dh, hv, hd, 0.0, 0, 0)
    check_cycle(g, o, 0.0, DELTA, tag=f"model planted {depth}")
    assert list(g["n_accept"]) == [depth, (depth + 4) % 8]


def test_model_verify_logits_all_within_tolerance(bf16_model):
    wl, _, head, W, dh = bf16_model
    rng = np.random.default_rng(7)
    h_v, h_d = synth.make_hidden(rng, 2, wl.k, wl.d)
    hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
    g, o = _run(wl, W, dh, hv, hd, 1.0, 1234, 5)
    z = o["verify"]["logits"]
    err = np.abs(g["logits"].astype(np.float64) - z)
    print("max |dz| verify:", err.max(), " draft:",
          np.abs(g["draft_logits"].astype(np.float64) - np.stack([r["logits"] for r in o["draft"]], 1)).max())
    assert err.max() <= DELTA
    check_cycle(g, o, 1.0, DELTA, tag="model sampled")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_q4_cycle(q4_model, T):
    wl, _, head, W, dh = q4_model
    rng = np.random.default_rng(31)
    h_v, h_d = synth.make_hidden(rng, 2, wl.k, wl.d)
    targets = rng.integers(3, wl.n_draft, size=(2, wl.k + 1))
    synth.plant_rows(head, h_v, h_d, [2, 6], targets, (targets + 5) % wl.n_draft, margin=10.0)
    hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
    g, o = _run(wl, W, dh, hv, hd, T, 1234, 1)
    check_cycle(g, o, T, DELTA, tag=f"q4 T{T}")
    if T > 0:
        assert np.abs(g["logits"].astype(np.float64) - o["verify"]["logits"]).max() <= DELTA
    else:
        assert list(g["n_accept"]) == [2, 6]


def test_commit_at_model_state_size():
    wl = synth.WORKLOADS["batched_commit"]
    B, k, S = wl.B, wl.k, wl.state_bytes
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(3)
    snaps = torch.randint(0, 256, (B, k + 1, S), dtype=torch.uint8, device=dev, generator=gen)
    live = torch.zeros(B, S, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(0)
    kv_len_np = rng.integers(0, wl.kv_max_rows - k, size=B).astype(np.int32)
    kv = torch.randint(1, 256, (B, wl.n_attn_layers, 2, wl.kv_max_rows, wl.kv_row_bytes), dtype=torch.uint8,
                       device=dev, generator=gen)
    n_acc_np = np.array([b % (k + 1) for b in range(B)], dtype=np.int32)       # every depth, twice
    kv_before = kv.cpu().numpy()
    kv_len = torch.from_numpy(kv_len_np).to(dev)
    mtp.mtp_commit_state(B, k, torch.from_numpy(n_acc_np).to(dev), snaps, live, S, kv, wl.n_attn_layers,
                         wl.kv_max_rows, wl.kv_row_bytes, kv_len)
    torch.cuda.synchronize()
    # oracle on sampled 64 KiB chunks of every request's state, whole KV and kv_len
    for b in range(B):
        for off in [0, S // 3, S - 65536, int(rng.integers(0, S - 65536))]:
            sl = slice(off, off + 65536)
            small_snaps = snaps[b:b + 1, :, sl].cpu().numpy()
            want, _, _ = O.commit(small_snaps, np.zeros((1, 65536), np.uint8), np.zeros((1, 0, 2, 1, 16), np.uint8),
                                  np.zeros(1, np.int32), n_acc_np[b:b + 1], k)
            assert np.array_equal(live[b, sl].cpu().numpy(), want[0]), (b, off)
        # every byte equal via a device-side comparison too (not an oracle, a cross-check)
        assert torch.equal(live[b], snaps[b, n_acc_np[b]])
    _, want_kv, want_len = O.commit(np.zeros((B, k + 1, 16), np.uint8), np.zeros((B, 16), np.uint8), kv_before,
                                    kv_len_np, n_acc_np, k)
    assert np.array_equal(kv.cpu().numpy(), want_kv)
    assert np.array_equal(kv_len.cpu().numpy(), want_len)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_model_tiled_head_cycle(bf16_tiled, T):
    # the bench's head layout: tiled bf16, raw workload rows and a sampled cycle
    wl, (hv, hd), head, W, dh = bf16_tiled
    g, o, _ = _raw_cycles(wl, W, dh, hv, hd, T, 1234, 2, f"model tiled T{T}")
    if T > 0:
        assert np.abs(g["logits"].astype(np.float64) - o["verify"]["logits"]).max() <= DELTA


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_q4_tiled_cycle(q4_model, T):
    wl, _, head, W, dh = q4_model
    th = mtp.tiled_head(dh)
    rng = np.random.default_rng(41)
    h_v, h_d = synth.make_hidden(rng, 2, wl.k, wl.d)
    targets = rng.integers(3, wl.n_draft, size=(2, wl.k + 1))
    synth.plant_rows(head, h_v, h_d, [1, 7], targets, (targets + 5) % wl.n_draft, margin=10.0)
    hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
    g, o = _run(wl, W, th, hv, hd, T, 1234, 3)
    check_cycle(g, o, T, DELTA, tag=f"q4 tiled T{T}")
    if T == 0:
        assert list(g["n_accept"]) == [1, 7]
