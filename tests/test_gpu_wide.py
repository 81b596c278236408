"""GPU parity of the verify pass for 17..128 hidden rows (several requests' k+1 rows per
launch, up to 16 requests x 8 rows), which runs a kernel of its own.

  * whole cycles against the fp64 oracle for every head layout, greedy and sampled, with a
    ragged vocabulary and ragged row counts (18, 32, 128 rows), planted acceptance depths;
  * logits, argmax, Gumbel sample, drafted-id logit, max and flags bit-identical to the
    launches of up to 16 rows on the same rows (log-sum-exp to fp32 summation order);
  * a row's results do not depend on how many rows (17..128) share the launch or where;
  * non-finite logits (NaN, +inf, -inf rows) in a wide launch;
  * the batched model-scale cycle (16 x 8 rows, V = 152,064, d = 2560, tiled bf16 head),
    then the commit of each request's accepted snapshot.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
import synth
from gpu_cycle import GpuCycle, dev_head, dev_hidden
from oracle import mtp_oracle as O
from parity import check_cycle, close

pytestmark = pytest.mark.gpu

DELTA = {"f32": 1e-4, "bf16": 2e-2, "q4a32": 2e-2}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _planted_case(wtype, V, d, nd, B, k, seed):
    rng = np.random.default_rng(seed)
    head = synth.make_head(rng, V, d, wtype, keep_source=(wtype == "q4a32"))
    h_v, h_d = synth.make_hidden(rng, B, k, d)
    depths = [int(x) for x in rng.integers(0, k + 1, size=B)]
    targets = rng.integers(3, nd, size=(B, k + 1))
    synth.plant_rows(head, h_v, h_d, depths, targets, (targets + 7) % nd, margin=10.0)
    htype = "f32" if wtype == "f32" else "bf16"
    return head, synth.encode_hidden(h_v, htype), synth.encode_hidden(h_d, htype), htype, depths


def _oracle_cycle(head, nd, hv, hd, htype, T, seed, cycle, delta):
    W = O.head_weights_f64(head)
    return O.cycle(W, nd, O.hidden_f64(hd, htype), O.hidden_f64(hv, htype), T, seed, cycle, -1, delta)


@pytest.mark.parametrize("layout", ["f32", "bf16", "q4a32", "bf16_tiled", "q4a32_tiled"])
@pytest.mark.parametrize("B,k", [(3, 5), (4, 7), (16, 7)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_wide_cycle_against_oracle(layout, B, k, T):
    wtype = layout.replace("_tiled", "")
    V, d, nd = 1013, 256, 400
    head, hv, hd, htype, depths = _planted_case(wtype, V, d, nd, B, k, seed=B * 10 + k)
    o = _oracle_cycle(head, nd, hv, hd, htype, T, 77, 3, DELTA[wtype])
    gc = GpuCycle(dev_head(head, tiled=layout.endswith("_tiled")), nd, B, k, T, seed=77)
    g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=3)
    check_cycle(g, o, T, DELTA[wtype], tag=f"wide {layout} B{B} k{k} T{T}")
    if T == 0:
        assert list(g["n_accept"]) == depths


def _verify(dh, hv, B, k, drafts, T, request_base, nd=None):
    """One verify launch over B requests; returns (row stats int32 [M][8], logits [M][V])."""
    gc = GpuCycle(dh, nd or dh.vocab, B, k, T, seed=11)
    gc.draft_tokens[:, :k] = torch.as_tensor(np.asarray(drafts), dtype=torch.int32, device="cuda")
    gc.verify(dev_hidden(hv), cycle=2, request_base=request_base)
    torch.cuda.synchronize()
    M = B * (k + 1)
    lg = gc.logits.reshape(M, -1).cpu().numpy() if gc.logits is not None else None
    return gc.row_stats.reshape(M, 8).cpu().numpy(), lg


@pytest.mark.parametrize("layout", ["f32", "bf16", "q4a32", "bf16_tiled", "q4a32_tiled"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_wide_equals_narrow_launches(layout, T):
    """16 requests x 8 rows in one launch against 8 launches of 2 requests (16 rows)."""
    wtype = layout.replace("_tiled", "")
    V, d, k, B = 2011, 512, 7, 16
    rng = np.random.default_rng(5)
    head = synth.make_head(rng, V, d, wtype)
    dh = dev_head(head, tiled=layout.endswith("_tiled"))
    htype = "f32" if wtype == "f32" else "bf16"
    hv = synth.encode_hidden(rng.standard_normal((B, k + 1, d)).astype(np.float32), htype)
    drafts = rng.integers(0, V, size=(B, k))
    wide_st, wide_lg = _verify(dh, hv, B, k, drafts, T, request_base=40)
    for c in range(B // 2):
        sl = slice(2 * c, 2 * c + 2)
        st, lg = _verify(dh, hv[sl], 2, k, drafts[sl], T, request_base=40 + 2 * c)
        rows = slice(2 * c * (k + 1), (2 * c + 2) * (k + 1))
        w = wide_st[rows]
        # max, z_tok, argmax, sample, flags, n_posinf: identical bits
        assert np.array_equal(w[:, [0, 2, 3, 4, 5, 6]], st[:, [0, 2, 3, 4, 5, 6]]), c
        lse_w, lse_n = w[:, 1].view(np.float32), st[:, 1].view(np.float32)
        assert np.allclose(lse_w, lse_n, rtol=2e-6, atol=2e-6), (c, np.abs(lse_w - lse_n).max())
        if T > 0:
            assert np.array_equal(wide_lg[rows].view(np.uint32), lg.view(np.uint32)), c


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
def test_wide_batch_invariance_bitwise(wtype):
    """One request's rows at several positions of launches of 18..128 rows: identical bits."""
    V, d, k = 2000, 256, 7
    rng = np.random.default_rng(13)
    head = synth.make_head(rng, V, d, wtype)
    dh = dev_head(head)
    htype = "f32" if wtype == "f32" else "bf16"
    probe = synth.encode_hidden(rng.standard_normal((1, k + 1, d)).astype(np.float32), htype)
    filler = synth.encode_hidden(rng.standard_normal((1, k + 1, d)).astype(np.float32), htype)
    pdraft = rng.integers(0, V, size=(1, k))
    ref = None
    for B in (3, 5, 16):
        for pos in sorted({0, B // 2, B - 1}):
            hv = np.repeat(filler, B, axis=0)
            hv[pos] = probe[0]
            drafts = np.repeat(pdraft, B, axis=0)
            # the probe keeps Philox request id 100 wherever it sits
            st, lg = _verify(dh, hv, B, k, drafts, 1.0, request_base=100 - pos)
            rows = slice(pos * (k + 1), (pos + 1) * (k + 1))
            cur = (st[rows], lg[rows])
            if ref is None:
                ref = cur
            assert np.array_equal(cur[0], ref[0]), (B, pos)
            assert np.array_equal(cur[1].view(np.uint32), ref[1].view(np.uint32)), (B, pos)


def _nonfinite_head(V, d):
    rng = np.random.default_rng(3)
    return (rng.standard_normal((V, d)) * 0.05).astype(np.float32)


@pytest.mark.parametrize("kind", ["nan_rows", "posinf", "all_nan", "neginf"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_wide_nonfinite_rows(kind, T):
    V, d, nd, k, B = 640, 64, 200, 3, 6
    w = _nonfinite_head(V, d)
    h_v = np.abs(np.random.default_rng(4).standard_normal((B, k + 1, d))).astype(np.float32) + 0.1
    h_d = np.abs(np.random.default_rng(6).standard_normal((B, k, d))).astype(np.float32) + 0.1
    if kind == "nan_rows":
        w[[7, 150, 400]] = np.nan
    elif kind == "posinf":
        w[[30, 190, 500], 0] = np.inf
    elif kind == "all_nan":
        w[:, 5] = np.nan
    elif kind == "neginf":
        w[:, 0] = -np.inf
        w[:50, 0] = 0.0
    head = synth.Head("f32", V, d, w)
    W = O.head_weights_f64(head)
    o = O.cycle(W, nd, h_d.astype(np.float64), h_v.astype(np.float64), T, 9, 0, -1, 1e-4)
    gc = GpuCycle(dev_head(head), nd, B, k, T, seed=9)
    g = gc.run(dev_hidden(h_d), dev_hidden(h_v))
    check_cycle(g, o, T, 1e-4, tag=f"wide nonfinite {kind} T{T}")
    assert np.array_equal(g["vstats"]["n_posinf"], np.isposinf(O.logits_f64(W, h_v.astype(np.float64))).sum(-1))


def test_wide_rejects_more_than_128_rows():
    V, d = 256, 64
    head = synth.make_head(np.random.default_rng(0), V, d, "f32")
    dh = dev_head(head)
    hv = dev_hidden(np.zeros((17, 8, d), np.float32))
    gc = GpuCycle(dh, V, 16, 7, 0.0)
    drafts = torch.zeros(17, 7, dtype=torch.int32, device="cuda")
    stats = mtp.row_stats_empty(17, 8)
    with pytest.raises(mtp.MtpError):
        mtp.mtp_verify_logits(dh, hv, 7, drafts, 7, gc.smp(), stats, None, gc.ws)


@pytest.mark.slow
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_batched_model_cycle_and_commit(T):
    """16 requests x 8 verify rows at V = 152,064, d = 2560 (tiled bf16 head), planted depths
    for half the requests, then each request's accepted snapshot committed."""
    wl = synth.WORKLOADS["batched_commit"]
    rng = np.random.default_rng(wl.seed)
    head = synth.make_head(rng, wl.V, wl.d, wl.wtype)
    h_v, h_d = synth.make_hidden(rng, wl.B, wl.k, wl.d)
    planted = list(range(0, wl.B, 2))
    depths = [int(x) for x in rng.integers(0, wl.k + 1, size=len(planted))]
    targets = rng.integers(3, wl.n_draft, size=(len(planted), wl.k + 1))
    hv_p, hd_p = h_v[planted], h_d[planted]
    synth.plant_rows(head, hv_p, hd_p, depths, targets, (targets + 9) % wl.n_draft, margin=10.0)
    h_v[planted], h_d[planted] = hv_p, hd_p
    hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
    W = O.head_weights_f64(head)
    o = O.cycle(W, wl.n_draft, O.hidden_f64(hd, "bf16"), O.hidden_f64(hv, "bf16"), T, 1234, 9, -1, 2e-2)
    gc = GpuCycle(dev_head(head, tiled=True), wl.n_draft, wl.B, wl.k, T, seed=1234)
    g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=9)
    check_cycle(g, o, T, 2e-2, tag=f"batched model T{T}")
    if T == 0:
        assert [int(g["n_accept"][b]) for b in planted] == depths
    # commit on the GPU's own accept counts: the accepted row's snapshot, trimmed KV
    S = 1 << 20
    snaps = torch.randint(0, 256, (wl.B, wl.k + 1, S), dtype=torch.uint8, device="cuda",
                          generator=torch.Generator(device="cuda").manual_seed(1))
    live = torch.zeros(wl.B, S, dtype=torch.uint8, device="cuda")
    kv = torch.randint(1, 256, (wl.B, wl.n_attn_layers, 2, wl.kv_max_rows, wl.kv_row_bytes), dtype=torch.uint8,
                       device="cuda", generator=torch.Generator(device="cuda").manual_seed(2))
    kv_len_np = np.random.default_rng(3).integers(0, wl.kv_max_rows - wl.k, size=wl.B).astype(np.int32)
    kv_before = kv.cpu().numpy()
    kv_len = torch.from_numpy(kv_len_np).cuda()
    mtp.mtp_commit_state(wl.B, wl.k, gc.n_accept, snaps, live, S, kv, wl.n_attn_layers, wl.kv_max_rows,
                         wl.kv_row_bytes, kv_len)
    torch.cuda.synchronize()
    n_acc = g["n_accept"]
    want_live, want_kv, want_len = O.commit(snaps.cpu().numpy(), np.zeros((wl.B, S), np.uint8), kv_before,
                                            kv_len_np, n_acc, wl.k)
    assert np.array_equal(live.cpu().numpy(), want_live)
    assert np.array_equal(kv.cpu().numpy(), want_kv)
    assert np.array_equal(kv_len.cpu().numpy(), want_len)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_large_hidden_size_verify_takes_the_wide_kernel(T):
    """d = 5120: 16 staged bf16 hidden rows (160 KiB) do not fit the 16-row kernel's LDS, so
    every verify of this head, at any row count, runs the wide kernel: whole cycles against
    the oracle at 16 and 8 verify rows, and request 0's logits and statistics identical
    across the two launch sizes."""
    V, d, nd, k = 1013, 5120, 400, 7
    head, hv, hd, htype, depths = _planted_case("bf16", V, d, nd, 2, k, seed=91)
    dh = dev_head(head)
    outs = []
    for B in (2, 1):
        o = _oracle_cycle(head, nd, hv[:B], hd[:B], htype, T, 77, 3, 2e-2)
        gc = GpuCycle(dh, nd, B, k, T, seed=77)
        g = gc.run(dev_hidden(np.ascontiguousarray(hd[:B])), dev_hidden(np.ascontiguousarray(hv[:B])), cycle=3)
        check_cycle(g, o, T, 2e-2, tag=f"d5120 B{B} T{T}")
        if T == 0:
            assert list(g["n_accept"]) == depths[:B]
        outs.append((gc.row_stats.cpu().numpy(), None if gc.logits is None else gc.logits.cpu().numpy()))
    st2, st1 = outs[0][0][0], outs[1][0][0]
    assert np.array_equal(st1[:, [0, 1, 3, 5, 6]], st2[:, [0, 1, 3, 5, 6]])
    if T > 0:
        assert np.array_equal(outs[0][1][0].view(np.uint32), outs[1][1][0].view(np.uint32))
