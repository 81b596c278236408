"""The allocation-free verify entry point (mtp_verify_logits_noalloc, for callers that cannot
allocate device memory) against mtp_verify_logits with a caller's workspace: two calls in a
row on the library's per-device scratch, the second smaller than the first (a 128-row wide
launch with sampled logits, then a 4-row launch of the 16-row kernel at T = 0), and a third
at the first size again; row statistics and logits identical bit for bit.  The same under
HIP graph capture, alone and inside a whole captured cycle.  Argument checks run before
any device call."""
import ctypes

import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
import synth
from gpu_cycle import dev_head, dev_hidden


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    if torch.cuda.is_available():
        torch.cuda.synchronize()


def _inputs(rng, head, B, k, d, V):
    h_v, _ = synth.make_hidden(rng, B, k, d)
    hv = dev_hidden(synth.encode_hidden(h_v, "bf16"))
    drafts = torch.from_numpy(rng.integers(0, V, size=(B, 7)).astype(np.int32)).cuda()
    return hv, drafts


def _both(dh, hv, drafts, B, k, T, V, stream=None):
    smp = mtp.sampling(T, -1, 4321, 7, 0)
    out = []
    for noalloc in (False, True):
        st = mtp.row_stats_empty(B, k + 1)
        lg = torch.full((B, k + 1, V), 7.0, dtype=torch.float32, device="cuda") if T > 0 else None
        torch.cuda.synchronize()
        if noalloc:
            mtp.mtp_verify_logits_noalloc(dh, hv, k, drafts, 7, smp, st, lg, stream)
        else:
            ws = mtp.workspace(mtp.workspace_bytes(mtp.OP_VERIFY, B * (k + 1), V, B))
            mtp.mtp_verify_logits(dh, hv, k, drafts, 7, smp, st, lg, ws)
        torch.cuda.synchronize()
        out.append((st.cpu().numpy(), None if lg is None else lg.cpu().numpy()))
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("tiled", [False, True])
def test_noalloc_verify_equals_the_workspace_verify(tiled):
    V, d = 4099, 256
    rng = np.random.default_rng(17)
    head = synth.make_head(rng, V, d, "bf16")
    dh = dev_head(head, tiled=tiled)
    for B, k, T in ((16, 7, 1.0), (1, 3, 0.0), (16, 7, 1.0)):
        hv, drafts = _inputs(rng, head, B, k, d, V)
        (st_ws, lg_ws), (st_na, lg_na) = _both(dh, hv, drafts, B, k, T, V)
        assert np.array_equal(st_ws, st_na), (B, k, T)
        if T > 0:
            assert np.array_equal(lg_ws.view(np.uint32), lg_na.view(np.uint32)), (B, k, T)
        assert np.all(st_na.reshape(-1, 8)[:, 3] >= 0)          # every row has an argmax


@pytest.mark.gpu
def test_noalloc_verify_at_model_scale():
    """The model-scale verify (152,064 x 2560 bf16, tiled) on the scratch array: one request's
    8 rows, then 16 requests x 8 rows (the 128-row kernel over 198 blocks, the most scratch a
    call of this head uses), then 8 rows again."""
    wl = synth.WORKLOADS["model_greedy"]
    rng = np.random.default_rng(wl.seed)
    head = synth.make_head(rng, wl.V, wl.d, wl.wtype)
    dh = dev_head(head, tiled=True)
    for B in (1, 16, 1):
        hv, drafts = _inputs(rng, head, B, wl.k, wl.d, wl.V)
        (st_ws, _), (st_na, _) = _both(dh, hv, drafts, B, wl.k, 0.0, wl.V)
        assert np.array_equal(st_ws, st_na), B


@pytest.mark.gpu
def test_noalloc_verify_on_a_side_stream():
    """The scratch array is found through the stream's own device (not only the null stream),
    and calls on another stream of the same device, ordered by synchronisation, give the
    same bits."""
    V, d = 4099, 256
    rng = np.random.default_rng(29)
    head = synth.make_head(rng, V, d, "bf16")
    dh = dev_head(head, tiled=True)
    side = torch.cuda.Stream()
    for B, k, T in ((16, 7, 1.0), (2, 5, 0.0)):
        hv, drafts = _inputs(rng, head, B, k, d, V)
        (st_ws, lg_ws), (st_na, lg_na) = _both(dh, hv, drafts, B, k, T, V, stream=side)
        assert np.array_equal(st_ws, st_na), (B, k, T)
        if T > 0:
            assert np.array_equal(lg_ws.view(np.uint32), lg_na.view(np.uint32)), (B, k, T)


@pytest.mark.gpu
def test_noalloc_verify_replays_under_graph_capture():
    """The allocation-free verify captured into a HIP graph (its callers' reason to exist):
    every replay, with eager work and a synchronisation between replays, gives the eager
    workspace verify's bits."""
    V, d, B, k, T = 4099, 256, 2, 7, 1.0
    rng = np.random.default_rng(41)
    head = synth.make_head(rng, V, d, "bf16")
    dh = dev_head(head, tiled=True)
    hv, drafts = _inputs(rng, head, B, k, d, V)
    (st_ref, lg_ref), _ = _both(dh, hv, drafts, B, k, T, V)
    smp = mtp.sampling(T, -1, 4321, 7, 0)
    st = mtp.row_stats_empty(B, k + 1)
    lg = torch.zeros(B, k + 1, V, dtype=torch.float32, device="cuda")
    mtp.mtp_verify_logits_noalloc(dh, hv, k, drafts, 7, smp, st, lg)     # set-up happens outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mtp.mtp_verify_logits_noalloc(dh, hv, k, drafts, 7, smp, st, lg)
    for rep in range(4):
        st.fill_(-3)
        lg.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(st.cpu().numpy(), st_ref), rep
        assert np.array_equal(lg.cpu().numpy().view(np.uint32), lg_ref.view(np.uint32)), rep


@pytest.mark.gpu
def test_whole_cycle_replays_under_graph_capture():
    """A whole sampled cycle -- k draft-head calls, the allocation-free verify, acceptance with
    its residual draw over several slices, and the commit with its KV trim -- captured into
    one HIP graph; each replay (live state, KV and lengths reset eagerly in between) equals
    the same cycle run eagerly through the workspace entry points."""
    V, d, nd, B, k, T = 4099, 256, 1024, 2, 3, 1.0
    state_bytes, layers, rows, row_bytes = 64 * 1024, 2, 64, 512
    rng = np.random.default_rng(43)
    head = synth.make_head(rng, V, d, "bf16")
    dh = dev_head(head, tiled=True)
    h_v, h_d = synth.make_hidden(rng, B, k, d)
    hv = dev_hidden(synth.encode_hidden(h_v, "bf16"))
    hds = [dev_hidden(np.ascontiguousarray(synth.encode_hidden(h_d, "bf16")[:, i])) for i in range(k)]
    smp = mtp.sampling(T, -1, 99, 5, 0)
    g = torch.Generator(device="cuda").manual_seed(7)
    snaps = torch.randint(0, 256, (B, k + 1, state_bytes), dtype=torch.uint8, device="cuda", generator=g)
    kv_init = torch.randint(1, 256, (B, layers, 2, rows, row_bytes), dtype=torch.uint8, device="cuda", generator=g)
    ws = mtp.workspace(max(mtp.workspace_bytes(mtp.OP_DRAFT, B, nd, B), mtp.workspace_bytes(mtp.OP_VERIFY, B * (k + 1), V, B),
                           mtp.workspace_bytes(mtp.OP_ACCEPT, 0, V, B)))
    bufs = dict(dtok=torch.zeros(B, k, dtype=torch.int32, device="cuda"), dst=mtp.row_stats_empty(B, k),
                dlg=torch.zeros(B, k, nd, dtype=torch.float32, device="cuda"), vst=mtp.row_stats_empty(B, k + 1),
                vlg=torch.zeros(B, k + 1, V, dtype=torch.float32, device="cuda"),
                out=torch.zeros(B, k + 1, dtype=torch.int32, device="cuda"),
                nacc=torch.zeros(B, dtype=torch.int32, device="cuda"), nemit=torch.zeros(B, dtype=torch.int32, device="cuda"),
                flg=torch.zeros(B, dtype=torch.int32, device="cuda"),
                live=torch.zeros(B, state_bytes, dtype=torch.uint8, device="cuda"), kv=kv_init.clone(),
                kvlen=torch.full((B,), 10, dtype=torch.int32, device="cuda"))

    def reset():
        for name in ("dtok", "dst", "vst", "out", "nacc", "nemit", "flg", "live"):
            bufs[name].zero_()
        bufs["dlg"].fill_(3.0)
        bufs["vlg"].fill_(3.0)
        bufs["kv"].copy_(kv_init)
        bufs["kvlen"].fill_(10)

    def cycle(noalloc):
        for i in range(k):
            mtp.mtp_draft_head(dh, nd, hds[i], i, k, smp, bufs["dtok"], bufs["dst"], bufs["dlg"], ws)
        if noalloc:
            mtp.mtp_verify_logits_noalloc(dh, hv, k, bufs["dtok"], k, smp, bufs["vst"], bufs["vlg"])
        else:
            mtp.mtp_verify_logits(dh, hv, k, bufs["dtok"], k, smp, bufs["vst"], bufs["vlg"], ws)
        mtp.mtp_accept_sample(B, k, k, V, nd, smp, bufs["dtok"], bufs["dst"], bufs["dlg"], bufs["vst"], bufs["vlg"],
                              bufs["out"], bufs["nacc"], bufs["nemit"], bufs["flg"], ws)
        mtp.mtp_commit_state(B, k, bufs["nacc"], snaps, bufs["live"], state_bytes, bufs["kv"], layers, rows, row_bytes,
                             bufs["kvlen"])

    def snapshot():
        return {name: t.cpu().numpy().copy() for name, t in bufs.items()}

    reset()
    cycle(noalloc=False)
    torch.cuda.synchronize()
    ref = snapshot()
    assert ref["nacc"].min() >= 0 and (ref["kvlen"] == 10 + ref["nacc"] + 1).all()
    reset()
    cycle(noalloc=True)                     # warm-up outside capture (the scratch array's set-up)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cycle(noalloc=True)
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for name in ref:
            assert np.array_equal(got[name], ref[name]), (rep, name)


def test_noalloc_rejects_bad_arguments_before_touching_a_device():
    if not __import__("os").path.exists(mtp.LIB_PATH):
        pytest.skip("libmtp.so not built")
    if torch.cuda.is_available():
        pytest.skip("checks with fake pointers run on CPU-only hosts")
    lib = mtp.load_library()
    FAKE = 0x10000
    h = mtp.mtp._Head(mtp.W_BF16, 256, 1024, 0, FAKE, None, None, None)
    smp = mtp.sampling(0.0, -1, 0, 0, 0)
    args = lambda B, k, hd=FAKE: (ctypes.byref(h), hd, mtp.H_BF16, B, k, FAKE, 7, ctypes.byref(smp), FAKE, None, None)
    assert lib.mtp_verify_logits_noalloc(*args(17, 7)) == -2          # 136 rows: more than one launch takes
    assert lib.mtp_verify_logits_noalloc(*args(1, 8)) == -2           # k > 7
    assert lib.mtp_verify_logits_noalloc(*args(1, 3, None)) == -1     # no hidden rows
    assert lib.mtp_verify_logits_noalloc(None, FAKE, mtp.H_BF16, 1, 3, FAKE, 7, ctypes.byref(smp), FAKE,
                                         None, None) == -1
