"""GPU parity of the four entry points against the oracle at sizes the oracle finishes in
seconds: several tiles plus ragged tails, exactly representable inputs (bit-exact logits),
planted ties, planted acceptance depths and EOS, non-finite rows, batch invariance,
determinism, and the commit."""
import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
import synth
from gpu_cycle import GpuCycle, dev_head, dev_hidden
from oracle import mtp_oracle as O
from parity import add_results, check_cycle, check_excluded, close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _exact_case(wtype, V, d, B, k, seed, tie_rows=(5, 9)):
    """W entries m/256 (|m| <= 127) or 4-bit codes with scale 1/16, min -1/2; hidden in
    {-3..3}: every partial sum is exact in fp32, so GPU logits must equal the fp64 oracle's."""
    rng = np.random.default_rng(seed)
    h_v = rng.integers(-3, 4, size=(B, k + 1, d)).astype(np.float32)
    h_d = rng.integers(-3, 4, size=(B, k, d)).astype(np.float32)
    if wtype == "q4a32":
        q = rng.integers(0, 16, size=(V, d)).astype(np.uint8)
        sgn = (np.sign(h_v[0, 0]) * 7 + 8).astype(np.uint8)     # planted tie rows aligned with row 0
        for x in tie_rows:
            q[x] = sgn
        nib = q[:, 0::2] | (q[:, 1::2] << 4)
        sc = np.full((V, d // 32), 0x3D80, np.uint16)           # 1/16
        mn = np.full((V, d // 32), 0xBF00, np.uint16)           # -1/2
        head = synth.Head("q4a32", V, d, nib, sc, mn)
    else:
        m = rng.integers(-127, 128, size=(V, d)).astype(np.float32)
        for x in tie_rows:
            m[x] = 127 * np.sign(h_v[0, 0])
        w = m / 256.0
        head = synth.Head(wtype, V, d, w if wtype == "f32" else synth.bf16_bits(w))
    htype = "f32" if wtype == "f32" else "bf16"
    return head, synth.encode_hidden(h_v, htype), synth.encode_hidden(h_d, htype), htype


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
@pytest.mark.parametrize("B,k", [(1, 1), (1, 7), (2, 3), (4, 3), (2, 7)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_exact_inputs_bit_exact_logits_and_lowest_id_ties(wtype, B, k, T):
    V, d, nd = 1013, 256, 333
    head, hv, hd, htype = _exact_case(wtype, V, d, B, k, seed=B * 10 + k)
    W = O.head_weights_f64(head)
    o = O.cycle(W, nd, O.hidden_f64(hd, htype), O.hidden_f64(hv, htype), T, 77, 3, -1, 1e-4)
    gc = GpuCycle(dev_head(head), nd, B, k, T, seed=77)
    g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=3)
    z = O.logits_f64(W, O.hidden_f64(hv, htype))
    if T > 0:
        assert np.array_equal(g["logits"].astype(np.float64), z)           # bit-exact
        zd = np.stack([O.logits_f64(W[:nd], O.hidden_f64(hd[:, i], htype)) for i in range(k)], axis=1)
        assert np.array_equal(g["draft_logits"].astype(np.float64), zd)
    # planted exact tie at ids 5 and 9 on verify row 0 of request 0: the lowest id wins
    if z[0, 0, 5] == z[0, 0].max():
        assert g["vstats"]["argmax"][0, 0] == 5
    if T == 0:
        # exact logits: greedy decisions (lowest id on exact ties) must agree everywhere
        assert np.array_equal(g["drafts"], o["drafts"])
        assert np.array_equal(g["vstats"]["argmax"], o["verify"]["argmax"])
        assert np.array_equal(g["tokens"], o["accept"]["tokens"])
        assert np.array_equal(g["n_accept"], o["accept"]["n_accept"])
    # logits on a grid (1/256, or 1/16 for the 4-bit codes); at T = 0 the planted tie on row 0
    # of request 0 is on the path, and every decision was compared exactly above
    check_cycle(g, o, T, 1e-4, tag=f"{wtype} B{B} k{k} T{T}", lattice=1 / 16 if wtype == "q4a32" else 1 / 256,
                certain_ties=1 if T == 0 else 0, min_clean=0 if (T == 0 and B == 1) else 1)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_tiny_cycle_against_oracle(T):
    # the tiny workload: d=256, V=4096, 1024 draft rows, k=3, fp32 N(0, 0.02) head, seed 0
    wl = synth.WORKLOADS["tiny_greedy"]
    rng = np.random.default_rng(wl.seed)
    head = synth.make_head(rng, wl.V, wl.d, wl.wtype)
    h_v, h_d = synth.make_hidden(rng, 1, wl.k, wl.d)
    W = O.head_weights_f64(head)
    seed = 1234 if T > 0 else 0
    gc = GpuCycle(dev_head(head), wl.n_draft, 1, wl.k, T, seed=seed, eos=2 if T > 0 else -1)
    total = None
    for cyc in range(20):
        o = O.cycle(W, wl.n_draft, h_d.astype(np.float64), h_v.astype(np.float64), T, seed, cyc,
                    2 if T > 0 else -1, 1e-4)
        g = gc.run(dev_hidden(h_d), dev_hidden(h_v), cycle=cyc)
        total = add_results(total, check_cycle(g, o, T, 1e-4, tag=f"tiny T{T} cycle {cyc}", bound=False))
    check_excluded(total, f"tiny T{T}")


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_planted_depths_and_eos(wtype, T):
    """Every acceptance depth 0..k over 2 requests x 8 cycles; EOS planted at some positions."""
    V, d, nd, k, B = 4096, 256, 1024, 7, 2
    rng = np.random.default_rng(5)
    head = synth.make_head(rng, V, d, wtype, keep_source=True)
    W = O.head_weights_f64(head)
    htype = "f32" if wtype == "f32" else "bf16"
    delta = 1e-4 if wtype == "f32" else 2e-2
    gc = GpuCycle(dev_head(head), nd, B, k, T, seed=1234, eos=2)
    seen = set()
    total = None
    for cyc in range(8):
        h_v, h_d = synth.make_hidden(rng, B, k, d)
        depths = [(cyc + b * 4) % (k + 1) for b in range(B)]
        targets = rng.integers(3, nd, size=(B, k + 1))
        alts = (targets + 17) % nd
        if cyc % 3 == 2:
            targets[0, depths[0] if depths[0] < k else k - 1] = 2        # EOS on the path
        synth.plant_rows(head, h_v, h_d, depths, targets, alts, margin=12.0)
        hv, hd = synth.encode_hidden(h_v, htype), synth.encode_hidden(h_d, htype)
        o = O.cycle(W, nd, O.hidden_f64(hd, htype), O.hidden_f64(hv, htype), T, 1234, cyc, 2, delta)
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cyc)
        total = add_results(total, check_cycle(g, o, T, delta, tag=f"{wtype} T{T} cycle {cyc}", bound=False))
        seen.update(int(a) for a in g["n_accept"])
        if T == 0:
            for b in range(B):
                a = depths[b]
                eos_at = [i for i in range(k) if targets[b, i] == 2 and i <= a]
                want = eos_at[0] if eos_at and eos_at[0] < a else a
                assert g["n_accept"][b] == want
    check_excluded(total, f"{wtype} T{T} planted")
    if T == 0:
        assert len(seen) >= 6


@pytest.mark.parametrize("V", [2050, 5003])
def test_residual_draw_over_several_slices(V):
    """Ratio acceptance at T = 1 over a vocabulary that is not a multiple of 4 and spans several
    of the accept kernel's residual slices (2050: 3 slices of 684 ids; 5003: 5 slices, the
    last one short): planted rejections at every depth, tokens, counts and flags against the
    oracle."""
    d, nd, k, B = 256, 1500, 7, 3
    rng = np.random.default_rng(V)
    head = synth.make_head(rng, V, d, "bf16", keep_source=True)
    W = O.head_weights_f64(head)
    gc = GpuCycle(dev_head(head), nd, B, k, 1.0, seed=99, eos=-1)
    total = None
    for cyc in range(6):
        h_v, h_d = synth.make_hidden(rng, B, k, d)
        depths = [(cyc + 3 * b) % (k + 1) for b in range(B)]
        targets = rng.integers(3, nd, size=(B, k + 1))
        synth.plant_rows(head, h_v, h_d, depths, targets, (targets + 11) % nd, margin=12.0)
        hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
        o = O.cycle(W, nd, O.hidden_f64(hd, "bf16"), O.hidden_f64(hv, "bf16"), 1.0, 99, cyc, -1, 2e-2)
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cyc)
        total = add_results(total, check_cycle(g, o, 1.0, 2e-2, tag=f"V{V} cycle {cyc}", bound=False))
    check_excluded(total, f"V{V}")


def _nonfinite_head(V, d):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
    return w


@pytest.mark.parametrize("kind", ["nan_rows", "posinf", "all_nan", "neginf"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_nonfinite_rows(kind, T):
    V, d, nd, k = 640, 64, 200, 3
    w = _nonfinite_head(V, d)
    h_v = np.abs(np.random.default_rng(4).standard_normal((1, k + 1, d))).astype(np.float32) + 0.1
    h_d = np.abs(np.random.default_rng(6).standard_normal((1, k, d))).astype(np.float32) + 0.1
    if kind == "nan_rows":
        w[[7, 150, 400]] = np.nan
    elif kind == "posinf":
        w[[30, 190, 500], 0] = np.inf            # hidden > 0: those logits are +inf
    elif kind == "all_nan":
        w[:, 5] = np.nan                          # every logit NaN -> rows invalid
    elif kind == "neginf":
        w[:, 0] = -np.inf                         # every logit -inf -> rows invalid
        w[:50, 0] = 0.0
    head = synth.Head("f32", V, d, w)
    W = O.head_weights_f64(head)
    o = O.cycle(W, nd, h_d.astype(np.float64), h_v.astype(np.float64), T, 9, 0, -1, 1e-4)
    gc = GpuCycle(dev_head(head), nd, 1, k, T, seed=9)
    g = gc.run(dev_hidden(h_d), dev_hidden(h_v))
    check_cycle(g, o, T, 1e-4, tag=f"nonfinite {kind} T{T}")
    assert np.array_equal(g["dstats"]["flags"][:, :k].astype(np.uint32),
                          np.stack([o["draft"][i]["flags"] for i in range(k)], axis=1))
    assert np.array_equal(g["vstats"]["n_posinf"], np.isposinf(O.logits_f64(W, h_v.astype(np.float64))).sum(-1))


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
def test_batch_invariance_bitwise(wtype):
    """A row's logits and statistics do not depend on how many rows share the launch or on
    the row's position (verify M = 2..16, draft B = 1..16)."""
    V, d, nd = 2000, 256, 700
    rng = np.random.default_rng(12)
    head = synth.make_head(rng, V, d, wtype)
    dh = dev_head(head)
    htype = "f32" if wtype == "f32" else "bf16"
    rows = synth.encode_hidden(rng.standard_normal((16, d)).astype(np.float32), htype)
    ref = None
    for B, k in [(1, 1), (1, 3), (1, 7), (2, 3), (2, 7), (4, 3), (8, 1)]:
        M = B * (k + 1)
        for pos in sorted({0, M - 1, M // 2}):
            hv = np.repeat(rows[1:2], M, axis=0)
            hv[pos] = rows[0]
            gc = GpuCycle(dh, nd, B, k, 1.0, seed=5)
            gc.draft_tokens.zero_()
            gc.verify(dev_hidden(hv.reshape(B, k + 1, d)))
            torch.cuda.synchronize()
            lg = gc.logits.reshape(M, V)[pos].cpu().numpy()
            st = gc.row_stats.reshape(M, 8)[pos].cpu().numpy()
            if ref is None:
                ref = (lg, st)
            assert np.array_equal(lg.view(np.uint32), ref[0].view(np.uint32)), (B, k, pos)
            # max, lse, argmax and flags are identical bits (z_tok/sample depend on the position)
            assert np.array_equal(st[[0, 1, 3, 5, 6]], ref[1][[0, 1, 3, 5, 6]]), (B, k, pos)
    # draft head over all V rows at any batch position equals the verify row
    for B in (1, 5, 16):
        hd = np.repeat(rows[1:2], B, axis=0)
        hd[B - 1] = rows[0]
        gc = GpuCycle(dh, V, B, 1, 1.0, seed=5)
        gc.draft(0, dev_hidden(hd))
        torch.cuda.synchronize()
        lg = gc.draft_logits[B - 1, 0].cpu().numpy()
        st = gc.draft_stats[B - 1, 0].cpu().numpy()
        assert np.array_equal(lg.view(np.uint32), ref[0].view(np.uint32))
        assert np.array_equal(st[[0, 1, 3, 5]], ref[1][[0, 1, 3, 5]])


def test_draft_equal_target_accepts_everything_on_gpu():
    # n_draft = V and h_d = h_v: q = p bit for bit on the GPU, so u*q <= p always holds
    V, d, k, B = 2048, 256, 3, 4
    rng = np.random.default_rng(2)
    head = synth.make_head(rng, V, d, "bf16")
    hv = synth.encode_hidden(rng.standard_normal((B, k + 1, d)).astype(np.float32), "bf16")
    hd = np.ascontiguousarray(hv[:, :k])
    gc = GpuCycle(dev_head(head), V, B, k, 1.0, seed=11)
    for cyc in range(5):
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cyc)
        assert np.all(g["n_accept"] == k) and np.all(g["flags"] & mtp.ACC_ALL_ACCEPTED)


def test_seeded_runs_are_bit_identical():
    wl = synth.WORKLOADS["tiny_sampled"]
    rng = np.random.default_rng(0)
    head = synth.make_head(rng, wl.V, wl.d, "bf16")
    h_v, h_d = synth.make_hidden(rng, 4, wl.k, wl.d)
    hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
    outs = []
    for _ in range(2):
        gc = GpuCycle(dev_head(head), wl.n_draft, 4, wl.k, 1.0, seed=1234, eos=2)
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=7)
        outs.append(g)
    for key in ("drafts", "tokens", "n_accept", "flags", "logits", "draft_logits"):
        assert np.array_equal(outs[0][key], outs[1][key]), key
    for key in ("max", "lse", "z_tok", "sample"):
        assert np.array_equal(outs[0]["vstats"][key], outs[1]["vstats"][key]), key
    gc = GpuCycle(dev_head(head), wl.n_draft, 4, wl.k, 1.0, seed=1234, eos=2)
    g2 = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=8)
    assert not np.array_equal(outs[0]["drafts"], g2["drafts"])


@pytest.mark.parametrize("k", [1, 3, 7])
def test_commit_every_depth_with_guards(k):
    rng = np.random.default_rng(k)
    B, S, L, R, rb = 8, 4096 + 48, 3, 24, 64
    snaps, live, kv, kv_len = synth.make_state(rng, B, k, S, L, R, rb)
    n_acc = np.array([b % (k + 1) for b in range(B)], dtype=np.int32)
    n_acc[-1] = 99       # out of range: clamped to k
    want_live, want_kv, want_len = O.commit(snaps, live, kv, kv_len, n_acc, k)
    d_snaps = torch.from_numpy(snaps).cuda()
    # guard bytes on both sides of the live state and KV buffers
    g_live = torch.full((B * S + 256,), 0xA5, dtype=torch.uint8, device="cuda")
    g_live[128:128 + B * S] = torch.from_numpy(live.reshape(-1)).cuda()
    g_kv = torch.full((kv.size + 256,), 0x5A, dtype=torch.uint8, device="cuda")
    g_kv[128:128 + kv.size] = torch.from_numpy(kv.reshape(-1)).cuda()
    d_len = torch.from_numpy(kv_len).cuda()
    mtp.mtp_commit_state(B, k, torch.from_numpy(n_acc).cuda(), d_snaps, g_live[128:128 + B * S], S,
                         g_kv[128:128 + kv.size], L, R, rb, d_len)
    torch.cuda.synchronize()
    gl = g_live.cpu().numpy()
    gk = g_kv.cpu().numpy()
    assert np.all(gl[:128] == 0xA5) and np.all(gl[-128:] == 0xA5)
    assert np.all(gk[:128] == 0x5A) and np.all(gk[-128:] == 0x5A)
    assert np.array_equal(gl[128:-128].reshape(B, S), want_live)
    assert np.array_equal(gk[128:-128].reshape(kv.shape), want_kv)
    assert np.array_equal(d_len.cpu().numpy(), want_len)


# ---------------------------------------------------------------------------------
# tiled weight layouts
# ---------------------------------------------------------------------------------
def _tiled_bf16_reference(w_bits: np.ndarray) -> np.ndarray:
    """The tiled bf16 layout written out from its definition in include/mtp.h."""
    V, d = w_bits.shape
    T = (V + 15) // 16
    pad = np.zeros((T * 16, d), np.uint16)
    pad[:V] = w_bits
    out = np.zeros((T, d // 32, 64, 8), np.uint16)
    for l in range(64):
        rows = np.arange(T) * 16 + (l % 16)
        for s in range(d // 32):
            out[:, s, l, :] = pad[rows, 32 * s + 8 * (l // 16): 32 * s + 8 * (l // 16) + 8]
    return out.reshape(-1).view(np.uint8)


def _tiled_q4_reference(nib: np.ndarray, sc: np.ndarray, mn: np.ndarray):
    V, half = nib.shape
    d = half * 2
    T = (V + 15) // 16
    pn = np.zeros((T * 16, half), np.uint8)
    pn[:V] = nib
    w = np.zeros((T, d // 128, 64, 16), np.uint8)
    for l in range(64):
        rows = np.arange(T) * 16 + (l % 16)
        for q in range(d // 128):
            for u in range(4):
                b0 = 16 * (4 * q + u) + 4 * (l // 16)
                w[:, q, l, 4 * u:4 * u + 4] = pn[rows, b0:b0 + 4]

    def tile_sc(a):
        p = np.zeros((T * 16, d // 32), np.uint16)
        p[:V] = a
        o = np.zeros((T, d // 256, 16, 8), np.uint16)
        for c in range(d // 256):
            o[:, c, :, :] = p.reshape(T, 16, d // 32)[:, :, 8 * c:8 * c + 8]
        return o.reshape(-1).view(np.uint8)
    return w.reshape(-1), tile_sc(sc), tile_sc(mn)


@pytest.mark.parametrize("wtype", ["bf16", "q4a32"])
@pytest.mark.parametrize("V", [1013, 4096])
def test_pack_head_matches_layout_definition(wtype, V):
    rng = np.random.default_rng(V)
    head = synth.make_head(rng, V, 256, wtype)
    th = dev_head(head, tiled=True)
    if wtype == "bf16":
        assert np.array_equal(th.w.cpu().numpy(), _tiled_bf16_reference(head.w))
    else:
        w, sc, mn = _tiled_q4_reference(head.w, head.scale, head.minv)
        assert np.array_equal(th.w.cpu().numpy(), w)
        assert np.array_equal(th.scale.cpu().numpy(), sc)
        assert np.array_equal(th.minv.cpu().numpy(), mn)


@pytest.mark.parametrize("wtype", ["bf16", "q4a32"])
@pytest.mark.parametrize("B,k", [(1, 7), (2, 3), (4, 3)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_tiled_head_is_bit_identical_to_row_major(wtype, B, k, T):
    V, d, nd = 3001, 512, 1111
    rng = np.random.default_rng(B * 100 + k)
    head = synth.make_head(rng, V, d, wtype)
    h_v, h_d = synth.make_hidden(rng, B, k, d)
    hv, hd = dev_hidden(synth.encode_hidden(h_v, "bf16")), dev_hidden(synth.encode_hidden(h_d, "bf16"))
    outs = []
    for tiled in (False, True):
        gc = GpuCycle(dev_head(head, tiled=tiled), nd, B, k, T, seed=3, eos=2)
        g = gc.run(hd, hv, cycle=4)
        g["raw_vstats"] = gc.row_stats.cpu().numpy()
        g["raw_dstats"] = gc.draft_stats.cpu().numpy()
        outs.append(g)
    a, b = outs
    for key in ("drafts", "tokens", "n_accept", "n_emit", "flags", "raw_vstats", "raw_dstats"):
        assert np.array_equal(a[key], b[key]), key
    if T > 0:
        assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
        assert np.array_equal(a["draft_logits"].view(np.uint32), b["draft_logits"].view(np.uint32))


@pytest.mark.parametrize("wtype", ["bf16", "q4a32"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_tiled_planted_depths_against_oracle(wtype, T):
    V, d, nd, k, B = 4096, 256, 1024, 7, 2
    rng = np.random.default_rng(15)
    head = synth.make_head(rng, V, d, wtype, keep_source=True)
    W = O.head_weights_f64(head)
    gc = GpuCycle(dev_head(head, tiled=True), nd, B, k, T, seed=1234, eos=2)
    total = None
    for cyc in range(4):
        h_v, h_d = synth.make_hidden(rng, B, k, d)
        depths = [(2 * cyc + b * 3) % (k + 1) for b in range(B)]
        targets = rng.integers(3, nd, size=(B, k + 1))
        synth.plant_rows(head, h_v, h_d, depths, targets, (targets + 9) % nd, margin=12.0)
        hv, hd = synth.encode_hidden(h_v, "bf16"), synth.encode_hidden(h_d, "bf16")
        o = O.cycle(W, nd, O.hidden_f64(hd, "bf16"), O.hidden_f64(hv, "bf16"), T, 1234, cyc, 2, 2e-2)
        g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=cyc)
        total = add_results(total, check_cycle(g, o, T, 2e-2, tag=f"tiled {wtype} T{T} cycle {cyc}", bound=False))
    check_excluded(total, f"tiled {wtype} T{T}")
