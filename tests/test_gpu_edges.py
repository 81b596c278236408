"""GPU parity at degenerate shapes, on exactly representable inputs (logits bit-exact
against the fp64 oracle): a vocabulary of one row, vocabularies shorter than one 16-row
tile or one tile plus a ragged row, a hidden size of one 32-value K-step and one that
leaves a ragged chunk, a draft head of one row and one over the whole vocabulary, and the
widest launch (16 requests x 8 verify rows, the 128-row kernel) on all of them."""
import numpy as np
import pytest
import torch

import synth
from gpu_cycle import GpuCycle, dev_head, dev_hidden
from oracle import mtp_oracle as O
from parity import check_cycle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _exact_inputs(wtype, V, d, B, k, seed):
    """W entries m/256 (|m| <= 127) or 4-bit codes with scale 1/16 and min -1/2, hidden values
    in {-3..3}: every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    h_v = rng.integers(-3, 4, size=(B, k + 1, d)).astype(np.float32)
    h_d = rng.integers(-3, 4, size=(B, k, d)).astype(np.float32)
    if wtype == "q4a32":
        q = rng.integers(0, 16, size=(V, d)).astype(np.uint8)
        nib = q[:, 0::2] | (q[:, 1::2] << 4)
        sc = np.full((V, d // 32), 0x3D80, np.uint16)           # 1/16
        mn = np.full((V, d // 32), 0xBF00, np.uint16)           # -1/2
        head = synth.Head("q4a32", V, d, nib, sc, mn)
    else:
        w = rng.integers(-127, 128, size=(V, d)).astype(np.float32) / 256.0
        head = synth.Head(wtype, V, d, w if wtype == "f32" else synth.bf16_bits(w))
    htype = "f32" if wtype == "f32" else "bf16"
    return head, synth.encode_hidden(h_v, htype), synth.encode_hidden(h_d, htype), htype


# (V, n_draft): one row; less than a tile; a tile and one row, drafting one row or all of them
SHAPES = [(1, 1), (5, 3), (17, 1), (17, 17), (40, 16)]


@pytest.mark.parametrize("wtype,d,tiled", [("f32", 32, False), ("f32", 96, False), ("bf16", 32, False),
                                           ("bf16", 96, True), ("q4a32", 256, False), ("q4a32", 256, True)])
@pytest.mark.parametrize("V,nd", SHAPES)
@pytest.mark.parametrize("B,k", [(1, 1), (3, 3), (16, 7)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_degenerate_shapes_against_oracle(wtype, d, tiled, V, nd, B, k, T):
    head, hv, hd, htype = _exact_inputs(wtype, V, d, B, k, seed=V * 100 + nd * 10 + B + k)
    W = O.head_weights_f64(head)
    o = O.cycle(W, nd, O.hidden_f64(hd, htype), O.hidden_f64(hv, htype), T, 91, 2, -1, 1e-4)
    gc = GpuCycle(dev_head(head, tiled=tiled), nd, B, k, T, seed=91)
    g = gc.run(dev_hidden(hd), dev_hidden(hv), cycle=2)
    if T > 0:
        z = O.logits_f64(W, O.hidden_f64(hv, htype))
        assert np.array_equal(g["logits"].astype(np.float64), z)                      # bit-exact
        zd = np.stack([O.logits_f64(W[:nd], O.hidden_f64(hd[:, i], htype)) for i in range(k)], axis=1)
        assert np.array_equal(g["draft_logits"].astype(np.float64), zd)
    else:
        # exact logits: every greedy decision (lowest id on exact ties) agrees
        assert np.array_equal(g["drafts"], o["drafts"])
        assert np.array_equal(g["vstats"]["argmax"], o["verify"]["argmax"])
        assert np.array_equal(g["tokens"], o["accept"]["tokens"])
        assert np.array_equal(g["n_accept"], o["accept"]["n_accept"])
        assert np.array_equal(g["n_emit"], o["accept"]["n_emit"])
    if V == 1:
        # one id: every draft is id 0, accepted, and the bonus is id 0 too
        assert (g["drafts"] == 0).all() and (g["n_accept"] == k).all() and (g["tokens"] == 0).all()
    lattice = 1 / 16 if wtype == "q4a32" else 1 / 256
    check_cycle(g, o, T, 1e-4, tag=f"{wtype} d{d} V{V} nd{nd} B{B} k{k} T{T}", lattice=lattice,
                min_clean=0 if T == 0 else 1)
