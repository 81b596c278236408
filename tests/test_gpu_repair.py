"""The GPU commit against an ordinary-forward repair, on the toy trunk with short-
convolution state rows (DS4Server issue "Add Qwen3.8 Flash Next native MTP speculation",
"Implementation", "Verification" and "Completion requirements": capture-commit and the
repair fallback are both correct, compared at logit, token and complete cache-state
level).  The capture path commits with mtp_commit_state on the device; the repair path
replays the accepted tokens on the host; every cycle must leave identical bytes."""
import numpy as np
import pytest
import torch

import speculative_decoding_head_amd as mtp
from repair_paths import ordinary, speculative
from test_oracle_repair import _same_cycles
from toy_trunk import ToyTrunkConv

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def gpu_commit(snaps, live, kv, kv_len, n_accept, k):
    B, K1, S = snaps.shape
    d_snaps = torch.from_numpy(np.ascontiguousarray(snaps)).cuda()
    d_live = torch.from_numpy(np.ascontiguousarray(live)).cuda()
    d_kv = torch.from_numpy(np.ascontiguousarray(kv)).cuda()
    d_len = torch.from_numpy(np.asarray(kv_len, dtype=np.int32).copy()).cuda()
    d_acc = torch.from_numpy(np.asarray(n_accept, dtype=np.int32)).cuda()
    mtp.mtp_commit_state(B, k, d_acc, d_snaps, d_live, S, d_kv, kv.shape[1], kv.shape[3], kv.shape[4], d_len)
    torch.cuda.synchronize()
    return d_live.cpu().numpy(), d_kv.cpu().numpy(), d_len.cpu().numpy()


@pytest.mark.parametrize("k", [2, 7])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_gpu_capture_commit_equals_host_repair(k, T):
    tt = ToyTrunkConv(3)
    assert tt.size * 8 % 16 == 0 and tt.kv_dim * 8 % 16 == 0
    n = 100
    want, _, _ = ordinary(tt, 0, n + k + 2, T, seed=7)
    got_c, cyc_c, _ = speculative(tt, 0, n, k, "capture", T, seed=7, commit=gpu_commit)
    got_r, cyc_r, _ = speculative(tt, 0, n, k, "repair", T, seed=7)
    assert got_c == want[:n] and got_r == want[:n]
    _same_cycles(cyc_c, cyc_r)
