"""Drive the HIP path through the C ABI from tests: upload synthetic inputs, run the
draft -> verify -> accept (-> commit) calls, read results back.  No arithmetic of the
method happens here."""
from __future__ import annotations

import numpy as np
import torch

import speculative_decoding_head_amd as mtp

WT = {"f32": mtp.W_F32, "bf16": mtp.W_BF16, "q4a32": mtp.W_Q4A32}


def dev_head(head, tiled: bool = False) -> mtp.Head:
    """Upload a synth head; ``tiled`` repacks bf16 / 4-bit heads on the device."""
    h = _dev_head_row_major(head)
    if tiled:
        h = mtp.tiled_head(h)
        torch.cuda.synchronize()
    return h


def _dev_head_row_major(head) -> mtp.Head:
    if head.wtype == "f32":
        w = torch.from_numpy(np.ascontiguousarray(head.w, dtype=np.float32)).cuda()
        return mtp.Head(mtp.W_F32, head.d, head.V, w)
    if head.wtype == "bf16":
        return mtp.Head(mtp.W_BF16, head.d, head.V, torch.from_numpy(head.w.view(np.int16)).cuda())
    return mtp.Head(mtp.W_Q4A32, head.d, head.V, torch.from_numpy(head.w).cuda(),
                    torch.from_numpy(head.scale.view(np.int16)).cuda(),
                    torch.from_numpy(head.minv.view(np.int16)).cuda())


def dev_hidden(h: np.ndarray) -> torch.Tensor:
    """f32 array or bf16 bit patterns (uint16) -> device tensor the binding accepts."""
    if h.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(h)).cuda()
    if h.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).cuda()
    raise TypeError(h.dtype)


class GpuCycle:
    """Device buffers for one cycle of B requests with k drafts."""

    def __init__(self, dhead: mtp.Head, n_draft: int, B: int, k: int, temperature: float, seed: int = 0,
                 eos: int = -1, k_max: int | None = None, rule: int = mtp.ACCEPT_RATIO,
                 draft_head: mtp.Head | None = None, draft_row_of: torch.Tensor | None = None):
        """``draft_head``: a head gathered from a set of ids (row_ids set) for the draft
        calls, with ``draft_row_of`` its inverse map; default: the first n_draft rows of
        ``dhead``."""
        self.h, self.n_draft, self.B, self.k = dhead, n_draft, B, k
        self.dh = dhead if draft_head is None else draft_head
        self.row_of = draft_row_of
        self.rule = rule
        self.positions = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.k_max = k if k_max is None else k_max
        self.T, self.seed, self.eos = temperature, seed, eos
        V = dhead.vocab
        dev = "cuda"
        self.draft_tokens = torch.full((B, self.k_max), -7, dtype=torch.int32, device=dev)
        self.draft_stats = mtp.row_stats_empty(B, self.k_max)
        self.draft_logits = (torch.zeros(B, self.k_max, n_draft, dtype=torch.float32, device=dev)
                             if temperature > 0 else None)
        self.row_stats = mtp.row_stats_empty(B, k + 1)
        self.logits = torch.zeros(B, k + 1, V, dtype=torch.float32, device=dev) if temperature > 0 else None
        self.out_tokens = torch.zeros(B, k + 1, dtype=torch.int32, device=dev)
        self.n_accept = torch.zeros(B, dtype=torch.int32, device=dev)
        self.n_emit = torch.zeros(B, dtype=torch.int32, device=dev)
        self.flags = torch.zeros(B, dtype=torch.int32, device=dev)
        nb = max(mtp.workspace_bytes(mtp.OP_DRAFT, min(B, 16), n_draft, B),
                 mtp.workspace_bytes(mtp.OP_VERIFY, min(B * (k + 1), 128), V, B),
                 mtp.workspace_bytes(mtp.OP_ACCEPT, 0, V, B))
        self.ws = mtp.workspace(nb)

    def set_positions(self, positions) -> None:
        """Absolute position verify row 0 of each request predicts (exact-match rule)."""
        self.positions.copy_(torch.as_tensor(np.asarray(positions, dtype=np.int32)))

    def smp(self, cycle=0, request_base=0):
        return mtp.sampling(self.T, self.eos, self.seed, cycle, request_base, self.rule, self.positions)

    def draft(self, slot: int, h_slot: torch.Tensor, cycle=0, request_base=0):
        mtp.mtp_draft_head(self.dh, self.n_draft, h_slot, slot, self.k_max, self.smp(cycle, request_base),
                           self.draft_tokens, self.draft_stats, self.draft_logits, self.ws)

    def verify(self, h_v: torch.Tensor, cycle=0, request_base=0):
        mtp.mtp_verify_logits(self.h, h_v, self.k, self.draft_tokens, self.k_max, self.smp(cycle, request_base),
                              self.row_stats, self.logits, self.ws)

    def accept(self, cycle=0, request_base=0):
        mtp.mtp_accept_sample(self.B, self.k, self.k_max, self.h.vocab, self.n_draft, self.smp(cycle, request_base),
                              self.draft_tokens, self.draft_stats, self.draft_logits, self.row_stats, self.logits,
                              self.out_tokens, self.n_accept, self.n_emit, self.flags, self.ws,
                              draft_row_of=self.row_of)

    def run(self, h_d: torch.Tensor, h_v: torch.Tensor, cycle=0, request_base=0, drafts=None) -> dict:
        """h_d [B][k][d], h_v [B][k+1][d] on the device."""
        for i in range(self.k):
            self.draft(i, h_d[:, i].contiguous(), cycle, request_base)
        if drafts is not None:
            self.draft_tokens[:, :self.k] = torch.as_tensor(np.asarray(drafts), dtype=torch.int32, device="cuda")
        self.verify(h_v, cycle, request_base)
        self.accept(cycle, request_base)
        torch.cuda.synchronize()
        return self.results()

    def results(self) -> dict:
        ds = {k: v.cpu().numpy() for k, v in mtp.row_stats_fields(self.draft_stats).items()}
        vs = {k: v.cpu().numpy() for k, v in mtp.row_stats_fields(self.row_stats).items()}
        out = dict(drafts=self.draft_tokens.cpu().numpy()[:, :self.k], dstats=ds, vstats=vs,
                   tokens=self.out_tokens.cpu().numpy(), n_accept=self.n_accept.cpu().numpy(),
                   n_emit=self.n_emit.cpu().numpy(), flags=self.flags.cpu().numpy().astype(np.uint32))
        if self.logits is not None:
            out["logits"] = self.logits.cpu().numpy()
            out["draft_logits"] = self.draft_logits.cpu().numpy()[:, :self.k]
        return out
