"""Seeded synthetic workloads for one speculative cycle.

Everything here is input construction: random weights and hidden rows, their
encoding into the stored formats (fp32, bf16 bit patterns, 4-bit affine packing),
planted edits that force a chosen acceptance depth or an EOS position, and random
state/KV bytes.  The arithmetic of the cycle itself lives elsewhere, twice: once in
the oracle and once in the HIP kernels.

Draw order (one ``numpy.random.default_rng(seed)`` per workload):
  1. W  [V][d]      normal(0, sigma) in fp32, then encoded (bf16 round-to-nearest-even,
                    or 4-bit affine packing per 32-value group);
  2. h_v [B][k+1][d] standard normal (verify rows);
  3. h_d [B][k][d]   standard normal (draft rows).
Planted edits are applied after the draws, before encoding the hidden rows.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "WT_F32", "WT_BF16", "WT_Q4A32", "HT_F32", "HT_BF16",
    "bf16_bits", "pack_q4a32", "Head", "make_head", "Workload", "WORKLOADS",
    "make_hidden", "encode_hidden", "plant_rows", "make_state", "identity_head",
]

WT_F32, WT_BF16, WT_Q4A32 = "f32", "bf16", "q4a32"
HT_F32, HT_BF16 = "f32", "bf16"
Q4_GROUP = 32


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN stays NaN (quiet bit forced); +-inf stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def _bf16_to_f32_for_construction(bits: np.ndarray) -> np.ndarray:
    # Used only to aim planted hidden rows at stored weight rows.
    return (bits.astype(np.uint32) << 16).view(np.float32)


def pack_q4a32(w: np.ndarray):
    """Pack fp32 weights [V][d] into the 4-bit affine, 32-value-group format.

    Per group of 32 consecutive elements along d:
      minv  = bf16(min w),  scale = bf16((max w - min w) / 15),
      q     = clamp(round_half_even((w - minv) / scale), 0, 15)   (q = 0 if scale == 0)
    Storage (structure of arrays):
      nibbles uint8 [V][d/2]   element 2j in the low nibble of byte j, 2j+1 in the high nibble
      scale   uint16 [V][d/32] bf16 bit patterns
      minv    uint16 [V][d/32] bf16 bit patterns
    The packed bytes, not the fp32 source, define the weights.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    V, d = w.shape
    if d % Q4_GROUP:
        raise ValueError("d must be a multiple of 32 for the 4-bit affine format")
    G = d // Q4_GROUP
    nib = np.empty((V, d // 2), dtype=np.uint8)
    scale_bits = np.empty((V, G), dtype=np.uint16)
    min_bits = np.empty((V, G), dtype=np.uint16)
    step = max(1, (1 << 24) // d)
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        g = w[r0:r1].reshape(r1 - r0, G, Q4_GROUP).astype(np.float64)
        lo = g.min(axis=2)
        hi = g.max(axis=2)
        mb = bf16_bits(lo.astype(np.float32))
        sb = bf16_bits(((hi - lo) / 15.0).astype(np.float32))
        mval = _bf16_to_f32_for_construction(mb).astype(np.float64)
        sval = _bf16_to_f32_for_construction(sb).astype(np.float64)
        safe = np.where(sval > 0, sval, 1.0)
        q = np.rint((g - mval[..., None]) / safe[..., None])
        q = np.where(sval[..., None] > 0, q, 0.0)
        q = np.clip(q, 0, 15).astype(np.uint8).reshape(r1 - r0, d)
        nib[r0:r1] = q[:, 0::2] | (q[:, 1::2] << 4)
        scale_bits[r0:r1] = sb
        min_bits[r0:r1] = mb
    return nib, scale_bits, min_bits


@dataclasses.dataclass
class Head:
    """A shared LM head W[V][d] in one stored format.

    wtype f32:   w float32 [V][d]
    wtype bf16:  w uint16  [V][d]   (bf16 bit patterns)
    wtype q4a32: w uint8   [V][d/2] + scale uint16 [V][d/32] + minv uint16 [V][d/32]
    ``source`` optionally keeps the fp32 draw the stored format was encoded from; it is
    used only to aim planted hidden rows.
    """
    wtype: str
    V: int
    d: int
    w: np.ndarray
    scale: Optional[np.ndarray] = None
    minv: Optional[np.ndarray] = None
    source: Optional[np.ndarray] = None

    def row_f32_for_construction(self, x: int) -> np.ndarray:
        if self.source is not None:
            return self.source[x].astype(np.float32)
        if self.wtype == WT_F32:
            return self.w[x].astype(np.float32)
        if self.wtype == WT_BF16:
            return _bf16_to_f32_for_construction(self.w[x])
        raise ValueError("4-bit heads need the fp32 source to aim planted rows")

    @property
    def nbytes(self) -> int:
        n = self.w.nbytes
        if self.scale is not None:
            n += self.scale.nbytes + self.minv.nbytes
        return n


def make_head(rng: np.random.Generator, V: int, d: int, wtype: str,
              sigma: float = 0.02, keep_source: bool = False) -> Head:
    w = rng.standard_normal((V, d), dtype=np.float32)
    w *= np.float32(sigma)
    if wtype == WT_F32:
        return Head(wtype, V, d, w, source=None)
    if wtype == WT_BF16:
        return Head(wtype, V, d, bf16_bits(w), source=w if keep_source else None)
    if wtype == WT_Q4A32:
        nib, sc, mn = pack_q4a32(w)
        return Head(wtype, V, d, nib, sc, mn, source=w if keep_source else None)
    raise ValueError(wtype)


def identity_head(V: int) -> Head:
    """fp32 identity head (d = V): logits equal the hidden row exactly."""
    return Head(WT_F32, V, V, np.eye(V, dtype=np.float32))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d: int
    V: int
    n_draft: int
    k: int
    B: int
    wtype: str
    htype: str
    temperature: float
    seed: int            # numpy draw seed
    philox_seed: int     # key of the counter-based generator
    eos: int = -1
    sigma: float = 0.02
    accept_rule: str = "ratio"   # at T > 0: "ratio" (u q <= p) or "exact" (draft == the trunk's draw)
    # recurrent state / KV (commit); zero means no state in this workload
    n_state_layers: int = 0
    state_heads: int = 0
    state_dim: int = 0
    n_attn_layers: int = 0
    kv_max_rows: int = 0
    kv_heads: int = 0
    kv_head_dim: int = 0

    @property
    def state_bytes(self) -> int:
        return self.n_state_layers * self.state_heads * self.state_dim * self.state_dim * 4

    @property
    def kv_row_bytes(self) -> int:
        return self.kv_heads * self.kv_head_dim * 2


WORKLOADS: Dict[str, Workload] = {
    # tiny greedy cycle
    "tiny_greedy": Workload("tiny_greedy", d=256, V=4096, n_draft=1024, k=3, B=1,
                            wtype=WT_F32, htype=HT_F32, temperature=0.0, seed=0, philox_seed=0),
    # greedy verify at model scale (152,064-row bf16 head, 64,000 draft rows, k=7)
    "model_greedy": Workload("model_greedy", d=2560, V=152064, n_draft=64000, k=7, B=1,
                             wtype=WT_BF16, htype=HT_BF16, temperature=0.0, seed=0, philox_seed=0),
    # sampled exact speculation at the tiny shapes, EOS id 2
    "tiny_sampled": Workload("tiny_sampled", d=256, V=4096, n_draft=1024, k=3, B=1,
                             wtype=WT_F32, htype=HT_F32, temperature=1.0, seed=0,
                             philox_seed=1234, eos=2),
    # 4-bit affine head at model scale, greedy and sampled
    "q4_greedy": Workload("q4_greedy", d=2560, V=152064, n_draft=64000, k=7, B=1,
                          wtype=WT_Q4A32, htype=HT_BF16, temperature=0.0, seed=0, philox_seed=1234),
    "q4_sampled": Workload("q4_sampled", d=2560, V=152064, n_draft=64000, k=7, B=1,
                           wtype=WT_Q4A32, htype=HT_BF16, temperature=1.0, seed=0, philox_seed=1234),
    # sampled verify at model scale with exact-match acceptance (the trunk's draws keyed
    # by position): argmax drafts, no draft logits, no residual
    "exact_sampled": Workload("exact_sampled", d=2560, V=152064, n_draft=64000, k=7, B=1,
                              wtype=WT_BF16, htype=HT_BF16, temperature=1.0, seed=0, philox_seed=1234,
                              accept_rule="exact"),
    # 16 requests x 8 verify rows, per-request acceptance, commit of 36-layer fp32 state
    "batched_commit": Workload("batched_commit", d=2560, V=152064, n_draft=64000, k=7, B=16,
                               wtype=WT_BF16, htype=HT_BF16, temperature=0.0, seed=0, philox_seed=0,
                               n_state_layers=36, state_heads=16, state_dim=128,
                               n_attn_layers=12, kv_max_rows=64, kv_heads=4, kv_head_dim=256),
}


def make_hidden(rng: np.random.Generator, B: int, k: int, d: int):
    """Standard-normal fp32 hidden rows, verify rows first, then draft rows."""
    h_v = rng.standard_normal((B, k + 1, d), dtype=np.float32)
    h_d = rng.standard_normal((B, k, d), dtype=np.float32)
    return h_v, h_d


def encode_hidden(h: np.ndarray, htype: str) -> np.ndarray:
    if htype == HT_F32:
        return np.ascontiguousarray(h, dtype=np.float32)
    if htype == HT_BF16:
        return bf16_bits(h)
    raise ValueError(htype)


def _aim(head: Head, x: int) -> np.ndarray:
    r = head.row_f32_for_construction(x).astype(np.float64)
    return (r / max(float(r @ r), 1e-30)).astype(np.float32)


def plant_rows(head: Head, h_v: np.ndarray, h_d: np.ndarray, depths: Sequence[int],
               targets: np.ndarray, alt_targets: np.ndarray, margin: float = 8.0) -> None:
    """Force an acceptance depth per request, in place (fp32 hidden rows).

    For request b with depth a = depths[b] (0..k):
      rows i < a:  h_v[b][i] += margin * aim(targets[b][i]); h_d[b][i] = h_v[b][i]
                   (draft and target agree on targets[b][i]);
      row  a < k:  h_v[b][a] += margin * aim(targets[b][a]);
                   h_d[b][a] = old h_v[b][a] + margin * aim(alt_targets[b][a])
                   (the draft prefers another id, so the draft is rejected there);
      row  k:      h_v[b][k] += margin * aim(targets[b][k]) (bonus row).
    aim(x) = W[x] / |W[x]|^2, so the planted row's logit at x rises by ``margin``.
    targets must be draft ids (< n_draft) for rows < k.
    """
    B, k1, _ = h_v.shape
    k = k1 - 1
    for b in range(B):
        a = int(depths[b])
        for i in range(k + 1):
            base = h_v[b, i].copy()
            h_v[b, i] = base + np.float32(margin) * _aim(head, int(targets[b, i]))
            if i < k:
                if i < a:
                    h_d[b, i] = h_v[b, i]
                elif i == a:
                    h_d[b, i] = base + np.float32(margin) * _aim(head, int(alt_targets[b, i]))


def make_state(rng: np.random.Generator, B: int, k: int, state_bytes: int, n_layers: int,
               max_rows: int, kv_row_bytes: int, kv_len: Optional[np.ndarray] = None):
    """Random recurrent-state snapshots and a KV cache after a verify pass.

    snapshots uint8 [B][k+1][state_bytes]: random, distinct per (b, r) with overwhelming
                                           probability (snapshot r = state after verify row r);
    live      uint8 [B][state_bytes]:      random (the pre-cycle state; overwritten by commit);
    kv        uint8 [B][n_layers][2][max_rows][kv_row_bytes]: rows [0, kv_len+k+1) random
                                           (prefix plus the k+1 rows the verify appended), rest 0;
    kv_len    int32 [B]                    drawn in [0, max_rows - k - 1] unless given.
    """
    snaps = np.frombuffer(rng.bytes(B * (k + 1) * state_bytes), dtype=np.uint8)
    snaps = snaps.reshape(B, k + 1, state_bytes).copy()
    live = np.frombuffer(rng.bytes(B * state_bytes), dtype=np.uint8).reshape(B, state_bytes).copy()
    if kv_len is None:
        kv_len = rng.integers(0, max_rows - k, size=B).astype(np.int32)
    kv = np.zeros((B, n_layers, 2, max_rows, kv_row_bytes), dtype=np.uint8)
    for b in range(B):
        n = int(kv_len[b]) + k + 1
        kv[b, :, :, :n, :] = np.frombuffer(
            rng.bytes(n_layers * 2 * n * kv_row_bytes), dtype=np.uint8
        ).reshape(n_layers, 2, n, kv_row_bytes)
    return snaps, live, kv, np.asarray(kv_len, dtype=np.int32)
