"""Thin Python binding of libmtp.so (argument marshalling only).

Every step of the cycle runs in the HIP kernels behind the C ABI; this module checks
tensors (device, dtype, contiguity, 16-byte alignment), passes raw device pointers and
the current HIP stream, and maps status codes to exceptions.  PyTorch supplies device
memory and streams only.  There is no CPU fallback: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmtp.so")

# mirrors of include/mtp.h
MTP_OK = 0
W_F32, W_BF16, W_Q4A32, W_BF16_TILED, W_Q4A32_TILED = 0, 1, 2, 3, 4
H_F32, H_BF16 = 0, 1
OP_DRAFT, OP_VERIFY, OP_ACCEPT = 0, 1, 2
ROW_NONFINITE, ROW_POSINF, ROW_INVALID = 0x1, 0x2, 0x4
ACC_ALL_ACCEPTED, ACC_EOS, ACC_RESID_FALLBACK, ACC_ROW_INVALID = 0x01, 0x02, 0x04, 0x08
ACC_NONFINITE_TARGET, ACC_NONFINITE_DRAFT, ACC_DRAFT_INVALID, ACC_EOS_DRAFT = 0x10, 0x20, 0x40, 0x80
ROW_STATS_WORDS = 8   # sizeof(mtp_row_stats) / 4
ACCEPT_RATIO, ACCEPT_EXACT = 0, 1

EXPORTED = ("mtp_draft_head", "mtp_verify_logits", "mtp_accept_sample", "mtp_commit_state",
            "mtp_workspace_bytes", "mtp_tiled_bytes", "mtp_pack_head", "mtp_status_str", "mtp_abi_version",
            "mtp_width_init", "mtp_width_observe", "mtp_width_expected_tokens", "mtp_width_cost",
            "mtp_width_choose", "mtp_gather_rows", "mtp_verify_logits_noalloc")


class MtpError(RuntimeError):
    pass


class _WidthCtl(ctypes.Structure):
    _fields_ = [("k_max", ctypes.c_int32), ("reserved", ctypes.c_int32), ("decay", ctypes.c_double),
                ("slope_prior", ctypes.c_double), ("alpha", ctypes.c_double * 7),
                ("weight", ctypes.c_double * 7), ("sw", ctypes.c_double),
                ("sk", ctypes.c_double), ("skk", ctypes.c_double), ("st", ctypes.c_double), ("skt", ctypes.c_double),
                ("verifier_passes", ctypes.c_uint64), ("cycles", ctypes.c_uint64), ("drafted", ctypes.c_uint64),
                ("accepted", ctypes.c_uint64), ("depth_hist", ctypes.c_uint64 * 8)]


class _Head(ctypes.Structure):
    _fields_ = [("wtype", ctypes.c_int32), ("d", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("w", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("minv", ctypes.c_void_p), ("row_ids", ctypes.c_void_p)]


class _Sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("eos_id", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("cycle", ctypes.c_uint32), ("request_base", ctypes.c_uint32), ("accept_rule", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("positions", ctypes.c_void_p)]


_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmtp.so (once).  Raises MtpError if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise MtpError(f"{path} is missing: build it with `python -m speculative_decoding_head_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    hp, sp = ctypes.POINTER(_Head), ctypes.POINTER(_Sampling)
    lib.mtp_draft_head.argtypes = [hp, i32, vp, i32, i32, i32, i32, sp, vp, vp, vp, vp, sz, vp]
    lib.mtp_verify_logits.argtypes = [hp, vp, i32, i32, i32, vp, i32, sp, vp, vp, vp, sz, vp]
    lib.mtp_verify_logits_noalloc.argtypes = [hp, vp, i32, i32, i32, vp, i32, sp, vp, vp, vp]
    lib.mtp_accept_sample.argtypes = [i32, i32, i32, i32, i32, sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mtp_gather_rows.argtypes = [hp, vp, i32, vp, vp, vp, vp]
    lib.mtp_gather_rows.restype = ctypes.c_int
    lib.mtp_commit_state.argtypes = [i32, i32, vp, vp, vp, sz, vp, i32, i32, sz, vp, vp]
    for f in ("mtp_draft_head", "mtp_verify_logits", "mtp_verify_logits_noalloc", "mtp_accept_sample",
              "mtp_commit_state", "mtp_abi_version"):
        getattr(lib, f).restype = ctypes.c_int
    lib.mtp_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.mtp_workspace_bytes.restype = sz
    lib.mtp_tiled_bytes.argtypes = [i32, i32, i32, i32]
    lib.mtp_tiled_bytes.restype = sz
    lib.mtp_pack_head.argtypes = [hp, vp, vp, vp, vp]
    lib.mtp_pack_head.restype = ctypes.c_int
    lib.mtp_status_str.argtypes = [ctypes.c_int]
    lib.mtp_status_str.restype = ctypes.c_char_p
    lib.mtp_abi_version.argtypes = []
    wp, f64 = ctypes.POINTER(_WidthCtl), ctypes.c_double
    lib.mtp_width_init.argtypes = [wp, i32, f64, f64, f64]
    lib.mtp_width_init.restype = ctypes.c_int
    lib.mtp_width_observe.argtypes = [wp, i32, i32, vp, vp, f64]
    lib.mtp_width_observe.restype = ctypes.c_int
    for f in ("mtp_width_expected_tokens", "mtp_width_cost"):
        getattr(lib, f).argtypes = [wp, i32]
        getattr(lib, f).restype = f64
    lib.mtp_width_choose.argtypes = [wp]
    lib.mtp_width_choose.restype = i32
    _lib_handle = lib
    return lib


def _check(status: int) -> None:
    if status != MTP_OK:
        msg = load_library().mtp_status_str(status).decode()
        raise MtpError(f"mtp status {status}: {msg}")


# ---------------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor], dtypes=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise MtpError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MtpError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise MtpError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    p = t.data_ptr()
    if p % 16:
        raise MtpError(f"{name} is not 16-byte aligned")
    return p


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _htype(h: torch.Tensor) -> int:
    if h.dtype == torch.float32:
        return H_F32
    if h.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return H_BF16
    raise MtpError(f"hidden rows must be float32 or bf16, got {h.dtype}")


@dataclass
class Head:
    """Device-resident shared LM head.  w: float32 [V][d] | bf16 [V][d] | uint8 [V][d/2]."""
    wtype: int
    d: int
    vocab: int
    w: torch.Tensor
    scale: Optional[torch.Tensor] = None
    minv: Optional[torch.Tensor] = None
    row_ids: Optional[torch.Tensor] = None   # int32 [vocab]: vocabulary id of each row (gathered draft heads)

    def _struct(self) -> _Head:
        return _Head(self.wtype, self.d, self.vocab, 0, _ptr(self.w, name="w"),
                     _ptr(self.scale, name="scale"), _ptr(self.minv, name="minv"),
                     _ptr(self.row_ids, (torch.int32,), "row_ids"))


def sampling(temperature: float = 0.0, eos_id: int = -1, seed: int = 0, cycle: int = 0,
             request_base: int = 0, accept_rule: int = ACCEPT_RATIO,
             positions: Optional[torch.Tensor] = None) -> _Sampling:
    """mtp_sampling.  ``positions`` (device int32 [B], for ACCEPT_EXACT at T > 0) must stay
    alive until the stream has run the calls that use it."""
    return _Sampling(float(temperature), int(eos_id), int(seed) & (2**64 - 1), int(cycle) & 0xFFFFFFFF,
                     int(request_base) & 0xFFFFFFFF, int(accept_rule), 0,
                     _ptr(positions, (torch.int32,), "positions"))


def row_stats_empty(*shape, device="cuda") -> torch.Tensor:
    """Storage for mtp_row_stats: int32 [..., 8]."""
    return torch.zeros(*shape, ROW_STATS_WORDS, dtype=torch.int32, device=device)


def row_stats_fields(t: torch.Tensor) -> dict:
    """Split an int32 [..., 8] mtp_row_stats tensor into named fields (views)."""
    f = t.view(torch.float32)
    return dict(max=f[..., 0], lse=f[..., 1], z_tok=f[..., 2], argmax=t[..., 3], sample=t[..., 4],
                flags=t[..., 5], n_posinf=t[..., 6])


def workspace_bytes(op: int, rows: int, n_vocab_rows: int, B: int) -> int:
    return int(load_library().mtp_workspace_bytes(op, rows, n_vocab_rows, B))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled, 256-byte aligned workspace of at least nbytes."""
    t = torch.zeros(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + max(int(nbytes), 256)]


def mtp_tiled_bytes(wtype: int, d: int, vocab: int, part: int) -> int:
    return int(load_library().mtp_tiled_bytes(wtype, d, vocab, part))


def mtp_pack_head(src: Head, dst_w: torch.Tensor, dst_scale: Optional[torch.Tensor] = None,
                  dst_minv: Optional[torch.Tensor] = None, stream=None) -> None:
    """Repack a row-major bf16 / 4-bit head into its tiled layout (device buffers given)."""
    lib = load_library()
    h = src._struct()
    _check(lib.mtp_pack_head(ctypes.byref(h), _ptr(dst_w, name="dst_w"), _ptr(dst_scale, name="dst_scale"),
                             _ptr(dst_minv, name="dst_minv"), _stream(stream)))


def tiled_head(src: Head, stream=None) -> Head:
    """Allocate device buffers and repack ``src`` into the tiled layout."""
    if src.wtype not in (W_BF16, W_Q4A32):
        raise MtpError("only row-major bf16 and 4-bit heads can be tiled")
    dev = src.w.device
    nb = [mtp_tiled_bytes(src.wtype, src.d, src.vocab, p) for p in range(3)]
    w = torch.empty(nb[0], dtype=torch.uint8, device=dev)
    sc = torch.empty(nb[1], dtype=torch.uint8, device=dev) if nb[1] else None
    mn = torch.empty(nb[2], dtype=torch.uint8, device=dev) if nb[2] else None
    mtp_pack_head(src, w, sc, mn, stream)
    return Head(W_BF16_TILED if src.wtype == W_BF16 else W_Q4A32_TILED, src.d, src.vocab, w, sc, mn, src.row_ids)


def gather_rows(src: Head, ids: torch.Tensor, stream=None) -> Head:
    """mtp_gather_rows: a row-major head of the rows ``ids`` (device int32, strictly
    ascending) of the row-major head ``src``, with row_ids = ids."""
    if src.wtype not in (W_F32, W_BF16, W_Q4A32):
        raise MtpError("gather from a row-major head")
    n = int(ids.numel())
    dev = src.w.device
    if src.wtype == W_Q4A32:
        w = torch.empty(n, src.d // 2, dtype=torch.uint8, device=dev)
        sc = torch.empty(n, src.d // 32, dtype=torch.int16, device=dev)
        mn = torch.empty(n, src.d // 32, dtype=torch.int16, device=dev)
    else:
        w = torch.empty(n, src.d, dtype=torch.float32 if src.wtype == W_F32 else torch.int16, device=dev)
        sc = mn = None
    h = src._struct()
    _check(load_library().mtp_gather_rows(ctypes.byref(h), _ptr(ids, (torch.int32,), "ids"), n, _ptr(w, name="w"),
                                          _ptr(sc, name="scale"), _ptr(mn, name="minv"), _stream(stream)))
    return Head(src.wtype, src.d, n, w, sc, mn, ids)


# ---------------------------------------------------------------------------------
# the four calls (same names as the C ABI)
# ---------------------------------------------------------------------------------
def mtp_draft_head(head: Head, n_draft: int, hidden: torch.Tensor, slot: int, k_max: int, smp: _Sampling,
                   draft_tokens: torch.Tensor, draft_stats: torch.Tensor, draft_logits: Optional[torch.Tensor],
                   ws: torch.Tensor, stream=None) -> None:
    lib = load_library()
    B = hidden.shape[0]
    h = head._struct()
    _check(lib.mtp_draft_head(ctypes.byref(h), int(n_draft), _ptr(hidden, name="hidden"), _htype(hidden), int(B),
                              int(slot), int(k_max), ctypes.byref(smp), _ptr(draft_tokens, (torch.int32,), "draft_tokens"),
                              _ptr(draft_stats, (torch.int32,), "draft_stats"),
                              _ptr(draft_logits, (torch.float32,), "draft_logits"),
                              _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


def mtp_verify_logits(head: Head, hidden: torch.Tensor, k: int, draft_tokens: torch.Tensor, k_max: int,
                      smp: _Sampling, row_stats: torch.Tensor, logits: Optional[torch.Tensor],
                      ws: torch.Tensor, stream=None) -> None:
    lib = load_library()
    B = hidden.shape[0] if hidden.dim() == 3 else hidden.shape[0] // (k + 1)
    h = head._struct()
    _check(lib.mtp_verify_logits(ctypes.byref(h), _ptr(hidden, name="hidden"), _htype(hidden), int(B), int(k),
                                 _ptr(draft_tokens, (torch.int32,), "draft_tokens"), int(k_max), ctypes.byref(smp),
                                 _ptr(row_stats, (torch.int32,), "row_stats"),
                                 _ptr(logits, (torch.float32,), "logits"),
                                 _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


def mtp_verify_logits_noalloc(head: Head, hidden: torch.Tensor, k: int, draft_tokens: torch.Tensor, k_max: int,
                              smp: _Sampling, row_stats: torch.Tensor, logits: Optional[torch.Tensor],
                              stream=None) -> None:
    """mtp_verify_logits on the library's own per-device scratch: no workspace argument,
    nothing allocated (calls on one GPU must not overlap)."""
    lib = load_library()
    B = hidden.shape[0] if hidden.dim() == 3 else hidden.shape[0] // (k + 1)
    h = head._struct()
    _check(lib.mtp_verify_logits_noalloc(ctypes.byref(h), _ptr(hidden, name="hidden"), _htype(hidden), int(B),
                                         int(k), _ptr(draft_tokens, (torch.int32,), "draft_tokens"), int(k_max),
                                         ctypes.byref(smp), _ptr(row_stats, (torch.int32,), "row_stats"),
                                         _ptr(logits, (torch.float32,), "logits"), _stream(stream)))


def mtp_accept_sample(B: int, k: int, k_max: int, vocab: int, n_draft: int, smp: _Sampling,
                      draft_tokens: torch.Tensor, draft_stats: torch.Tensor, draft_logits: Optional[torch.Tensor],
                      row_stats: torch.Tensor, logits: Optional[torch.Tensor], out_tokens: torch.Tensor,
                      n_accept: torch.Tensor, n_emit: torch.Tensor, flags: torch.Tensor,
                      ws: Optional[torch.Tensor], stream=None, draft_row_of: Optional[torch.Tensor] = None) -> None:
    lib = load_library()
    _check(lib.mtp_accept_sample(int(B), int(k), int(k_max), int(vocab), int(n_draft), ctypes.byref(smp),
                                 _ptr(draft_tokens, (torch.int32,), "draft_tokens"),
                                 _ptr(draft_stats, (torch.int32,), "draft_stats"),
                                 _ptr(draft_logits, (torch.float32,), "draft_logits"),
                                 _ptr(row_stats, (torch.int32,), "row_stats"),
                                 _ptr(logits, (torch.float32,), "logits"),
                                 _ptr(draft_row_of, (torch.int32,), "draft_row_of"),
                                 _ptr(out_tokens, (torch.int32,), "out_tokens"),
                                 _ptr(n_accept, (torch.int32,), "n_accept"), _ptr(n_emit, (torch.int32,), "n_emit"),
                                 _ptr(flags, (torch.int32,), "flags"),
                                 _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(stream)))


def mtp_commit_state(B: int, k: int, n_accept: torch.Tensor, snapshots: Optional[torch.Tensor],
                     live: Optional[torch.Tensor], state_bytes: int, kv: Optional[torch.Tensor], n_layers: int,
                     max_rows: int, kv_row_bytes: int, kv_len: torch.Tensor, stream=None) -> None:
    lib = load_library()
    _check(lib.mtp_commit_state(int(B), int(k), _ptr(n_accept, (torch.int32,), "n_accept"),
                                _ptr(snapshots, name="snapshots"), _ptr(live, name="live"), int(state_bytes),
                                _ptr(kv, name="kv"), int(n_layers), int(max_rows), int(kv_row_bytes),
                                _ptr(kv_len, (torch.int32,), "kv_len"), _stream(stream)))


# ---------------------------------------------------------------------------------
# adaptive verify width (host side; same names as the C ABI's mtp_width_*)
# ---------------------------------------------------------------------------------
class WidthController:
    """One mtp_width_ctl: feed it each cycle's acceptance outputs and time, ask it for k."""

    def __init__(self, k_max: int = 7, decay: float = 0.1, alpha0: float = 0.8, slope_prior: float = 0.1):
        self._c = _WidthCtl()
        _check(load_library().mtp_width_init(ctypes.byref(self._c), int(k_max), float(decay), float(alpha0),
                                             float(slope_prior)))

    def observe(self, k: int, n_accept, flags, seconds: float) -> None:
        import numpy as np
        a = np.ascontiguousarray(np.asarray(n_accept.cpu() if hasattr(n_accept, "cpu") else n_accept, dtype=np.int32))
        f = np.ascontiguousarray(np.asarray(flags.cpu() if hasattr(flags, "cpu") else flags).astype(np.uint32))
        if a.shape != f.shape or a.ndim != 1:
            raise MtpError("n_accept and flags must be [B]")
        _check(load_library().mtp_width_observe(ctypes.byref(self._c), int(k), int(a.size), a.ctypes.data,
                                                f.ctypes.data, float(seconds)))

    def expected_tokens(self, k: int) -> float:
        return load_library().mtp_width_expected_tokens(ctypes.byref(self._c), int(k))

    def cost(self, k: int) -> float:
        return load_library().mtp_width_cost(ctypes.byref(self._c), int(k))

    def choose(self) -> int:
        return int(load_library().mtp_width_choose(ctypes.byref(self._c)))

    @property
    def alpha(self):
        return list(self._c.alpha)

    @property
    def weight(self):
        return list(self._c.weight)

    @property
    def counters(self) -> dict:
        c = self._c
        return dict(verifier_passes=c.verifier_passes, cycles=c.cycles, drafted=c.drafted, accepted=c.accepted,
                    depth_hist=list(c.depth_hist))
