"""ctypes binding of libtq.so (include/tq.h): argument marshalling only.

Every computation of the packed-key path runs in the HIP library; this module
only converts torch device tensors to raw pointers, checks return codes and
allocates caller-owned buffers with torch. If libtq.so is missing, importing
the binding raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_OK, TQ_ERR_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_DEVICE, TQ_ERR_WORKSPACE = 0, -1, -2, -3, -4
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_OP_ENCODE, TQ_OP_SCORE, TQ_OP_TOPK, TQ_OP_ATTEND = 0, 1, 2, 3
TQ_APPEND_PREPARED = 1


class TQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} -> {code} ({tq_status_string(code)})")
        self.code = code


class tq_params(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("m", ctypes.c_int32), ("n_groups", ctypes.c_int32),
        ("group_dim", ctypes.c_int32 * 2), ("group_bits", ctypes.c_int32 * 2),
        ("centroids", (ctypes.c_float * 16) * 2), ("thresholds", (ctypes.c_float * 15) * 2),
        ("group_chan", ctypes.c_void_p), ("rot", ctypes.c_void_p), ("proj", ctypes.c_void_p),
        ("norm_dtype", ctypes.c_int32),
    ]


class tq_bank(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("rnorms", ctypes.c_void_p)]


EXPORTS = ["tq_make_codebook", "tq_make_codebook_sphere", "tq_make_rotation", "tq_make_rotation_hadamard",
           "tq_bank_layout", "tq_workspace_bytes", "tq_encode", "tq_encode_append", "tq_encode_append_noalloc",
           "tq_prepare_queries",
           "tq_score_prepared", "tq_score", "tq_topk", "tq_decode", "tq_attend", "tq_fp32_logits", "tq_copy",
           "tq_status_string"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m kv_cache_inner_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER(tq_params)
    B = ctypes.POINTER(tq_bank)
    sig = {
        "tq_make_codebook": (ctypes.c_int, [ctypes.c_int, vp, vp, vp]),
        "tq_make_rotation": (ctypes.c_int, [ctypes.c_int, vp, vp]),
        "tq_make_codebook_sphere": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, vp, vp, vp]),
        "tq_make_rotation_hadamard": (ctypes.c_int, [ctypes.c_int, vp, vp]),
        "tq_bank_layout": (ctypes.c_int, [P, i64, vp, vp, vp]),
        "tq_workspace_bytes": (sz, [ctypes.c_int, P, i64, i64, i32, i32]),
        "tq_encode": (ctypes.c_int, [P, vp, ctypes.c_int, i64, i64, B, vp, sz, vp]),
        "tq_encode_append": (ctypes.c_int, [P, vp, ctypes.c_int, i64, i64, vp, i64, B, ctypes.c_int, vp, sz, vp]),
        "tq_encode_append_noalloc": (ctypes.c_int, [P, vp, ctypes.c_int, i64, i64, vp, i64, B, vp]),
        "tq_prepare_queries": (ctypes.c_int, [P, vp, i64, i32, vp, sz, vp]),
        "tq_score_prepared": (ctypes.c_int, [P, B, i64, i64, i32, vp, vp, vp]),
        "tq_score": (ctypes.c_int, [P, B, i64, i64, vp, i32, vp, vp, sz, vp]),
        "tq_topk": (ctypes.c_int, [P, B, i64, i64, vp, i32, i32, vp, vp, vp, sz, vp]),
        "tq_decode": (ctypes.c_int, [P, B, i64, i64, vp, vp]),
        "tq_attend": (ctypes.c_int, [P, B, P, B, i64, i64, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]),
        "tq_fp32_logits": (ctypes.c_int, [vp, i64, i64, i32, vp, i32, vp, vp]),
        "tq_copy": (ctypes.c_int, [vp, vp, sz, vp]),
        "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()


def lib():
    return _lib


def tq_status_string(code: int) -> str:
    return _lib.tq_status_string(code).decode()


def _check(fn: str, rc: int):
    if rc != TQ_OK:
        raise TQError(fn, rc)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Context in which the binding allocates a call's workspace and outputs: the launch
    stream, so that torch's caching allocator orders any later reuse of those blocks after
    the kernels that use them (a block freed on another stream could be handed out while
    the kernels still run)."""
    import contextlib

    import torch

    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


# ------------------------------------------------------------------------------------------
# host-only entry points
# ------------------------------------------------------------------------------------------

def tq_make_codebook(bits: int) -> Tuple[np.ndarray, np.ndarray, float]:
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(max(L - 1, 1), np.float32)
    mse = ctypes.c_double()
    _check("tq_make_codebook", _lib.tq_make_codebook(bits, c.ctypes.data, t.ctypes.data, ctypes.addressof(mse)))
    return c, t[: L - 1], mse.value


def tq_make_rotation(gauss: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(gauss, dtype=np.float32)
    d = g.shape[0]
    out = np.zeros((d, d), np.float32)
    _check("tq_make_rotation", _lib.tq_make_rotation(d, g.ctypes.data, out.ctypes.data))
    return out


def tq_make_codebook_sphere(bits: int, d: int) -> Tuple[np.ndarray, np.ndarray, float]:
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(max(L - 1, 1), np.float32)
    mse = ctypes.c_double()
    _check("tq_make_codebook_sphere", _lib.tq_make_codebook_sphere(bits, d, c.ctypes.data, t.ctypes.data,
                                                                   ctypes.addressof(mse)))
    return c, t[: L - 1], mse.value


def tq_make_rotation_hadamard(signs: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(signs, dtype=np.float32)
    d = s.shape[0]
    out = np.zeros((d, d), np.float32)
    _check("tq_make_rotation_hadamard", _lib.tq_make_rotation_hadamard(d, s.ctypes.data, out.ctypes.data))
    return out


class Params:
    """tq_params plus the device tensors it points to (kept alive here)."""

    def __init__(self, d: int, m: int, groups: Sequence[Tuple[int, int]], rot, proj, chan=None,
                 codebooks: Optional[List[Tuple[np.ndarray, np.ndarray]]] = None, norm16: bool = False):
        self.d, self.m = d, m
        self.norm16 = bool(norm16)
        self.groups = [(int(a), int(b)) for a, b in groups]
        self.rot, self.proj, self.chan = rot, proj, chan
        s = tq_params()
        s.d, s.m, s.n_groups = d, m, len(self.groups)
        self.codebooks = []
        for g, (dg, b) in enumerate(self.groups):
            s.group_dim[g], s.group_bits[g] = dg, b
            c, t = codebooks[g] if codebooks else tq_make_codebook(b)[:2]
            self.codebooks.append((c, t))
            for i, v in enumerate(c):
                s.centroids[g][i] = float(v)
            for i, v in enumerate(t):
                s.thresholds[g][i] = float(v)
        s.group_chan = _ptr(chan)
        s.rot, s.proj = _ptr(rot), _ptr(proj)
        s.norm_dtype = TQ_F16 if self.norm16 else TQ_F32
        self.struct = s

    @property
    def ref(self):
        return ctypes.byref(self.struct)

    @property
    def ng(self) -> int:
        return len(self.groups)

    def layout(self, n: int) -> Tuple[int, int, int]:
        w, npad, bpk = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check("tq_bank_layout", _lib.tq_bank_layout(self.ref, n, ctypes.addressof(w), ctypes.addressof(npad),
                                                     ctypes.addressof(bpk)))
        return w.value, npad.value, bpk.value

    def workspace_bytes(self, op: int, banks: int, n: int, G: int = 1, k: int = 1) -> int:
        return int(_lib.tq_workspace_bytes(op, self.ref, banks, n, G, k))


def make_params(d: int, m: int, groups: Sequence[Tuple[int, int]], gaussians: Sequence[np.ndarray], proj: np.ndarray,
                chan: Optional[np.ndarray] = None, device="cuda", rotations: Optional[Sequence[np.ndarray]] = None,
                codebooks: Optional[List[Tuple[np.ndarray, np.ndarray]]] = None, norm16: bool = False) -> Params:
    """Host construction of R (tq_make_rotation per group, unless explicit `rotations` are
    given) and the codebooks (tq_make_codebook unless `codebooks` are given), uploaded with
    S and the channel list. norm16: banks of these parameters store binary16 norms."""
    import torch

    rots = list(rotations) if rotations is not None else [tq_make_rotation(g) for g in gaussians]
    rot = torch.from_numpy(np.concatenate([r.ravel() for r in rots])).to(device)
    pj = None if proj is None else torch.from_numpy(np.ascontiguousarray(proj, dtype=np.float32)).to(device)
    ch = None if chan is None else torch.from_numpy(np.ascontiguousarray(chan, dtype=np.int32)).to(device)
    return Params(d, m, groups, rot, pj, ch, codebooks=codebooks, norm16=norm16)


class Bank:
    """Caller-owned device arrays of `banks` packed banks of n keys."""

    def __init__(self, params: Params, banks: int, n: int, device="cuda"):
        import torch

        W, npad, _ = params.layout(n)
        self.banks, self.n, self.n_pad, self.W = banks, n, npad, W
        self.bits = torch.zeros((banks, npad // 16, W, 16), dtype=torch.int32, device=device)
        nt = torch.float16 if params.norm16 else torch.float32
        self.norms = torch.zeros((banks, npad, params.ng), dtype=nt, device=device)
        self.rnorms = torch.zeros((banks, npad), dtype=nt, device=device)
        self.struct = tq_bank(self.bits.data_ptr(), self.norms.data_ptr(), self.rnorms.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def _workspace(nbytes: int, device):
    import torch

    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------
# device entry points (asynchronous on the current torch stream unless one is given; the
# workspace and outputs a call allocates itself are allocated on the launch stream)
# ------------------------------------------------------------------------------------------

def tq_encode(params: Params, keys, bank: Bank, workspace=None, stream=None):
    import torch

    assert keys.is_contiguous() and keys.dim() == 3 and keys.shape[2] == params.d
    dtype = TQ_BF16 if keys.dtype == torch.bfloat16 else TQ_F32
    assert keys.dtype in (torch.bfloat16, torch.float32)
    banks, n = keys.shape[0], keys.shape[1]
    ws_bytes = params.workspace_bytes(TQ_OP_ENCODE, banks, n)
    with _on(stream):
        ws = workspace if workspace is not None else _workspace(ws_bytes, keys.device)
    _check("tq_encode", _lib.tq_encode(params.ref, keys.data_ptr(), dtype, banks, n, bank.ref, ws.data_ptr(),
                                       ws.numel(), _stream(stream)))
    return bank


def tq_encode_append(params: Params, keys, bank: Bank, pos, workspace=None, prepared=False, stream=None):
    """Encodes keys [banks][count][d] into slots pos[b] .. pos[b] + count - 1 of each bank of
    `bank` (allocated for bank.n slots per bank); pos: device int32 tensor [banks].
    prepared=True: `workspace` already holds S' from an earlier encode with these params."""
    import torch

    assert keys.is_contiguous() and keys.dim() == 3 and keys.shape[2] == params.d
    assert keys.dtype in (torch.bfloat16, torch.float32)
    assert pos.dtype == torch.int32 and pos.is_contiguous() and pos.numel() == keys.shape[0] == bank.banks
    dtype = TQ_BF16 if keys.dtype == torch.bfloat16 else TQ_F32
    banks, count = keys.shape[0], keys.shape[1]
    ws_bytes = params.workspace_bytes(TQ_OP_ENCODE, banks, count)
    with _on(stream):
        ws = workspace if workspace is not None else _workspace(ws_bytes, keys.device)
    _check("tq_encode_append", _lib.tq_encode_append(params.ref, keys.data_ptr(), dtype, banks, count, pos.data_ptr(),
                                                     bank.n, bank.ref, TQ_APPEND_PREPARED if prepared else 0,
                                                     ws.data_ptr(), ws.numel(), _stream(stream)))
    return bank


def tq_encode_append_noalloc(params: Params, keys, bank: Bank, pos, stream=None):
    """tq_encode_append without a workspace: S' is formed in the library's own device array
    (d, m <= 128). Calls that overlap on one device race (they share that array)."""
    import torch

    assert keys.is_contiguous() and keys.dim() == 3 and keys.shape[2] == params.d
    assert keys.dtype in (torch.bfloat16, torch.float32)
    assert pos.dtype == torch.int32 and pos.is_contiguous() and pos.numel() == keys.shape[0] == bank.banks
    dtype = TQ_BF16 if keys.dtype == torch.bfloat16 else TQ_F32
    _check("tq_encode_append_noalloc", _lib.tq_encode_append_noalloc(params.ref, keys.data_ptr(), dtype, keys.shape[0],
                                                                     keys.shape[1], pos.data_ptr(), bank.n, bank.ref,
                                                                     _stream(stream)))
    return bank


def tq_prepare_queries(params: Params, q, workspace, stream=None):
    assert q.is_contiguous() and q.dim() == 3 and q.shape[2] == params.d
    _check("tq_prepare_queries", _lib.tq_prepare_queries(params.ref, q.data_ptr(), q.shape[0], q.shape[1],
                                                         workspace.data_ptr(), workspace.numel(), _stream(stream)))


def tq_score_prepared(params: Params, bank: Bank, G: int, workspace, scores, stream=None):
    _check("tq_score_prepared", _lib.tq_score_prepared(params.ref, bank.ref, bank.banks, bank.n, G,
                                                       workspace.data_ptr(), scores.data_ptr(), _stream(stream)))
    return scores


def score_workspace(params: Params, bank: Bank, G: int):
    return _workspace(params.workspace_bytes(TQ_OP_SCORE, bank.banks, bank.n, G), bank.bits.device)


def tq_score(params: Params, bank: Bank, q, scores=None, workspace=None, stream=None):
    import torch

    assert q.is_contiguous() and q.dim() == 3 and q.shape[0] == bank.banks and q.shape[2] == params.d
    G = q.shape[1]
    with _on(stream):
        if scores is None:
            scores = torch.empty((bank.banks, G, bank.n), dtype=torch.float32, device=q.device)
        ws = workspace if workspace is not None else score_workspace(params, bank, G)
    _check("tq_score", _lib.tq_score(params.ref, bank.ref, bank.banks, bank.n, q.data_ptr(), G, scores.data_ptr(),
                                     ws.data_ptr(), ws.numel(), _stream(stream)))
    return scores


def tq_topk(params: Params, bank: Bank, q, k: int, workspace=None, stream=None):
    import torch

    assert q.is_contiguous() and q.dim() == 3 and q.shape[0] == bank.banks and q.shape[2] == params.d
    G = q.shape[1]
    with _on(stream):
        vals = torch.empty((bank.banks, G, k), dtype=torch.float32, device=q.device)
        idx = torch.empty((bank.banks, G, k), dtype=torch.int32, device=q.device)
        ws = workspace if workspace is not None else _workspace(
            params.workspace_bytes(TQ_OP_TOPK, bank.banks, bank.n, G, k), q.device)
    _check("tq_topk", _lib.tq_topk(params.ref, bank.ref, bank.banks, bank.n, q.data_ptr(), G, k, vals.data_ptr(),
                                   idx.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    return vals, idx


def tq_decode(params: Params, bank: Bank, out=None, stream=None):
    """Stage-1 reconstruction x_hat [banks, n, d] (float32, channel order) of a packed bank."""
    import torch

    if out is None:
        with _on(stream):
            out = torch.empty((bank.banks, bank.n, params.d), dtype=torch.float32, device=bank.bits.device)
    _check("tq_decode", _lib.tq_decode(params.ref, bank.ref, bank.banks, bank.n, out.data_ptr(), _stream(stream)))
    return out


def attend_workspace(kparams: Params, bank: Bank, G: int):
    return _workspace(kparams.workspace_bytes(TQ_OP_ATTEND, bank.banks, bank.n, G), bank.bits.device)


def tq_attend(kparams: Params, kbank: Bank, vparams: Params, vbank: Bank, q, scale: float, lengths=None, out=None,
              workspace=None, stream=None):
    """Decode attention: softmax(scale * estimated logits) over the tokens of each bank,
    applied to the decompressed values. q [banks, G, d_k] -> out [banks, G, d_v].
    lengths: optional device int32 tensor [banks], the number of leading slots each bank
    attends over (default: all kbank.n)."""
    import torch

    assert q.is_contiguous() and q.dim() == 3 and q.shape[0] == kbank.banks and q.shape[2] == kparams.d
    assert vbank.banks == kbank.banks and vbank.n == kbank.n
    if lengths is not None:
        assert lengths.dtype == torch.int32 and lengths.is_contiguous() and lengths.numel() == kbank.banks
    G = q.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty((kbank.banks, G, vparams.d), dtype=torch.float32, device=q.device)
        ws = workspace if workspace is not None else attend_workspace(kparams, kbank, G)
    _check("tq_attend", _lib.tq_attend(kparams.ref, kbank.ref, vparams.ref, vbank.ref, kbank.banks, kbank.n,
                                       _ptr(lengths), q.data_ptr(), G, float(scale), out.data_ptr(), ws.data_ptr(),
                                       ws.numel(), _stream(stream)))
    return out


def tq_fp32_logits(keys, q, scores=None, stream=None):
    import torch

    banks, n, d = keys.shape
    G = q.shape[1]
    if scores is None:
        with _on(stream):
            scores = torch.empty((banks, G, n), dtype=torch.float32, device=keys.device)
    _check("tq_fp32_logits", _lib.tq_fp32_logits(keys.data_ptr(), banks, n, d, q.data_ptr(), G, scores.data_ptr(),
                                                 _stream(stream)))
    return scores


def tq_copy(src, dst, stream=None):
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    _check("tq_copy", _lib.tq_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream)))
