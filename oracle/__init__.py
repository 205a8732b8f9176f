"""TurboQuant CPU oracle (fp64) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``tq_oracle.c`` (plain C, fp64,
OpenMP over keys) through ctypes and shares no code with the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile the oracle with gcc (-O2, OpenMP). Returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-D_DEFAULT_SOURCE", "-Wall", "-shared", "-fPIC",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("m", ctypes.c_int), ("ng", ctypes.c_int),
                ("gdim", ctypes.c_int * 2), ("gbits", ctypes.c_int * 2),
                ("chan", ctypes.POINTER(ctypes.c_int)), ("norm16", ctypes.c_int)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def set_threads(n: int) -> int:
    """Threads of the oracle's OpenMP loops from now on; returns the previous count."""
    return int(lib().orc_set_threads(int(n)))


def _p(a: np.ndarray, ct=ctypes.c_void_p):
    return a.ctypes.data_as(ct)


class Spec:
    """Shape of one encoding: dimension d, sign-sketch rows m (0 = MSE-only),
    channel groups [(d_g, b_g)] with b_g the codebook bits of group g, and the
    channel list (group 0's channels then group 1's; None = identity). norm16: the
    format variant whose norms are stored at binary16 precision (the binary16 rounding of
    the float32 norm; the residual is taken against the reconstruction from that stored
    norm)."""

    def __init__(self, d: int, m: int, groups: Sequence[tuple], chan: Optional[np.ndarray] = None,
                 norm16: bool = False):
        self.d, self.m = d, m
        self.norm16 = bool(norm16)
        self.groups = [(int(a), int(b)) for a, b in groups]
        self.chan = None if chan is None else np.ascontiguousarray(chan, dtype=np.int32)
        c = _Cfg()
        c.d, c.m, c.ng = d, m, len(self.groups)
        for g, (dg, bg) in enumerate(self.groups):
            c.gdim[g], c.gbits[g] = dg, bg
        c.chan = _p(self.chan, ctypes.POINTER(ctypes.c_int)) if self.chan is not None else None
        c.norm16 = int(self.norm16)
        self._c = c

    @property
    def words(self) -> int:
        return self.m // 32 + sum(b * (dg // 32) for dg, b in self.groups)

    @property
    def ng(self) -> int:
        return len(self.groups)

    def ref(self):
        return ctypes.byref(self._c)


def codebook(bits: int):
    """Lloyd-Max for N(0,1): (centroids[2^b], thresholds[2^b - 1], mse, iterations)."""
    L = 1 << bits
    c = np.zeros(L, np.float64)
    t = np.zeros(max(L - 1, 1), np.float64)
    mse = ctypes.c_double()
    it = ctypes.c_int()
    rc = lib().orc_codebook(bits, _p(c), _p(t), ctypes.byref(mse), ctypes.byref(it))
    if rc:
        raise ValueError(f"orc_codebook({bits}) -> {rc}")
    return c, t[: L - 1], mse.value, it.value


def rotation(gauss: np.ndarray) -> np.ndarray:
    """Sign-fixed Householder Q of a square Gaussian matrix (fp64)."""
    g = np.ascontiguousarray(gauss, dtype=np.float32)
    d = g.shape[0]
    out = np.zeros((d, d), np.float64)
    if lib().orc_rotation(d, _p(g), _p(out)):
        raise ValueError("orc_rotation")
    return out


def codebook_sphere(bits: int, d: int, tol: float = 1e-14):
    """Lloyd-Max, in z units (z = sqrt(d) t), for one coordinate t of a uniformly random
    unit vector in R^d: t^2 ~ Beta(1/2, (d-1)/2), the law of a squared coordinate of a
    uniform point on the sphere (turboquant-pytorch write-up, stage 1: the codebook is fitted
    to the distribution of the rotated coordinates; its large-d limit is N(0,1)). Cell
    masses and moments from the regularised incomplete beta function, the Lloyd fixed
    point iterated on the positive half (the law is symmetric). Returns
    (centroids[2^b], thresholds[2^b - 1], mse)."""
    from scipy.special import betainc, betaln

    L, H = 1 << bits, 1 << (bits - 1)
    beta = 0.5 * (d - 1)
    top = np.sqrt(d)

    def moments(a, b):  # over a <= z <= b, z >= 0: mass, E[z 1], E[z^2 1]
        ua, ub = min(a * a / d, 1.0), min(b * b / d, 1.0)  # (sqrt(d))^2 / d may round above 1
        m0 = 0.5 * (betainc(0.5, beta, ub) - betainc(0.5, beta, ua))
        r1 = np.exp(betaln(1.0, beta) - betaln(0.5, beta))  # E[sqrt(u)] over the whole law
        m1 = 0.5 * np.sqrt(d) * r1 * (betainc(1.0, beta, ub) - betainc(1.0, beta, ua))
        m2 = 0.5 * (betainc(1.5, beta, ub) - betainc(1.5, beta, ua))  # E[z^2] = d E[u] = 1 overall
        return m0, m1, m2

    c = np.array([min(3.0, top) * (k + 0.5) / H for k in range(H)])
    for _ in range(1_000_000):
        t = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [top]])
        nc = np.array([moments(t[k], t[k + 1])[1] / moments(t[k], t[k + 1])[0] for k in range(H)])
        done = np.max(np.abs(nc - c)) < tol
        c = nc
        if done:
            break
    t = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [top]])
    mse = 0.0
    for k in range(H):
        m0, m1, m2 = moments(t[k], t[k + 1])
        mse += 2.0 * (m2 - 2.0 * c[k] * m1 + c[k] * c[k] * m0)
    cent = np.concatenate([-c[::-1], c])
    thr = np.concatenate([-t[1:H][::-1], [0.0], t[1:H]])
    return cent, thr, mse


def hadamard_rotation(signs: np.ndarray) -> np.ndarray:
    """Randomised Walsh-Hadamard rotation H_d diag(sign(s)) / sqrt(d), d a power of two,
    with H_d the Sylvester Hadamard matrix (tistory series part 11, on community GPU
    implementations: structured Walsh-Hadamard rotations). fp64."""
    from scipy.linalg import hadamard

    s = np.sign(np.asarray(signs, np.float64))
    d = s.shape[0]
    return hadamard(d).astype(np.float64) * s[None, :] / np.sqrt(d)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (butterflies)."""
    y = np.array(x, np.float64, copy=True)
    n, h = y.shape[-1], 1
    while h < n:
        y = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(*y.shape[:-3], n)
        h *= 2
    return y


class Params:
    """The oracle's own parameters: rotations from its own QR (or the given rotation
    matrices), codebooks from its own Lloyd-Max (or the given (centroids, thresholds) per
    group), the projection S as drawn (float32)."""

    def __init__(self, spec: Spec, gaussians: Sequence[np.ndarray], proj: Optional[np.ndarray],
                 rotations: Optional[Sequence[np.ndarray]] = None, codebooks: Optional[Sequence[tuple]] = None):
        self.spec = spec
        self.rots = ([np.asarray(r, np.float64) for r in rotations] if rotations is not None
                     else [rotation(g) for g in gaussians])
        self.rot = np.ascontiguousarray(np.concatenate([r.ravel() for r in self.rots]))
        m = spec.m
        self.proj = np.ascontiguousarray(proj, dtype=np.float32) if m > 0 else np.zeros((1, spec.d), np.float32)
        self.cent = np.zeros((2, 16), np.float64)
        self.thr = np.zeros((2, 15), np.float32)
        for g, (_, b) in enumerate(spec.groups):
            c, t = codebooks[g][:2] if codebooks is not None else codebook(b)[:2]
            self.cent[g, : len(c)] = c
            self.thr[g, : len(t)] = np.asarray(t, np.float64).astype(np.float32)


def n_pad(n: int) -> int:
    return 16 * ((n + 15) // 16)


def encode(prm: Params, keys: np.ndarray):
    """keys [n, d] float32 -> (bits [n_pad/16, W, 16] uint32, norms [n_pad, ng], rnorms [n_pad])."""
    sp = prm.spec
    k = np.ascontiguousarray(keys, dtype=np.float32)
    n = k.shape[0]
    npd = n_pad(n)
    bits = np.zeros((npd // 16, sp.words, 16), np.uint32)
    norms = np.zeros((npd, sp.ng), np.float32)
    rnorms = np.zeros(npd, np.float32)
    rc = lib().orc_encode(sp.ref(), _p(prm.rot), _p(prm.proj), _p(prm.cent), _p(prm.thr), _p(k),
                          ctypes.c_long(n), _p(bits), _p(norms), _p(rnorms))
    if rc:
        raise ValueError("orc_encode")
    return bits, norms, rnorms


def encode_trace(prm: Params, keys: np.ndarray):
    """encode() plus the fp64 values every decision was taken on: z [n, d] (group
    order, unit variance) and the sketch projections p [n, m]."""
    sp = prm.spec
    k = np.ascontiguousarray(keys, dtype=np.float32)
    n = k.shape[0]
    npd = n_pad(n)
    bits = np.zeros((npd // 16, sp.words, 16), np.uint32)
    norms = np.zeros((npd, sp.ng), np.float32)
    rnorms = np.zeros(npd, np.float32)
    z = np.zeros((n, sp.d), np.float64)
    p = np.zeros((n, max(sp.m, 1)), np.float64)
    rc = lib().orc_encode_trace(sp.ref(), _p(prm.rot), _p(prm.proj), _p(prm.cent), _p(prm.thr), _p(k),
                                ctypes.c_long(n), _p(bits), _p(norms), _p(rnorms), _p(z), _p(p))
    if rc:
        raise ValueError("orc_encode_trace")
    return bits, norms, rnorms, z, p[:, : sp.m]


def decode(prm: Params, bits: np.ndarray, norms: np.ndarray, n: int) -> np.ndarray:
    sp = prm.spec
    out = np.zeros((n, sp.d), np.float64)
    rc = lib().orc_decode(sp.ref(), _p(prm.rot), _p(prm.cent), _p(np.ascontiguousarray(bits, np.uint32)),
                          _p(np.ascontiguousarray(norms, np.float32)), ctypes.c_long(n), _p(out))
    if rc:
        raise ValueError("orc_decode")
    return out


def attend(kprm: Params, kbank, vprm: Params, vbank, n: int, q: np.ndarray, scale: float) -> np.ndarray:
    """Decode attention of queries q [G, d_k] over one bank of n stored tokens (fp64):
    out [G, d_v] = softmax(scale * est) @ xhat_v.

    turboquant-pytorch write-up (discuss.pytorch.kr), usage example and the two-stage
    section: the keys are held by the inner-product quantiser, whose estimates est =
    score(...) stand in for the logits q . k; the values are held by the MSE quantiser and
    enter through its decompression xhat_v = decode(...). The softmax and the weighted sum
    are the ordinary attention definition. kbank / vbank: (bits, norms, rnorms) of one bank."""
    s = score(kprm, kbank[0], kbank[1], kbank[2], n, q)
    v = decode(vprm, vbank[0], vbank[1], n)
    z = scale * s
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def unpack(spec: Spec, bits: np.ndarray, n: int):
    codes = np.zeros((n, spec.d), np.int32)
    signs = np.zeros((n, max(spec.m, 1)), np.uint8)
    if lib().orc_unpack(spec.ref(), _p(np.ascontiguousarray(bits, np.uint32)), ctypes.c_long(n), _p(codes), _p(signs)):
        raise ValueError("orc_unpack")
    return codes, signs[:, : spec.m]


def score(prm: Params, bits, norms, rnorms, n: int, q: np.ndarray) -> np.ndarray:
    """Estimated inner products [G, n] (fp64) of queries q [G, d] against one bank."""
    sp = prm.spec
    qq = np.ascontiguousarray(q, dtype=np.float32)
    G = qq.shape[0]
    out = np.zeros((G, n), np.float64)
    rc = lib().orc_score(sp.ref(), _p(prm.rot), _p(prm.proj), _p(prm.cent), _p(np.ascontiguousarray(bits, np.uint32)),
                         _p(np.ascontiguousarray(norms, np.float32)), _p(np.ascontiguousarray(rnorms, np.float32)),
                         ctypes.c_long(n), _p(qq), G, _p(out))
    if rc:
        raise ValueError("orc_score")
    return out


def score_pairs(prm: Params, bits, norms, rnorms, q: np.ndarray, qi: np.ndarray, ki: np.ndarray) -> np.ndarray:
    sp = prm.spec
    qq = np.ascontiguousarray(q, dtype=np.float32)
    qi = np.ascontiguousarray(qi, dtype=np.int32)
    ki = np.ascontiguousarray(ki, dtype=np.int64)
    out = np.zeros(len(qi), np.float64)
    rc = lib().orc_score_pairs(sp.ref(), _p(prm.rot), _p(prm.proj), _p(prm.cent),
                               _p(np.ascontiguousarray(bits, np.uint32)), _p(np.ascontiguousarray(norms, np.float32)),
                               _p(np.ascontiguousarray(rnorms, np.float32)), _p(qq), qq.shape[0], _p(qi), _p(ki),
                               ctypes.c_long(len(qi)), _p(out))
    if rc:
        raise ValueError("orc_score_pairs")
    return out


def topk(scores: np.ndarray, k: int):
    s = np.ascontiguousarray(scores, dtype=np.float64)
    G, n = s.shape
    vals = np.zeros((G, k), np.float64)
    idx = np.zeros((G, k), np.int64)
    if lib().orc_topk(_p(s), ctypes.c_long(n), G, k, _p(vals), _p(idx)):
        raise ValueError("orc_topk")
    return vals, idx


def lloyd_empirical(points: np.ndarray, L: int, start: np.ndarray, weights: Optional[np.ndarray] = None,
                    max_iter: int = 100000):
    """Lloyd iteration on a weighted empirical set: (centroids, thresholds, mse, iterations)."""
    pts = np.ascontiguousarray(points, dtype=np.float64)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float64)
    c = np.ascontiguousarray(start, dtype=np.float64).copy()
    t = np.zeros(max(L - 1, 1), np.float64)
    mse = ctypes.c_double()
    it = lib().orc_lloyd_empirical(_p(pts), _p(w) if w is not None else None, ctypes.c_long(len(pts)), L, _p(c), _p(t),
                                   ctypes.byref(mse), max_iter)
    if it < 0:
        raise ValueError("orc_lloyd_empirical")
    return c, t[: L - 1], mse.value, it


def bucketize(z: float, thresholds: np.ndarray) -> int:
    t = np.ascontiguousarray(thresholds, dtype=np.float32)
    lib().orc_bucketize.argtypes = [ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
    return lib().orc_bucketize(ctypes.c_float(z), _p(t), len(t) + 1)


def round_binary16(x: float) -> float:
    """The IEEE binary16 value nearest to the float32 x (ties to even), as a float."""
    f = lib().orc_round_binary16
    f.argtypes = [ctypes.c_float]
    f.restype = ctypes.c_float
    return float(f(ctypes.c_float(x)))
