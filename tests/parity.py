"""Helpers for the GPU-vs-oracle parity tests.

Both sides receive the same seeded inputs (keys, queries, the Gaussian matrices
the method draws). Each side builds its own parameters from them: the GPU path
through the library's host builders (tq_make_rotation / tq_make_codebook), the
oracle through its own QR and Lloyd-Max. Expected values come from the oracle
only.

Tolerances (decision band and score tolerance as the task fixes them; the
residual-norm tolerance derived from fp32 arithmetic):
  - codes: every GPU/oracle disagreement must lie within 1e-5 of a decision
    threshold in unit-variance z units, and at most 1e-4 of all coordinates
    may disagree;
  - signs (keys whose codes all agree): every disagreement must have
    |p_i| / rho < 1e-5, at most 1e-4 of all signs;
  - norms: |nu_gpu - nu| <= 1e-6 nu; residual norms (keys whose codes agree):
    |rho_gpu - rho| <= 1e-5 |x| + 1e-6 rho (fp32 MFMA rotation error bound);
  - binary16 norms: each side rounds its own float32 norm, and float32 norms 1e-6
    apart round apart only across a binary16 tie: such keys differ by one unit in
    the last place (2^-10 nu at most), at most 1e-3 of the keys, and are left out
    of the sign and residual checks (their reconstructions differ by that unit);
    residual norms of the other keys: |rho_gpu - rho| <= 1e-5 |x| + 2^-10 rho;
  - scores on identical bank bytes: |s_gpu - s| <= 1e-4 + 1e-3 |s|.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads

BAND = 1e-5
MAX_FLIP_FRAC = 1e-4
SCORE_ATOL, SCORE_RTOL = 1e-4, 1e-3


def tq_mod():
    import kv_cache_inner_amd as tq

    return tq


def groups_of(cfg: workloads.Config, bits: int):
    """(d_g, codebook bits) per group for total budget `bits` (the sign sketch takes 1)."""
    if cfg.groups is None:
        return [(cfg.d, bits - 1)]
    return [(dg, b - 1) for dg, b in cfg.groups]


def both_params(cfg: workloads.Config, bits: int, layer: int = 0, device="cuda", norm16: bool = False):
    tq = tq_mod()
    groups = groups_of(cfg, bits)
    chan = workloads.group_channels(cfg)
    gauss = workloads.rotation_gaussians(cfg.cfg_id, [g[0] for g in groups], layer)
    S = workloads.projection(cfg.cfg_id, cfg.m, cfg.d, layer)
    gpu = tq.make_params(cfg.d, cfg.m, groups, gauss, S, chan, device, norm16=norm16)
    orc = oracle.Params(oracle.Spec(cfg.d, cfg.m, groups, chan, norm16=norm16), gauss, S)
    return gpu, orc


def upload_bank(tq, gpu_params, bits, norms, rnorms, n, device="cuda"):
    """A device bank holding the given host arrays ([banks, ...] stacked)."""
    import torch

    banks = bits.shape[0]
    b = tq.Bank(gpu_params, banks, n, device)
    b.bits.copy_(torch.from_numpy(bits.view(np.int32)))
    b.norms.copy_(torch.from_numpy(norms))
    b.rnorms.copy_(torch.from_numpy(rnorms))
    return b


def download_bank(bank):
    return (bank.bits.cpu().numpy().view(np.uint32), bank.norms.cpu().numpy(), bank.rnorms.cpu().numpy())


def unpack(bits_tiles: np.ndarray, groups, m: int, n: int):
    """Bank tile array [n_pad/16, W, 16] -> codes [n, d] (group order), signs [n, m]."""
    W = bits_tiles.shape[1]
    words = bits_tiles.transpose(0, 2, 1).reshape(-1, W)[:n]
    flat = ((words[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(n, W * 32).astype(np.int32)
    codes, off = [], 0
    for dg, b in groups:
        idx = np.zeros((n, dg), np.int32)
        for p in range(b):
            idx |= flat[:, off + p * dg: off + (p + 1) * dg] << p
        codes.append(idx)
        off += b * dg
    return np.concatenate(codes, axis=1), flat[:, off: off + m]


def check_encode(gpu_bank, ref, orc: oracle.Params, n: int, report: dict = None):
    """gpu_bank: (bits, norms, rnorms) of ONE bank from the GPU; ref: oracle.encode_trace output."""
    spec = orc.spec
    gb, gn, gr = gpu_bank
    rb, rn, rr, z, p = ref
    cg, sg = unpack(gb, spec.groups, spec.m, n)
    cr, sr = unpack(rb, spec.groups, spec.m, n)
    # codes: disagreements only within the decision band
    rows = []
    for g, (dg, b) in enumerate(spec.groups):
        t = np.full(15, np.inf)
        t[: (1 << b) - 1] = orc.thr[g, : (1 << b) - 1]
        rows.append(np.repeat(t[None], dg, axis=0))
    thr = np.concatenate(rows, axis=0)  # [d, 15], unused slots at infinity
    mism = cg != cr
    nflip = int(mism.sum())
    if nflip:
        kk, jj = np.nonzero(mism)
        dist = np.abs(z[kk, jj][:, None] - thr[jj]).min(axis=1)
        assert (dist < BAND).all(), f"code flips outside the band: max dist {dist.max():.3e}"
        assert (np.abs(cg[kk, jj] - cr[kk, jj]) == 1).all()
    assert nflip <= MAX_FLIP_FRAC * cg.size + 1, f"{nflip} code flips of {cg.size}"
    clean = ~mism.any(axis=1)
    gn, gr = gn.astype(np.float32), gr.astype(np.float32)
    if spec.norm16:
        off = gn[:n] != rn[:n]
        assert (np.abs(gn[:n] - rn[:n]) <= 2.0 ** -10 * rn[:n]).all(), "binary16 norms beyond one unit"
        tie = off.any(axis=1)
        assert tie.sum() <= 1e-3 * n + 1, f"{int(tie.sum())} keys with differently rounded norms"
        clean &= ~tie
    # signs, on keys whose codes agree
    smis = (sg != sr) & clean[:, None]
    nsflip = int(smis.sum())
    if nsflip:
        kk, ii = np.nonzero(smis)
        rel = np.abs(p[kk, ii]) / np.maximum(rr[kk], 1e-30)
        assert (rel < BAND).all(), f"sign flips outside the band: max |p|/rho {rel.max():.3e}"
    assert nsflip <= MAX_FLIP_FRAC * sg.size + 1, f"{nsflip} sign flips of {sg.size}"
    # norms
    if not spec.norm16:
        np.testing.assert_allclose(gn[:n], rn[:n], rtol=1e-6, atol=0)
    xn = np.sqrt((rn[:n].astype(np.float64) ** 2).sum(axis=1))
    dr = np.abs(gr[:n].astype(np.float64) - rr[:n])
    tol = 1e-5 * xn + (2.0 ** -10 if spec.norm16 else 1e-6) * rr[:n]
    assert (dr[clean] <= tol[clean]).all(), f"rho off by {np.max(dr[clean] / np.maximum(xn[clean], 1e-30)):.3e} |x|"
    # padding slots: zero-vector encodings, identical bytes
    npad = gb.shape[0] * 16
    if npad > n:
        g_pad = gb.transpose(0, 2, 1).reshape(-1, gb.shape[1])[n:]
        r_pad = rb.transpose(0, 2, 1).reshape(-1, rb.shape[1])[n:]
        np.testing.assert_array_equal(g_pad, r_pad)
        assert (gn[n:] == 0).all() and (gr[n:] == 0).all()
    if report is not None:
        report["code_flips"] = report.get("code_flips", 0) + nflip
        report["sign_flips"] = report.get("sign_flips", 0) + nsflip
        report["coords"] = report.get("coords", 0) + cg.size
        report["signs"] = report.get("signs", 0) + sg.size
    return nflip, nsflip


def check_scores(got: np.ndarray, ref: np.ndarray, what: str = "scores"):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    tol = SCORE_ATOL + SCORE_RTOL * np.abs(ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} beyond tolerance; "
                           f"worst excess {np.max(err - tol):.3e}, max err {err.max():.3e}")
    return float(err.max())


def check_topk(vals: np.ndarray, idx: np.ndarray, ref: np.ndarray, k: int, what: str = "topk"):
    """Top-k protocol on one bank. vals/idx [G, k] from the GPU, ref [G, n] oracle
    estimates on the same bank bytes. Every returned index must be a true top-k member
    up to the score tolerance (oracle score >= s_k - tol(s_k), s_k the oracle's k-th best),
    every returned value must match the oracle's estimate for its index (score
    tolerance), and a list must be distinct indices, best first. Returns the fraction of
    returned indices that equal the oracle's own top-k (ties by lower index)."""
    G, n = ref.shape
    idx = np.asarray(idx, np.int64)
    vals = np.asarray(vals, np.float64)
    assert idx.shape == (G, k) and vals.shape == (G, k)
    assert ((idx >= 0) & (idx < n)).all(), f"{what}: index out of range"
    order = np.lexsort((np.arange(n)[None, :].repeat(G, 0), -ref), axis=1)[:, :k]
    sk = np.take_along_axis(ref, order[:, k - 1:k], axis=1)
    got_ref = np.take_along_axis(ref, idx, axis=1)
    tol_k = SCORE_ATOL + SCORE_RTOL * np.abs(sk)
    assert (got_ref >= sk - tol_k).all(), (f"{what}: returned index below the k-th best by "
                                           f"{np.max(sk - tol_k - got_ref):.3e}")
    check_scores(vals, got_ref, f"{what} values")
    for g in range(G):
        assert len(set(idx[g].tolist())) == k, f"{what}: repeated index in query {g}"
    assert (np.diff(vals, axis=1) <= 0).all(), f"{what}: list not best first"
    same = np.mean([len(set(idx[g].tolist()) & set(order[g].tolist())) / k for g in range(G)])
    return float(same)
