"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test here checks the oracle against something other than itself: closed
forms, a textbook table, direct numerical minimisation, brute force on tiny
inputs, the statistics the method guarantees (unbiasedness, the closed-form
variance of the sign sketch, the 2/pi shrinkage of an MSE-only 1-bit
quantiser), the 3-bit distortion the turboquant-pytorch write-up reports, and
hand-built inputs whose encoding is known bit by bit.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import integrate, optimize, stats

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------
# codebook (Lloyd-Max for N(0,1))
# ------------------------------------------------------------------------------------

def test_codebook_one_bit_closed_form():
    c, t, mse, _ = oracle.codebook(1)
    a = math.sqrt(2 / math.pi)  # E|X| for X ~ N(0,1)
    np.testing.assert_allclose(c, [-a, a], rtol=0, atol=1e-14)
    assert t[0] == 0.0
    assert abs(mse - (1 - 2 / math.pi)) < 1e-14


def _read_max_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "gaussian_lloyd_max_max1960.txt")):
        if line.startswith("#") or not line.strip():
            continue
        L, c, t, mse = [f.strip() for f in line.split("|")]
        rows[int(L)] = ([float(v) for v in c.split()], [] if t == "-" else [float(v) for v in t.split()], float(mse))
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_textbook_table(bits):
    L = 1 << bits
    cpos, tpos, mse_tab = _read_max_table()[L]
    c, t, mse, _ = oracle.codebook(bits)
    np.testing.assert_allclose(c[L // 2:], cpos, atol=1.5e-3)
    np.testing.assert_allclose(t[L // 2:], tpos, atol=1.5e-3)
    assert abs(mse - mse_tab) / mse_tab < 0.05


def _cond_mean(a, b):
    m0 = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
    m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    return m1 / m0


def _mse_of_thresholds(tpos):
    """MSE of the symmetric quantizer with positive thresholds tpos (0 is always a
    threshold for an even level count), each cell represented by its conditional
    mean; integrals by adaptive quadrature (no closed form)."""
    edges = [0.0] + list(tpos) + [np.inf]
    tot = 0.0
    for a, b in zip(edges[:-1], edges[1:]):
        c = _cond_mean(a, b)
        tot += integrate.quad(lambda x: (x - c) ** 2 * stats.norm.pdf(x), a, b, epsabs=1e-14, epsrel=1e-12)[0]
    return 2 * tot


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_is_the_direct_minimiser(bits):
    """Minimise the quadrature MSE over the free thresholds directly (no Lloyd
    iteration involved) and compare with the oracle's fixed point."""
    L = 1 << bits
    c, t, mse, _ = oracle.codebook(bits)
    x0 = t[L // 2:] * (1 + 0.03 * np.linspace(-1, 1, L // 2 - 1))  # perturbed start
    if L == 4:
        r = optimize.minimize_scalar(lambda v: _mse_of_thresholds([v]), bounds=(0.5, 1.5), method="bounded",
                                     options={"xatol": 1e-10})
        tbest = np.array([r.x])
    else:
        r = optimize.minimize(lambda v: _mse_of_thresholds(np.sort(v)), x0, method="Nelder-Mead",
                              options={"xatol": 1e-9, "fatol": 1e-15, "maxiter": 20000})
        tbest = np.sort(r.x)
    np.testing.assert_allclose(tbest, t[L // 2:], atol=2e-4)
    assert abs(_mse_of_thresholds(tbest) - mse) < 1e-9


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_fixed_point_conditions(bits):
    """Centroid = conditional mean of its cell (by quadrature); threshold = midpoint."""
    L = 1 << bits
    c, t, _, _ = oracle.codebook(bits)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(L):
        assert abs(_cond_mean(edges[k], edges[k + 1]) - c[k]) < 1e-10
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    np.testing.assert_array_equal(c, -c[::-1])  # symmetric, middle threshold exactly 0


def _brute_force_partition(x, L):
    """Global optimum of the L-cell quantizer of a tiny sorted set: exhaustive
    over contiguous partitions."""
    n = len(x)
    best = (np.inf, None)
    for cuts in itertools.combinations(range(1, n), L - 1):
        parts = np.split(x, cuts)
        sse = sum(((p - p.mean()) ** 2).sum() for p in parts)
        if sse < best[0]:
            best = (sse, np.array([p.mean() for p in parts]))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_lloyd_brute_force_tiny_sets(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(5, 11))
    L = int(g.integers(2, 5))
    x = np.sort(g.standard_normal(n) * g.uniform(0.5, 2.0))
    sse, cents = _brute_force_partition(x, L)
    # the optimum is a fixed point of the iteration
    c, t, mse, it = oracle.lloyd_empirical(x, L, cents)
    np.testing.assert_allclose(c, cents, atol=1e-12)
    assert abs(mse - sse) < 1e-10
    # from a generic start the iteration reaches a fixed point no better than the optimum
    c2, t2, mse2, _ = oracle.lloyd_empirical(x, L, np.linspace(x[0], x[-1], L))
    assert mse2 >= sse - 1e-10
    for k in range(L):
        lo = -np.inf if k == 0 else t2[k - 1]
        hi = np.inf if k == L - 1 else t2[k]
        cell = x[(x >= lo) & (x < hi)]
        if len(cell):
            assert abs(cell.mean() - c2[k]) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_bucketize_is_nearest_centroid(bits):
    """Thresholds are midpoints, so the bucket is the nearest centroid; exhaustive
    over the float32 neighbours of every threshold, plus random draws."""
    c, t, _, _ = oracle.codebook(bits)
    tf = t.astype(np.float32)
    zs = []
    for tau in tf:
        v = np.float32(tau)
        zs.append(v)
        up, dn = v, v
        for _ in range(4):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            zs += [up, dn]
    zs += list(np.random.default_rng(0).standard_normal(2000).astype(np.float32) * 1.5)
    for z in zs:
        k = oracle.bucketize(float(z), tf)
        if np.any(tf == z):   # exactly on a float32 threshold: ties go up
            assert k == int(np.nonzero(tf == z)[0][0]) + 1
        else:
            dist = np.abs(float(z) - c)
            order = np.argsort(dist)
            if dist[order[1]] - dist[order[0]] > 1e-12:
                assert k == int(order[0])
            else:  # equidistant in fp64 arithmetic (z within ~1e-12 of a midpoint)
                assert k in (int(order[0]), int(order[1]))


# ------------------------------------------------------------------------------------
# rotation
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("d", [32, 96, 128, 768])
def test_rotation_is_sign_fixed_q_factor(d):
    G = np.random.default_rng(d).standard_normal((d, d)).astype(np.float32)
    R = oracle.rotation(G)
    assert np.abs(R @ R.T - np.eye(d)).max() < 1e-12
    T = R.T @ G.astype(np.float64)          # the triangular factor
    assert np.abs(np.tril(T, -1)).max() < 1e-10 * np.abs(T).max()
    assert (np.diag(T) > 0).all()
    # the same unique factor as a library QR with the signs fixed
    Q, Rq = np.linalg.qr(G.astype(np.float64))
    assert np.abs(Q * np.sign(np.diag(Rq)) - R).max() < 1e-10


def _perm_upper(d, seed):
    """G = P U with P a permutation (not an involution) and U upper triangular with a
    positive diagonal: its sign-fixed Q factor is exactly P."""
    g = np.random.default_rng(seed)
    perm = np.roll(np.arange(d), 1 + seed % (d - 1))
    P = np.eye(d)[perm]               # P[j, perm[j]] = 1
    U = np.triu(g.uniform(-1, 1, (d, d)))
    np.fill_diagonal(U, g.uniform(0.5, 2.0, d))
    return (P @ U).astype(np.float32), P, perm


def test_rotation_of_permuted_triangular_is_the_permutation():
    Gm, P, _ = _perm_upper(64, 5)
    R = oracle.rotation(Gm)
    assert np.abs(R - P).max() < 1e-12


# ------------------------------------------------------------------------------------
# packed format and encode, on inputs whose encoding is known bit by bit
# ------------------------------------------------------------------------------------

def _half_odd_key(d, seed):
    """A key of +-0.5 / +-1.5 entries with sum of squares exactly d, so that with an
    identity rotation z = sqrt(d) x / |x| = x exactly."""
    g = np.random.default_rng(seed)
    n1 = 5 * d // 8   # 0.25*n1 + 2.25*(d-n1) = d
    mag = np.array([0.5] * n1 + [1.5] * (d - n1))
    g.shuffle(mag)
    return (mag * g.choice([-1.0, 1.0], d)).astype(np.float32)


def _identity_gauss(d, seed=0):
    g = np.random.default_rng(seed)
    U = np.triu(g.uniform(-1, 1, (d, d)))
    np.fill_diagonal(U, g.uniform(0.5, 2.0, d))
    return U.astype(np.float32)


def test_format_bit_positions_and_zero_padding():
    d = m = 64
    spec = oracle.Spec(d, m, [(d, 2)])
    prm = oracle.Params(spec, [_identity_gauss(d)], np.eye(m, d, dtype=np.float32))
    assert np.abs(prm.rots[0] - np.eye(d)).max() < 1e-14
    keys = np.zeros((7, d), np.float32)
    x = _half_odd_key(d, 1)
    keys[5] = x
    bits, norms, rnorms = oracle.encode(prm, keys)
    assert bits.shape == (1, 2 * 2 + 2, 16)
    c = prm.cent[0, :4]
    # expected bucket per coordinate: thresholds are -0.98, 0, 0.98
    idx = np.where(x < -1, 0, np.where(x < 0, 1, np.where(x < 1, 2, 3)))
    resid = x - c[idx]                 # |x| = 8 = sqrt(d): xhat = c[idx] exactly scaled by 1
    sgn = (resid >= 0).astype(np.uint32)
    for j in range(d):
        for p in range(2):
            assert (bits[0, p * 2 + j // 32, 5] >> (j % 32)) & 1 == (idx[j] >> p) & 1
        assert (bits[0, 4 + j // 32, 5] >> (j % 32)) & 1 == sgn[j]
    assert norms[5, 0] == 8.0
    assert abs(rnorms[5] - np.linalg.norm(resid)) < 1e-6
    # zero-vector slots (keys 0..4, 6 and padding 7..15): bucket L/2 = 2, all signs +
    for i in list(range(5)) + list(range(6, 16)):
        assert list(bits[0, :, i]) == [0, 0, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF]
        assert norms[i, 0] == 0.0 and rnorms[i] == 0.0


def test_rotation_convention_row_j_gives_coordinate_j():
    """z_j = <R[j,:], x>: with R = P, coordinate j is x[perm[j]] (a transposed
    rotation would read x[perm^-1[j]])."""
    d = 64
    Gm, P, perm = _perm_upper(d, 7)
    spec = oracle.Spec(d, 0, [(d, 2)])
    prm = oracle.Params(spec, [Gm], None)
    x = _half_odd_key(d, 3)
    bits, _, _ = oracle.encode(prm, x[None])
    codes, _ = oracle.unpack(spec, bits, 1)
    z = x[perm]
    want = np.where(z < -1, 0, np.where(z < 0, 1, np.where(z < 1, 2, 3)))
    np.testing.assert_array_equal(codes[0], want)


def test_two_groups_follow_the_channel_list():
    d = 64
    chan = np.random.default_rng(2).permutation(d).astype(np.int32)
    spec = oracle.Spec(d, 0, [(32, 2), (32, 1)], chan)
    prm = oracle.Params(spec, [_identity_gauss(32, 1), _identity_gauss(32, 2)], None)
    x = np.zeros(d, np.float32)
    x[chan[:32]] = _half_odd_key(32, 4)
    x[chan[32:]] = _half_odd_key(32, 5)
    bits, norms, _ = oracle.encode(prm, x[None])
    codes, _ = oracle.unpack(spec, bits, 1)
    z0, z1 = x[chan[:32]], x[chan[32:]]
    np.testing.assert_array_equal(codes[0, :32], np.where(z0 < -1, 0, np.where(z0 < 0, 1, np.where(z0 < 1, 2, 3))))
    np.testing.assert_array_equal(codes[0, 32:], (z1 >= 0).astype(int))
    np.testing.assert_allclose(norms[0], [math.sqrt(32)] * 2, rtol=1e-7)


# ------------------------------------------------------------------------------------
# consistency of the stages with the decoder (random small shapes)
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_residual_signs_and_norms_are_those_of_the_decoder(seed):
    g = np.random.default_rng(100 + seed)
    d = int(g.choice([32, 64, 96, 128]))
    m = int(g.choice([32, 128]))
    b = int(g.integers(1, 4))
    spec = oracle.Spec(d, m, [(d, b)])
    S = g.standard_normal((m, d)).astype(np.float32)
    prm = oracle.Params(spec, [g.standard_normal((d, d)).astype(np.float32)], S)
    x = (g.standard_normal((40, d)) * g.uniform(0.1, 5, (40, 1))).astype(np.float32)
    bits, norms, rnorms = oracle.encode(prm, x)
    xhat = oracle.decode(prm, bits, norms, 40)
    r = x.astype(np.float64) - xhat
    np.testing.assert_allclose(rnorms[:40], np.linalg.norm(r, axis=1), rtol=1e-6)
    np.testing.assert_allclose(norms[:40, 0], np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-7)
    _, signs = oracle.unpack(spec, bits, 40)
    p = r @ S.astype(np.float64).T
    clear = np.abs(p) > 1e-9 * np.abs(p).max()
    np.testing.assert_array_equal(signs[clear], (p[clear] >= 0).astype(np.uint8))
    # MSE-only scores are exactly <q, decode(x)>
    spec0 = oracle.Spec(d, 0, [(d, b)])
    prm0 = oracle.Params(spec0, [g.standard_normal((d, d)).astype(np.float32)], None)
    b0, n0, r0 = oracle.encode(prm0, x)
    q = g.standard_normal((3, d)).astype(np.float32)
    s0 = oracle.score(prm0, b0, n0, r0, 40, q)
    ref = q.astype(np.float64) @ oracle.decode(prm0, b0, n0, 40).T
    np.testing.assert_allclose(s0, ref, rtol=1e-11, atol=1e-11)


def test_binary16_rounding_is_the_ieee_nearest_value():
    # against numpy's float16 conversion (an independent implementation of IEEE 754
    # round-to-nearest-even), over many binades, the subnormal range, ties and overflow
    g = np.random.default_rng(77)
    x = (g.standard_normal(20000) * 10.0 ** g.integers(-9, 5, 20000)).astype(np.float32)
    edge = np.float32([0.0, 65504.0, 65519.0, 65520.0, 65536.0, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25,
                       1.5 * 2.0 ** -25, 1e-9, -3.5, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2049.0, 2051.0])
    for v in np.concatenate([x, edge]):
        with np.errstate(over="ignore"):
            ref = float(np.float16(v))
        assert oracle.round_binary16(float(v)) == ref, v


@pytest.mark.parametrize("seed", range(4))
def test_binary16_norm_variant_stores_rounded_norms_and_corrects_their_reconstruction(seed):
    # the format variant: stored norms are the binary16 roundings of the float32 norms; the
    # codes are those of the float32 format; the residual (its norm and its signs) is the one
    # left by the reconstruction from the stored bytes
    g = np.random.default_rng(300 + seed)
    d = int(g.choice([64, 128]))
    m = int(g.choice([32, 128]))
    b = int(g.integers(1, 4))
    G = g.standard_normal((d, d)).astype(np.float32)
    S = g.standard_normal((m, d)).astype(np.float32)
    x = (g.standard_normal((40, d)) * g.uniform(0.01, 50, (40, 1))).astype(np.float32)
    spec32 = oracle.Spec(d, m, [(d, b)])
    spec16 = oracle.Spec(d, m, [(d, b)], norm16=True)
    b32, n32, _ = oracle.encode(oracle.Params(spec32, [G], S), x)
    prm = oracle.Params(spec16, [G], S)
    bits, norms, rnorms = oracle.encode(prm, x)
    np.testing.assert_array_equal(norms, n32.astype(np.float16).astype(np.float32))
    np.testing.assert_array_equal(norms[:40, 0],
                                  np.linalg.norm(x.astype(np.float64), axis=1).astype(np.float32)
                                  .astype(np.float16).astype(np.float32))
    codes32, _ = oracle.unpack(spec32, b32, 40)
    codes16, signs = oracle.unpack(spec16, bits, 40)
    np.testing.assert_array_equal(codes16, codes32)
    r = x.astype(np.float64) - oracle.decode(prm, bits, norms, 40)
    rho16 = np.linalg.norm(r, axis=1).astype(np.float32).astype(np.float16).astype(np.float32)
    assert np.abs(rnorms[:40] - rho16).max() <= 2.0 ** -10 * rho16.max()
    assert (rnorms[:40] == rho16).mean() > 0.9
    p = r @ S.astype(np.float64).T
    clear = np.abs(p) > 1e-9 * np.abs(p).max()
    np.testing.assert_array_equal(signs[clear], (p[clear] >= 0).astype(np.uint8))


def test_zero_key_contributes_nothing():
    spec = oracle.Spec(128, 128, [(128, 3)])
    g = np.random.default_rng(9)
    prm = oracle.Params(spec, [g.standard_normal((128, 128)).astype(np.float32)],
                        g.standard_normal((128, 128)).astype(np.float32))
    bits, norms, rnorms = oracle.encode(prm, np.zeros((1, 128), np.float32))
    codes, signs = oracle.unpack(spec, bits, 1)
    assert (codes == 4).all() and (signs == 1).all() and norms[0, 0] == 0 and rnorms[0] == 0
    assert oracle.score(prm, bits, norms, rnorms, 1, g.standard_normal((2, 128)).astype(np.float32)).tolist() == [[0.0], [0.0]]


# ------------------------------------------------------------------------------------
# two permuted channel groups (tambur.pub article: mixed bit widths per channel, the
# 3.5 / 2.5 bits-per-channel paragraph), and the pair scorer the full-size checks use
# ------------------------------------------------------------------------------------

def _np_unpack(spec, bits, n):
    """Bucket indices [n, d] (group order) and sign bits [n, m] read straight from the
    packed words with numpy: key i is lane i % 16 of tile i // 16; for group g the
    plane-p word of coordinate j is word0_g + p * d_g / 32 + j // 32, bit j % 32; the
    sign words follow the code words."""
    b = np.asarray(bits, np.uint32)
    keys = np.arange(n)
    tile, lane = keys // 16, keys % 16
    codes = np.zeros((n, spec.d), np.int64)
    off = word0 = 0
    for dg, bg in spec.groups:
        for j in range(dg):
            for p in range(bg):
                w = b[tile, word0 + p * (dg // 32) + j // 32, lane]
                codes[:, off + j] |= ((w >> np.uint32(j % 32)) & np.uint32(1)).astype(np.int64) << p
        word0 += bg * (dg // 32)
        off += dg
    signs = np.zeros((n, spec.m), np.uint8)
    for i in range(spec.m):
        w = b[tile, word0 + i // 32, lane]
        signs[:, i] = (w >> np.uint32(i % 32)) & np.uint32(1)
    return codes, signs


def _longctx_split(seed, m=128, d0=32, b0=2, d1=96, b1=1):
    """Parameters of the long-context layout (32 channels with a 2-bit codebook, 96 with
    a 1-bit one, one sign sketch over all 128) on a random channel permutation."""
    g = np.random.default_rng(seed)
    d = d0 + d1
    chan = g.permutation(d).astype(np.int32)
    spec = oracle.Spec(d, m, [(d0, b0), (d1, b1)], chan)
    gs = [g.standard_normal((d0, d0)).astype(np.float32), g.standard_normal((d1, d1)).astype(np.float32)]
    S = g.standard_normal((max(m, 1), d)).astype(np.float32) if m else None
    return spec, gs, S, chan, g


def _np_decode(prm, codes, norms, chan):
    """x_hat in channel order: group g's (nu_g / sqrt(d_g)) R_g^T c_g[idx_g] scattered to
    the channels the list gives that group (numpy, from the pinned rotation and codebook)."""
    n = codes.shape[0]
    d = prm.spec.d
    out = np.zeros((n, d))
    off = 0
    for gi, (dg, bg) in enumerate(prm.spec.groups):
        c = oracle.codebook(bg)[0]
        R = prm.rots[gi]
        yhat = c[codes[:, off:off + dg]]                      # [n, d_g] rotated reconstruction
        xg = (yhat @ R) * (norms[:n, gi].astype(np.float64) / math.sqrt(dg))[:, None]
        out[:, chan[off:off + dg]] = xg
        off += dg
    return out


@pytest.mark.parametrize("seed", range(3))
def test_two_group_decode_is_the_scatter_of_each_groups_reconstruction(seed):
    spec, gs, S, chan, g = _longctx_split(40 + seed)
    prm = oracle.Params(spec, gs, S)
    n = 37
    x = (g.standard_normal((n, spec.d)) * g.uniform(0.2, 4, (n, 1))).astype(np.float32)
    x[:, chan[:32]] *= 8.0                                    # outlier group, as in the workload
    bits, norms, rnorms = oracle.encode(prm, x)
    codes, signs = _np_unpack(spec, bits, n)
    c2, s2 = oracle.unpack(spec, bits, n)
    np.testing.assert_array_equal(codes, c2)
    np.testing.assert_array_equal(signs, s2)
    # norms per group over the channels the list assigns it
    xd = x.astype(np.float64)
    np.testing.assert_allclose(norms[:n, 0], np.linalg.norm(xd[:, chan[:32]], axis=1), rtol=1e-7)
    np.testing.assert_allclose(norms[:n, 1], np.linalg.norm(xd[:, chan[32:]], axis=1), rtol=1e-7)
    # codes: nearest centroid of the unit-variance rotated coordinates of each group
    off = 0
    for gi, (dg, bg) in enumerate(spec.groups):
        z = math.sqrt(dg) * (xd[:, chan[off:off + dg]] @ prm.rots[gi].T) / np.linalg.norm(
            xd[:, chan[off:off + dg]], axis=1, keepdims=True)
        c = oracle.codebook(bg)[0]
        near = np.argmin(np.abs(z[..., None] - c), axis=-1)
        clear = np.min(np.abs(z[..., None] - oracle.codebook(bg)[1]), axis=-1) > 1e-9 if bg > 0 else True
        np.testing.assert_array_equal(codes[:, off:off + dg][clear], near[clear])
        off += dg
    # decode against the numpy scatter
    np.testing.assert_allclose(oracle.decode(prm, bits, norms, n), _np_decode(prm, codes, norms, chan),
                               rtol=0, atol=1e-12 * np.abs(xd).max())
    # the residual: its norm and signs are those of x - decode(bytes), S in channel order
    r = xd - _np_decode(prm, codes, norms, chan)
    np.testing.assert_allclose(rnorms[:n], np.linalg.norm(r, axis=1), rtol=1e-6)
    p = r @ S.astype(np.float64).T
    clear = np.abs(p) > 1e-9 * np.abs(p).max()
    np.testing.assert_array_equal(signs[clear], (p[clear] >= 0).astype(np.uint8))


def test_two_group_encoding_is_equivariant_under_channel_relabelling():
    """Encoding x with channel list chan equals encoding x[chan] (groups now contiguous)
    with the identity list and S's columns taken in the same order: a scatter through the
    inverse list, or a residual or projection in the wrong channel order, breaks it."""
    spec, gs, S, chan, g = _longctx_split(47)
    n = 50
    x = g.standard_normal((n, spec.d)).astype(np.float32)
    b1, n1, r1, z1, p1 = oracle.encode_trace(oracle.Params(spec, gs, S), x)
    spec_id = oracle.Spec(spec.d, spec.m, spec.groups, None)
    b2, n2, r2, z2, p2 = oracle.encode_trace(oracle.Params(spec_id, gs, np.ascontiguousarray(S[:, chan])),
                                             np.ascontiguousarray(x[:, chan]))
    c1, s1 = oracle.unpack(spec, b1, n)
    c2, s2 = oracle.unpack(spec_id, b2, n)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(n1, n2)
    np.testing.assert_allclose(z1, z2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r1, r2, rtol=1e-7)
    np.testing.assert_allclose(p1, p2, rtol=0, atol=1e-10 * np.abs(p1).max())
    clear = np.abs(p1) > 1e-9 * np.abs(p1).max()
    np.testing.assert_array_equal(s1[clear], s2[clear])
    # and the relabelled list does matter: the identity list on the unpermuted keys differs
    b3, _, _ = oracle.encode(oracle.Params(spec_id, gs, S), x)
    assert (oracle.unpack(spec_id, b3, n)[0] != c1).any()


@pytest.mark.parametrize("seed", range(3))
def test_two_group_mse_only_score_is_the_inner_product_with_the_decode(seed):
    spec, gs, _, chan, g = _longctx_split(60 + seed, m=0)
    prm = oracle.Params(spec, gs, None)
    n = 41
    x = g.standard_normal((n, spec.d)).astype(np.float32)
    bits, norms, rnorms = oracle.encode(prm, x)
    q = g.standard_normal((5, spec.d)).astype(np.float32)
    codes, _ = _np_unpack(spec, bits, n)
    ref = q.astype(np.float64) @ _np_decode(prm, codes, norms, chan).T
    np.testing.assert_allclose(oracle.score(prm, bits, norms, rnorms, n, q), ref, rtol=1e-11, atol=1e-11)


def test_two_group_sketch_term_is_the_signed_projection_sum():
    """est - <q, x_hat> is sqrt(pi/2)/m * rho * <S q, 2 s - 1> with S q taken over the
    original channel order (a query read in group order would differ)."""
    spec, gs, S, chan, g = _longctx_split(70, m=64)
    prm = oracle.Params(spec, gs, S)
    n = 23
    x = g.standard_normal((n, spec.d)).astype(np.float32)
    bits, norms, rnorms = oracle.encode(prm, x)
    q = g.standard_normal((3, spec.d)).astype(np.float32)
    codes, signs = _np_unpack(spec, bits, n)
    qd = q.astype(np.float64)
    mse = qd @ _np_decode(prm, codes, norms, chan).T
    qs = qd @ S.astype(np.float64).T                                     # [G, m]
    sk = math.sqrt(math.pi / 2) / spec.m * rnorms[:n].astype(np.float64) * (qs @ (2.0 * signs - 1).T)
    np.testing.assert_allclose(oracle.score(prm, bits, norms, rnorms, n, q), mse + sk, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("two_groups", [False, True])
def test_score_pairs_is_the_score_matrix_entry(two_groups):
    """The pair scorer (used by the full-size checks) returns score[qi, ki] exactly, with
    m different from d so that an offset by d instead of m in the projected query shows."""
    g = np.random.default_rng(80 + two_groups)
    if two_groups:
        spec, gs, S, chan, _ = _longctx_split(81, m=96)
    else:
        spec = oracle.Spec(64, 160, [(64, 3)])
        gs, S = [g.standard_normal((64, 64)).astype(np.float32)], g.standard_normal((160, 64)).astype(np.float32)
    prm = oracle.Params(spec, gs, S)
    n, G = 45, 7
    x = g.standard_normal((n, spec.d)).astype(np.float32)
    bits, norms, rnorms = oracle.encode(prm, x)
    q = g.standard_normal((G, spec.d)).astype(np.float32)
    full = oracle.score(prm, bits, norms, rnorms, n, q)
    qi = g.integers(0, G, 400)
    ki = g.integers(0, n, 400)
    qi[:2], ki[:2] = [0, G - 1], [n - 1, 0]
    got = oracle.score_pairs(prm, bits, norms, rnorms, q, qi, ki)
    np.testing.assert_array_equal(got, full[qi, ki])


@pytest.mark.slow
def test_two_group_estimator_unbiased_over_projections_and_rotations():
    g = np.random.default_rng(91)
    d = 128
    chan = g.permutation(d).astype(np.int32)
    spec = oracle.Spec(d, d, [(32, 2), (96, 1)], chan)
    x = g.standard_normal(d).astype(np.float32)
    x[chan[:32]] *= 8.0
    q = (x / 4 + g.standard_normal(d)).astype(np.float32)
    truth = float(q.astype(np.float64) @ x.astype(np.float64))
    vals = np.empty(1500)
    for s in range(len(vals)):
        h = np.random.default_rng(11000 + s)
        prm = oracle.Params(spec, [h.standard_normal((32, 32)).astype(np.float32),
                                   h.standard_normal((96, 96)).astype(np.float32)],
                            h.standard_normal((d, d)).astype(np.float32))
        b_, n_, r_ = oracle.encode(prm, x[None])
        vals[s] = oracle.score(prm, b_, n_, r_, 1, q[None])[0, 0]
    assert abs(vals.mean() - truth) < 4 * vals.std(ddof=1) / math.sqrt(len(vals))
    # over projections alone (rotations fixed): the MSE part is fixed, the sketch unbiased
    h = np.random.default_rng(12)
    gs = [h.standard_normal((32, 32)).astype(np.float32), h.standard_normal((96, 96)).astype(np.float32)]
    prm = oracle.Params(spec, gs, np.zeros((d, d), np.float32))
    for s in range(len(vals)):
        prm.proj = np.random.default_rng(13000 + s).standard_normal((d, d)).astype(np.float32)
        b_, n_, r_ = oracle.encode(prm, x[None])
        vals[s] = oracle.score(prm, b_, n_, r_, 1, q[None])[0, 0]
    assert abs(vals.mean() - truth) < 4 * vals.std(ddof=1) / math.sqrt(len(vals))


# ------------------------------------------------------------------------------------
# distortion (turboquant-pytorch write-up, performance section: 0.034 measured, 0.043 bound)
# ------------------------------------------------------------------------------------

def _sphere_marginal_mse(bits, d):
    """E[(z - Q(z))^2] for z = sqrt(d) u_1, u uniform on the unit sphere in R^d
    (u_1 has density proportional to (1-t^2)^((d-3)/2)), by quadrature."""
    c, t, _, _ = oracle.codebook(bits)
    logB = math.lgamma(0.5) + math.lgamma((d - 1) / 2) - math.lgamma(d / 2)
    f = lambda s: math.exp(((d - 3) / 2) * math.log1p(-s * s / d) - logB) / math.sqrt(d)  # density of z
    edges = np.concatenate([[-math.sqrt(d)], t, [math.sqrt(d)]])
    tot = 0.0
    for k in range(len(c)):
        tot += integrate.quad(lambda s: (s - c[k]) ** 2 * f(s), edges[k], edges[k + 1], epsabs=1e-13, epsrel=1e-11)[0]
    return tot


def _unit_gaussian_distortion(bits, d, n, seed):
    g = np.random.default_rng(seed)
    spec = oracle.Spec(d, 0, [(d, bits)])
    prm = oracle.Params(spec, [g.standard_normal((d, d)).astype(np.float32)], None)
    x = g.standard_normal((n, d))
    x = (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)
    bits_, norms, _ = oracle.encode(prm, x)
    err = ((x.astype(np.float64) - oracle.decode(prm, bits_, norms, n)) ** 2).sum(axis=1)
    return err.mean(), err.std() / math.sqrt(n)


def test_three_bit_distortion_matches_the_reported_value():
    gold = dict(l.split() for l in open(os.path.join(GOLDEN, "p3_mse_distortion.txt")) if not l.startswith("#"))
    d, b = int(gold["d"]), int(gold["bits"])
    mean, se = _unit_gaussian_distortion(b, d, 6000, 11)
    assert round(mean, 3) == float(gold["measured"])
    assert mean < float(gold["bound"])
    assert abs(mean - _sphere_marginal_mse(b, d)) < 4 * se + 1e-5


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_distortion_equals_sphere_marginal_expectation(bits):
    mean, se = _unit_gaussian_distortion(bits, 128, 4000, 20 + bits)
    assert abs(mean - _sphere_marginal_mse(bits, 128)) < 4 * se + 1e-5
    assert mean < math.sqrt(3) * math.pi / 2 * 4.0 ** (-bits)


# ------------------------------------------------------------------------------------
# variants: the exact sphere-marginal codebook, the randomised Walsh-Hadamard rotation
# ------------------------------------------------------------------------------------

def _sphere_law_mse(c, t, d):
    """E[(z - Q(z))^2] under the sphere marginal of z = sqrt(d) u_1 for the codebook (c, t),
    by adaptive quadrature of the density."""
    logB = math.lgamma(0.5) + math.lgamma((d - 1) / 2) - math.lgamma(d / 2)
    f = lambda s: math.exp(((d - 3) / 2) * math.log1p(-min(s * s / d, 1.0)) - logB) / math.sqrt(d)
    edges = np.concatenate([[-math.sqrt(d)], t, [math.sqrt(d)]])
    return sum(integrate.quad(lambda s: (s - c[k]) ** 2 * f(s), edges[k], edges[k + 1], epsabs=1e-13,
                              epsrel=1e-11)[0] for k in range(len(c)))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_sphere_codebook_in_three_dimensions_is_the_uniform_quantiser(bits):
    # d = 3: a coordinate of a uniform point on the 2-sphere is uniform on [-1, 1]
    # (Archimedes), so z is uniform on [-sqrt 3, sqrt 3], whose optimal quantiser is uniform
    L = 1 << bits
    c, t, mse = oracle.codebook_sphere(bits, 3)
    r3 = math.sqrt(3.0)
    np.testing.assert_allclose(c, r3 * (2 * np.arange(L) + 1 - L) / L, atol=1e-12)
    np.testing.assert_allclose(t, r3 * (2 * np.arange(1, L) - L) / L, atol=1e-12)
    assert abs(mse - 1.0 / L ** 2) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_sphere_codebook_tends_to_the_normal_one(bits):
    c, t, mse = oracle.codebook_sphere(bits, 10 ** 8)
    cg, tg, mg, _ = oracle.codebook(bits)
    assert np.abs(c - cg).max() < 1e-5 and np.abs(t - tg).max() < 1e-5 and abs(mse - mg) < 1e-6


@pytest.mark.parametrize("bits,d", [(2, 8), (3, 16), (3, 128), (4, 32)])
def test_sphere_codebook_by_quadrature(bits, d):
    c, t, mse = oracle.codebook_sphere(bits, d)
    # the distortion by adaptive quadrature of the density (not the beta moments)
    assert abs(_sphere_law_mse(c, t, d) - mse) < 1e-9
    # centroid conditions by quadrature: c_k = E[z | cell k]
    logB = math.lgamma(0.5) + math.lgamma((d - 1) / 2) - math.lgamma(d / 2)
    f = lambda s: math.exp(((d - 3) / 2) * math.log1p(-min(s * s / d, 1.0)) - logB) / math.sqrt(d)
    edges = np.concatenate([[-math.sqrt(d)], t, [math.sqrt(d)]])
    for k in range(len(c)):
        m0 = integrate.quad(f, edges[k], edges[k + 1], epsabs=1e-14)[0]
        m1 = integrate.quad(lambda s: s * f(s), edges[k], edges[k + 1], epsabs=1e-14)[0]
        assert abs(m1 / m0 - c[k]) < 1e-9
    # and it beats the normal codebook on this law
    cg, tg, _, _ = oracle.codebook(bits)
    assert mse < _sphere_law_mse(cg, tg, d)


def test_sphere_codebook_is_the_monte_carlo_optimum():
    """Lloyd on coordinates of sampled uniform unit vectors (d = 12) reaches the same codebook."""
    d, bits = 12, 2
    g = np.random.default_rng(5)
    x = g.standard_normal((100000, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    z = (math.sqrt(d) * x).ravel()
    z = np.concatenate([z, -z])  # the law is symmetric; so is its sample, then
    c, t, mse = oracle.codebook_sphere(bits, d)
    ce, te, msee, _ = oracle.lloyd_empirical(z, 1 << bits, oracle.codebook(bits)[0])
    assert np.abs(ce - c).max() < 3e-3 and abs(msee / len(z) - mse) < 1e-3


@pytest.mark.parametrize("d", [1, 2, 8, 128])
def test_hadamard_rotation_is_orthogonal_and_the_fast_transform(d):
    g = np.random.default_rng(d)
    s = np.where(g.standard_normal(d) > 0, 1.0, -1.0)
    R = oracle.hadamard_rotation(s)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-13)
    assert np.allclose(np.abs(R), 1 / math.sqrt(d))
    x = g.standard_normal((5, d))
    np.testing.assert_allclose(x @ R.T, oracle.fwht(x * s) / math.sqrt(d), atol=1e-12)
    # entry (j, k) = (-1)^popcount(j & k) s_k / sqrt(d)
    j, k = g.integers(0, d, 2)
    assert R[j, k] * math.sqrt(d) == (-1) ** bin(int(j) & int(k)).count("1") * s[k]


def test_hadamard_rotation_three_bit_distortion():
    """The rotated coordinates of Gaussian keys are Gaussian for any fixed rotation, so the
    3-bit distortion with a Walsh-Hadamard rotation is the reported value too."""
    d, b, n = 128, 3, 6000
    g = np.random.default_rng(12)
    spec = oracle.Spec(d, 0, [(d, b)])
    prm = oracle.Params(spec, [], None, rotations=[oracle.hadamard_rotation(np.where(g.random(d) > 0.5, 1, -1))])
    x = g.standard_normal((n, d))
    x = (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)
    bits_, norms, _ = oracle.encode(prm, x)
    err = ((x.astype(np.float64) - oracle.decode(prm, bits_, norms, n)) ** 2).sum(axis=1)
    se = err.std() / math.sqrt(n)
    assert abs(err.mean() - _sphere_marginal_mse(b, d)) < 4 * se + 1e-5
    assert round(err.mean(), 3) == 0.034


# ------------------------------------------------------------------------------------
# the estimator: unbiased, with the sign sketch's closed-form variance; MSE-only is biased
# ------------------------------------------------------------------------------------

def _est_over_S(x, q, rot_gauss, bits, nseeds, seed0):
    d = x.shape[0]
    spec = oracle.Spec(d, d, [(d, bits)])
    prm = oracle.Params(spec, [rot_gauss], np.zeros((d, d), np.float32))
    out = np.empty(nseeds)
    for s in range(nseeds):
        prm.proj = np.random.default_rng(seed0 + s).standard_normal((d, d)).astype(np.float32)
        b_, n_, r_ = oracle.encode(prm, x[None])
        out[s] = oracle.score(prm, b_, n_, r_, 1, q[None])[0, 0]
    return out, prm


@pytest.mark.slow
def test_estimator_unbiased_with_closed_form_variance_over_projections():
    g = np.random.default_rng(31)
    d = 128
    x = (g.standard_normal(d) * 2).astype(np.float32)
    G = g.standard_normal((d, d)).astype(np.float32)
    # a query with a large component along the residual so that a wrong sketch
    # scale or sign would show as a bias
    spec0 = oracle.Spec(d, 0, [(d, 2)])
    prm0 = oracle.Params(spec0, [G], None)
    b0, n0, _ = oracle.encode(prm0, x[None])
    r = x - oracle.decode(prm0, b0, n0, 1)[0]
    rho = np.linalg.norm(r)
    q = (3 * r / rho + g.standard_normal(d)).astype(np.float32)
    est, prm = _est_over_S(x, q, G, 2, 3000, 5000)
    truth = float(q.astype(np.float64) @ x.astype(np.float64))
    se = est.std(ddof=1) / math.sqrt(len(est))
    assert abs(est.mean() - truth) < 4 * se
    qd = q.astype(np.float64)
    var = ((math.pi / 2) * rho ** 2 * (qd @ qd) - (qd @ r) ** 2) / d
    rel = est.var(ddof=1) / var
    assert abs(rel - 1) < 4 * math.sqrt(2 / (len(est) - 1))


@pytest.mark.slow
def test_binary16_norm_variant_estimator_stays_unbiased():
    # with the residual taken against the rounded-norm reconstruction the sketch corrects
    # the rounding too: the estimate stays unbiased over projections
    g = np.random.default_rng(37)
    d = 128
    x = (g.standard_normal(d) * 7).astype(np.float32)
    q = (x / 3 + g.standard_normal(d)).astype(np.float32)
    G = g.standard_normal((d, d)).astype(np.float32)
    spec = oracle.Spec(d, d, [(d, 1)], norm16=True)
    prm = oracle.Params(spec, [G], np.zeros((d, d), np.float32))
    est = np.empty(3000)
    for s in range(len(est)):
        prm.proj = np.random.default_rng(7000 + s).standard_normal((d, d)).astype(np.float32)
        b_, n_, r_ = oracle.encode(prm, x[None])
        est[s] = oracle.score(prm, b_, n_, r_, 1, q[None])[0, 0]
    truth = float(q.astype(np.float64) @ x.astype(np.float64))
    assert abs(est.mean() - truth) < 4 * est.std(ddof=1) / math.sqrt(len(est))


@pytest.mark.slow
def test_estimator_unbiased_over_rotations_and_projections():
    g = np.random.default_rng(41)
    d = 64
    x = g.standard_normal(d).astype(np.float32)
    q = (x + g.standard_normal(d)).astype(np.float32)
    spec = oracle.Spec(d, d, [(d, 1)])
    vals = []
    for s in range(1500):
        h = np.random.default_rng(9000 + s)
        prm = oracle.Params(spec, [h.standard_normal((d, d)).astype(np.float32)],
                            h.standard_normal((d, d)).astype(np.float32))
        b_, n_, r_ = oracle.encode(prm, x[None])
        vals.append(oracle.score(prm, b_, n_, r_, 1, q[None])[0, 0])
    vals = np.array(vals)
    truth = float(q.astype(np.float64) @ x.astype(np.float64))
    assert abs(vals.mean() - truth) < 4 * vals.std(ddof=1) / math.sqrt(len(vals))


@pytest.mark.slow
def test_mse_only_one_bit_shrinks_inner_products_by_two_over_pi():
    """The bias the sign sketch removes (tambur.pub article: an MSE-optimal quantiser
    gives a biased inner-product estimate)."""
    g = np.random.default_rng(51)
    d = 128
    spec = oracle.Spec(d, 0, [(d, 1)])
    ratios = []
    for s in range(300):
        h = np.random.default_rng(7000 + s)
        prm = oracle.Params(spec, [h.standard_normal((d, d)).astype(np.float32)], None)
        x = h.standard_normal((8, d)).astype(np.float32)
        b_, n_, r_ = oracle.encode(prm, x)
        xhat = oracle.decode(prm, b_, n_, 8)
        ratios += list((x.astype(np.float64) * xhat).sum(1) / (x.astype(np.float64) ** 2).sum(1))
    assert abs(np.mean(ratios) - 2 / math.pi) < 0.01


# ------------------------------------------------------------------------------------
# decode attention: softmax of the estimated logits over MSE-decoded values
# ------------------------------------------------------------------------------------

def _attend_setup(n, G, seed, kbits=2, vbits=3, key_scale=1.0):
    g = np.random.default_rng(seed)
    d = 64
    kspec = oracle.Spec(d, d, [(d, kbits)])
    vspec = oracle.Spec(d, 0, [(d, vbits)])
    kprm = oracle.Params(kspec, [g.standard_normal((d, d)).astype(np.float32)],
                         g.standard_normal((d, d)).astype(np.float32))
    vprm = oracle.Params(vspec, [g.standard_normal((d, d)).astype(np.float32)], None)
    keys = (key_scale * g.standard_normal((n, d))).astype(np.float32)
    vals = g.standard_normal((n, d)).astype(np.float32)
    q = g.standard_normal((G, d)).astype(np.float32)
    return kprm, vprm, oracle.encode(kprm, keys), oracle.encode(vprm, vals), q


def test_attend_over_equal_logits_is_the_mean_decoded_value():
    """Zero keys give estimate 0 for every token (zero norms), and a zero scale flattens
    any logits: either way the softmax is uniform and attention is the plain mean."""
    kprm, vprm, kb, vb, q = _attend_setup(37, 3, 1)
    n = 37
    mean = oracle.decode(vprm, vb[0], vb[1], n).mean(axis=0)
    out0 = oracle.attend(kprm, kb, vprm, vb, n, q, 0.0)
    np.testing.assert_allclose(out0, np.repeat(mean[None], 3, axis=0), rtol=1e-13, atol=1e-15)
    zb = oracle.encode(kprm, np.zeros((n, 64), np.float32))
    out1 = oracle.attend(kprm, zb, vprm, vb, n, q, 0.125)
    np.testing.assert_allclose(out1, np.repeat(mean[None], 3, axis=0), rtol=1e-13, atol=1e-15)


def test_attend_over_two_tokens_is_the_logistic_blend():
    """Two tokens: the softmax weight of the first is 1 / (1 + e^(scale (s2 - s1)))."""
    kprm, vprm, kb, vb, q = _attend_setup(2, 4, 2)
    s = oracle.score(kprm, kb[0], kb[1], kb[2], 2, q)
    v = oracle.decode(vprm, vb[0], vb[1], 2)
    scale = 0.3
    w1 = 1.0 / (1.0 + np.exp(scale * (s[:, 1] - s[:, 0])))
    expect = w1[:, None] * v[0][None] + (1.0 - w1)[:, None] * v[1][None]
    np.testing.assert_allclose(oracle.attend(kprm, kb, vprm, vb, 2, q, scale), expect, rtol=1e-12, atol=1e-14)


def test_attend_with_one_dominant_logit_returns_that_value():
    """One key far along the query direction takes all the weight."""
    g = np.random.default_rng(3)
    kprm, vprm, _, vb, q = _attend_setup(50, 1, 3)
    keys = (0.1 * g.standard_normal((50, 64))).astype(np.float32)
    keys[17] = 40.0 * q[0] / np.linalg.norm(q[0])
    kb = oracle.encode(kprm, keys)
    out = oracle.attend(kprm, kb, vprm, vb, 50, q, 1.0)
    v17 = oracle.decode(vprm, vb[0], vb[1], 50)[17]
    np.testing.assert_allclose(out[0], v17, rtol=0, atol=1e-9 * np.abs(v17).max())


def test_attend_over_one_repeated_value_returns_it():
    """A convex combination of copies of one vector is that vector, whatever the logits."""
    g = np.random.default_rng(4)
    kprm, vprm, kb, _, q = _attend_setup(40, 5, 4, key_scale=3.0)
    x = g.standard_normal(64).astype(np.float32)
    vb = oracle.encode(vprm, np.repeat(x[None], 40, axis=0))
    xhat = oracle.decode(vprm, vb[0], vb[1], 1)[0]
    out = oracle.attend(kprm, kb, vprm, vb, 40, q, 0.7)
    np.testing.assert_allclose(out, np.repeat(xhat[None], 5, axis=0), rtol=1e-12, atol=1e-14)


def test_attend_is_a_convex_combination_of_the_decoded_values():
    """Every output coordinate lies between the smallest and largest decoded value, and
    with n = d tokens whose decoded values are linearly independent the weights can be
    recovered from the output: they sum to one and their log-ratios are the scaled logit
    differences (the softmax's defining property)."""
    kprm, vprm, kb, vb, q = _attend_setup(64, 2, 5)
    v = oracle.decode(vprm, vb[0], vb[1], 64)
    out = oracle.attend(kprm, kb, vprm, vb, 64, q, 0.5)
    assert (out >= v.min(axis=0) - 1e-12).all() and (out <= v.max(axis=0) + 1e-12).all()
    # recover the weights: out = p @ v with v square and invertible
    p = np.linalg.solve(v.T, out.T).T
    s = oracle.score(kprm, kb[0], kb[1], kb[2], 64, q)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-9)
    np.testing.assert_allclose(np.log(p[:, 1:] / p[:, :1]), 0.5 * (s[:, 1:] - s[:, :1]), rtol=0, atol=1e-4)


# ------------------------------------------------------------------------------------
# top-k
# ------------------------------------------------------------------------------------

def test_topk_orders_by_score_then_lower_index():
    g = np.random.default_rng(3)
    s = np.round(g.standard_normal((5, 400)), 1)     # many exact ties
    vals, idx = oracle.topk(s, 17)
    for q in range(5):
        order = np.lexsort((np.arange(400), -s[q]))[:17]
        np.testing.assert_array_equal(idx[q], order)
        np.testing.assert_array_equal(vals[q], s[q, order])


def test_workload_generators_are_method_free_and_seeded():
    cfg = workloads.CONFIGS["decode3b"]
    a = workloads.keys(cfg, n=64)
    b = workloads.keys(cfg, n=64)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (2, 64, 128)
    # bf16-representable values
    back = (workloads.bf16_bits(a).astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(back, a)
