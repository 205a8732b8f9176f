"""Decompression (tq_decode) and decode attention (tq_attend) on the GPU against the oracle.

Both sides read identical bank bytes: the oracle encodes keys (inner-product quantiser)
and values (MSE-only quantiser, m = 0), the bytes are uploaded, and the GPU output is
compared with oracle.decode / oracle.attend on the same bytes.

Tolerances, derived from the arithmetic:
  - decode: fp32 accumulation of d_g products per channel,
    |x_gpu - x| <= 4 d_g 2^-24 (nu_g / sqrt(d_g)) sum_j |R_g[j][k]| max|c_g|;
  - attend: the logits the GPU uses differ from the oracle's by at most e (measured here
    with tq_score on the same bytes, and itself checked against the score tolerance).
    Perturbing every logit by at most e moves each softmax weight by a factor within
    e^(+-2 scale e), so |o_gpu - o| <= (e^(2 scale e) - 1) A + 1e-6 (A + s) with
    A_j = sum_i p_i |x_hat_ij| and s the rms decoded value coordinate: the second term
    covers the kernel's own rounding (30-bit fixed-point weights, fp32 partials).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import both_params, check_encode, check_scores, download_bank, upload_bank

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tq():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_inner_amd as tq

    return tq


def value_params(tq, cfg, groups, chan=None, layer=0, d=None):
    """MSE-only (m = 0) parameters for the values, both sides, from the value rotation draws."""
    d = cfg.d if d is None else d
    gauss = workloads.value_rotation_gaussians(cfg.cfg_id, [g[0] for g in groups], layer)
    gpu = tq.make_params(d, 0, groups, gauss, None, chan)
    orc = oracle.Params(oracle.Spec(d, 0, groups, chan), gauss, None)
    return gpu, orc


def _encode_banks(orc, x):
    refs = [oracle.encode(orc, x[b]) for b in range(x.shape[0])]
    return [np.stack([r[i] for r in refs]) for i in range(3)]


def _decode_tol(orc, norms_b, n):
    """Per (vector, channel) bound of the fp32 decoder's rounding (channel order)."""
    sp = orc.spec
    tol = np.zeros((n, sp.d))
    off = 0
    for g, (dg, b) in enumerate(sp.groups):
        colsum = np.abs(orc.rots[g]).sum(axis=0)  # sum_j |R[j][k]|
        cmax = np.abs(orc.cent[g, : 1 << b]).max()
        t = 4 * dg * 2.0 ** -24 * (norms_b[:n, g:g + 1].astype(np.float64) / np.sqrt(dg)) * colsum[None] * cmax
        chans = sp.chan[off:off + dg] if sp.chan is not None else np.arange(off, off + dg)
        tol[:, chans] = t
        off += dg
    return tol


def _check_attend(got, ref, v, p, e, scale, what):
    A = p @ np.abs(v)                           # [G, d]
    s = np.sqrt((v ** 2).mean())
    tol = (np.expm1(2 * scale * e)) * A + 1e-6 * (A + s)
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} beyond tolerance; worst excess "
                           f"{np.max(err - tol):.3e}, max err {err.max():.3e}, logit err {e:.3e}")
    return float(err.max())


def _attend_case(tq, kgpu, korc, vgpu, vorc, kb, vb, q, scale, n, banks_to_check=None):
    """Runs tq_attend and tq_score on uploaded banks; compares every (checked) bank with the oracle."""
    import torch

    banks = kb[0].shape[0]
    kbank = upload_bank(tq, kgpu, kb[0], kb[1], kb[2], n)
    vbank = upload_bank(tq, vgpu, vb[0], vb[1], vb[2], n)
    qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    out = tq.tq_attend(kgpu, kbank, vgpu, vbank, qd, scale).cpu().numpy()
    logits = tq.tq_score(kgpu, kbank, qd).cpu().numpy()
    worst = 0.0
    for b in (range(banks) if banks_to_check is None else banks_to_check):
        s_ref = oracle.score(korc, kb[0][b], kb[1][b], kb[2][b], n, q[b])
        e = check_scores(logits[b], s_ref, f"logits bank {b}")
        v = oracle.decode(vorc, vb[0][b], vb[1][b], n)
        z = scale * s_ref
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ref = oracle.attend(korc, (kb[0][b], kb[1][b], kb[2][b]), vorc, (vb[0][b], vb[1][b], vb[2][b]), n, q[b], scale)
        worst = max(worst, _check_attend(out[b], ref, v, p, e, scale, f"bank {b}"))
    return worst


# ------------------------------------------------------------------------------------------
# MSE-only encoding (m = 0) of the values by the GPU encoder
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["bf16_b3", "f32_b2", "two_groups", "d64_unaligned"])
def test_encode_mse_only_values(tq, case):
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    n, d, chan, groups, banks = 1000, cfg.d, None, [(cfg.d, 3)], [0, 7]
    dtype = torch.bfloat16
    if case == "f32_b2":
        groups, dtype = [(cfg.d, 2)], torch.float32
    elif case == "two_groups":
        lcfg = workloads.CONFIGS["longctx"]
        chan = workloads.group_channels(lcfg)
        groups = [(32, 3), (96, 2)]
    elif case == "d64_unaligned":
        n, d, groups = 999, 64, [(64, 3)]
    say(f"encode values m=0 {case}: n={n} d={d} groups={groups}")
    gpu, orc = value_params(tq, cfg, groups, chan, d=d)
    x = workloads.values(cfg, n=n, banks=banks, d=d)   # bf16-valued floats
    bank = tq.Bank(gpu, len(banks), n)
    tq.tq_encode(gpu, torch.from_numpy(x).cuda().to(dtype), bank)
    torch.cuda.synchronize()
    gb = download_bank(bank)
    report = {}
    for b in range(len(banks)):
        check_encode((gb[0][b], gb[1][b], gb[2][b]), oracle.encode_trace(orc, x[b]), orc, n, report)
    say("report", report)


# ------------------------------------------------------------------------------------------
# decompression
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["keys_b4", "values_b3", "values_b1", "two_groups", "d768"])
def test_decode_matches_oracle(tq, case):
    cfg = workloads.CONFIGS["decode8b"]
    n = 1000
    if case == "keys_b4":
        gpu, orc = both_params(cfg, 4)
        x = workloads.keys(cfg, n=n, banks=[0, 5])
    elif case == "d768":
        scfg = workloads.CONFIGS["search"]
        gpu, orc = both_params(scfg, 2)
        x = workloads.keys(scfg, n=100, banks=[0])
        n = 100
    elif case == "two_groups":
        lcfg = workloads.CONFIGS["longctx"]
        chan = workloads.group_channels(lcfg)
        gpu, orc = value_params(tq, lcfg, [(32, 3), (96, 2)], chan)
        x = workloads.values(lcfg, n=n, banks=[3])
    else:
        bits = 3 if case == "values_b3" else 1
        gpu, orc = value_params(tq, cfg, [(cfg.d, bits)])
        x = workloads.values(cfg, n=n, banks=[1, 2])
    say(f"decode {case}: {x.shape}")
    bits_, norms, rnorms = _encode_banks(orc, x)
    bank = upload_bank(tq, gpu, bits_, norms, rnorms, n)
    got = tq.tq_decode(gpu, bank).cpu().numpy()
    for b in range(x.shape[0]):
        ref = oracle.decode(orc, bits_[b], norms[b], n)
        tol = _decode_tol(orc, norms[b], n)
        err = np.abs(got[b].astype(np.float64) - ref)
        assert (err <= tol).all(), f"bank {b}: worst excess {np.max(err - tol):.3e}, max err {err.max():.3e}"


# ------------------------------------------------------------------------------------------
# decode attention
# ------------------------------------------------------------------------------------------

def test_attend_several_chunks_ragged(tq):
    """3 banks x 2500 tokens (two full 1024-token chunks and a ragged one, a ragged last
    tile), G = 6 (a full and a partial group of four queries), 3-bit keys + sketch, 3-bit
    values."""
    cfg = workloads.CONFIGS["decode8b"]
    n, G = 2500, 6
    say(f"attend 3 banks x {n}, G={G}")
    kgpu, korc = both_params(cfg, 4)
    vgpu, vorc = value_params(tq, cfg, [(cfg.d, 3)])
    kb = _encode_banks(korc, workloads.keys(cfg, n=n, banks=[0, 9, 63]))
    vb = _encode_banks(vorc, workloads.values(cfg, n=n, banks=[0, 9, 63]))
    q = workloads.queries(cfg, banks=[0, 9, 63], G=G)
    say("max err", _attend_case(tq, kgpu, korc, vgpu, vorc, kb, vb, q, 1.0 / np.sqrt(cfg.d), n))


@pytest.mark.parametrize("case", ["v1", "v2", "two_groups", "d64", "one_token", "sharp"])
def test_attend_value_layouts_and_edges(tq, case):
    cfg = workloads.CONFIGS["decode3b"]
    n, G, scale, d = 300, 4, 1.0 / np.sqrt(cfg.d), cfg.d
    chan = None
    groups = [(cfg.d, 3)]
    if case == "v1":
        groups = [(cfg.d, 1)]
    elif case == "v2":
        groups = [(cfg.d, 2)]
    elif case == "two_groups":
        lcfg = workloads.CONFIGS["longctx"]
        chan = workloads.group_channels(lcfg)
        groups = [(32, 3), (96, 2)]
    elif case == "d64":
        d, groups = 64, [(64, 3)]
    elif case == "one_token":
        n, G = 1, 3
    elif case == "sharp":
        scale = 2.0      # nearly one-hot weights
    say(f"attend {case}: n={n} G={G} groups={groups} d_v={d}")
    kgpu, korc = both_params(cfg, 3)
    vgpu, vorc = value_params(tq, cfg, groups, chan, d=d)
    kb = _encode_banks(korc, workloads.keys(cfg, n=n, banks=[1]))
    vb = _encode_banks(vorc, workloads.values(cfg, n=n, banks=[1], d=d))
    q = workloads.queries(cfg, banks=[1], G=G)
    say("max err", _attend_case(tq, kgpu, korc, vgpu, vorc, kb, vb, q, scale, n))


def test_attend_equal_logits_is_the_mean_value(tq):
    """Zero keys give logit 0 for every token: the output is the mean decoded value."""
    import torch

    cfg = workloads.CONFIGS["decode3b"]
    n = 1500
    kgpu, korc = both_params(cfg, 4)
    vgpu, vorc = value_params(tq, cfg, [(cfg.d, 3)])
    kb = _encode_banks(korc, np.zeros((1, n, cfg.d), np.float32))
    vb = _encode_banks(vorc, workloads.values(cfg, n=n, banks=[0]))
    kbank = upload_bank(tq, kgpu, kb[0], kb[1], kb[2], n)
    vbank = upload_bank(tq, vgpu, vb[0], vb[1], vb[2], n)
    q = torch.from_numpy(workloads.queries(cfg, banks=[0], G=5)).cuda()
    out = tq.tq_attend(kgpu, kbank, vgpu, vbank, q, 0.1).cpu().numpy()[0]
    v = oracle.decode(vorc, vb[0][0], vb[1][0], n)
    mean = v.mean(axis=0)
    tol = 1e-6 * (np.abs(v).mean(axis=0) + np.sqrt((v ** 2).mean()))
    assert (np.abs(out - mean[None]) <= tol[None]).all()


def test_attend_full_decode8b_layer_sampled(tq):
    """One full 8B-class layer (64 banks x 32768 tokens, G = 4) on random bank bytes for
    keys and values, in the launch configuration the benchmark uses; three banks checked
    against the oracle."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    n = cfg.tokens
    say("attend full decode8b layer, random banks")
    kgpu, korc = both_params(cfg, 4)
    vgpu, vorc = value_params(tq, cfg, [(cfg.d, 3)])
    kW, npad, _ = kgpu.layout(n)
    vW, _, _ = vgpu.layout(n)
    kb = workloads.random_bank(cfg.cfg_id, cfg.banks, npad, kW, 1, layer=0)
    vbits, vnorms, vr = workloads.random_bank(cfg.cfg_id, cfg.banks, npad, vW, 1, layer=1)
    vb = (vbits, vnorms, np.zeros_like(vr))
    q = workloads.queries(cfg)
    say("max err", _attend_case(tq, kgpu, korc, vgpu, vorc, kb, vb, q, 1.0 / np.sqrt(cfg.d), n,
                                banks_to_check=[0, 37, 63]))


def test_attend_prefix_lengths_over_garbage_slots(tq):
    """Banks of 1200 slots whose first 1102 hold oracle-encoded tokens and whose other slots
    hold NaN norms and random bits; per-bank lengths pick the attended prefix: a partial last
    chunk, exactly one chunk, one token, none (output 0), and one past n (clamped to n)."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    n_cap, n_fill, G = 1200, 1102, 4
    lengths = [n_fill, 512, 1, 0, 700, 5000]
    banks = len(lengths)
    say(f"attend prefix lengths {lengths} over {n_cap} slots")
    kgpu, korc = both_params(cfg, 4)
    vgpu, vorc = value_params(tq, cfg, [(cfg.d, 3)])
    bsel = list(range(banks))
    kb = _encode_banks(korc, workloads.keys(cfg, n=n_fill, banks=bsel))
    vb = _encode_banks(vorc, workloads.values(cfg, n=n_fill, banks=bsel))
    g = np.random.default_rng(11)

    def padded(prm, arrs):
        W, npad, _ = prm.layout(n_cap)
        bits = g.integers(0, 2**32, size=(banks, npad // 16, W, 16), dtype=np.uint64).astype(np.uint32)
        norms = np.full((banks, npad, prm.ng), np.nan, np.float32)
        rn = np.full((banks, npad), np.nan, np.float32)
        t = arrs[0].shape[1]
        bits[:, :t] = arrs[0]  # whole tiles of the filled part (its padding slots included)
        norms[:, : t * 16] = arrs[1]
        rn[:, : t * 16] = arrs[2]
        # slots n_fill .. end of its tile: garbage as well
        bits_flat = bits.transpose(0, 1, 3, 2).reshape(banks, -1, W)
        bits_flat[:, n_fill:] = g.integers(0, 2**32, size=bits_flat[:, n_fill:].shape, dtype=np.uint64)
        bits = bits_flat.reshape(banks, npad // 16, 16, W).transpose(0, 1, 3, 2).copy()
        norms[:, n_fill:] = np.nan
        rn[:, n_fill:] = np.nan
        return upload_bank(tq, prm, bits, norms, rn, n_cap)

    kbank, vbank = padded(kgpu, kb), padded(vgpu, vb)
    q = workloads.queries(cfg, banks=bsel, G=G)
    scale = 1.0 / np.sqrt(cfg.d)
    out = tq.tq_attend(kgpu, kbank, vgpu, vbank, torch.from_numpy(q).cuda(), scale,
                       lengths=torch.tensor(lengths, dtype=torch.int32, device="cuda")).cpu().numpy()
    logits = tq.tq_score(kgpu, kbank, torch.from_numpy(q).cuda()).cpu().numpy()
    assert np.isfinite(out).all()
    for b, L in enumerate(lengths):
        L = min(L, n_cap)
        if L == 0:
            assert (out[b] == 0).all()
            continue
        if L > n_fill:  # clamped to n: the garbage slots take part; only finiteness is checked
            continue
        s_ref = oracle.score(korc, kb[0][b], kb[1][b], kb[2][b], L, q[b])
        e = check_scores(logits[b][:, :L], s_ref, f"logits bank {b}")
        v = oracle.decode(vorc, vb[0][b], vb[1][b], L)
        z = scale * s_ref
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ref = oracle.attend(korc, (kb[0][b], kb[1][b], kb[2][b]), vorc, (vb[0][b], vb[1][b], vb[2][b]), L, q[b], scale)
        say(f"bank {b} len {L} max err", _check_attend(out[b], ref, v, p, e, scale, f"bank {b}"))


@pytest.mark.parametrize("unaligned", [False, True])
def test_append_mse_only_values(tq, unaligned):
    """A decode step's value appends: MSE-only (m = 0) values appended at per-bank slots by
    tq_encode_append match the oracle's encoding; untouched slots keep their bytes."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    gpu, orc = value_params(tq, cfg, [(cfg.d, 3)])
    n_cap, banks, count = 80, 2, 21
    vals = workloads.values(cfg, n=count, banks=[4, 5])
    bank = tq.Bank(gpu, banks, n_cap)
    bank.bits.fill_(0x5A5A5A5A)
    bank.norms.fill_(-1.0)
    bank.rnorms.fill_(-2.0)
    pos = np.array([3, 40], np.int64)
    vv = torch.from_numpy(vals).cuda().to(torch.bfloat16)
    if unaligned:
        flat = torch.zeros(vv.numel() + 1, dtype=torch.bfloat16, device="cuda")
        flat[1:] = vv.reshape(-1)
        vv = flat[1:].view(vv.shape)
    tq.tq_encode_append(gpu, vv, bank, torch.from_numpy(pos.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    gb, gn, gr = download_bank(bank)
    W = gb.shape[2]
    report = {}
    for b in range(banks):
        slots = np.arange(pos[b], pos[b] + count)
        words = gb[b].transpose(0, 2, 1).reshape(-1, W)[slots]
        ref = oracle.encode_trace(orc, vals[b])
        ref_rows = ref[0].transpose(0, 2, 1).reshape(-1, W)
        pad = (-count) % 16
        tiles = np.concatenate([words, ref_rows[count:]]).reshape(-1, 16, W).transpose(0, 2, 1)
        check_encode((tiles, np.concatenate([gn[b][slots], np.zeros((pad, 1), np.float32)]),
                      np.concatenate([gr[b][slots], np.zeros(pad, np.float32)])), ref, orc, count, report)
        untouched = np.setdiff1d(np.arange(bank.n_pad), slots)
        assert (gb[b].transpose(0, 2, 1).reshape(-1, W)[untouched] == 0x5A5A5A5A).all()
        assert (gn[b][untouched] == -1.0).all() and (gr[b][untouched] == -2.0).all()
    say("report", report)
