"""The 16-bit norm format (tq_params.norm_dtype = TQ_F16) on the GPU against the oracle.

Encoding: the GPU encoder's binary16 norms, codes and signs against oracle.encode_trace
with norm16 (tolerances in tests/parity.py: each side rounds its own float32 norm, so a
key whose float32 norms straddle a binary16 tie is one unit apart and is left out of the
sign and residual checks). Every reader (the ring, fused, prepared and top-k scorers,
decode, attention) on oracle-encoded binary16 bytes, with the tolerances of the float32
format: both sides read the same stored values.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import both_params, check_encode, check_scores, check_topk, download_bank, upload_bank

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


def _dev(cfg, x):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if cfg.key_dtype == "bf16" else t


def _encode_banks(orc, x):
    refs = [oracle.encode(orc, x[b]) for b in range(x.shape[0])]
    return [np.stack([r[i] for r in refs]) for i in range(3)]


@pytest.mark.parametrize("name,bits,n", [("tiny", 3, 1000), ("decode3b", 4, 1500), ("decode8b", 3, 1503),
                                         ("longctx", 3, 777)])
def test_half_norm_encode(tq, name, bits, n):
    import torch

    cfg = workloads.CONFIGS[name]
    say(f"half-norm encode {name} b={bits} n={n}")
    gpu, orc = both_params(cfg, bits, norm16=True)
    x = workloads.keys(cfg, n=n, banks=[0, 1])
    bank = tq.Bank(gpu, 2, n)
    assert bank.norms.dtype == torch.float16 and bank.rnorms.dtype == torch.float16
    tq.tq_encode(gpu, _dev(cfg, x), bank)
    torch.cuda.synchronize()
    gb = download_bank(bank)
    rep = {}
    for b in range(2):
        check_encode((gb[0][b], gb[1][b], gb[2][b]), oracle.encode_trace(orc, x[b]), orc, n, rep)
    say("report", rep)


def test_half_norm_append_equals_encode(tq):
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    n = 200
    gpu, _ = both_params(cfg, 3, norm16=True)
    x = workloads.keys(cfg, n=n, banks=[2])
    whole = tq.Bank(gpu, 1, n)
    tq.tq_encode(gpu, _dev(cfg, x), whole)
    grown = tq.Bank(gpu, 1, n)
    xd = _dev(cfg, x)
    for lo, hi in [(0, 1), (1, 17), (17, 200)]:
        pos = torch.full((1,), lo, dtype=torch.int32, device="cuda")
        tq.tq_encode_append(gpu, xd[:, lo:hi].contiguous(), grown, pos)
    torch.cuda.synchronize()
    # slots 0..n-1 (appends write only the slots they are given; the padding slots of the
    # whole-bank encode hold zero-vector records)
    (wb, wn, wr), (gb, gn, gr) = download_bank(whole), download_bank(grown)
    W = wb.shape[2]
    np.testing.assert_array_equal(wb[0].transpose(0, 2, 1).reshape(-1, W)[:n],
                                  gb[0].transpose(0, 2, 1).reshape(-1, W)[:n])
    np.testing.assert_array_equal(wn[0][:n], gn[0][:n])
    np.testing.assert_array_equal(wr[0][:n], gr[0][:n])


@pytest.mark.parametrize("G", [1, 3, 4, 7, 16, 20])
def test_half_norm_scores(tq, G):
    """G = 4: the ring scorer; 1..16: the fused scorers; 20: prepared operands."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    n = 2000 + 9
    gpu, orc = both_params(cfg, 3, norm16=True)
    x = workloads.keys(cfg, n=n, banks=[0, 3])
    q = workloads.queries(cfg, banks=[0, 3], G=G)
    say(f"half-norm scores G={G} n={n}")
    kb = _encode_banks(orc, x)
    bank = upload_bank(tq, gpu, kb[0], kb[1], kb[2], n)
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
    for b in range(2):
        check_scores(got[b], oracle.score(orc, kb[0][b], kb[1][b], kb[2][b], n, q[b]), f"bank {b}")


def test_half_norm_scores_two_groups_and_topk(tq):
    import torch

    cfg = workloads.CONFIGS["longctx"]
    n, G, k = 3000, 4, 10
    gpu, orc = both_params(cfg, 3, norm16=True)
    x = workloads.keys(cfg, n=n, banks=[1])
    q = workloads.queries(cfg, banks=[1], G=G)
    kb = _encode_banks(orc, x)
    bank = upload_bank(tq, gpu, kb[0], kb[1], kb[2], n)
    qd = torch.from_numpy(q).cuda()
    ref = oracle.score(orc, kb[0][0], kb[1][0], kb[2][0], n, q[0])
    check_scores(tq.tq_score(gpu, bank, qd).cpu().numpy()[0], ref, "two groups")
    vals, idx = tq.tq_topk(gpu, bank, qd, k)
    check_topk(vals.cpu().numpy()[0], idx.cpu().numpy()[0], ref, k)


def test_half_norm_decode_and_attend(tq):
    """Keys (inner-product quantiser) and values (MSE-only) both with binary16 norms."""
    import torch

    cfg = workloads.CONFIGS["decode3b"]
    n, G, scale = 1300, 4, 1.0 / np.sqrt(128)
    kgpu, korc = both_params(cfg, 4, norm16=True)
    groups = [(cfg.d, 3)]
    vg = workloads.value_rotation_gaussians(cfg.cfg_id, [cfg.d])
    vgpu = tq.make_params(cfg.d, 0, groups, vg, None, norm16=True)
    vorc = oracle.Params(oracle.Spec(cfg.d, 0, groups, norm16=True), vg, None)
    kb = _encode_banks(korc, workloads.keys(cfg, n=n, banks=[0, 1]))
    vb = _encode_banks(vorc, workloads.values(cfg, n=n, banks=[0, 1]))
    kbank = upload_bank(tq, kgpu, kb[0], kb[1], kb[2], n)
    vbank = upload_bank(tq, vgpu, vb[0], vb[1], vb[2], n)
    dec = tq.tq_decode(vgpu, vbank).cpu().numpy()
    q = workloads.queries(cfg, banks=[0, 1], G=G)
    qd = torch.from_numpy(q).cuda()
    out = tq.tq_attend(kgpu, kbank, vgpu, vbank, qd, scale).cpu().numpy()
    logits = tq.tq_score(kgpu, kbank, qd).cpu().numpy()
    for b in range(2):
        v = oracle.decode(vorc, vb[0][b], vb[1][b], n)
        # fp32 decoder: d products of |c| nu / sqrt(d) per channel
        tol = 4 * cfg.d * 2.0 ** -24 * vb[1][b][:n, :1].astype(np.float64) / np.sqrt(cfg.d) * \
            np.abs(vorc.rots[0]).sum(axis=0)[None] * np.abs(vorc.cent[0, :8]).max()
        assert (np.abs(dec[b] - v) <= tol).all()
        s_ref = oracle.score(korc, kb[0][b], kb[1][b], kb[2][b], n, q[b])
        e = check_scores(logits[b], s_ref, f"logits bank {b}")
        z = scale * s_ref
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ref = oracle.attend(korc, (kb[0][b], kb[1][b], kb[2][b]), vorc, (vb[0][b], vb[1][b], vb[2][b]), n, q[b],
                            scale)
        A = p @ np.abs(v)
        tol = np.expm1(2 * scale * e) * A + 1e-6 * (A + np.sqrt((v ** 2).mean()))
        err = np.abs(out[b].astype(np.float64) - ref)
        assert (err <= tol).all(), f"bank {b}: worst excess {np.max(err - tol):.3e}"


def test_half_norm_full_decode8b_layer_sampled(tq):
    """The full 8B-class layer (64 banks x 32768 keys, G = 4) with binary16 norms, in the
    benchmark's launch configuration, on random bank bytes (binary16 norms of random
    positive values); sampled pairs against the oracle."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    gpu, orc = both_params(cfg, 3, norm16=True)
    W, npad, bpk = gpu.layout(cfg.tokens)
    assert bpk == 4 * W + 4
    rb, rn, rr = workloads.random_bank(cfg.cfg_id, cfg.banks, npad, W, 1, layer=3)
    rn = rn.astype(np.float16).astype(np.float32)  # values the format can hold
    rr = rr.astype(np.float16).astype(np.float32)
    bank = upload_bank(tq, gpu, rb, rn, rr, cfg.tokens)
    q = workloads.queries(cfg, layer=3)
    say("half-norm full layer, random bank")
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
    g = np.random.default_rng(16)
    for b in g.choice(cfg.banks, 6, replace=False):
        ki = np.concatenate([g.integers(0, cfg.tokens, 250), [0, cfg.tokens - 1]])
        qi = g.integers(0, cfg.G, len(ki))
        ref = oracle.score_pairs(orc, rb[b], rn[b], rr[b], q[b], qi, ki)
        check_scores(got[b, qi, ki], ref, f"bank {b}")


# ------------------------------------------------------------------------------------------
# keys above 128 dimensions (the two-GEMM encoder and the large-operand readers) and key rows
# at unaligned addresses (the tile-per-work-group encoder), with binary16 norms
# ------------------------------------------------------------------------------------------

def _cfg_with(base, **kw):
    import dataclasses

    return dataclasses.replace(workloads.CONFIGS[base], **kw)


def _encode_check(tq, cfg, bits, x, unaligned=False):
    import torch

    gpu, orc = both_params(cfg, bits, norm16=True)
    banks, n = x.shape[0], x.shape[1]
    bank = tq.Bank(gpu, banks, n)
    t = _dev(cfg, x)
    if unaligned:  # the same values one element off a 16-byte boundary
        flat = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        flat[1:] = t.reshape(-1)
        t = flat[1:].view(t.shape)
    tq.tq_encode(gpu, t, bank)
    torch.cuda.synchronize()
    gb = download_bank(bank)
    assert bank.norms.dtype == torch.float16 and bank.rnorms.dtype == torch.float16
    rep = {}
    for b in range(banks):
        check_encode((gb[0][b], gb[1][b], gb[2][b]), oracle.encode_trace(orc, x[b]), orc, n, rep)
    return rep


@pytest.mark.parametrize("case", ["search_b4", "search_b2", "d256_two_groups_bf16", "m256_bf16"])
def test_half_norm_encode_large_keys(tq, case):
    """The two-GEMM encoder writes binary16 norms, its residual taken against the rounded
    norm: d = 768 fp32 unit vectors (search), two permuted channel groups at d = 256 with
    a partial row tile, and m above 128 at d = 128."""
    if case.startswith("search"):
        cfg, bits, n = workloads.CONFIGS["search"], int(case[-1]), 301
    elif case == "d256_two_groups_bf16":
        groups = ((64, 3), (192, 2))
        cfg, bits, n = _cfg_with("longctx", d=256, m=160, key_dtype="bf16", cfg_id=81, outliers=64,
                                 groups=groups), 3, 1100
    else:
        cfg, bits, n = _cfg_with("decode8b", d=128, m=256, key_dtype="bf16", cfg_id=82), 3, 1100
    say(f"half-norm encode, large keys: {case} d={cfg.d} m={cfg.m} n={n}")
    x = workloads.keys(cfg, n=n, banks=[0] if cfg.banks == 1 else [0, 1])
    say("   report", _encode_check(tq, cfg, bits, x))


@pytest.mark.parametrize("name,bits", [("decode3b", 3), ("search", 4)])
def test_half_norm_encode_unaligned_keys(tq, name, bits):
    """Key rows off a 16-byte boundary take the tile-per-work-group encoder, which writes
    binary16 norms as well (d = 128 and d = 768)."""
    cfg = workloads.CONFIGS[name]
    n = 333 if name == "search" else 1000
    say(f"half-norm encode, unaligned keys: {name} b={bits} n={n}")
    x = workloads.keys(cfg, n=n, banks=[0])
    say("   report", _encode_check(tq, cfg, bits, x, unaligned=True))


@pytest.mark.parametrize("bits,n,G,k", [(4, 3003, 37, 10), (2, 2001, 9, 10), (4, 700, 3, 64)])
def test_half_norm_search_readers(tq, bits, n, G, k):
    """Top-k, scores (prepared operands in LDS; G <= 16 through the register-operand
    scorer) and decompression of 768-dimensional keys with binary16 norms, on
    oracle-encoded bytes."""
    import torch

    cfg = workloads.CONFIGS["search"]
    say(f"half-norm search readers: b={bits} n={n} G={G} k={k}")
    gpu, orc = both_params(cfg, bits, norm16=True)
    x = workloads.keys(cfg, n=n)
    q = workloads.queries(cfg, G=G)
    kb = _encode_banks(orc, x)
    bank = upload_bank(tq, gpu, kb[0], kb[1], kb[2], n)
    qd = torch.from_numpy(q).cuda()
    ref = oracle.score(orc, kb[0][0], kb[1][0], kb[2][0], n, q[0])
    vals, idx = tq.tq_topk(gpu, bank, qd, k)
    check_topk(vals.cpu().numpy()[0], idx.cpu().numpy()[0], ref, k)
    check_scores(tq.tq_score(gpu, bank, qd).cpu().numpy()[0], ref, "scores")
    # decompression of the same bytes, within the fp32 decoder's rounding bound
    dec = tq.tq_decode(gpu, bank).cpu().numpy()[0]
    v = oracle.decode(orc, kb[0][0], kb[1][0], n)
    cb = 1 << (bits - 1)
    tol = 4 * cfg.d * 2.0 ** -24 * kb[1][0][:n, :1].astype(np.float64) / np.sqrt(cfg.d) * \
        np.abs(orc.rots[0]).sum(axis=0)[None] * np.abs(orc.cent[0, :cb]).max()
    assert (np.abs(dec - v) <= tol).all()


@pytest.mark.parametrize("G", [4, 20])
def test_half_norm_scores_d256(tq, G):
    import torch

    cfg = _cfg_with("decode8b", d=256, m=256, key_dtype="bf16", cfg_id=83)
    n = 1234
    say(f"half-norm scores d=256 G={G}")
    gpu, orc = both_params(cfg, 3, norm16=True)
    x = workloads.keys(cfg, n=n, banks=[0, 1])
    q = workloads.queries(cfg, banks=[0, 1], G=G)
    kb = _encode_banks(orc, x)
    bank = upload_bank(tq, gpu, kb[0], kb[1], kb[2], n)
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
    for b in range(2):
        check_scores(got[b], oracle.score(orc, kb[0][b], kb[1][b], kb[2][b], n, q[b]), f"bank {b}")
