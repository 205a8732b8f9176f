"""GPU (gfx950 HIP path, through the C ABI) against the CPU oracle.

Sizes the oracle finishes in seconds span many 16-key tiles and a ragged tail;
the full-size workloads are checked on sampled outputs the oracle computes one
by one. See tests/parity.py for the tolerances.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import (both_params, check_encode, check_scores, download_bank, groups_of, unpack, upload_bank)

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


def _dev_keys(cfg, keys):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(keys)).cuda()
    return t.to(torch.bfloat16) if cfg.key_dtype == "bf16" else t


def _encode_check(tq, cfg, bits, keys, layer=0, report=None):
    import torch

    banks, n = keys.shape[0], keys.shape[1]
    gpu, orc = both_params(cfg, bits, layer)
    bank = tq.Bank(gpu, banks, n)
    tq.tq_encode(gpu, _dev_keys(cfg, keys), bank)
    torch.cuda.synchronize()
    gb = download_bank(bank)
    report = {} if report is None else report
    for b in range(banks):
        ref = oracle.encode_trace(orc, keys[b])
        check_encode((gb[0][b], gb[1][b], gb[2][b]), ref, orc, n, report)
    return gpu, orc, bank, report


def _score_check(tq, cfg, bits, keys, q, layer=0):
    import torch

    banks, n = keys.shape[0], keys.shape[1]
    gpu, orc = both_params(cfg, bits, layer)
    refs = [oracle.encode(orc, keys[b]) for b in range(banks)]
    bank = upload_bank(tq, gpu, np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs]),
                       np.stack([r[2] for r in refs]), n)
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
    worst = 0.0
    for b in range(banks):
        ref = oracle.score(orc, *refs[b], n, q[b])
        worst = max(worst, check_scores(got[b], ref, f"bank {b}"))
    return worst


# ------------------------------------------------------------------------------------------
# scorer on oracle-encoded banks (identical bank bytes on both sides)
# ------------------------------------------------------------------------------------------

def test_score_tiny_full(tq):
    cfg = workloads.CONFIGS["tiny"]
    say("score tiny: n=1024 G=16 b=3")
    keys = workloads.keys(cfg)
    q = workloads.queries(cfg)
    say("max err", _score_check(tq, cfg, 3, keys, q))


@pytest.mark.parametrize("bits", [3, 4])
def test_score_decode3b_full(tq, bits):
    cfg = workloads.CONFIGS["decode3b"]
    say(f"score decode3b: 2 banks x 8192, G=8, b={bits}")
    keys = workloads.keys(cfg)
    q = workloads.queries(cfg)
    say("max err", _score_check(tq, cfg, bits, keys, q))


def test_score_longctx_two_groups(tq):
    cfg = workloads.CONFIGS["longctx"]
    say("score longctx two groups: 3 banks x 2000, G=4")
    keys = workloads.keys(cfg, n=2000, banks=[0, 3, 7])
    q = workloads.queries(cfg, banks=[0, 3, 7])
    say("max err", _score_check(tq, cfg, 3, keys, q))


@pytest.mark.parametrize("G", [1, 3, 8, 16, 20])
def test_score_longctx_two_groups_other_G(tq, G):
    """Two permuted channel groups at query counts other than the ring scorer's four: the
    fused scorers (G = 1..16, operands in registers) and prepared operands in LDS (G = 20),
    on a ragged bank length."""
    cfg = workloads.CONFIGS["longctx"]
    say(f"score longctx two groups: 2 banks x 1500, G={G}")
    keys = workloads.keys(cfg, n=1500, banks=[2, 5])
    q = workloads.queries(cfg, banks=[2, 5], G=G)
    say("max err", _score_check(tq, cfg, 3, keys, q))


@pytest.mark.parametrize("name,bits,G", [("decode8b", 3, 4), ("decode3b", 4, 7), ("longctx", 3, 5), ("search", 4, 9)])
def test_prepared_operands_reused(tq, name, bits, G):
    """The split scorer's public pair: tq_prepare_queries once, then tq_score_prepared on
    two different sets of banks with the same operands (they depend on the queries and the
    parameters only); both against the oracle."""
    import torch

    cfg = workloads.CONFIGS[name]
    n = 700 if name == "search" else 1200
    banks = [0] if name == "search" else [0, 1]
    gpu, orc = both_params(cfg, bits)
    q = workloads.queries(cfg, banks=banks, G=G)
    qd = torch.from_numpy(q).cuda()
    say(f"prepared operands: {name} b={bits} G={G} n={n}")
    ws = torch.empty(gpu.workspace_bytes(tq.TQ_OP_SCORE, len(banks), n, G), dtype=torch.uint8, device="cuda")
    tq.tq_prepare_queries(gpu, qd, ws)
    for layer in (0, 1):
        keys = workloads.keys(cfg, layer=layer, n=n, banks=banks)
        refs = [oracle.encode(orc, keys[b]) for b in range(len(banks))]
        bank = upload_bank(tq, gpu, np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs]),
                           np.stack([r[2] for r in refs]), n)
        scores = torch.full((len(banks), G, n), float("nan"), dtype=torch.float32, device="cuda")
        got = tq.tq_score_prepared(gpu, bank, G, ws, scores).cpu().numpy()
        for b in range(len(banks)):
            check_scores(got[b], oracle.score(orc, *refs[b], n, q[b]), f"keys of layer {layer}, bank {b}")


@pytest.mark.parametrize("n,G", [(1, 1), (15, 3), (16, 4), (17, 5), (33, 16), (1000, 2), (999, 13)])
def test_score_ragged_shapes(tq, n, G):
    cfg = workloads.CONFIGS["decode8b"]
    say(f"score ragged n={n} G={G}")
    keys = workloads.keys(cfg, n=n, banks=[1, 2])
    q = workloads.queries(cfg, banks=[1, 2], G=G)
    _score_check(tq, cfg, 3, keys, q)


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("d", [64, 256])
def test_score_other_head_dims(tq, d, bits):
    """d = 64 and 256 at G = 4 and G = 1 (the fused scorer with operands in registers;
    1024-thread work-groups at G = 1)."""
    import dataclasses

    cfg = dataclasses.replace(workloads.CONFIGS["decode8b"], d=d, m=d, cfg_id=40 + d // 64)
    keys = workloads.keys(cfg, n=300, banks=[0])
    for G in (4, 1):
        say(f"score d={d} b={bits} G={G}")
        q = workloads.queries(cfg, banks=[0], G=G)
        _score_check(tq, cfg, bits, keys, q)


def test_score_random_banks_full_decode8b_layer(tq):
    """Full 8B-class layer (64 banks x 32768 keys, G=4) on random bank bytes, in the
    launch configuration the benchmark uses; sampled pairs against the oracle."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    for bits in (3, 4):
        say(f"score full layer random bank b={bits}")
        gpu, orc = both_params(cfg, bits)
        W, npad, _ = gpu.layout(cfg.tokens)
        rb, rn, rr = workloads.random_bank(cfg.cfg_id, cfg.banks, npad, W, 1)
        bank = upload_bank(tq, gpu, rb, rn, rr, cfg.tokens)
        q = workloads.queries(cfg)
        got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
        g = np.random.default_rng(bits)
        for b in g.choice(cfg.banks, 6, replace=False):
            ki = np.concatenate([g.integers(0, cfg.tokens, 250), [0, cfg.tokens - 1]])
            qi = g.integers(0, cfg.G, len(ki))
            ref = oracle.score_pairs(orc, rb[b], rn[b], rr[b], q[b], qi, ki)
            check_scores(got[b, qi, ki], ref, f"bank {b}")


@pytest.mark.parametrize("offset", [0, 1])
def test_score_ring_steady_state_every_output(tq, offset):
    """256 banks x 4100 keys (one work-group per bank, 17 tiles on most waves: the ring's
    steady state with its grouped stores, then a ragged last tile), G = 4, on random bank
    bytes; every score against the oracle. offset = 1 places the score rows 4 bytes off a
    16-byte boundary (the per-tile store path)."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    banks, n = 256, 4100
    gpu, orc = both_params(cfg, 3)
    W, npad, _ = gpu.layout(n)
    rb, rn, rr = workloads.random_bank(cfg.cfg_id, banks, npad, W, 1, layer=5)
    bank = upload_bank(tq, gpu, rb, rn, rr, n)
    q = np.random.default_rng(11).standard_normal((banks, 4, cfg.d)).astype(np.float32)
    flat = torch.full((banks * 4 * n + offset,), float("nan"), dtype=torch.float32, device="cuda")
    scores = flat[offset:].view(banks, 4, n)
    say(f"ring steady state: {banks} x {n}, score offset {offset}")
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda(), scores=scores).cpu().numpy()
    for b in range(banks):
        check_scores(got[b], oracle.score(orc, rb[b], rn[b], rr[b], n, q[b]), f"bank {b}")


@pytest.mark.parametrize("case", ["b3_one_wg", "b3_four_wgs", "b3_offset", "b4_one_wg", "longctx_one_wg"])
def test_score_ring_full_runs_every_output(tq, case):
    """Work-group runs of whole tiles (every key below n, 16 waves with equal runs):
    256 banks x 4096 keys (one work-group per bank) and 64 banks x 16384 keys (four per
    bank), at b = 3 (grouped 16-byte stores; offset: the per-tile stores), b = 4 (3-tile
    ring halves) and two channel groups; random bank bytes, every score against the
    oracle."""
    import torch

    name = "longctx" if case.startswith("longctx") else "decode8b"
    cfg = workloads.CONFIGS[name]
    bits = 4 if case.startswith("b4") else 3
    banks, n = (64, 16384) if case == "b3_four_wgs" else (256, 4096)
    offset = 1 if case == "b3_offset" else 0
    gpu, orc = both_params(cfg, bits)
    W, npad, _ = gpu.layout(n)
    rb, rn, rr = workloads.random_bank(cfg.cfg_id, banks, npad, W, len(orc.spec.groups), layer=6)
    bank = upload_bank(tq, gpu, rb, rn, rr, n)
    q = np.random.default_rng(12).standard_normal((banks, 4, cfg.d)).astype(np.float32)
    flat = torch.full((banks * 4 * n + offset,), float("nan"), dtype=torch.float32, device="cuda")
    scores = flat[offset:].view(banks, 4, n)
    say(f"ring full runs: {case}: {banks} x {n}, b={bits}, score offset {offset}")
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda(), scores=scores).cpu().numpy()
    for b in range(banks):
        check_scores(got[b], oracle.score(orc, rb[b], rn[b], rr[b], n, q[b]), f"bank {b}")


# ------------------------------------------------------------------------------------------
# encoder against the oracle's encoding of the same keys
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_tiny_full(tq, bits):
    """fp32 keys at every codebook width the encoder is compiled for (1, 2, 3 bits + sketch)."""
    cfg = workloads.CONFIGS["tiny"]
    say(f"encode tiny b={bits}")
    _, _, _, rep = _encode_check(tq, cfg, bits, workloads.keys(cfg))
    say("report", rep)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_decode3b_full(tq, bits):
    cfg = workloads.CONFIGS["decode3b"]
    say(f"encode decode3b b={bits}")
    _, _, _, rep = _encode_check(tq, cfg, bits, workloads.keys(cfg))
    say("report", rep)


def test_encode_longctx_two_groups(tq):
    cfg = workloads.CONFIGS["longctx"]
    say("encode longctx two groups")
    _, _, _, rep = _encode_check(tq, cfg, 3, workloads.keys(cfg, n=3000, banks=[0, 5]))
    say("report", rep)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 100])
def test_encode_ragged(tq, n):
    cfg = workloads.CONFIGS["decode8b"]
    say(f"encode ragged n={n}")
    _encode_check(tq, cfg, 4, workloads.keys(cfg, n=n, banks=[3, 4, 5]))


@pytest.mark.parametrize("name", ["longctx", "search"])
def test_encode_degenerate_keys(tq, name):
    """Zero keys, a key zero in one channel group only, and very large / small norms; the
    search shape (d = 768) takes the two-GEMM encoder."""
    cfg = workloads.CONFIGS[name]
    keys = workloads.keys(cfg, n=64, banks=[0])
    keys[0, 3] = 0.0
    if name == "longctx":
        chan = workloads.group_channels(cfg)
        keys[0, 5, chan[:32]] = 0.0
        keys[0, 6, chan[32:]] = 0.0
    else:
        keys[0, 5, :400] = 0.0
    keys[0, 7] *= 1024.0
    keys[0, 8] /= 1024.0
    say(f"encode degenerate keys: {name}")
    gpu, orc, bank, _ = _encode_check(tq, cfg, 3 if name == "longctx" else 4, keys)
    _, _, rr = download_bank(bank)
    assert rr[0, 3] == 0.0


def test_encode_bf16_and_f32_inputs_agree(tq):
    import torch

    cfg = workloads.CONFIGS["decode3b"]
    gpu, _ = both_params(cfg, 3)
    keys = workloads.keys(cfg, n=500)  # bf16-representable values
    out = []
    for dt in (torch.bfloat16, torch.float32):
        bank = tq.Bank(gpu, 2, 500)
        tq.tq_encode(gpu, torch.from_numpy(keys).cuda().to(dt), bank)
        out.append(download_bank(bank))
    for a, b in zip(*out):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_encode_unaligned_keys(tq, dt):
    """Keys at an address that is not a multiple of the vector-load width take the
    tile-per-block encoder instead of the register-resident one: both meet the oracle,
    and their outputs are compared word by word."""
    import torch

    cfg = workloads.CONFIGS["longctx"]
    keys = workloads.keys(cfg, n=700, banks=[1, 2])
    gpu, orc = both_params(cfg, 3)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dense = torch.from_numpy(keys).cuda().to(tdt)
    flat = torch.zeros(dense.numel() + 1, dtype=tdt, device="cuda")
    flat[1:] = dense.reshape(-1)
    shifted = flat[1:].view(dense.shape)
    assert shifted.data_ptr() % 8 != 0
    out = []
    for src in (dense, shifted):
        bank = tq.Bank(gpu, 2, 700)
        tq.tq_encode(gpu, src, bank)
        torch.cuda.synchronize()
        out.append(download_bank(bank))
    say(f"encode unaligned {dt}")
    report = {}
    for b in range(2):
        ref = oracle.encode_trace(orc, keys[b])
        check_encode((out[1][0][b], out[1][1][b], out[1][2][b]), ref, orc, 700, report)
    diff = int((out[0][0] != out[1][0]).sum())
    say("report", report, "words differing between the two encoders:", diff)
    for b in range(2):  # the aligned call meets the oracle too
        check_encode((out[0][0][b], out[0][1][b], out[0][2][b]), oracle.encode_trace(orc, keys[b]), orc, 700)


def test_determinism(tq):
    import torch

    cfg = workloads.CONFIGS["decode3b"]
    gpu, _ = both_params(cfg, 4)
    keys = _dev_keys(cfg, workloads.keys(cfg, n=4000))
    q = torch.from_numpy(workloads.queries(cfg)).cuda()
    res = []
    for _ in range(2):
        bank = tq.Bank(gpu, 2, 4000)
        tq.tq_encode(gpu, keys, bank)
        s = tq.tq_score(gpu, bank, q)
        res.append((download_bank(bank), s.cpu().numpy()))
    for a, b in zip(res[0][0], res[1][0]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(res[0][1], res[1][1])


def test_end_to_end_against_oracle_pipeline(tq):
    """GPU encode + GPU score vs oracle encode + oracle score. Codes may differ inside
    the decision band, so the difference is reported; it must stay rare."""
    import torch

    cfg = workloads.CONFIGS["decode3b"]
    keys = workloads.keys(cfg, n=4096)
    q = workloads.queries(cfg)
    for bits in (3, 4):
        gpu, orc = both_params(cfg, bits)
        bank = tq.Bank(gpu, 2, 4096)
        tq.tq_encode(gpu, _dev_keys(cfg, keys), bank)
        got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
        beyond = 0
        for b in range(2):
            ref = oracle.score(orc, *oracle.encode(orc, keys[b]), 4096, q[b])
            err = np.abs(got[b] - ref)
            beyond += int((err > 1e-4 + 1e-3 * np.abs(ref)).sum())
        say(f"end-to-end b={bits}: {beyond} of {got.size} scores beyond the score tolerance")
        assert beyond <= 1e-3 * got.size


def test_encode_full_decode8b_layer_sampled(tq):
    """Full 8B-class layer encoded on the GPU (64 banks x 32768 bf16 keys, drawn on the
    device); 2048 sampled keys re-encoded by the oracle and compared record by record."""
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    layer = 31
    keys = workloads.keys_device(cfg, layer, "cuda")
    for bits in (3, 4):
        say(f"encode full layer b={bits}")
        gpu, orc = both_params(cfg, bits, layer)
        bank = tq.Bank(gpu, cfg.banks, cfg.tokens)
        tq.tq_encode(gpu, keys, bank)
        g = np.random.default_rng(7 + bits)
        bi = g.integers(0, cfg.banks, 2048)
        ki = g.integers(0, cfg.tokens, 2048)
        ki[:2] = [0, cfg.tokens - 1]
        bt, kt = torch.from_numpy(bi).cuda(), torch.from_numpy(ki).cuda()
        sk = keys[bt, kt].float().cpu().numpy()
        gbits = bank.bits[bt, kt // 16, :, kt % 16].cpu().numpy().view(np.uint32)  # [2048, W]
        gathered = np.ascontiguousarray(gbits.reshape(128, 16, -1).transpose(0, 2, 1))
        gn = bank.norms[bt, kt].cpu().numpy()
        gr = bank.rnorms[bt, kt].cpu().numpy()
        rep = {}
        check_encode((gathered, gn, gr), oracle.encode_trace(orc, sk), orc, 2048, rep)
        say("report", rep)


def test_longctx_full_size_sampled(tq):
    """Long-context workload at full size (8 banks x 131072 bf16 keys, two channel groups
    at 2 and 1 codebook bits, one 128-row sketch): GPU encoding on 2048 sampled keys against
    the oracle's encoding of them, and GPU scores at full size on random bank bytes (every
    byte pattern with positive norms is a valid scorer input) on sampled pairs against the
    oracle's estimates for the same bytes."""
    import torch

    cfg = workloads.CONFIGS["longctx"]
    gpu, orc = both_params(cfg, 3)
    keys = workloads.keys_device(cfg, 0, "cuda")
    q = workloads.queries_device(cfg, 0, "cuda")
    say(f"longctx full size: {cfg.banks} x {cfg.tokens}")
    bank = tq.Bank(gpu, cfg.banks, cfg.tokens)
    tq.tq_encode(gpu, keys, bank)
    scores = tq.tq_score(gpu, bank, q).cpu().numpy()
    g = np.random.default_rng(4)
    bi = g.integers(0, cfg.banks, 2048)
    ki = g.integers(0, cfg.tokens, 2048)
    ki[:2] = [0, cfg.tokens - 1]
    bt, kt = torch.from_numpy(bi).cuda(), torch.from_numpy(ki).cuda()
    sk = keys[bt, kt].float().cpu().numpy()
    gbits = bank.bits[bt, kt // 16, :, kt % 16].cpu().numpy().view(np.uint32)
    gathered = np.ascontiguousarray(gbits.reshape(128, 16, -1).transpose(0, 2, 1))
    rep = {}
    check_encode((gathered, bank.norms[bt, kt].cpu().numpy(), bank.rnorms[bt, kt].cpu().numpy()),
                 oracle.encode_trace(orc, sk), orc, 2048, rep)
    say("report", rep)
    del bank, scores
    W, npad, _ = gpu.layout(cfg.tokens)
    rb, rn, rr = workloads.random_bank(cfg.cfg_id, cfg.banks, npad, W, 2)
    rbank = upload_bank(tq, gpu, rb, rn, rr, cfg.tokens)
    scores = tq.tq_score(gpu, rbank, q).cpu().numpy()
    qh = q.cpu().numpy()
    for b in g.choice(cfg.banks, 4, replace=False):
        kk = np.concatenate([g.integers(0, cfg.tokens, 400), [0, cfg.tokens - 1]])
        qi = g.integers(0, cfg.G, len(kk))
        ref = oracle.score_pairs(orc, rb[b], rn[b], rr[b], qh[b], qi, kk)
        check_scores(scores[b, qi, kk], ref, f"bank {b}")


# ------------------------------------------------------------------------------------------
# streaming append: keys encoded into chosen slots of preallocated banks
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,unaligned", [("longctx", False), ("longctx", True), ("search", False)])
def test_encode_append_slots(tq, name, unaligned):
    """Appends in three calls at different per-bank positions (not multiples of 16), one of
    them running past the capacity; appended slots match the oracle's encoding of their keys
    and every other slot keeps its previous bytes. Unaligned key rows take the
    tile-per-block encoder, aligned ones the persistent one; 768-dimensional vectors (new
    rows of a search database, b = 4) take the tile-per-block encoder."""
    import torch

    cfg = workloads.CONFIGS[name]
    gpu, orc = both_params(cfg, 4 if name == "search" else 3)
    n_cap, banks = 100, 2
    keys = workloads.keys(cfg, n=64, banks=[2, 3])
    bank = tq.Bank(gpu, banks, n_cap)
    bank.bits.fill_(0x5A5A5A5A)
    bank.norms.fill_(-1.0)
    bank.rnorms.fill_(-2.0)
    start = np.array([0, 5], np.int64)
    calls = [(0, 37), (37, 38), (38, 64)]  # [key range) per call
    filled = {0: {}, 1: {}}  # bank -> slot -> key index
    ws = torch.empty(gpu.workspace_bytes(tq.TQ_OP_ENCODE, banks, 64), dtype=torch.uint8, device="cuda")
    for k0, k1 in calls:
        pos = start + k0
        if k0 == 38:
            pos[1] = n_cap - 7  # bank 1: only 7 of these 26 keys fit (the rest are skipped)
        kk = torch.from_numpy(np.ascontiguousarray(keys[:, k0:k1])).cuda()
        if cfg.key_dtype == "bf16":
            kk = kk.to(torch.bfloat16)
        if unaligned:  # the same values at an address that is not a multiple of 8 bytes
            flat = torch.zeros(kk.numel() + 1, dtype=kk.dtype, device="cuda")
            flat[1:] = kk.reshape(-1)
            kk = flat[1:].view(kk.shape)
        say(f"append keys [{k0}, {k1}) at slots {pos.tolist()}")
        # the first call forms S' in the workspace, the later ones reuse it
        tq.tq_encode_append(gpu, kk, bank, torch.from_numpy(pos.astype(np.int32)).cuda(), workspace=ws,
                            prepared=k0 > 0)
        for b in range(banks):
            for j in range(k1 - k0):
                sl = int(pos[b]) + j
                if 0 <= sl < bank.n_pad:
                    filled[b][sl] = k0 + j
    torch.cuda.synchronize()
    gb, gn, gr = download_bank(bank)
    report = {}
    for b in range(banks):
        slots = np.array(sorted(filled[b]), np.int64)
        kidx = np.array([filled[b][s] for s in slots], np.int64)
        # the appended records, gathered into a fresh tile array in slot order
        W = gb.shape[2]
        words = gb[b].transpose(0, 2, 1).reshape(-1, W)[slots]
        n_new = len(slots)
        pad = (-n_new) % 16
        ref = oracle.encode_trace(orc, keys[b][kidx])
        # the gathered array's padding rows are the oracle's (zero-vector records)
        ref_rows = ref[0].transpose(0, 2, 1).reshape(-1, W)
        tiles = np.concatenate([words, ref_rows[n_new:]]).reshape(-1, 16, W).transpose(0, 2, 1)
        check_encode((tiles, np.concatenate([gn[b][slots], np.zeros((pad, gn.shape[2]), np.float32)]),
                      np.concatenate([gr[b][slots], np.zeros(pad, np.float32)])), ref, orc, n_new, report)
        untouched = np.setdiff1d(np.arange(bank.n_pad), slots)
        assert (gb[b].transpose(0, 2, 1).reshape(-1, W)[untouched] == 0x5A5A5A5A).all()
        assert (gn[b][untouched] == -1.0).all() and (gr[b][untouched] == -2.0).all()
    assert len(filled[1]) == 37 + 1 + 7 + (bank.n_pad - n_cap)
    say("report", report)


# ------------------------------------------------------------------------------------------
# variants: randomised Walsh-Hadamard rotation, exact sphere-marginal codebook
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["hadamard", "sphere", "both"])
def test_variant_encode_and_score(tq, variant):
    """The kernels take any orthogonal rotation and any symmetric codebook: encoding and
    scoring with the Walsh-Hadamard rotation and/or the sphere-marginal codebook, each side
    with its own construction of them."""
    import torch

    cfg = workloads.CONFIGS["decode3b"]
    groups = groups_of(cfg, 3)
    d, m, b = cfg.d, cfg.m, groups[0][1]
    gauss = workloads.rotation_gaussians(cfg.cfg_id, [d])
    S = workloads.projection(cfg.cfg_id, m, d)
    signs = np.where(np.random.default_rng(77).random(d) < 0.5, -1.0, 1.0).astype(np.float32)
    had, sph = variant in ("hadamard", "both"), variant in ("sphere", "both")
    gpu = tq.make_params(d, m, groups, gauss, S, None, rotations=[tq.tq_make_rotation_hadamard(signs)] if had else None,
                         codebooks=[tq.tq_make_codebook_sphere(b, d)[:2]] if sph else None)
    orc = oracle.Params(oracle.Spec(d, m, groups, None), gauss, S,
                        rotations=[oracle.hadamard_rotation(signs)] if had else None,
                        codebooks=[oracle.codebook_sphere(b, d)] if sph else None)
    keys = workloads.keys(cfg, n=1500, banks=[0, 1])
    q = workloads.queries(cfg, banks=[0, 1])
    say(f"variant {variant}: encode")
    bank = tq.Bank(gpu, 2, 1500)
    tq.tq_encode(gpu, _dev_keys(cfg, keys), bank)
    torch.cuda.synchronize()
    gb = download_bank(bank)
    rep = {}
    for bk in range(2):
        check_encode((gb[0][bk], gb[1][bk], gb[2][bk]), oracle.encode_trace(orc, keys[bk]), orc, 1500, rep)
    say("report", rep)
    say(f"variant {variant}: score")
    refs = [oracle.encode(orc, keys[bk]) for bk in range(2)]
    ob = upload_bank(tq, gpu, np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs]),
                     np.stack([r[2] for r in refs]), 1500)
    got = tq.tq_score(gpu, ob, torch.from_numpy(q).cuda()).cpu().numpy()
    for bk in range(2):
        check_scores(got[bk], oracle.score(orc, *refs[bk], 1500, q[bk]), f"bank {bk}")
