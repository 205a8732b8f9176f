"""GPU top-k and the large-operand scorer (vector-search shapes, many queries) against
the CPU oracle, through the C ABI. Small cases are compared on oracle-encoded banks
(identical bank bytes on both sides); the full 2,000,000 x 768 database is encoded on
the GPU and checked on sampled queries, the oracle scoring every key of the GPU's bank
for them."""
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


def _oracle_bank(tq, cfg, bits, keys, layer=0):
    gpu, orc = both_params(cfg, bits, layer)
    refs = [oracle.encode(orc, keys[b]) for b in range(keys.shape[0])]
    bank = upload_bank(tq, gpu, np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs]),
                       np.stack([r[2] for r in refs]), keys.shape[1])
    return gpu, orc, refs, bank


@pytest.mark.parametrize("bits", [2, 4])
def test_encode_search_small(tq, bits):
    """768-dimensional unit vectors: GPU encoding against the oracle's, record by record."""
    import torch

    cfg = workloads.CONFIGS["search"]
    n = 301
    say(f"encode search-shaped d=768 b={bits} n={n}")
    keys = workloads.keys(cfg, n=n)
    gpu, orc = both_params(cfg, bits)
    bank = tq.Bank(gpu, 1, n)
    tq.tq_encode(gpu, torch.from_numpy(keys).cuda(), bank)
    gb = download_bank(bank)
    rep = {}
    check_encode((gb[0][0], gb[1][0], gb[2][0]), oracle.encode_trace(orc, keys[0]), orc, n, rep)
    say("   report", rep)


@pytest.mark.parametrize("bits,n,G,k", [(4, 5003, 37, 10), (2, 3001, 9, 10), (4, 700, 5, 64), (2, 900, 3, 1),
                                        (4, 33, 5, 10), (2, 40, 6, 7)])
def test_topk_search_small(tq, bits, n, G, k):
    import torch

    cfg = workloads.CONFIGS["search"]
    say(f"topk search-shaped: d=768 b={bits} n={n} G={G} k={k}")
    keys = workloads.keys(cfg, n=n)
    q = workloads.queries(cfg, G=G)
    gpu, orc, refs, bank = _oracle_bank(tq, cfg, bits, keys)
    vals, idx = tq.tq_topk(gpu, bank, torch.from_numpy(q).cuda(), k)
    ref = oracle.score(orc, *refs[0], n, q[0])
    same = check_topk(vals.cpu().numpy()[0], idx.cpu().numpy()[0], ref, k)
    say(f"   returned indices equal to the oracle's top-{k}: {same:.4f}")


def test_topk_several_banks_decode_shapes(tq):
    import torch

    cfg = workloads.CONFIGS["decode8b"]
    n, k = 1000, 10
    say("topk decode-shaped banks: 3 banks x 1000, G=4, b=3")
    keys = workloads.keys(cfg, n=n, banks=[0, 9, 17])
    q = workloads.queries(cfg, banks=[0, 9, 17])
    gpu, orc, refs, bank = _oracle_bank(tq, cfg, 3, keys)
    vals, idx = tq.tq_topk(gpu, bank, torch.from_numpy(q).cuda(), k)
    for b in range(3):
        ref = oracle.score(orc, *refs[b], n, q[b])
        check_topk(vals.cpu().numpy()[b], idx.cpu().numpy()[b], ref, k, f"bank {b}")


def test_topk_ties_by_lower_index(tq):
    """Duplicate keys give equal estimates: the lower index must come first."""
    import torch

    cfg = workloads.CONFIGS["search"]
    n, k = 640, 12
    keys = workloads.keys(cfg, n=n)
    keys[0, 300:310] = keys[0, 5]  # ten copies of key 5 later in the bank
    q = workloads.queries(cfg, G=4)
    q[0, 0] = keys[0, 5]  # a query whose best match is key 5 and its copies
    gpu, orc, refs, bank = _oracle_bank(tq, cfg, 4, keys)
    vals, idx = tq.tq_topk(gpu, bank, torch.from_numpy(q).cuda(), k)
    ref = oracle.score(orc, *refs[0], n, q[0])
    check_topk(vals.cpu().numpy()[0], idx.cpu().numpy()[0], ref, k)
    first = idx.cpu().numpy()[0, 0, :11].tolist()
    assert first == [5] + list(range(300, 310)), first


@pytest.mark.parametrize("cfg_name,bits,n,G", [("decode3b", 3, 777, 40), ("search", 4, 1500, 4), ("search", 2, 333, 21),
                                              ("search", 4, 1, 4), ("search", 4, 17, 6)])
def test_score_large_operands(tq, cfg_name, bits, n, G):
    """tq_score where the operands go through LDS: more than 16 queries per bank, or
    768-dimensional keys (down to one key: most waves get no tile, the one batch is partial)."""
    import torch

    cfg = workloads.CONFIGS[cfg_name]
    say(f"score {cfg_name} b={bits} n={n} G={G}")
    banks = [0] if cfg.banks == 1 else [0, 1]
    keys = workloads.keys(cfg, n=n, banks=banks)
    q = workloads.queries(cfg, banks=banks, G=G)
    gpu, orc, refs, bank = _oracle_bank(tq, cfg, bits, keys)
    got = tq.tq_score(gpu, bank, torch.from_numpy(q).cuda()).cpu().numpy()
    for b in range(len(banks)):
        say("   max err", check_scores(got[b], oracle.score(orc, *refs[b], n, q[b]), f"bank {b}"))


@pytest.mark.parametrize("bits", [4, 2])
def test_topk_full_search_sampled(tq, bits):
    """Full search size: 2,000,000 x 768, 1024 queries, top-10. The GPU encodes the unit
    vectors and its top-10's recall@10 against the exact inner products is reported (no pin:
    the pages print none). Parity at full size runs on random database bytes of the same
    layout (any byte pattern with positive norms is a valid scorer input): the GPU top-10
    against the oracle's estimates of all 2,000,000 keys for sampled queries."""
    import torch

    cfg = workloads.CONFIGS["search"]
    n, k = cfg.tokens, cfg.topk
    say(f"full search b={bits}: {n} x {cfg.d}, G={cfg.G}, k={k}")
    gpu, orc = both_params(cfg, bits)
    keys = workloads.keys_device(cfg, 0, "cuda")
    q = workloads.queries_device(cfg, 0, "cuda")
    bank = tq.Bank(gpu, 1, n)
    tq.tq_encode(gpu, keys, bank)
    vals, idx = tq.tq_topk(gpu, bank, q, k)
    torch.cuda.synchronize()
    # recall@10 against exact fp32 inner products
    exact = torch.topk(q[0] @ keys[0].T, k, dim=1).indices
    hits = (idx[0].long()[:, :, None] == exact[:, None, :]).any(dim=2).float().mean().item()
    say(f"   recall@{k} vs exact inner products: {hits:.4f}")
    del keys, bank
    torch.cuda.empty_cache()
    W, npad, _ = gpu.layout(n)
    rb, rn, rr = workloads.random_bank(cfg.cfg_id, 1, npad, W, 1, layer=bits)
    rbank = upload_bank(tq, gpu, rb, rn, rr, n)
    vals, idx = tq.tq_topk(gpu, rbank, q, k)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    g = np.random.default_rng(bits)
    for qi in g.choice(cfg.G, 6, replace=False):
        ref = oracle.score(orc, rb[0], rn[0], rr[0], n, qh[0, qi:qi + 1])
        same = check_topk(vals.cpu().numpy()[0, qi:qi + 1], idx.cpu().numpy()[0, qi:qi + 1], ref, k, f"query {qi}")
        say(f"   query {qi}: overlap with the oracle's top-{k} {same:.2f}")


def _sample_rows(n, chunk, count, seed):
    """Rows to check in a bank of n keys: the first and last, both sides of every
    residual-chunk boundary of the large-key encoder, then seeded random rows up to
    `count` (a multiple of 16), sorted."""
    rows = {0, n - 1}
    for b in range(chunk, n, chunk):
        rows.update((b - 1, b))
    g = np.random.default_rng(seed)
    while len(rows) < count:
        rows.update(g.integers(0, n, count - len(rows)).tolist())
    return np.array(sorted(rows)[:count], np.int64)


@pytest.mark.parametrize("bits", [2, 4])
def test_encode_full_search_sampled(tq, bits):
    """The full 2,000,000 x 768 search database encoded by the GPU (the launch sequence the
    benchmark times: 62 residual chunks of 32768 rows); 2048 rows, including the first, the
    last and both sides of every chunk boundary, re-encoded by the oracle and compared
    record by record (codes within the decision band, signs, norms)."""
    import torch

    cfg = workloads.CONFIGS["search"]
    n = cfg.tokens
    say(f"encode full search b={bits}: {n} x {cfg.d}")
    gpu, orc = both_params(cfg, bits)
    keys = workloads.keys_device(cfg, 0, "cuda")
    bank = tq.Bank(gpu, 1, n)
    tq.tq_encode(gpu, keys, bank)
    torch.cuda.synchronize()
    rows = _sample_rows(n, 32768, 2048, 500 + bits)
    assert len(rows) == 2048 and rows[0] == 0 and rows[-1] == n - 1
    r = torch.from_numpy(rows).cuda()
    # the sampled records gathered into a compact bank of 2048 keys (128 whole tiles)
    W = bank.W
    sb = bank.bits[0][r // 16, :, r % 16].reshape(128, 16, W).permute(0, 2, 1).contiguous()
    sub = (sb.cpu().numpy().view(np.uint32), bank.norms[0][r].cpu().numpy(), bank.rnorms[0][r].cpu().numpy())
    kh = keys[0][r].cpu().numpy()
    del keys, bank
    torch.cuda.empty_cache()
    rep = {}
    check_encode(sub, oracle.encode_trace(orc, kh), orc, len(rows), rep)
    say("   report", rep)


# ------------------------------------------------------------------------------------------
# encoder for keys above 128 dimensions (tiled two-GEMM path): partial tiles, two channel
# groups with a channel permutation, bf16 and fp32 keys, several residual chunks
# ------------------------------------------------------------------------------------------

def _large_cfg(d, m, groups, key_dtype, cfg_id):
    import dataclasses

    base = workloads.CONFIGS["longctx"] if groups else workloads.CONFIGS["decode8b"]
    extra = dict(outliers=groups[0][0], groups=groups) if groups else {}
    return dataclasses.replace(base, d=d, m=m, key_dtype=key_dtype, cfg_id=cfg_id, **extra)


def _encode_vs_oracle(tq, cfg, bits, keys):
    import torch

    gpu, orc = both_params(cfg, bits)
    banks, n = keys.shape[0], keys.shape[1]
    bank = tq.Bank(gpu, banks, n)
    t = torch.from_numpy(np.ascontiguousarray(keys)).cuda()
    tq.tq_encode(gpu, t.to(torch.bfloat16) if cfg.key_dtype == "bf16" else t, bank)
    torch.cuda.synchronize()
    gb = download_bank(bank)
    rep = {}
    for b in range(banks):
        check_encode((gb[0][b], gb[1][b], gb[2][b]), oracle.encode_trace(orc, keys[b]), orc, n, rep)
    return rep


@pytest.mark.parametrize("d,m,groups,dt", [
    (256, 160, ((64, 3), (192, 2)), "bf16"),  # two groups, permuted channels, partial row tile
    (160, 288, None, "f32"),                  # partial coordinate and row tiles, fp32 keys
    (256, 128, ((96, 2), (160, 3)), "f32"),   # d above 128 with m at 128
    (128, 256, None, "bf16"),                 # m above 128 with d at 128
])
def test_encode_large_keys(tq, d, m, groups, dt):
    cfg = _large_cfg(d, m, groups, dt, 60 + d // 32 + m // 32)
    keys = workloads.keys(cfg, n=1500, banks=[0, 1])
    say(f"encode large keys d={d} m={m} groups={groups} {dt}")
    bits = 3 if groups is None else cfg.bits[0]
    say("   report", _encode_vs_oracle(tq, cfg, bits, keys))


def test_encode_large_keys_several_chunks(tq):
    """More key rows than one residual chunk (32768): the chunk boundary falls inside a bank."""
    cfg = _large_cfg(256, 256, None, "bf16", 71)
    keys = workloads.keys(cfg, n=11111, banks=[0, 1, 2])
    say("encode large keys, 3 x 11111 keys (two residual chunks)")
    say("   report", _encode_vs_oracle(tq, cfg, 3, keys))


@pytest.mark.parametrize("op", ["topk", "score"])
def test_side_stream_results_survive_default_stream_allocations(tq, op):
    """A call on a side stream allocates its workspace and outputs on that stream: memory
    the default stream allocates and overwrites while the kernels still run must not be
    the call's workspace (a block freed to the current stream's pool could be)."""
    import torch

    cfg = workloads.CONFIGS["search"]
    n, G, k, bits = 60000, 40, 10, 4
    say(f"side stream {op}: d=768 b={bits} n={n} G={G}")
    keys = workloads.keys(cfg, n=n)
    q = workloads.queries(cfg, G=G)
    gpu, orc, refs, bank = _oracle_bank(tq, cfg, bits, keys)
    qd = torch.from_numpy(q).cuda()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws_bytes = gpu.workspace_bytes(tq.TQ_OP_TOPK if op == "topk" else tq.TQ_OP_SCORE, 1, n, G, k)
    outs = []
    for rep in range(3):
        if op == "topk":
            outs.append(tq.tq_topk(gpu, bank, qd, k, stream=side))
        else:
            outs.append((tq.tq_score(gpu, bank, qd, stream=side),))
        # while the side stream runs: allocate and scribble on the default stream
        for _ in range(4):
            junk = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
            junk.fill_(0xA5)
            junk2 = torch.empty((1, G, max(k, n)), dtype=torch.float32, device="cuda")
            junk2.fill_(-1e30)
            del junk, junk2
    torch.cuda.synchronize()
    ref = oracle.score(orc, *refs[0], n, q[0])
    for o in outs:
        if op == "topk":
            check_topk(o[0].cpu().numpy()[0], o[1].cpu().numpy()[0], ref, k)
        else:
            check_scores(o[0].cpu().numpy()[0], ref)
