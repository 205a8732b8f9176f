"""The allocation-free append (tq_encode_append_noalloc) against tq_encode_append, through
the C ABI: two calls in a row, the second smaller, on the persistent encoder (aligned keys,
float32 and binary16 norms, one and two channel groups) and on the tile encoder (unaligned
keys). Both entry points run the same kernels on the same inputs, so every byte of the two
banks must be equal; the first call's records are also checked against the oracle."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import both_params, check_encode, download_bank

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


def _keys_on_device(keys, dtype, unaligned):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(keys)).cuda().to(dtype)
    if unaligned:  # the same values at an address that is not a multiple of 8 bytes
        flat = torch.zeros(t.numel() + 1, dtype=dtype, device="cuda")
        flat[1:] = t.reshape(-1)
        t = flat[1:].view(t.shape)
    return t


@pytest.mark.parametrize("cfg_name,bits,norm16,unaligned,f32", [
    ("decode8b", 3, False, False, False),   # the decode-step shape: persistent encoder
    ("decode8b", 4, True, False, False),    # binary16 norms
    ("longctx", 3, False, False, True),     # two permuted channel groups, float32 keys
    ("decode3b", 3, False, True, False),    # unaligned rows: the tile encoder
])
def test_noalloc_append_equals_the_workspace_append(tq, cfg_name, bits, norm16, unaligned, f32):
    import torch

    cfg = workloads.CONFIGS[cfg_name]
    gpu, orc = both_params(cfg, bits, norm16=norm16)
    banks, n_cap = 6, 200
    dtype = torch.float32 if f32 else torch.bfloat16
    keys = workloads.keys(cfg, n=40, banks=range(banks))
    ref_bank = tq.Bank(gpu, banks, n_cap)
    got_bank = tq.Bank(gpu, banks, n_cap)
    for bk in (ref_bank, got_bank):
        bk.bits.fill_(0x3C3C3C3C)
        bk.norms.fill_(-1.0)
        bk.rnorms.fill_(-2.0)
    ws = torch.empty(gpu.workspace_bytes(tq.TQ_OP_ENCODE, banks, 40), dtype=torch.uint8, device="cuda")
    # call 1: 40 keys per bank at per-bank slots; call 2: 9 keys (a smaller input) elsewhere,
    # one bank partly past the capacity
    calls = [(0, 40, np.array([0, 7, 33, 100, 150, 3], np.int32)),
             (40 - 9, 40, np.array([60, 90, 5, 170, n_cap - 4, 120], np.int32))]
    for i, (k0, k1, pos) in enumerate(calls):
        kk = _keys_on_device(keys[:, k0:k1], dtype, unaligned)
        pd = torch.from_numpy(pos).cuda()
        say(f"{cfg_name} b={bits} norm16={norm16} unaligned={unaligned}: call {i}, {k1 - k0} keys at {pos.tolist()}")
        tq.tq_encode_append(gpu, kk, ref_bank, pd, workspace=ws)
        tq.tq_encode_append_noalloc(gpu, kk, got_bank, pd)
        torch.cuda.synchronize()
        for a, b in zip(download_bank(ref_bank), download_bank(got_bank)):
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))
        if i == 0:
            # the appended records of bank 0 (slots 0..39) against the oracle's encoding
            gb, gn, gr = download_bank(got_bank)
            ref = oracle.encode_trace(orc, keys[0, :40])
            W = gb.shape[2]
            rows = gb[0].transpose(0, 2, 1).reshape(-1, W)[:48].copy()
            rows[40:] = ref[0].transpose(0, 2, 1).reshape(-1, W)[40:48]
            tiles = rows.reshape(3, 16, W).transpose(0, 2, 1)
            nrm = np.concatenate([gn[0][:40], ref[1][40:48].astype(gn.dtype)])
            rn = np.concatenate([gr[0][:40], ref[2][40:48].astype(gr.dtype)])
            rep = {}
            check_encode((tiles, nrm, rn), ref, orc, 40, rep)
            say("   oracle report", rep)


def test_noalloc_append_rejects_layouts_beyond_its_array(tq):
    import torch

    cfg = workloads.CONFIGS["search"]
    gpu, _ = both_params(cfg, 2)
    bank = tq.Bank(gpu, 1, 32)
    keys = torch.zeros((1, 4, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_encode_append_noalloc(gpu, keys, bank, torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert e.value.code == tq.TQ_ERR_UNSUPPORTED
