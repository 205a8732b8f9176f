"""The measurement kernels against plain references, through the C ABI: the fp32
unquantized-key logits (the comparator the benchmark times beside the packed scorer)
against fp64 inner products of the same fp32 values, and the device copy."""
import sys

import numpy as np
import pytest

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


@pytest.mark.parametrize("banks,n,d,G", [
    (3, 1000, 128, 4), (2, 17, 128, 4), (1, 1, 128, 4), (5, 4099, 128, 3), (2, 32, 128, 1),  # streaming kernel
    (64, 2048, 128, 4),                                                                     # many waves per bank
    (2, 333, 64, 8), (1, 100, 256, 4),                                                      # staged kernel
])
def test_fp32_logits_are_the_inner_products(tq, banks, n, d, G):
    import torch

    say(f"fp32 logits banks={banks} n={n} d={d} G={G}")
    g = np.random.default_rng(n + 7 * d + G)
    keys = g.standard_normal((banks, n, d)).astype(np.float32) * g.uniform(0.1, 3, (1, 1, d)).astype(np.float32)
    q = g.standard_normal((banks, G, d)).astype(np.float32)
    got = tq.tq_fp32_logits(torch.from_numpy(keys).cuda(), torch.from_numpy(q).cuda()).cpu().numpy()
    ref = np.einsum("bgc,bnc->bgn", q.astype(np.float64), keys.astype(np.float64))
    mag = np.einsum("bgc,bnc->bgn", np.abs(q).astype(np.float64), np.abs(keys).astype(np.float64))
    # fp32 sums of d products: each term rounded at most about log2(d) + 2 times
    bound = (np.log2(d) + 3) * 2.0 ** -24 * mag
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"max excess {np.max(err - bound):.3e}"


def test_copy_moves_the_bytes(tq):
    import torch

    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    tq.tq_copy(src[: 12345 * 4], dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[: 12345 * 4], src[: 12345 * 4]) and (dst[12345 * 4:] == 0).all()
