"""Host-side checks of libtq.so that need no GPU: exported symbols, the host
parameter builders against the oracle's independent implementations, bank
geometry, workspace planning and argument validation (no kernel is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    from kv_cache_inner_amd import build as b

    if not os.path.exists(b.LIB):
        b.build()
    import kv_cache_inner_amd as tq

    return tq


def _declared_functions():
    txt = open(os.path.join(ROOT, "include", "tq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol(tq):
    names = _declared_functions()
    assert len(names) == 18
    lib = ctypes.CDLL(tq.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm
    assert sorted(tq.EXPORTS) == names


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle(tq, bits):
    c, t, mse = tq.tq_make_codebook(bits)
    oc, ot, omse, _ = oracle.codebook(bits)
    np.testing.assert_array_equal(c, oc.astype(np.float32))
    np.testing.assert_allclose(t, ot.astype(np.float32), atol=1e-7)
    assert abs(mse - omse) < 1e-12
    np.testing.assert_array_equal(c, -c[::-1])
    np.testing.assert_array_equal(t, -t[::-1])


@pytest.mark.parametrize("d", [32, 96, 128, 768])
def test_rotation_matches_oracle(tq, d):
    G = np.random.default_rng(1000 + d).standard_normal((d, d)).astype(np.float32)
    R = tq.tq_make_rotation(G)
    Ro = oracle.rotation(G)
    assert np.abs(R.astype(np.float64) - Ro).max() < 1e-6
    assert np.abs(R.astype(np.float64) @ R.T.astype(np.float64) - np.eye(d)).max() < 1e-5


def test_rotation_rejects_rank_deficient(tq):
    G = np.ones((32, 32), np.float32)
    with pytest.raises(tq.TQError) as e:
        tq.tq_make_rotation(G)
    assert e.value.code == tq.TQ_ERR_ARG


def _params(tq, d=128, m=128, groups=((128, 2),), codebooks=None):
    return tq.Params(d, m, groups, rot=None, proj=None, codebooks=codebooks)


class _FakePtr:
    def __init__(self, v):
        self.v = v

    def data_ptr(self):
        return self.v


def _with_fake_ptrs(tq, **kw):
    p = _params(tq, **kw)
    p.struct.rot = 0x10000
    p.struct.proj = 0x20000
    return p


@pytest.mark.parametrize("groups,m,W,bpk", [
    (((128, 2),), 128, 12, 56),     # d=128, b=3 (2-bit codebook + sketch)
    (((128, 3),), 128, 16, 72),     # d=128, b=4
    (((32, 2), (96, 1)), 128, 9, 48),  # two groups, 2.25 bits/channel of codes+sketch
    (((768, 1),), 768, 48, 200),    # search, b=2
    (((768, 3),), 768, 96, 392),    # search, b=4
])
def test_bank_geometry(tq, groups, m, W, bpk):
    d = sum(g[0] for g in groups)
    p = _with_fake_ptrs(tq, d=d, m=m, groups=groups)
    w, npad, b = p.layout(1000)
    assert (w, npad, b) == (W, 1008, bpk)
    assert p.layout(0)[1] == 0 and p.layout(16)[1] == 16 and p.layout(17)[1] == 32


@pytest.mark.parametrize("groups,m,W,bpk", [
    (((128, 2),), 128, 12, 52),        # d=128, b=3 with binary16 norms: 4 bytes fewer per key
    (((32, 2), (96, 1)), 128, 9, 42),  # two groups: two norms and the residual norm, 2 bytes each
    (((256, 2),), 256, 24, 100),       # keys above 128 dimensions (the two-GEMM encoder)
    (((768, 3),), 768, 96, 388),       # the search layout at b = 4
])
def test_bank_geometry_with_half_norms(tq, groups, m, W, bpk):
    d = sum(g[0] for g in groups)
    p = _with_fake_ptrs(tq, d=d, m=m, groups=groups)
    p.struct.norm_dtype = tq.TQ_F16
    assert p.layout(1000) == (W, 1008, bpk)


def test_workspace_sizes(tq):
    p = _with_fake_ptrs(tq)
    assert p.workspace_bytes(tq.TQ_OP_ENCODE, 4, 100) == 128 * 128 * 4
    s = p.workspace_bytes(tq.TQ_OP_SCORE, 64, 32768, 4)
    assert s > 0 and s % 256 == 0
    assert p.workspace_bytes(tq.TQ_OP_SCORE, 64, 32768, 0) == 0
    assert p.workspace_bytes(tq.TQ_OP_TOPK, 1, 1000, 16, 10) > p.workspace_bytes(tq.TQ_OP_SCORE, 1, 1000, 16)
    assert p.workspace_bytes(tq.TQ_OP_TOPK, 1, 1000, 16, 65) == 0
    # search shapes: the top-k partial lists come on top of the query operands
    v = _with_fake_ptrs(tq, d=768, m=768, groups=((768, 3),))
    t = v.workspace_bytes(tq.TQ_OP_TOPK, 1, 2_000_000, 1024, 10)
    assert t > v.workspace_bytes(tq.TQ_OP_SCORE, 1, 2_000_000, 1024) and t % 256 == 0
    assert v.workspace_bytes(tq.TQ_OP_TOPK, 1, 2_000_000, 1024, 64) > t
    # a valid shape without a compiled scorer layout
    q = _with_fake_ptrs(tq, d=160, m=128, groups=((160, 2),))
    assert q.workspace_bytes(tq.TQ_OP_SCORE, 1, 100, 4) == 0


def test_search_key_chunks_stay_within_a_32bit_byte_range(tq):
    """The search kernel reads a work-group's key chunk through one buffer resource (a
    32-bit byte range), so the plan must split a bank into chunks of at most 2 GiB of bit
    words. The top-k workspace beyond the query operands (two partial lists of k entries per
    wave, 8 waves per work-group, per chunk) gives the chunk count the plan chose."""
    v = _with_fake_ptrs(tq, d=768, m=768, groups=((768, 3),))  # 96 words = 384 B per key
    G, k = 8192, 10  # 1024 query blocks: on its own the plan would keep one chunk per bank
    per_chunk = 2 * G * 8 * k * 4
    for n, want in ((1_000_000, 1), (4_000_000, 1), (6_000_000, 2), (12_000_000, 3)):
        extra = v.workspace_bytes(tq.TQ_OP_TOPK, 1, n, G, k) - v.workspace_bytes(tq.TQ_OP_SCORE, 1, n, G)
        assert extra % per_chunk == 0
        kc = extra // per_chunk
        chunk_tiles = -(-(-(-n // 16)) // kc)
        assert chunk_tiles * 96 * 64 <= 2**31 - 1, (n, kc)
        assert kc == want, (n, kc)


def _rc(fn, *a):
    return fn(*a)


def test_argument_validation_returns_before_any_launch(tq):
    L = tq._lib.lib()
    good = _with_fake_ptrs(tq)
    bank = tq.tq_bank(0x30000, 0x40000, 0x50000)
    nullbank = tq.tq_bank(None, None, None)
    # invalid parameter structs
    def patched(**fields):
        p = _with_fake_ptrs(tq)
        for k, v in fields.items():
            if k in ("group_dim", "group_bits"):
                getattr(p.struct, k)[0] = v
            else:
                setattr(p.struct, k, v)
        return p

    for p in [patched(d=100, group_dim=100), patched(m=100), patched(m=16), patched(group_bits=4),
              patched(group_bits=0), patched(group_dim=64), patched(n_groups=3), patched(d=2048, group_dim=2048)]:
        assert L.tq_encode(p.ref, 0x1000, 0, 1, 10, ctypes.byref(bank), 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
        assert L.tq_score(p.ref, ctypes.byref(bank), 1, 10, 0x1000, 4, 0x2000, 0x3000, 1 << 20, None) == tq.TQ_ERR_ARG
    # m = 0 (codes and norms only) is a valid encoding but has no estimator
    mse_only = patched(m=0)
    assert L.tq_bank_layout(mse_only.ref, 10, None, None, None) == tq.TQ_OK
    assert L.tq_score(mse_only.ref, ctypes.byref(bank), 1, 10, 0x1000, 4, 0x2000, 0x3000, 1 << 20,
                      None) == tq.TQ_ERR_UNSUPPORTED
    # missing matrices
    p = _params(tq)
    assert L.tq_bank_layout(p.ref, 10, None, None, None) == tq.TQ_ERR_ARG
    # asymmetric codebook: valid but unsupported by the kernels
    c, t, _ = tq.tq_make_codebook(2)
    c2 = c.copy()
    c2[0] -= 0.01
    asym = _params(tq, codebooks=[(c2, t)])
    asym.struct.rot, asym.struct.proj = 0x10000, 0x20000
    assert L.tq_bank_layout(asym.ref, 10, None, None, None) == tq.TQ_ERR_UNSUPPORTED
    # thresholds outside their cells
    t2 = t.copy()
    t2[0] = c[0] - 1
    bad = _params(tq, codebooks=[(c, t2)])
    bad.struct.rot, bad.struct.proj = 0x10000, 0x20000
    assert L.tq_bank_layout(bad.ref, 10, None, None, None) == tq.TQ_ERR_ARG
    # null buffers, negative sizes, bad dtype, bad k, workspace too small
    assert L.tq_encode(good.ref, None, 0, 1, 10, ctypes.byref(bank), 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_encode(good.ref, 0x1000, 0, 1, 10, ctypes.byref(nullbank), 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_encode(good.ref, 0x1000, 7, 1, 10, ctypes.byref(bank), 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_encode(good.ref, 0x1000, 0, -1, 10, ctypes.byref(bank), 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_encode(good.ref, 0x1000, 0, 1, 10, ctypes.byref(bank), 0x2000, 16, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_encode(good.ref, 0x1000, 0, 1, 10, ctypes.byref(bank), 0x2001, 1 << 20, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_score(good.ref, ctypes.byref(bank), 1, 10, None, 4, 0x2000, 0x3000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_score(good.ref, ctypes.byref(bank), 1, 10, 0x1000, 0, 0x2000, 0x3000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_prepare_queries(good.ref, 0x1000, 1, 4, 0x3000, 8, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_prepare_queries(good.ref, 0x1000, 1, 4, 0x3001, 1 << 20, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, 10, 0x1000, 4, 11, 0x2000, 0x3000, 0x4000, 1 << 20,
                     None) == tq.TQ_ERR_ARG
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, 100, 0x1000, 4, 0, 0x2000, 0x3000, 0x4000, 1 << 20,
                     None) == tq.TQ_ERR_ARG
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, 100, 0x1000, 4, 65, 0x2000, 0x3000, 0x4000, 1 << 20,
                     None) == tq.TQ_ERR_ARG
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, 100, 0x1000, 4, 10, 0x2000, 0x3000, 0x4000, 64,
                     None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, 100, 0x1000, 4, 10, 0x2000, 0x3000, 0x4001, 1 << 20,
                     None) == tq.TQ_ERR_WORKSPACE
    # top-k returns int32 key indices: a bank of more than INT32_MAX keys is refused
    # (about 155 GB at d = 128, b = 3: it would fit in device memory)
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, 1 << 31, 0x1000, 4, 10, 0x2000, 0x3000, 0x4000, 1 << 40,
                     None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_topk(good.ref, ctypes.byref(bank), 1, (1 << 31) - 1, 0x1000, 4, 10, 0x2000, 0x3000, 0x4000, 64,
                     None) == tq.TQ_ERR_WORKSPACE
    # append: null keys or positions, negative sizes, bad dtype, small or misaligned workspace
    A = L.tq_encode_append
    assert A(good.ref, None, 0, 1, 1, 0x6000, 100, ctypes.byref(bank), 0, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert A(good.ref, 0x1000, 0, 1, 1, None, 100, ctypes.byref(bank), 0, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert A(good.ref, 0x1000, 0, 1, -1, 0x6000, 100, ctypes.byref(bank), 0, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert A(good.ref, 0x1000, 0, 1, 1, 0x6000, -5, ctypes.byref(bank), 0, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert A(good.ref, 0x1000, 3, 1, 1, 0x6000, 100, ctypes.byref(bank), 0, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert A(good.ref, 0x1000, 0, 1, 1, 0x6000, 100, ctypes.byref(nullbank), 0, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    assert A(good.ref, 0x1000, 0, 1, 1, 0x6000, 100, ctypes.byref(bank), 0, 0x2000, 64, None) == tq.TQ_ERR_WORKSPACE
    assert A(good.ref, 0x1000, 0, 1, 1, 0x6000, 100, ctypes.byref(bank), 0, 0x2010, 1 << 20, None) == tq.TQ_ERR_WORKSPACE
    assert A(good.ref, None, 0, 4, 0, None, 100, ctypes.byref(nullbank), 0, None, 0, None) == tq.TQ_OK
    assert A(good.ref, 0x1000, 0, 1, 1, 0x6000, 100, ctypes.byref(bank), 2, 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    # the no-allocation append: the same checks, and layouts beyond its device array refused
    N = L.tq_encode_append_noalloc
    assert N(good.ref, None, 0, 1, 1, 0x6000, 100, ctypes.byref(bank), None) == tq.TQ_ERR_ARG
    assert N(good.ref, 0x1000, 0, 1, 1, None, 100, ctypes.byref(bank), None) == tq.TQ_ERR_ARG
    assert N(good.ref, 0x1000, 3, 1, 1, 0x6000, 100, ctypes.byref(bank), None) == tq.TQ_ERR_ARG
    assert N(good.ref, 0x1000, 0, 1, 1, 0x6000, 100, ctypes.byref(nullbank), None) == tq.TQ_ERR_ARG
    assert N(good.ref, None, 0, 4, 0, None, 100, ctypes.byref(nullbank), None) == tq.TQ_OK
    for big in (_with_fake_ptrs(tq, d=256, m=128, groups=((256, 2),)),
                _with_fake_ptrs(tq, d=128, m=256, groups=((128, 2),)),
                _with_fake_ptrs(tq, d=768, m=768, groups=((768, 3),))):
        assert N(big.ref, 0x1000, 0, 1, 1, 0x6000, 100, ctypes.byref(bank), None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_fp32_logits(None, 1, 10, 128, 0x1000, 4, 0x2000, None) == tq.TQ_ERR_ARG
    assert L.tq_copy(0x1001, 0x2000, 64, None) == tq.TQ_ERR_ARG
    # decompression and attention: value params are MSE-only (m = 0), d_v <= 128
    vals = patched(m=0)
    D, At = L.tq_decode, L.tq_attend
    assert D(good.ref, ctypes.byref(nullbank), 1, 10, 0x7000, None) == tq.TQ_ERR_ARG
    assert D(good.ref, ctypes.byref(bank), 1, 10, None, None) == tq.TQ_ERR_ARG
    assert D(good.ref, ctypes.byref(bank), -1, 10, 0x7000, None) == tq.TQ_ERR_ARG
    assert D(patched(m=16).ref, ctypes.byref(bank), 1, 10, 0x7000, None) == tq.TQ_ERR_ARG
    assert D(vals.ref, ctypes.byref(nullbank), 0, 10, None, None) == tq.TQ_OK
    assert D(vals.ref, ctypes.byref(nullbank), 3, 0, None, None) == tq.TQ_OK
    kb, vb = ctypes.byref(bank), ctypes.byref(tq.tq_bank(0x60000, 0x70000, None))
    need = good.workspace_bytes(tq.TQ_OP_ATTEND, 2, 100, 4)
    assert need > good.workspace_bytes(tq.TQ_OP_SCORE, 2, 100, 4) and need % 256 == 0
    assert vals.workspace_bytes(tq.TQ_OP_ATTEND, 2, 100, 4) == 0  # no estimator for the logits
    assert good.workspace_bytes(tq.TQ_OP_ATTEND, 2, 0, 4) == 0
    def att(kp=good, keys=kb, vp=vals, values=vb, banks=2, n=100, q=0x1000, G=4, scale=0.125, out=0x8000,
            ws=0x100000, ws_bytes=need):
        return At(kp.ref, keys, vp.ref, values, banks, n, None, q, G, scale, out, ws, ws_bytes, None)
    assert att(kp=vals) == tq.TQ_ERR_UNSUPPORTED
    assert att(vp=patched(m=16)) == tq.TQ_ERR_ARG
    assert att(vp=_with_fake_ptrs(tq, d=256, m=0, groups=((256, 2),))) == tq.TQ_ERR_UNSUPPORTED
    assert att(n=0) == tq.TQ_ERR_ARG and att(G=0) == tq.TQ_ERR_ARG and att(banks=-1) == tq.TQ_ERR_ARG
    assert att(scale=float("inf")) == tq.TQ_ERR_ARG
    assert att(q=None) == tq.TQ_ERR_ARG and att(out=None) == tq.TQ_ERR_ARG
    assert att(values=ctypes.byref(nullbank)) == tq.TQ_ERR_ARG
    assert att(ws=None) == tq.TQ_ERR_WORKSPACE and att(ws=0x100010) == tq.TQ_ERR_WORKSPACE
    assert att(ws_bytes=need - 256) == tq.TQ_ERR_WORKSPACE
    assert att(banks=0, keys=ctypes.byref(nullbank), values=ctypes.byref(nullbank), q=None, out=None, ws=None,
               ws_bytes=0) == tq.TQ_OK
    # 16-byte alignment of the matrices and of the banks the scorers read
    odd = _with_fake_ptrs(tq)
    odd.struct.rot = 0x10004
    assert L.tq_bank_layout(odd.ref, 10, None, None, None) == tq.TQ_ERR_ARG
    oddbank = tq.tq_bank(0x30000, 0x40008, 0x50000)
    assert L.tq_score(good.ref, ctypes.byref(oddbank), 1, 10, 0x1000, 4, 0x2000, 0x3000, 1 << 20,
                      None) == tq.TQ_ERR_ARG
    assert L.tq_topk(good.ref, ctypes.byref(oddbank), 1, 100, 0x1000, 4, 10, 0x2000, 0x3000, 0x4000, 1 << 20,
                     None) == tq.TQ_ERR_ARG
    assert att(keys=ctypes.byref(oddbank)) == tq.TQ_ERR_ARG
    # the 16-bit norm format: other norm types are invalid
    for nd in (tq.TQ_BF16, 3, -1):
        bad = patched(norm_dtype=nd)
        assert L.tq_bank_layout(bad.ref, 10, None, None, None) == tq.TQ_ERR_ARG
        assert L.tq_encode(bad.ref, 0x1000, 0, 1, 10, ctypes.byref(bank), 0x2000, 1 << 20, None) == tq.TQ_ERR_ARG
    # empty inputs are valid no-ops
    assert L.tq_encode(good.ref, None, 0, 0, 10, ctypes.byref(nullbank), None, 0, None) == tq.TQ_OK
    assert L.tq_encode(good.ref, None, 0, 3, 0, ctypes.byref(nullbank), None, 0, None) == tq.TQ_OK
    assert L.tq_score(good.ref, ctypes.byref(nullbank), 3, 0, None, 4, None, None, 0, None) == tq.TQ_OK
    assert L.tq_copy(None, None, 0, None) == tq.TQ_OK
    for code in (0, -1, -2, -3, -4, 9):
        assert isinstance(tq.tq_status_string(code), str)


# ------------------------------------------------------------------------------------------
# host-side variants against the oracle's own constructions
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bits,d", [(1, 3), (2, 16), (3, 128), (4, 768), (3, 1 << 20)])
def test_sphere_codebook_matches_the_oracle(tq, bits, d):
    import oracle

    c, t, mse = tq.tq_make_codebook_sphere(bits, d)
    co, to, mo = oracle.codebook_sphere(bits, d)
    assert np.abs(c - co).max() < 1e-6 and np.abs(t - to).max() < 1e-6 and abs(mse - mo) < 1e-8
    assert (c[::-1] == -c).all()


def test_hadamard_rotation_matches_the_oracle(tq):
    import oracle

    g = np.random.default_rng(3)
    for d in (1, 4, 128, 1024):
        s = np.where(g.standard_normal(d) > 0, 1.0, -0.5).astype(np.float32)  # only the signs count
        np.testing.assert_allclose(tq.tq_make_rotation_hadamard(s), oracle.hadamard_rotation(s), atol=1e-7)
    L = tq._lib.lib()
    ones = np.ones(8, np.float32)
    out = np.zeros(64, np.float32)
    assert L.tq_make_rotation_hadamard(6, ones.ctypes.data, out.ctypes.data) == tq.TQ_ERR_ARG  # not a power of 2
    ones[3] = 0.0
    assert L.tq_make_rotation_hadamard(8, ones.ctypes.data, out.ctypes.data) == tq.TQ_ERR_ARG  # a zero sign
    c = np.zeros(16, np.float32)
    assert L.tq_make_codebook_sphere(2, 2, c.ctypes.data, c.ctypes.data, None) == tq.TQ_ERR_ARG
    assert L.tq_make_codebook_sphere(5, 128, c.ctypes.data, c.ctypes.data, None) == tq.TQ_ERR_ARG
