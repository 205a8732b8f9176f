"""Seeded synthetic inputs for the TurboQuant encode/score path.

This module is the only code shared by the GPU path's tests and the CPU
oracle. It draws random numbers and lays them out; it contains none of the
method's arithmetic (no rotation, no quantisation, no estimator).

Every array is derived from a seed ``1000*cfg + 10*role + layer`` so that a
workload can be regenerated piecewise (one layer, one bank) without drawing
the whole thing. Roles:

    1 keys, 2 queries, 3 rotation Gaussians, 4 projection S,
    5 outlier-channel choice, 6 per-channel scales, 7 random banks,
    8 values, 9 the value quantiser's rotation Gaussians

Workload shapes follow the problem statements of the source pages: KV-cache
keys of decode-time attention (batch, kv_head, token, head_dim) with GQA
query groups, and a normalised vector-search database (turboquant-pytorch
write-up on discuss.pytorch.kr, usage example and performance section;
tambur.pub article on Google's TurboQuant, paragraphs on the KV cache and on
vector search). No dataset is read: every input is synthetic.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

ROLE_KEYS, ROLE_QUERIES, ROLE_ROT, ROLE_PROJ, ROLE_CHAN, ROLE_SCALE, ROLE_BANK = 1, 2, 3, 4, 5, 6, 7
ROLE_VALUES, ROLE_VROT = 8, 9


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload. ``bits`` is the total bit budget per coordinate, the
    1-bit sign sketch included; the per-coordinate codebook gets ``bits-1``
    when ``m > 0``."""

    cfg_id: int
    name: str
    d: int
    m: int
    bits: Tuple[int, ...]          # bit budgets the workload is run at
    batch: int
    kv_heads: int
    q_heads: int                   # query heads; G = q_heads // kv_heads
    tokens: int                    # keys per bank
    layers: int = 1
    key_dtype: str = "bf16"
    unit_norm: bool = False        # rows L2-normalised (search)
    outliers: int = 0              # number of outlier channels
    outlier_scale: float = 1.0
    lognormal_sigma: float = 0.0   # per (layer, kv_head, channel) scale
    groups: Optional[Tuple[Tuple[int, int], ...]] = None  # (dim, bits) incl. outlier group first
    topk: int = 0

    @property
    def banks(self) -> int:
        return self.batch * self.kv_heads

    @property
    def G(self) -> int:
        return self.q_heads // self.kv_heads


CONFIGS = {
    # n=1024 keys, d=128, fp32 N(0,1), 16 queries, b=3 (2-bit codebook + 1-bit sign sketch), m=128
    "tiny": Config(1, "tiny", 128, 128, (3,), 1, 1, 16, 1024, key_dtype="f32"),
    # 3B-class decode: batch 1, 8192 tokens, 2 kv heads, 16 q heads, 4 outlier channels x10
    "decode3b": Config(2, "decode3b", 128, 128, (3, 4), 1, 2, 16, 8192, outliers=4, outlier_scale=10.0),
    # 8B-class decode batch: batch 8, 32K context, 8 kv heads, 32 q heads, 32 layers,
    # per-channel lognormal(0, 0.5) scales
    "decode8b": Config(3, "decode8b", 128, 128, (3, 4), 8, 8, 32, 32768, layers=32, lognormal_sigma=0.5),
    # long context, two channel groups: 32 outlier channels x8 at b=3, 96 channels at b=2
    "longctx": Config(4, "longctx", 128, 128, (3,), 1, 8, 32, 131072, outliers=32, outlier_scale=8.0,
                      groups=((32, 3), (96, 2))),
    # vector search: 2,000,000 x 768 unit vectors, 1024 unit queries, b in {2,4}, m=768, top-10
    "search": Config(5, "search", 768, 768, (2, 4), 1, 1, 1024, 2_000_000, key_dtype="f32",
                     unit_norm=True, topk=10),
}


def seed_of(cfg_id: int, role: int, layer: int = 0) -> int:
    return 1000 * cfg_id + 10 * role + layer


def rng(cfg_id: int, role: int, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_of(cfg_id, role, layer)))


# --------------------------------------------------------------------------------------
# parameters drawn by the method: Gaussian matrices (the rotation's QR input and S)
# --------------------------------------------------------------------------------------

def rotation_gaussians(cfg_id: int, dims: Sequence[int], layer: int = 0) -> List[np.ndarray]:
    """i.i.d. N(0,1) float32 matrices, one d_g x d_g per channel group.
    The orthogonal rotation is derived from each by QR (done by the callers)."""
    g = rng(cfg_id, ROLE_ROT, layer)
    return [g.standard_normal((dg, dg)).astype(np.float32) for dg in dims]


def projection(cfg_id: int, m: int, d: int, layer: int = 0) -> np.ndarray:
    """The sign-sketch projection S: m x d, i.i.d. N(0,1), float32."""
    return rng(cfg_id, ROLE_PROJ, layer).standard_normal((m, d)).astype(np.float32)


# --------------------------------------------------------------------------------------
# channel structure
# --------------------------------------------------------------------------------------

def outlier_channels(cfg: Config) -> np.ndarray:
    """Sorted indices of the outlier channels (the same for every head and layer)."""
    if cfg.outliers == 0:
        return np.zeros(0, dtype=np.int32)
    ch = rng(cfg.cfg_id, ROLE_CHAN).choice(cfg.d, size=cfg.outliers, replace=False)
    return np.sort(ch).astype(np.int32)


def group_channels(cfg: Config) -> Optional[np.ndarray]:
    """Channel list for two-group configs: the outlier group's channels ascending,
    then the remaining channels ascending. None for single-group configs."""
    if cfg.groups is None:
        return None
    out = outlier_channels(cfg)
    assert len(out) == cfg.groups[0][0]
    rest = np.setdiff1d(np.arange(cfg.d, dtype=np.int32), out)
    return np.concatenate([out, rest]).astype(np.int32)


def channel_scales(cfg: Config, layer: int = 0) -> np.ndarray:
    """Per (kv_head, channel) multiplicative scales, shape [kv_heads, d], float32."""
    s = np.ones((cfg.kv_heads, cfg.d), dtype=np.float64)
    if cfg.outliers:
        s[:, outlier_channels(cfg)] *= cfg.outlier_scale
    if cfg.lognormal_sigma > 0:
        s *= np.exp(cfg.lognormal_sigma * rng(cfg.cfg_id, ROLE_SCALE, layer).standard_normal((cfg.kv_heads, cfg.d)))
    return s.astype(np.float32)


# --------------------------------------------------------------------------------------
# keys and queries
# --------------------------------------------------------------------------------------

def _round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values already on the bf16 grid -> their raw uint16 bf16 encoding."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def keys(cfg: Config, layer: int = 0, n: Optional[int] = None, banks: Optional[Sequence[int]] = None) -> np.ndarray:
    """Keys [len(banks), n, d] as float32 values (already rounded to bf16 when the
    config stores bf16 keys). Bank index = batch * kv_heads + kv_head."""
    n = cfg.tokens if n is None else n
    banks = list(range(cfg.banks)) if banks is None else list(banks)
    scales = channel_scales(cfg, layer)
    out = np.empty((len(banks), n, cfg.d), dtype=np.float32)
    for i, b in enumerate(banks):
        g = rng(cfg.cfg_id, ROLE_KEYS, layer * 100_000 + b)
        x = g.standard_normal((n, cfg.d), dtype=np.float32)
        if cfg.unit_norm:
            x /= np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True).astype(np.float32)
        else:
            x *= scales[b % cfg.kv_heads][None, :]
        out[i] = _round_bf16(x) if cfg.key_dtype == "bf16" else x
    return out


def queries(cfg: Config, layer: int = 0, banks: Optional[Sequence[int]] = None, G: Optional[int] = None) -> np.ndarray:
    """Queries [len(banks), G, d] float32 (GQA: the G query heads sharing one kv head)."""
    banks = list(range(cfg.banks)) if banks is None else list(banks)
    G = cfg.G if G is None else G
    out = np.empty((len(banks), G, cfg.d), dtype=np.float32)
    for i, b in enumerate(banks):
        g = rng(cfg.cfg_id, ROLE_QUERIES, layer * 100_000 + b)
        q = g.standard_normal((G, cfg.d), dtype=np.float32)
        if cfg.unit_norm:
            q /= np.linalg.norm(q.astype(np.float64), axis=1, keepdims=True).astype(np.float32)
        out[i] = q
    return out


def values(cfg: Config, layer: int = 0, n: Optional[int] = None, banks: Optional[Sequence[int]] = None,
           d: Optional[int] = None) -> np.ndarray:
    """Values [len(banks), n, d] float32, i.i.d. N(0,1) (rounded to bf16 when the config
    stores bf16 keys): the tokens' value vectors of a decode-time KV cache, stored next to
    the keys by the MSE-only quantiser. Bank index as for :func:`keys`."""
    n = cfg.tokens if n is None else n
    d = cfg.d if d is None else d
    banks = list(range(cfg.banks)) if banks is None else list(banks)
    out = np.empty((len(banks), n, d), dtype=np.float32)
    for i, b in enumerate(banks):
        x = rng(cfg.cfg_id, ROLE_VALUES, layer * 100_000 + b).standard_normal((n, d), dtype=np.float32)
        out[i] = _round_bf16(x) if cfg.key_dtype == "bf16" else x
    return out


def value_rotation_gaussians(cfg_id: int, dims: Sequence[int], layer: int = 0) -> List[np.ndarray]:
    """As :func:`rotation_gaussians`, for the value quantiser's own rotation."""
    g = rng(cfg_id, ROLE_VROT, layer)
    return [g.standard_normal((dg, dg)).astype(np.float32) for dg in dims]


def keys_device(cfg: Config, layer: int, device, n: Optional[int] = None, dtype=None):
    """Full-size keys drawn directly on a torch device (for workloads too large to
    draw on the host). Same distribution as :func:`keys`, different stream:
    the seed is shared, the generator is torch's on that device."""
    import torch

    n = cfg.tokens if n is None else n
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(cfg.cfg_id, ROLE_KEYS, layer))
    x = torch.randn((cfg.banks, n, cfg.d), generator=gen, device=device, dtype=torch.float32)
    if cfg.unit_norm:
        x /= torch.linalg.vector_norm(x.double(), dim=2, keepdim=True).float()
    else:
        sc = torch.from_numpy(channel_scales(cfg, layer)).to(device)
        x *= sc.repeat(cfg.batch, 1)[:, None, :]
    if dtype is None:
        dtype = torch.bfloat16 if cfg.key_dtype == "bf16" else torch.float32
    return x.to(dtype)


def values_device(cfg: Config, layer: int, device, n: Optional[int] = None, dtype=None):
    """Full-size values drawn directly on a torch device: same distribution as
    :func:`values`, torch's generator seeded with the values' seed."""
    import torch

    n = cfg.tokens if n is None else n
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(cfg.cfg_id, ROLE_VALUES, layer))
    x = torch.randn((cfg.banks, n, cfg.d), generator=gen, device=device, dtype=torch.float32)
    if dtype is None:
        dtype = torch.bfloat16 if cfg.key_dtype == "bf16" else torch.float32
    return x.to(dtype)


def queries_device(cfg: Config, layer: int, device, G: Optional[int] = None):
    import torch

    G = cfg.G if G is None else G
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(cfg.cfg_id, ROLE_QUERIES, layer))
    q = torch.randn((cfg.banks, G, cfg.d), generator=gen, device=device, dtype=torch.float32)
    if cfg.unit_norm:
        q /= torch.linalg.vector_norm(q.double(), dim=2, keepdim=True).float()
    return q


# --------------------------------------------------------------------------------------
# random packed banks (the score is a pure function of the packed bytes, so a random
# byte pattern with positive norms is a valid scorer input of any size)
# --------------------------------------------------------------------------------------

def random_bank(cfg_id: int, banks: int, n_pad: int, words: int, n_groups: int, layer: int = 0):
    """Random bank content: bit words [banks, n_pad/16, words, 16] uint32, group norms
    [banks, n_pad, n_groups] float32 and residual norms [banks, n_pad] float32."""
    g = rng(cfg_id, ROLE_BANK, layer)
    bits = g.integers(0, 2**32, size=(banks, n_pad // 16, words, 16), dtype=np.uint64).astype(np.uint32)
    norms = (np.sqrt(g.chisquare(128, size=(banks, n_pad, n_groups)))).astype(np.float32)
    rnorms = (0.3 * np.sqrt(g.chisquare(128, size=(banks, n_pad)))).astype(np.float32)
    return bits, norms, rnorms
