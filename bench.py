"""Benchmark of the packed-key scorer on the 8B-class decode workload.

One step = one decode step of the whole model's attention logits: for each of
32 layers, tq_score (query preparation + the packed-key scorer) of the batch's
queries against that layer's packed keys: batch 8, 32768-token context, 8 kv
heads, 32 query heads (G = 4 per bank), d = 128, b = 3 (2-bit codebook + 1-bit
sketch, m = 128). Value = estimated inner products per second.

The same run also times the encoder over all 32 layers (keys/s), the b = 4
variant of the sweep, the fp32 unquantized-keys logits kernel on the same
shapes, the long-context and vector-search workloads, streaming appends, and
the CPU oracle on a bounded sample (rank 0). Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0


def encode_rates(keys, ms, d, m, groups, bf16_keys):
    """Encoder rates: algorithmic fp32 contraction flops (rotation 2 d_g^2 per group,
    projection 2 m d per key) and the bf16 matrix flops actually issued (every fp32 operand
    is three exact bf16 pieces; bf16 keys are one piece: rotation 3 products, otherwise 6;
    projection 6)."""
    rot = sum(2 * dg * dg for dg in groups)
    prj = 2 * m * d
    issued = rot * (3 if bf16_keys else 6) + prj * 6
    sec = ms * 1e-3
    return {
        "keys_per_s": keys / sec,
        "ms": ms,
        "fp32_equivalent_tflops": keys * (rot + prj) / sec / 1e12,
        "fp32_equivalent_frac_of_fp32_mfma_peak": keys * (rot + prj) / sec / 1e12 / FP32_MFMA_PEAK_TFLOPS,
        "bf16_mfma_issued_tflops": keys * issued / sec / 1e12,
        "bf16_mfma_frac": keys * issued / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS,
    }
METRIC = "packed-key inner products/sec + HBM GB/s (% peak), d=128 b=3, 32K ctx decode"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the sources the ring scorer is built from: its device code (the scorer, layout
    and device-helper headers) and its host launch function (grid and arguments)."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_inner_amd", "csrc")
    for f in ("tq_device.h", "tq_layout.h", "tq_score.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    lib = open(os.path.join(csrc, "tq_lib.hip")).read()
    m = re.search(r"static int launch_ring\(.*?\n}\n", lib, re.S)
    h.update((m.group(0) if m else "").encode())
    return h.hexdigest()[:16]


def counters_for(kernel: str, workload: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}|{workload}")
    except ValueError:
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def groups_of(cfg, bits):
    """(d_g, codebook bits) per channel group for a total budget of `bits` (1 bit is the sketch)."""
    return [(cfg.d, bits - 1)] if cfg.groups is None else [(dg, b - 1) for dg, b in cfg.groups]


def params_for(tq, cfg, bits, device, norm16=False):
    import workloads

    groups = groups_of(cfg, bits)
    gauss = workloads.rotation_gaussians(cfg.cfg_id, [g[0] for g in groups])
    S = workloads.projection(cfg.cfg_id, cfg.m, cfg.d)
    return tq.make_params(cfg.d, cfg.m, groups, gauss, S, workloads.group_channels(cfg), device, norm16=norm16)


def time_encode_layer(tq, params, cfg, device, reps=4):
    """ms per tq_encode of one decode8b layer (64 banks x 32768 bf16 keys), from `reps` calls
    issued back to back after one warm call, so the host's marshalling of a call overlaps the
    previous call on the device."""
    import torch

    import workloads

    keys = workloads.keys_device(cfg, 0, device)
    bank = tq.Bank(params, cfg.banks, cfg.tokens, device)
    ws = torch.empty(params.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), dtype=torch.uint8,
                     device=device)
    tq.tq_encode(params, keys, bank, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tq.tq_encode(params, keys, bank, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


class Sweep:
    """Packed banks of all layers for one bit budget, plus per-layer queries."""

    def __init__(self, tq, cfg, bits, layers, device, norm16=False):
        import torch

        self.cfg, self.bits, self.layers = cfg, bits, layers
        self.params = params_for(tq, cfg, bits, device, norm16)
        self.banks, self.queries = [], []
        W, npad, bpk = self.params.layout(cfg.tokens)
        self.bytes_per_key = bpk
        enc_ws = torch.empty(self.params.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), dtype=torch.uint8,
                             device=device)
        import workloads

        for layer in range(layers):
            keys = workloads.keys_device(cfg, layer, device)
            bank = tq.Bank(self.params, cfg.banks, cfg.tokens, device)
            tq.tq_encode(self.params, keys, bank, workspace=enc_ws)
            self.banks.append(bank)
            self.queries.append(workloads.queries_device(cfg, layer, device))
            del keys
        torch.cuda.synchronize()
        self.ws = tq.score_workspace(self.params, self.banks[0], cfg.G)
        self.scores = torch.empty((cfg.banks, cfg.G, cfg.tokens), dtype=torch.float32, device=device)

    def step(self, tq):
        """One decode step: per layer, one tq_score call (query preparation fused into the
        packed-key scorer: a single kernel launch). The C entry point is called with
        pre-marshalled arguments so that host-side Python overhead stays below the GPU time
        per layer."""
        import torch

        if not hasattr(self, "_calls"):
            lib = tq._lib.lib()
            stream = torch.cuda.current_stream().cuda_stream
            ws, wsn = self.ws.data_ptr(), self.ws.numel()
            self._calls = [(lib.tq_score, (self.params.ref, self.banks[l].ref, self.cfg.banks, self.cfg.tokens,
                                           self.queries[l].data_ptr(), self.cfg.G, self.scores.data_ptr(), ws, wsn,
                                           stream))
                           for l in range(self.layers)]
        for score, sa in self._calls:
            if score(*sa):
                raise RuntimeError("tq_score failed")


class EventPool(list):
    """Pre-created timing events (creating them inside the timed loop costs host time)."""

    def __init__(self, n):
        import torch

        super().__init__((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                         for _ in range(n))
        self.done = []


def timed(fn, steps, warmup, layers):
    """Runs `warmup` untimed steps, then `steps` timed ones between synchronizations.
    fn() runs one step (`layers` back-to-back launches on the current stream); a HIP event
    pair on that stream brackets every timed step, so the mean launch duration is the
    bracketed time over the launches inside it (an event pair around each launch would
    add its own gap between the kernels). Returns (wall seconds, per-launch ms list)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    events = EventPool(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        e0, e1 = events.pop()
        e0.record()
        fn()
        e1.record()
        events.done.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) / layers for a, b in events.done]
    return wall, kern_ms


def cpu_baseline(cfg, bits, banks, layers):
    """The oracle (fp64, OpenMP) on a bounded sample of the sweep: it encodes `banks`
    banks of layer 0 once, then scores them with the queries of `layers` layers, so
    the scored pair count equals that of a sweep of `layers` layers over `banks`
    banks (layer 0's keys stand in for every layer's)."""
    import oracle
    import workloads
    groups = groups_of(cfg, bits)
    orc = oracle.Params(oracle.Spec(cfg.d, cfg.m, groups, workloads.group_channels(cfg)),
                        workloads.rotation_gaussians(cfg.cfg_id, [g[0] for g in groups]),
                        workloads.projection(cfg.cfg_id, cfg.m, cfg.d))
    n = cfg.tokens
    keys = workloads.keys(cfg, 0, banks=range(banks))
    t0 = time.perf_counter()
    encs = [oracle.encode(orc, keys[b]) for b in range(banks)]
    t_enc = time.perf_counter() - t0
    del keys
    t_score = 0.0
    for layer in range(layers):
        q = workloads.queries(cfg, layer, banks=range(banks))
        t0 = time.perf_counter()
        for b in range(banks):
            oracle.score(orc, *encs[b], n, q[b])
        t_score += time.perf_counter() - t0
    pairs = banks * n * cfg.G * layers
    threads = oracle.set_threads(0)
    # one core, on one bank and one layer's queries
    prev = oracle.set_threads(1)
    q = workloads.queries(cfg, 0, banks=[0])
    t0 = time.perf_counter()
    oracle.score(orc, *encs[0], n, q[0])
    t_one = time.perf_counter() - t0
    oracle.set_threads(prev)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": pairs / t_score,
        "unit": "pairs/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{banks} banks x {n} keys of the 8B-class layer 0 (b={bits}) encoded once, scored against "
                  f"G={cfg.G} queries of each of {layers} layers ({pairs} pairs, score {t_score:.1f}s); "
                  f"oracle encode of those keys {t_enc:.1f}s ({banks * n / t_enc:.3g} keys/s)",
        "encode_keys_per_s": banks * n / t_enc,
        "cpu_model": cpu_model,
        "one_core": {"value": n * cfg.G / t_one, "unit": "pairs/s",
                     "sample": f"1 bank x {n} keys x G={cfg.G} queries, {t_one:.2f}s"},
    }


def copy_ceiling(tq, device, nbytes, reps=32):
    """Plain device copy moving the same total bytes as one score launch (half read, half
    written), cycled over distinct buffer pairs (about 1.2 GB in all, so that no launch is
    served from the 256 MB last-level cache) and launched back to back with pre-marshalled
    arguments, as the scorer's launches are: the HBM rate a streaming kernel of this size
    reaches on this device, launch overhead included."""
    import ctypes

    import torch

    half = (nbytes // 2 + 15) // 16 * 16
    copies = max(2, -(-int(1.2e9) // (2 * half)))
    buf = torch.empty((copies, 2, half), dtype=torch.uint8, device=device)
    lib = tq._lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    calls = [(buf[i % copies, 0].data_ptr(), buf[i % copies, 1].data_ptr(), half, stream)
             for i in range(max(reps, copies))]
    for c in calls[:copies]:
        if lib.tq_copy(*c):
            raise RuntimeError("tq_copy failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for c in calls:
        lib.tq_copy(*c)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / len(calls)
    del buf
    torch.cuda.empty_cache()
    return {"bytes": 2 * half, "ms": ms, "gbps": 2 * half / (ms * 1e-3) / 1e9, "copies_cycled": copies}


def longctx_extra(tq, device):
    """Long-context workload (8 banks x 131072 keys, two channel groups): encode rate, and
    score rate over 12 distinct copies of the banks cycled (about 600 MB, beyond the
    256 MB last-level cache, so every launch streams from HBM)."""
    import torch
    import workloads

    cfg = workloads.CONFIGS["longctx"]
    prm = params_for(tq, cfg, 3, device)
    keys = workloads.keys_device(cfg, 0, device)
    q = workloads.queries_device(cfg, 0, device)
    bank = tq.Bank(prm, cfg.banks, cfg.tokens, device)
    ws = torch.empty(prm.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), dtype=torch.uint8, device=device)
    tq.tq_encode(prm, keys, bank, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
    for a, b in ev:
        a.record()
        tq.tq_encode(prm, keys, bank, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    enc_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    copies = []
    for _ in range(12):
        c = tq.Bank(prm, cfg.banks, cfg.tokens, device)
        c.bits.copy_(bank.bits)
        c.norms.copy_(bank.norms)
        c.rnorms.copy_(bank.rnorms)
        copies.append(c)
    scores = torch.empty((cfg.banks, cfg.G, cfg.tokens), dtype=torch.float32, device=device)
    sws = tq.score_workspace(prm, bank, cfg.G)
    for c in copies[:2]:
        tq.tq_score(prm, c, q, scores=scores, workspace=sws)
    # back to back with pre-marshalled arguments, one event pair around all launches (as the
    # decode step runs its layers): host-side marshalling per call would otherwise leave the
    # GPU idle between launches shorter than it
    import ctypes

    lib = tq._lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    calls = [(prm.ref, copies[i % 12].ref, cfg.banks, cfg.tokens, q.data_ptr(), cfg.G, scores.data_ptr(),
              sws.data_ptr(), sws.numel(), stream) for i in range(48)]
    for c in calls[:12]:
        assert lib.tq_score(*c) == 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for c in calls:
        lib.tq_score(*c)
    b.record()
    torch.cuda.synchronize()
    sc_ms = a.elapsed_time(b) / len(calls)
    _, _, bpk = prm.layout(cfg.tokens)
    keys_n = cfg.banks * cfg.tokens
    return {
        "workload": "longctx: 8 banks x 131072 bf16 keys, groups (32 ch, 2-bit codebook) + (96 ch, 1-bit), "
                    "one 128-row sign sketch, G=4",
        "bytes_per_key": int(bpk),
        "encode": encode_rates(keys_n, enc_ms, cfg.d, cfg.m, [g[0] for g in cfg.groups], True),
        "score_pairs_per_s": keys_n * cfg.G / (sc_ms * 1e-3),
        "score_ms": sc_ms,
        "score_gbps": keys_n * (bpk + 4 * cfg.G) / (sc_ms * 1e-3) / 1e9,
    }


def append_extra(tq, device):
    """Streaming append on the 8B-class shapes: one new key per bank (64 banks, capacity
    32768 + 16 slots) per layer call, as in a decode step, and 16 keys per bank per call."""
    import torch
    import workloads

    cfg = workloads.CONFIGS["decode8b"]
    prm = params_for(tq, cfg, 3, device)
    n_cap = cfg.tokens + 16
    banks = [tq.Bank(prm, cfg.banks, n_cap, device) for _ in range(2)]
    out = {"workload": "decode8b: 64 banks of 32784 slots, b=3; keys appended at slot 32768 onwards"}
    for count in (1, 16):
        keys = torch.randn(cfg.banks, count, cfg.d, device=device).to(torch.bfloat16)
        pos = torch.full((cfg.banks,), cfg.tokens, dtype=torch.int32, device=device)
        ws = torch.empty(prm.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, count), dtype=torch.uint8, device=device)
        res = {}
        for prepared in (False, True):
            for i in range(4):
                tq.tq_encode_append(prm, keys, banks[i % 2], pos, workspace=ws, prepared=prepared and i > 0)
            calls = 64
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(calls):
                tq.tq_encode_append(prm, keys, banks[i % 2], pos, workspace=ws, prepared=prepared)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / calls
            res["prepared" if prepared else "with_projection_fold"] = {
                "us_per_call": us, "keys_per_s": cfg.banks * count / (us * 1e-6),
                "us_per_decode_step_32_layers": 32 * us}
        out[f"count{count}"] = res
    del banks
    torch.cuda.empty_cache()
    return out


def halfnorm_extra(tq, device, layers, steps, ref_launch_ms):
    """The headline sweep with the 16-bit norm format: the same decode8b layers (b=3) encoded
    with binary16 norms (4 bytes fewer per key) and scored by the same ring kernel."""
    import workloads

    cfg = workloads.CONFIGS["decode8b"]
    sw = Sweep(tq, cfg, 3, layers, device, norm16=True)
    wall, kern = timed(lambda: sw.step(tq), steps, 2, layers)
    nbytes = cfg.banks * cfg.tokens * (sw.bytes_per_key + 4 * cfg.G)
    kavg = float(np.mean(kern))
    gbps = nbytes / (kavg * 1e-3) / 1e9
    out = {
        "workload": "decode8b sweep as the headline, binary16 norms",
        "value": cfg.banks * cfg.tokens * cfg.G * layers / (wall / steps),
        "unit": "pairs/s",
        "bytes_per_key": sw.bytes_per_key,
        "avg_launch_ms": kavg,
        "kernel_gbps": gbps,
        "kernel_frac": gbps / HBM_PEAK_GBPS,
        "launch_speedup_vs_f32_norms": ref_launch_ms / kavg,
    }
    del sw
    return out


def variants_extra(tq, device):
    """One decode8b layer (b=3) encoded and scored with the randomised Walsh-Hadamard rotation
    and the exact sphere-marginal codebook (same kernels, other parameters)."""
    import torch
    import workloads

    cfg = workloads.CONFIGS["decode8b"]
    groups = groups_of(cfg, 3)
    signs = np.where(np.random.default_rng(77).random(cfg.d) < 0.5, -1.0, 1.0).astype(np.float32)
    prm = tq.make_params(cfg.d, cfg.m, groups, None, workloads.projection(cfg.cfg_id, cfg.m, cfg.d), None, device,
                         rotations=[tq.tq_make_rotation_hadamard(signs)],
                         codebooks=[tq.tq_make_codebook_sphere(groups[0][1], cfg.d)[:2]])
    keys = workloads.keys_device(cfg, 0, device)
    q = workloads.queries_device(cfg, 0, device)
    bank = tq.Bank(prm, cfg.banks, cfg.tokens, device)
    ws = torch.empty(prm.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), dtype=torch.uint8, device=device)
    tq.tq_encode(prm, keys, bank, workspace=ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        tq.tq_encode(prm, keys, bank, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    enc_ms = a.elapsed_time(b) / 3
    scores = torch.empty((cfg.banks, cfg.G, cfg.tokens), dtype=torch.float32, device=device)
    sws = tq.score_workspace(prm, bank, cfg.G)
    tq.tq_score(prm, bank, q, scores=scores, workspace=sws)
    a.record()
    for _ in range(10):
        tq.tq_score(prm, bank, q, scores=scores, workspace=sws)
    b.record()
    torch.cuda.synchronize()
    sc_us = a.elapsed_time(b) * 100
    n = cfg.banks * cfg.tokens
    return {"workload": "decode8b layer 0, b=3, Walsh-Hadamard rotation + sphere-marginal codebook (d=128)",
            "encode": encode_rates(n, enc_ms, cfg.d, cfg.m, [cfg.d], True),
            "score_us_per_launch_same_layer_repeated": sc_us,
            "codebook_mse_sphere_vs_normal": [tq.tq_make_codebook_sphere(groups[0][1], cfg.d)[2],
                                              tq.tq_make_codebook(groups[0][1])[2]]}


def fp32_comparator(tq, device, layers, steps, packed_launch_ms):
    """The fp32 unquantized-keys logits kernel on the decode8b shapes (528 B per key: the 32-bit
    keys the packed format replaces, and the G = 4 scores), 4 distinct fp32 layers (4.3 GB,
    far beyond the 256 MB last-level cache) cycled over the sweep's layer count. The speedup
    of the packed scorer is reported per launch and, beside it, the byte ratio that bounds it
    when both kernels stream at the same rate."""
    import torch
    import workloads

    cfg = workloads.CONFIGS["decode8b"]
    nfp = 4
    kf = [workloads.keys_device(cfg, l, device, dtype=torch.float32) for l in range(nfp)]
    qf = [workloads.queries_device(cfg, l, device) for l in range(nfp)]
    sf = torch.empty((cfg.banks, cfg.G, cfg.tokens), dtype=torch.float32, device=device)

    def fp32_step():
        for layer in range(layers):
            tq.tq_fp32_logits(kf[layer % nfp], qf[layer % nfp], sf)

    wallf, kernf = timed(fp32_step, steps, 1, layers)
    fbytes = cfg.banks * cfg.tokens * (4 * cfg.d + 4 * cfg.G)
    pbytes = cfg.banks * cfg.tokens * (56 + 4 * cfg.G)
    del kf
    return {
        "value": cfg.banks * cfg.tokens * cfg.G * layers / (wallf / steps),
        "unit": "pairs/s",
        "avg_launch_ms": float(np.mean(kernf)),
        "kernel_gbps": fbytes / (np.mean(kernf) * 1e-3) / 1e9,
        "speedup_of_packed_b3": float(np.mean(kernf)) / packed_launch_ms,
        "byte_ratio_b3": fbytes / pbytes,
        "context": "the pages quote up to 8x for 4-bit keys vs 32-bit keys on H100",
    }


def launch_sweep(tq, device, reps=32):
    """Launch-size sweep on the decode shapes (64 banks, G = 4, d = 128, b = 3): per launch
    size, the ring scorer and a plain copy moving the same algorithmic bytes (half read, half
    written), each cycled over distinct buffers (about 1.2 GB in all, so no launch is served
    from the 256 MB last-level cache) and timed back to back, as the decode step runs them.
    A least-squares fit t = t0 + B / BW_inf over the sizes separates the fixed cost of a
    launch (t0) from its asymptotic streaming rate (BW_inf)."""
    import ctypes

    import torch
    import workloads

    cfg = workloads.CONFIGS["decode8b"]
    prm = params_for(tq, cfg, 3, device)
    lib = tq._lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    banks, G = cfg.banks, cfg.G
    sizes = [4096, 8192, 16384, 32768, 65536, 131072]  # keys per bank
    q = workloads.queries_device(cfg, 0, device)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = []
    for n in sizes:
        W, npad, bpk = prm.layout(n)
        alg = banks * n * (bpk + 4 * G)
        copies = max(2, -(-int(1.2e9) // (banks * npad * bpk)))
        bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (copies * banks, npad // 16, W, 16), dtype=torch.int32,
                             device=device)
        norms = torch.rand((copies * banks, npad, 1), device=device) + 0.5
        rnorms = torch.rand((copies * banks, npad), device=device) * 0.5 + 0.1
        scores = [torch.empty((banks, G, n), dtype=torch.float32, device=device) for _ in range(2)]
        structs = [tq.tq_bank(bits[c * banks].data_ptr(), norms[c * banks].data_ptr(), rnorms[c * banks].data_ptr())
                   for c in range(copies)]
        calls = [(prm.ref, ctypes.byref(structs[i % copies]), banks, n, q.data_ptr(), G, scores[i % 2].data_ptr(),
                  None, 0, stream) for i in range(max(reps, copies))]
        for c in calls[:copies]:
            assert lib.tq_score(*c) == 0
        a.record()
        for c in calls:
            lib.tq_score(*c)
        b.record()
        torch.cuda.synchronize()
        score_us = a.elapsed_time(b) * 1e3 / len(calls)
        del bits, norms, rnorms, scores, structs, calls
        cp = copy_ceiling(tq, device, alg, reps)
        half = cp["bytes"] // 2
        copy_us = cp["ms"] * 1e3
        rows.append({"keys_per_launch": banks * n, "algorithmic_bytes": alg, "score_us": score_us,
                     "copy_us": copy_us, "score_gbps": alg / score_us / 1e3, "copy_gbps": 2 * half / copy_us / 1e3})

    def fit(key):
        x = np.array([r["algorithmic_bytes"] for r in rows], np.float64)
        y = np.array([r[key] for r in rows], np.float64)
        slope, t0 = np.polyfit(x, y, 1)
        bw = 1.0 / slope / 1e3  # bytes per microsecond -> GB/s
        return {"t0_us": float(t0), "bw_inf_gbps": float(bw), "bw_inf_frac_of_8tbs": float(bw / HBM_PEAK_GBPS),
                "max_rel_residual": float(np.max(np.abs(y - (t0 + slope * x)) / y))}

    return {"workload": "decode8b shapes, 64 banks x n keys, G=4, b=3 (72 algorithmic bytes per key); "
                        "random bank bytes, distinct buffers cycled",
            "rows": rows, "fit_score": fit("score_us"), "fit_copy": fit("copy_us")}


def attend_extra(tq, device, layers=4, reps=12):
    """Decode attention over decode8b layers (64 banks x 32768 tokens, G = 4): keys at b=4
    (3-bit codebook + sketch), values MSE-only at 3 bits; `layers` distinct layers cycled so
    that no layer's banks stay in the last-level cache. Per layer: the logits (tq_score), the
    chunk kernel (softmax weights and the integer product with the value planes) and the
    combine kernel."""
    import torch
    import workloads

    cfg = workloads.CONFIGS["decode8b"]
    kprm = params_for(tq, cfg, 4, device)
    vprm = tq.make_params(cfg.d, 0, [(cfg.d, 3)], workloads.value_rotation_gaussians(cfg.cfg_id, [cfg.d]), None,
                          None, device)
    kws = torch.empty(kprm.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), dtype=torch.uint8, device=device)
    vws = torch.empty(max(vprm.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), 256), dtype=torch.uint8,
                      device=device)
    kb, vb, qs = [], [], []
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    venc_ms = 0.0
    for layer in range(layers):
        kb.append(tq.tq_encode(kprm, workloads.keys_device(cfg, layer, device), tq.Bank(kprm, cfg.banks, cfg.tokens,
                                                                                        device), workspace=kws))
        vals = workloads.values_device(cfg, layer, device)
        vbank = tq.Bank(vprm, cfg.banks, cfg.tokens, device)
        tq.tq_encode(vprm, vals, vbank, workspace=vws)
        a.record()
        tq.tq_encode(vprm, vals, vbank, workspace=vws)
        b.record()
        torch.cuda.synchronize()
        venc_ms += a.elapsed_time(b)
        vb.append(vbank)
        qs.append(workloads.queries_device(cfg, layer, device))
        del vals
    out = torch.empty((cfg.banks, cfg.G, cfg.d), dtype=torch.float32, device=device)
    ws = tq.attend_workspace(kprm, kb[0], cfg.G)
    scale = 1.0 / math.sqrt(cfg.d)
    scores = torch.empty((cfg.banks, cfg.G, cfg.tokens), dtype=torch.float32, device=device)
    sws = tq.score_workspace(kprm, kb[0], cfg.G)

    def run(fn):
        for i in range(layers):
            fn(i)
        a.record()
        for i in range(reps):
            fn(i % layers)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    att_us = run(lambda i: tq.tq_attend(kprm, kb[i], vprm, vb[i], qs[i], scale, out=out, workspace=ws))
    sc_us = run(lambda i: tq.tq_score(kprm, kb[i], qs[i], scores=scores, workspace=sws))
    _, npad, kbpk = kprm.layout(cfg.tokens)
    _, _, vbpk = vprm.layout(cfg.tokens)
    n = cfg.banks * cfg.tokens
    logit_bytes = 4 * cfg.G * n
    return {
        "workload": "decode8b attention, 64 banks x 32768 tokens, G=4, keys b=4 (m=128), values MSE-only 3-bit, "
                    f"{layers} layers cycled",
        "us_per_layer": att_us,
        "logits_us_per_layer": sc_us,
        "softmax_and_values_us_per_layer": att_us - sc_us,
        "bytes_per_token": {"key": kbpk, "value": vbpk - 4, "logits_written_and_read": 2 * 4 * cfg.G},
        "gbps_whole_call": (n * (kbpk + vbpk - 4) + 2 * logit_bytes) / (att_us * 1e-6) / 1e9,
        "value_encode_keys_per_s": n / (venc_ms / layers * 1e-3),
    }


def small_extra(tq, device, reps=20):
    """The small workloads, whose banks stay in the last-level cache, so a call is bound by
    launch latency rather than HBM: microseconds per tq_encode and per tq_score call for
    tiny (1 x 1024 fp32 keys, G=16, b=3) and decode3b (2 x 8192 bf16 keys, G=8, b=3 and 4)."""
    import torch
    import workloads

    out = {}
    for name, bits in (("tiny", 3), ("decode3b", 3), ("decode3b", 4)):
        cfg = workloads.CONFIGS[name]
        prm = params_for(tq, cfg, bits, device)
        keys = torch.from_numpy(workloads.keys(cfg)).to(device)
        if cfg.key_dtype == "bf16":
            keys = keys.to(torch.bfloat16)
        q = torch.from_numpy(workloads.queries(cfg)).to(device)
        bank = tq.Bank(prm, cfg.banks, cfg.tokens, device)
        ews = torch.empty(max(prm.workspace_bytes(tq.TQ_OP_ENCODE, cfg.banks, cfg.tokens), 256), dtype=torch.uint8,
                          device=device)
        sws = tq.score_workspace(prm, bank, cfg.G)
        scores = torch.empty((cfg.banks, cfg.G, cfg.tokens), dtype=torch.float32, device=device)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        res = {}
        for label, fn in (("encode_us", lambda: tq.tq_encode(prm, keys, bank, workspace=ews)),
                          ("score_us", lambda: tq.tq_score(prm, bank, q, scores=scores, workspace=sws))):
            for _ in range(3):
                fn()
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            res[label] = a.elapsed_time(b) / reps * 1e3
        res["pairs"] = cfg.banks * cfg.tokens * cfg.G
        res["keys"] = cfg.banks * cfg.tokens
        out[f"{name}_b{bits}"] = res
    out["note"] = "cache-resident banks: per-call latency, not an HBM rate"
    return out


def search_extra(tq, device):
    """Vector search: 2,000,000 x 768 unit vectors, 1024 queries, top-10 per query, at
    b=4 and b=2; encode rate, top-k rate and recall@10 against the exact inner products."""
    import torch
    import workloads

    cfg = workloads.CONFIGS["search"]
    out = {"workload": "search: 2,000,000 x 768 fp32 unit vectors, 1024 unit queries, top-10, m=768"}
    for bits in (4, 2):
        prm = params_for(tq, cfg, bits, device)
        keys = workloads.keys_device(cfg, 0, device)
        q = workloads.queries_device(cfg, 0, device)
        bank = tq.Bank(prm, 1, cfg.tokens, device)
        ews = torch.empty(prm.workspace_bytes(tq.TQ_OP_ENCODE, 1, cfg.tokens), dtype=torch.uint8, device=device)
        tq.tq_encode(prm, keys, bank, workspace=ews)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tq.tq_encode(prm, keys, bank, workspace=ews)
        b.record()
        torch.cuda.synchronize()
        enc_ms = a.elapsed_time(b)
        exact = torch.topk(q[0] @ keys[0].T, cfg.topk, dim=1).indices
        del keys
        torch.cuda.empty_cache()
        ws = torch.empty(prm.workspace_bytes(tq.TQ_OP_TOPK, 1, cfg.tokens, cfg.G, cfg.topk), dtype=torch.uint8,
                         device=device)
        tq.tq_topk(prm, bank, q, cfg.topk, workspace=ws)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in ev:
            a.record()
            vals, idx = tq.tq_topk(prm, bank, q, cfg.topk, workspace=ws)
            b.record()
        torch.cuda.synchronize()
        tk_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        recall = (idx[0].long()[:, :, None] == exact[:, None, :]).any(dim=2).float().mean().item()
        pairs = cfg.tokens * cfg.G
        out[f"b{bits}"] = {
            "encode": encode_rates(cfg.tokens, enc_ms, cfg.d, cfg.m, [cfg.d], False),
            "topk_ms": tk_ms,
            "topk_pairs_per_s": pairs / (tk_ms * 1e-3),
            "topk_tflops_algorithmic": pairs * 2 * (cfg.d + cfg.m) / (tk_ms * 1e-3) / 1e12,
            "recall_at_10_vs_exact": recall,
        }
        del bank, ws, exact
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline sweep")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (calibrates the HBM traffic counters)")
    ap.add_argument("--only", choices=["attend", "longctx", "search", "append", "variants", "small", "halfnorm",
                                       "sweep", "fp32"],
                    help="run one extra section alone and print its JSON (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "one GPU only: every bank is independent, so more GPUs would each run "
                                   "this same single-GPU sweep on their own banks; run with --gpus 1"}))
        sys.exit(2)

    import torch

    import kv_cache_inner_amd as tq
    import workloads

    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.only:
        fn = {"attend": attend_extra, "longctx": longctx_extra, "search": search_extra, "append": append_extra,
              "variants": variants_extra, "small": small_extra, "sweep": launch_sweep,
              "fp32": lambda t, d: fp32_comparator(t, d, args.layers, max(args.steps // 4, 1), float("nan")),
              "halfnorm": lambda t, d: halfnorm_extra(t, d, args.layers, args.steps, float("nan"))}[args.only]
        print(json.dumps({args.only: fn(tq, device)}))
        return
    cfg = workloads.CONFIGS["decode8b"]
    L = args.layers
    if args.copy_mib:
        nbytes = args.copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        tq.tq_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    log(f"encode + pack {L} layers (b=3)")
    sw3 = Sweep(tq, cfg, 3, L, device)
    keys_total = cfg.banks * cfg.tokens * L
    enc_layer_ms = time_encode_layer(tq, sw3.params, cfg, device)
    enc_ms = enc_layer_ms * L
    log(f"encode: {enc_layer_ms:.3f} ms per layer ({enc_ms:.2f} ms for {keys_total} keys)")

    log("timed sweep b=3")
    wall, kern_ms = timed(lambda: sw3.step(tq), args.steps, args.warmup, L)
    ms_per_step = 1e3 * wall / args.steps
    pairs_per_step = cfg.banks * cfg.tokens * cfg.G * L
    value = pairs_per_step / (wall / args.steps)
    bytes_per_launch = cfg.banks * cfg.tokens * (sw3.bytes_per_key + 4 * cfg.G)
    kavg = float(np.mean(kern_ms))
    achieved = bytes_per_launch / (kavg * 1e-3) / 1e9
    step_gbps = bytes_per_launch * L / (wall / args.steps) / 1e9

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8-limb exact (i32 acc, f64 combine)",
        "data": "synthetic",
        "config": {
            "workload": "decode8b: 32 layers x batch 8 x 8 kv heads x 32768 keys, G=4 queries per kv head, "
                        "d=128, b=3 (2-bit codebook + 1-bit sign sketch, m=128), bf16 keys N(0,1) x "
                        "lognormal(0,0.5) channel scales",
            "layers": L, "banks_per_layer": cfg.banks, "keys_per_bank": cfg.tokens, "G": cfg.G, "d": cfg.d,
            "bits": 3, "bytes_per_key": sw3.bytes_per_key,
        },
        "step_ms_percentiles": {"p10": float(np.percentile(kern_ms, 10)) * L,
                                "median": float(np.median(kern_ms)) * L,
                                "p90": float(np.percentile(kern_ms, 90)) * L},
        "hbm_gbps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "roofline": {
            "bound": "hbm",
            "kernel": "score_ring_kernel",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": counters_for("score_ring_kernel", "decode8b_b3"),
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "avg_launch_ms": kavg,
            "launches": len(kern_ms) * L,
        },
        "hbm_copy_ceiling": copy_ceiling(tq, device, bytes_per_launch),
        "encode": dict(encode_rates(keys_total, enc_ms, cfg.d, cfg.m, [cfg.d], True), layers=L,
                       timed="one layer's keys encoded 4 times back to back (host marshalling overlapped), x layers"),
    }
    del sw3
    torch.cuda.empty_cache()

    if not args.no_extras:
        log("b=4 sweep")
        sw4 = Sweep(tq, cfg, 4, L, device)
        wall4, kern4 = timed(lambda: sw4.step(tq), max(args.steps // 2, 1), 2, L)
        b4_bytes = cfg.banks * cfg.tokens * (sw4.bytes_per_key + 4 * cfg.G)
        out["b4"] = {
            "value": pairs_per_step / (wall4 / max(args.steps // 2, 1)),
            "unit": "pairs/s",
            "bytes_per_key": sw4.bytes_per_key,
            "kernel_gbps": b4_bytes / (np.mean(kern4) * 1e-3) / 1e9,
            "kernel_frac": b4_bytes / (np.mean(kern4) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        }
        del sw4
        torch.cuda.empty_cache()
        log("binary16 norms")
        out["half_norms"] = halfnorm_extra(tq, device, L, max(args.steps // 2, 1), kavg)
        torch.cuda.empty_cache()

        log("fp32 unquantized-keys comparator")
        out["fp32_comparator"] = fp32_comparator(tq, device, L, max(args.steps // 4, 1), kavg)
        torch.cuda.empty_cache()
        log("launch-size sweep")
        out["launch_sweep"] = launch_sweep(tq, device)
        torch.cuda.empty_cache()

        log("long-context mixed bit widths")
        out["longctx"] = longctx_extra(tq, device)
        torch.cuda.empty_cache()
        log("vector search top-10")
        out["search"] = search_extra(tq, device)
        log("streaming append")
        out["append"] = append_extra(tq, device)
        torch.cuda.empty_cache()
        log("small workloads (latency)")
        out["small"] = small_extra(tq, device)
        log("decode attention")
        out["attend"] = attend_extra(tq, device)
        torch.cuda.empty_cache()
        log("rotation / codebook variants")
        out["variants"] = variants_extra(tq, device)
        torch.cuda.empty_cache()

    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(cfg, 3, cfg.banks, L)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
