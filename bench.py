"""FAVOR+ throughput on one MI355X.

One step = one bidirectional FAVOR+ pass over B=4 H=8 L=4096 (d=64, m=256,
one shared projection) plus one causal FAVOR+ pass over B=2 H=8 L=8192 (d=64,
m=256, one projection per head), bf16 inputs with fp32 accumulation, inputs
resident in device memory.  The metric is tokens (B*H*L) per second over the
whole step.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]

Besides the step, every workload (the small fp32 case, the two long
bidirectional ones, the two long causal ones) is timed on its own and
reported under "configs" with its algorithmic work and roofline fraction.

``python bench.py --summarise-counters FETCH_DIR WRITE_DIR`` turns two
rocprofv3 ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of this script
(with ``--calib-copy --no-configs``) into profiles/traffic.json;
``python bench.py --summarise-trace TRACE_DIR`` prints per-stage launch
times from a ``--kernel-trace`` run; ``python bench.py --summarise-sq D1 D2 D3``
prints per-wave SQ counters from three ``--pmc`` passes (the counter sets
listed in ``SQ_PASSES``).  ``python bench.py --workload NAME``
runs one workload alone (stage-timed calls), for profiling it.
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import glob
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import positive_random_feature_amd as favor  # noqa: E402
from positive_random_feature_amd import _lib  # noqa: E402
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0
# dense matrix-core peaks (TFLOP/s) by operand dtype
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
# kernels of the three stages of each op at the bench shapes (d=64, m=256)
STAGES = {"bidir": ["kv_partial", "merge_scan", "bidir_out"],
          "causal": ["kv_partial", "merge_scan", "causal_tile"]}
KERNEL_SOURCES = ["positive_random_feature_amd/csrc/favor_kernels.hip", "positive_random_feature_amd/csrc/favor_device.h",
                  "positive_random_feature_amd/csrc/favor_api.cpp"]


class Hip:
    """Minimal HIP event API through ctypes (events on any stream handle)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def record(self, e, stream):
        if self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def to_dev_bf16(bits, dev):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


class Op:
    def __init__(self, name, dev, feature="positive"):
        self.w = WORKLOADS[name]
        w = self.w
        inp = make_inputs(w)
        self.inp = inp
        if w.dtype == "bf16":
            self.q, self.k, self.v = (to_dev_bf16(b, dev) for b in (inp.q_bits, inp.k_bits, inp.v_bits))
        else:
            self.q, self.k, self.v = (torch.from_numpy(a).to(dev) for a in (inp.q, inp.k, inp.v))
        om = favor.orf_omega(w.seed, w.H if w.omega_per_head else 1, w.m, w.d)
        self.omega_host = om.numpy() if w.omega_per_head else om[0].numpy()
        self.omega = (om if w.omega_per_head else om[0]).contiguous().to(dev)
        self.out = torch.empty_like(self.q)
        self.shape = favor._shape(self.q, self.omega, feature)
        opcode = _lib.FAVOR_OP_BIDIR if w.op == "bidir" else _lib.FAVOR_OP_CAUSAL
        self.ws = torch.empty(favor.workspace_bytes(opcode, self.shape), dtype=torch.uint8, device=dev)

    def run(self, stream):
        lib = _lib.load()
        w = self.w
        if w.op == "bidir":
            st = lib.favor_bidir(ctypes.byref(self.shape), self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                 self.omega.data_ptr(), self.out.data_ptr(), self.ws.data_ptr(), self.ws.numel(), stream)
        else:
            st = lib.favor_causal(ctypes.byref(self.shape), self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                  self.omega.data_ptr(), self.out.data_ptr(), w.chunk, self.ws.data_ptr(),
                                  self.ws.numel(), stream)
        _lib.check(st, w.op)

    def run_profiled(self, stream, events):
        lib = _lib.load()
        w = self.w
        arr = (ctypes.c_void_p * len(events))(*[e.value for e in events])
        if w.op == "bidir":
            st = lib.favor_bidir_profiled(ctypes.byref(self.shape), self.q.data_ptr(), self.k.data_ptr(),
                                          self.v.data_ptr(), self.omega.data_ptr(), self.out.data_ptr(),
                                          self.ws.data_ptr(), self.ws.numel(), stream, arr, len(events))
        else:
            st = lib.favor_causal_profiled(ctypes.byref(self.shape), self.q.data_ptr(), self.k.data_ptr(),
                                           self.v.data_ptr(), self.omega.data_ptr(), self.out.data_ptr(), w.chunk,
                                           self.ws.data_ptr(), self.ws.numel(), stream, arr, len(events))
        _lib.check(st, w.op + " (profiled)")


def _strip_comments(text: str) -> str:
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_source_hash(kernel: str | None = None) -> str:
    """Hash of kernel source with comments and blank space removed, so that
    counters stay valid across comment-only edits.  With `kernel` (e.g.
    "causal_tile"), the kernel file is hashed without the definitions of the
    other kernels (its own definition, the shared helpers and the launchers
    stay in), together with the device header and the launch plan, so that
    edits to other kernels leave its counters valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        if kernel and p.endswith(".hip"):
            if f" {kernel}_kernel(" not in text:
                raise ValueError(kernel)
            spans = []
            for m in re.finditer(r"__global__[^\n]*?void (\w+)_kernel\(", text):
                if m.group(1) == kernel:
                    continue
                start = text.rindex("\ntemplate", 0, m.start()) + 1
                end = text.index("\n}\n", m.start()) + 3
                spans.append((start, end))
            for start, end in reversed(spans):
                text = text[:start] + text[end:]
        h.update(_strip_comments(text).encode())
    return h.hexdigest()[:16]


def traffic_kernel_hash(kernel: str):
    try:
        return kernel_source_hash(kernel)
    except ValueError:
        return None


def traffic_for(stage: str):
    """HBM bytes per launch of a stage ("<workload>:<kernel>") from the
    committed counter summary, or None when it is missing or was taken on a
    different source of that kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    entry = t.get("stages", {}).get(stage)
    try:
        current = kernel_source_hash(stage.split(":")[1])
    except ValueError:  # kernel not found in the sources
        return None
    if not entry or entry.get("kernel_hash") != current:
        return None
    return entry.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _rel_l2(got, want) -> float:
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def cpu_baseline(ops, dev, stream, min_seconds: float = 10.0, max_rounds: int = 50):
    """The plain-C fp64 oracle on the host cores, over whole steps' inputs,
    repeated until at least ``min_seconds`` of CPU work have been timed.  The
    oracle outputs it computes also give each workload's parity (rel L2 of
    the library's output against the oracle on the same inputs): the two step
    workloads and the other configurations over the whole output, the long
    causal one on sampled rows of four heads (its full-tensor check runs in
    the test suite)."""
    from oracle import native
    from oracle import reference as ref
    native.build(force=False)
    t_total = 0.0
    tokens = 0
    rounds = 0
    last = {}
    while rounds < max_rounds and (rounds == 0 or t_total < min_seconds):
        for op in ops:
            inp = op.inp
            fn = native.bidir if op.w.op == "bidir" else native.causal
            t0 = time.perf_counter()
            last[op.w.name] = fn(inp.q, inp.k, inp.v, op.omega_host)
            t_total += time.perf_counter() - t0
            tokens += op.w.tokens
        rounds += 1
    parity = {}
    for op in ops:
        op.run(stream)
        torch.cuda.synchronize()
        parity[op.w.name] = _rel_l2(op.out.float().cpu().numpy().astype(np.float64), last[op.w.name])
    for name in ("bidir_f32_tiny", "bidir_bf16_12k", "causal_bf16_64k"):
        op = Op(name, dev)
        op.run(stream)
        torch.cuda.synchronize()
        got = op.out.float().cpu().numpy().astype(np.float64)
        inp, w = op.inp, op.w
        if name == "causal_bf16_64k":
            rows = np.unique(np.concatenate([np.arange(0, w.L, 8192), np.arange(8191, w.L, 8192),
                                             np.random.default_rng(3).integers(0, w.L, 24)]))
            errs = []
            for h in (0, 5, 10, 15):
                want = ref.causal_rows(inp.q[0, h], inp.k[0, h], inp.v[0, h], op.omega_host[h], rows)
                errs.append(_rel_l2(got[0, h, rows], want))
            parity[name + " (sampled rows, 4 heads)"] = max(errs)
        else:
            fn = native.bidir if w.op == "bidir" else native.causal
            parity[name] = _rel_l2(got, fn(inp.q, inp.k, inp.v, op.omega_host))
        del op
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": native.num_threads(), "kind": "oracle",
            "sample": f"{rounds} full steps (bidir 4x8x4096 + causal 2x8x8192, d=64, m=256) back to back, "
                      "fp64 plain-C oracle, OpenMP over heads", "seconds": t_total,
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "parity_rel_l2": parity}


def alg_work(w):
    """Algorithmic FLOPs and HBM bytes of one call: per token 8md + 4m FLOPs
    (projections of q and k, phi(K)^T [V | 1], phi(Q) [KV | z]) and 4d
    elements moved (q, k, v read, out written), plus the projection read once
    per head (fp32)."""
    elem = 2 if w.dtype == "bf16" else 4
    flops = w.tokens * (8 * w.m * w.d + 4 * w.m)
    n_omega = w.H if w.omega_per_head else 1
    bytes_ = w.tokens * 4 * w.d * elem + n_omega * w.m * w.d * 4
    return flops, bytes_


# Exponential issue rate of the chip: one v_exp_f32 per wave64 takes about
# two fp32-FMA issue slots (measured), i.e. 32 exponentials per clock per
# compute unit (4 SIMDs x 16 lanes / 2), at 256 compute units and 2.4 GHz.
EXP_PEAK_PER_S = 256 * 2.4e9 * 32


def exp_roof_us(w, feature="positive"):
    """Diagnostic third roof: the 2m exponentials per token (q and k
    features) at the chip's exponential issue rate; ReLU features have none."""
    if feature == "relu":
        return 0.0
    return w.tokens * 2 * w.m / EXP_PEAK_PER_S * 1e6


def time_configs(hip, dev, stream, reps_target_ms: float = 20.0):
    """Each workload on its own: per-call time (events around back-to-back
    calls on one stream) and its fraction of the binding roofline; the two
    step workloads also with the generalised ReLU features ("<name>:relu",
    the same algorithmic work without the exponentials)."""
    res = {}
    runs = [(name, "positive") for name in WORKLOADS] + [("bidir_bf16_4k", "relu"), ("causal_bf16_8k", "relu"),
                                                         ("causal_bf16_8k", "chunk32")]
    for name, feature in runs:
        w = WORKLOADS[name]
        if feature == "chunk32":  # the causal chunk length as a tunable: 32-token scan
            w = w.replace(chunk=32)
            op = Op(name, dev)
            op.w = w
        else:
            op = Op(name, dev, feature)
        for _ in range(3):
            op.run(stream)
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        op.run(stream)
        hip.record(e1, stream)
        one = max(hip.elapsed_ms(e0, e1), 1e-3)
        n = int(min(2000, max(5, reps_target_ms / one)))
        hip.record(e0, stream)
        for _ in range(n):
            op.run(stream)
        hip.record(e1, stream)
        ms = hip.elapsed_ms(e0, e1) / n
        flops, bytes_ = alg_work(w)
        t_mfma = flops / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)
        t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
        bound = "mfma" if t_mfma > t_hbm else "hbm"
        t_roof = max(t_mfma, t_hbm)
        res[name if feature == "positive" else f"{name}:{feature}"] = {
                     "op": w.op, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "m": w.m, "dtype": w.dtype,
                     "chunk": (w.chunk or (64 if w.d == 64 and w.dtype == "bf16" and w.m <= 256 else 32))
                     if w.op == "causal" else None,
                     "calls": n, "us_per_call": ms * 1e3, "tokens_per_s": w.tokens / (ms * 1e-3),
                     "alg_gflop": flops / 1e9, "alg_mb": bytes_ / 1e6, "bound": bound,
                     "roof_us": t_roof * 1e6, "frac": t_roof / (ms * 1e-3),
                     "exp_roof_us": exp_roof_us(w, feature),
                     "achieved": (bytes_ / (ms * 1e-3) / 1e9) if bound == "hbm" else (flops / (ms * 1e-3) / 1e12),
                     "achieved_unit": "GB/s" if bound == "hbm" else "TFLOP/s"}
        del op
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def time_stages(hip, dev, name, calls, warmup):
    """One workload alone: `calls` stage-timed calls after `warmup` plain ones."""
    op = Op(name, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    for _ in range(warmup):
        op.run(stream)
    torch.cuda.synchronize()
    n_ev = _lib.FAVOR_N_STAGES + 1
    evs = [[hip.event() for _ in range(n_ev)] for _ in range(calls)]
    for i in range(calls):
        op.run_profiled(stream, evs[i])
    torch.cuda.synchronize()
    per_stage = np.zeros(_lib.FAVOR_N_STAGES)
    for i in range(calls):
        for j in range(_lib.FAVOR_N_STAGES):
            per_stage[j] += hip.elapsed_ms(evs[i][j], evs[i][j + 1])
    per_stage /= calls
    flops, bytes_ = alg_work(op.w)
    total_s = per_stage.sum() * 1e-3
    return {"workload": name, "calls": calls, "stage_us": [float(x * 1e3) for x in per_stage],
            "us_per_call": total_s * 1e6, "tokens_per_s": op.w.tokens / total_s,
            "alg_tflops": flops / total_s / 1e12, "alg_gbs": bytes_ / total_s / 1e9}


def time_hadamard(hip, dev, stream, n_heads=16, m=512, d=128, reps=50):
    """Device generation of a structured (Hadamard) projection of the long
    causal workload's size."""
    lib = _lib.load()
    out = torch.empty((n_heads, m, d), dtype=torch.float32, device=dev)
    for _ in range(3):
        _lib.check(lib.favor_hadamard_omega(1, n_heads, m, d, out.data_ptr(), stream), "favor_hadamard_omega")
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for i in range(reps):
        _lib.check(lib.favor_hadamard_omega(i, n_heads, m, d, out.data_ptr(), stream), "favor_hadamard_omega")
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) / reps * 1e3
    return {"heads": n_heads, "m": m, "d": d, "us_per_call": us, "gbs_written": n_heads * m * d * 4 / (us * 1e-6) / 1e9}


def time_givens(hip, dev, stream, n_heads=16, m=512, d=128, reps=20):
    """Device generation of a structured (Givens) projection of the long
    causal workload's size (d ceil(log2 d) rotations per block)."""
    lib = _lib.load()
    out = torch.empty((n_heads, m, d), dtype=torch.float32, device=dev)
    for _ in range(3):
        _lib.check(lib.favor_givens_omega(1, n_heads, m, d, 0, out.data_ptr(), stream), "favor_givens_omega")
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for i in range(reps):
        _lib.check(lib.favor_givens_omega(i, n_heads, m, d, 0, out.data_ptr(), stream), "favor_givens_omega")
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) / reps * 1e3
    return {"heads": n_heads, "m": m, "d": d, "us_per_call": us}


def time_structured_features(hip, dev, stream, B=4, H=8, L=4096, reps=50):
    """Stabilised bf16 features of B x H x L tokens (m = 4d, Hadamard
    projection per head) two ways: the dense matrix-core projection of the
    materialised projection (favor_features, its projection packing
    included) and fast Walsh-Hadamard transforms from the seed
    (favor_features_hadamard).  Both write the same fp32 features."""
    lib = _lib.load()
    rows = []
    for d in (16, 32, 64, 128):
        m = 4 * d
        g = torch.Generator(device="cpu").manual_seed(d)
        x = (torch.randn((B, H, L, d), generator=g) * d ** -0.25).to(torch.bfloat16).to(dev)
        om = favor.hadamard_omega(1, H, m, d, device=dev)
        shp = favor._shape(x, om)
        ws = torch.empty(favor.workspace_bytes(_lib.FAVOR_OP_FEATURES, shp), dtype=torch.uint8, device=dev)
        phi = torch.empty((B, H, L, m), dtype=torch.float32, device=dev)
        ls = torch.empty((B, H, L), dtype=torch.float32, device=dev)

        def dense():
            _lib.check(lib.favor_features(ctypes.byref(shp), x.data_ptr(), om.data_ptr(), phi.data_ptr(),
                                          ls.data_ptr(), 1, ws.data_ptr(), ws.numel(), stream), "favor_features")

        def fwht():
            _lib.check(lib.favor_features_hadamard(ctypes.byref(shp), x.data_ptr(), 1, phi.data_ptr(), ls.data_ptr(),
                                                   1, stream), "favor_features_hadamard")

        res = {"d": d, "m": m, "tokens": B * H * L, "phi_bytes": B * H * L * m * 4}
        for name, fn in (("dense_us", dense), ("fwht_us", fwht)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            for _ in range(reps):
                fn()
            hip.record(e1, stream)
            res[name] = hip.elapsed_ms(e0, e1) / reps * 1e3
        rows.append(res)
    return rows


def time_streaming(hip, dev, stream, name="causal_bf16_8k", pieces=8, reps=50):
    """The causal workload fed in `pieces` consecutive pieces, each call
    continuing from the previous call's carried state (favor_causal_state)."""
    op = Op(name, dev)
    w = op.w
    lib = _lib.load()
    n = favor.state_floats(w.m, w.d)
    step = (w.L + pieces - 1) // pieces
    parts = []
    for a in range(0, w.L, step):
        b = min(w.L, a + step)
        q, k, v = (t[:, :, a:b].contiguous() for t in (op.q, op.k, op.v))
        shape = favor._shape(q, op.omega)
        ws = torch.empty(favor.workspace_bytes(_lib.FAVOR_OP_CAUSAL, shape), dtype=torch.uint8, device=dev)
        parts.append((shape, q, k, v, torch.empty_like(q), ws))
    states = [torch.empty((w.B, w.H, n), dtype=torch.float32, device=dev) for _ in range(2)]

    def run_all():
        for i, (shape, q, k, v, out, ws) in enumerate(parts):
            sin = states[(i + 1) % 2].data_ptr() if i > 0 else None
            st = lib.favor_causal_state(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        op.omega.data_ptr(), out.data_ptr(), 0, sin, states[i % 2].data_ptr(),
                                        ws.data_ptr(), ws.numel(), stream)
            _lib.check(st, "favor_causal_state")

    for _ in range(3):
        run_all()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(reps):
        run_all()
    hip.record(e1, stream)
    ms = hip.elapsed_ms(e0, e1) / reps
    return {"workload": name, "pieces": len(parts), "tokens_per_piece": step * w.B * w.H,
            "us_per_sequence": ms * 1e3, "tokens_per_s": w.tokens / (ms * 1e-3)}


def time_decode(hip, dev, stream, name="causal_bf16_8k", B=64, H=16, steps=32, reps=20):
    """Decoding: B x H heads of the causal workload's shape, one token per
    call, each call continuing from the previous call's state
    (favor_causal_state, the one-launch path for calls of at most 32 tokens
    per head).  Every step must read and write the heads' fp32 states; their
    bytes per step over the step time is the reported rate."""
    w = WORKLOADS[name].replace(B=B, H=H, L=steps)
    inp = make_inputs(w)
    lib = _lib.load()
    toks = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    om = favor.orf_omega(w.seed, H if w.omega_per_head else 1, w.m, w.d)
    omega = (om if w.omega_per_head else om[0]).contiguous().to(dev)
    q1 = toks[0][:, :, :1].contiguous()
    shape = favor._shape(q1, omega)
    ws = torch.empty(favor.workspace_bytes(_lib.FAVOR_OP_CAUSAL, shape), dtype=torch.uint8, device=dev)
    n = favor.state_floats(w.m, w.d)
    states = [torch.zeros((B, H, n), dtype=torch.float32, device=dev) for _ in range(2)]
    pieces = [tuple(t[:, :, i:i + 1].contiguous() for t in toks) for i in range(steps)]
    out = torch.empty_like(q1)

    def run_all():
        for i, (q, k, v) in enumerate(pieces):
            sin = states[(i + 1) % 2].data_ptr() if i > 0 else None
            st = lib.favor_causal_state(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        omega.data_ptr(), out.data_ptr(), 0, sin, states[i % 2].data_ptr(),
                                        ws.data_ptr(), ws.numel(), stream)
            _lib.check(st, "favor_causal_state")

    for _ in range(2):
        run_all()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(reps):
        run_all()
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) / (reps * steps) * 1e3
    state_bytes = 2 * B * H * n * 4
    return {"heads": B * H, "d": w.d, "m": w.m, "tokens_per_call_per_head": 1, "us_per_step": us,
            "tokens_per_s": B * H / (us * 1e-6), "state_mb_per_step": state_bytes / 1e6,
            "state_gbs": state_bytes / (us * 1e-6) / 1e9}


# ---------------------------------------------------------------------------
# Profiler summaries (rocprofv3 CSV output of runs of this script)
# ---------------------------------------------------------------------------
def _read_csvs(root, suffix):
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {root}")
    return rows


def _stage_labels(names):
    """Label the favor kernel launches of bench runs: the output kernel names
    its operation (bidir_out: the bidirectional workload, causal_tile: the
    causal one), and the segment-sum and merge/scan launches belong to the
    output kernel that follows them, whatever order the operations ran in."""
    kinds = []
    for n in names:
        kinds.append(next((k for k in ("kv_partial", "merge_scan", "bidir_out", "causal_tile") if k + "_kernel" in n),
                          None))
    labels = [None] * len(names)
    nxt = None
    for i in range(len(names) - 1, -1, -1):
        k = kinds[i]
        if k in ("bidir_out", "causal_tile"):
            nxt = "bidir_bf16_4k" if k == "bidir_out" else "causal_bf16_8k"
            labels[i] = nxt + ":" + k
        elif k is not None and nxt is not None:
            labels[i] = nxt + ":" + k
    return labels


def summarise_counters(fetch_dir, write_dir):
    def per_dispatch(root, counter):
        rows = [r for r in _read_csvs(root, "counter_collection.csv") if r.get("Counter_Name") == counter]
        by = {}
        for r in rows:
            key = int(r["Dispatch_Id"])
            by.setdefault(key, [r["Kernel_Name"], 0.0])
            by[key][1] += float(r["Counter_Value"])
        return [by[k] for k in sorted(by)]

    out = {"source_hash": kernel_source_hash(), "calibration": {}, "stages": {}}
    copy_kib = (512 << 20) / 1024.0
    lines = []
    vals = {}
    for counter, root in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = per_dispatch(root, counter)
        other = [v for n, v in disp if "favor" not in n]
        if not other:
            raise SystemExit(f"{counter}: no calibration copy dispatch found (run with --calib-copy)")
        scale = copy_kib / max(other)
        out["calibration"]["fetch" if counter == "FETCH_SIZE" else "write"] = scale
        labels = _stage_labels([n for n, _ in disp])
        acc = {}
        for (n, v), lab in zip(disp, labels):
            if lab:
                acc.setdefault(lab, []).append(v)
        vals[counter] = {lab: (sum(v) / len(v), scale) for lab, v in acc.items()}
    for lab in vals["FETCH_SIZE"]:
        fk, fs = vals["FETCH_SIZE"][lab]
        wk, wsc = vals["WRITE_SIZE"].get(lab, (0.0, 1.0))
        b = (fk * fs + wk * wsc) * 1024.0
        out["stages"][lab] = {"fetch_kib": fk, "write_kib": wk, "bytes_per_launch": b,
                              "kernel_hash": kernel_source_hash(lab.split(":")[1])}
        lines.append(f"| {lab} | {fk:.1f} | {wk:.1f} | {b / 1e6:.2f} |")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}; calibration fetch x{out['calibration']['fetch']:.4f}, "
          f"write x{out['calibration']['write']:.4f}; source hash {out['source_hash']}")
    print("| stage (workload:kernel) | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled MB/dispatch |")
    print("|---|---|---|---|")
    print("\n".join(lines))


# Known-traffic runs for a per-kernel check of the HBM counters: every input
# is far larger than the 32 MB of L2, so each kernel's L2-miss reads are its
# input streams and its writes are its outputs.
CALIB_SHAPES = {
    "features": dict(B=8, H=8, L=16384, d=64, m=64),
    "bidir": dict(B=4, H=8, L=32768, d=64, m=256),
    "causal": dict(B=2, H=8, L=65536, d=64, m=256),
}
CALIB_COPY_BYTES = 512 << 20


def calib_expected():
    """(label, kernel, read bytes, write bytes, what) of each dispatch of the
    --calib-kernels run, in launch order (small operand streams -- packed
    projections, shifts -- are left out and named)."""
    f = CALIB_SHAPES["features"]
    x = f["B"] * f["H"] * f["L"] * f["d"] * 2
    phi = f["B"] * f["H"] * f["L"] * f["m"] * 4
    rows = [("features:features", "features_kernel", x, phi, "x read, phi written"),
            ("fwht:hadamard_features", "hadamard_features_kernel", x, phi, "x read, phi written")]
    for op in ("bidir", "causal"):
        c = CALIB_SHAPES[op]
        bh = c["B"] * c["H"]
        t = bh * c["L"] * c["d"] * 2
        nseg = -(-favor_kernels_target() // bh)
        part = bh * nseg * c["m"] * (c["d"] + 1) * 4
        rows.append((f"{op}:kv_partial", "kv_partial_kernel", 2 * t, part, "k, v read; segment sums written"))
        rows.append((f"{op}:merge_scan", "merge_scan_kernel", part, 0 if op == "bidir" else part,
                     "segment sums read" + ("" if op == "bidir" else "; carries written")))
        if op == "bidir":
            rows.append(("bidir:bidir_out", "bidir_out_kernel", t, t, "q read, out written"))
        else:
            rows.append(("causal:causal_tile", "causal_tile_kernel", 3 * t + part, t, "q, k, v, carries read; out written"))
    rows.append(("copy", None, CALIB_COPY_BYTES, CALIB_COPY_BYTES, "device copy"))
    return rows


def favor_kernels_target():
    """Workgroups the launch plan aims for (one per compute unit)."""
    return 256


def run_calib_kernels(dev):
    """One call of each known-traffic kernel, then the calibration copy."""
    g = torch.Generator(device="cpu").manual_seed(0)

    def rnd(B, H, L, d):
        return (torch.randn((B, H, L, d), generator=g) * d ** -0.25).to(torch.bfloat16).to(dev)

    f = CALIB_SHAPES["features"]
    x = rnd(f["B"], f["H"], f["L"], f["d"])
    om = favor.hadamard_omega(1, 1, f["m"], f["d"], device=dev)[0].contiguous()
    torch.cuda.synchronize()
    favor.features(x, om)
    favor.features_hadamard(x, 1, f["m"], per_head=False)
    torch.cuda.synchronize()
    del x
    for op in ("bidir", "causal"):
        c = CALIB_SHAPES[op]
        q, k, v = (rnd(c["B"], c["H"], c["L"], c["d"]) for _ in range(3))
        omc = favor.orf_omega(1, 1, c["m"], c["d"])[0].contiguous().to(dev)
        torch.cuda.synchronize()
        (favor.bidir if op == "bidir" else favor.causal)(q, k, v, omc)
        torch.cuda.synchronize()
        del q, k, v
    src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def summarise_calibration(dirs):
    """Per-kernel table of the --calib-kernels runs: the raw read-request
    counts and the derived FETCH_SIZE / WRITE_SIZE against each kernel's
    known bytes."""
    want = {"FETCH_SIZE", "WRITE_SIZE", "TCC_EA0_RDREQ_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_32B_sum",
            "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"}
    per = {}
    for root in dirs:
        rows = _read_csvs(root, "counter_collection.csv")
        disp = {}
        for r in rows:
            if r.get("Counter_Name") in want:
                d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ordered = [disp[k] for k in sorted(disp)]
        exp = calib_expected()
        i = 0
        for lab, kern, rb, wb, what in exp:
            if kern is None:
                cand = [d for d in ordered if "favor" not in d["name"]]
                d = cand[-1] if cand else None
            else:
                d = None
                while i < len(ordered):
                    if kern in ordered[i]["name"]:
                        d = ordered[i]
                        i += 1
                        break
                    i += 1
            if d is None:
                raise SystemExit(f"{root}: no dispatch for {lab}")
            per.setdefault(lab, {}).update({k: v for k, v in d.items() if k != "name"})
    print("| kernel | expected read MB | FETCH_SIZE MB (ratio) | read requests | BUBBLE | 32 B | expected B/request | "
          "expected write MB | WRITE_SIZE MB (ratio) | write requests | 64 B | what |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for lab, kern, rb, wb, what in calib_expected():
        c = per[lab]
        fs = c.get("FETCH_SIZE", float("nan")) * 1024
        ws = c.get("WRITE_SIZE", float("nan")) * 1024
        rq = c.get("TCC_EA0_RDREQ_sum", float("nan"))
        wr = c.get("TCC_EA0_WRREQ_sum", float("nan"))
        ratio_f = fs / rb if rb else float("nan")
        ratio_w = ws / wb if wb else float("nan")
        print(f"| {lab} | {rb / 1e6:.1f} | {fs / 1e6:.1f} ({ratio_f:.3f}) | {rq:.0f} | {c.get('TCC_BUBBLE_sum', float('nan')):.0f} | "
              f"{c.get('TCC_EA0_RDREQ_32B_sum', float('nan')):.0f} | {rb / rq if rq else float('nan'):.1f} | {wb / 1e6:.1f} | "
              f"{ws / 1e6:.1f} ({ratio_w:.3f}) | {wr:.0f} | {c.get('TCC_EA0_WRREQ_64B_sum', float('nan')):.0f} | {what} |")


SQ_PASSES = (
    ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
     "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY"),
    ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_LDS_BANK_CONFLICT",
     "SQ_INSTS_VALU_TRANS_F32", "SQ_WAIT_INST_LDS"),
    ("SQ_WAVES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VMEM_WR", "SQ_ACTIVE_INST_SCA",
     "SQ_INSTS_VMEM_RD", "SQ_INST_CYCLES_VMEM_RD", "SQ_ACTIVE_INST_MISC"),
)
SQ_KERNELS = ("kv_partial", "merge_scan", "bidir_out", "causal_tile", "causal_wide", "causal_chunk", "features")


def summarise_sq(dirs):
    """Per-wave SQ counters of each kernel from three rocprofv3 --pmc runs
    (one per entry of SQ_PASSES, in that order): every counter summed over
    the kernel's dispatches and divided by that pass's SQ_WAVES."""
    tot = [{} for _ in dirs]
    for p, d in enumerate(dirs):
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    k = next((k for k in SQ_KERNELS if k + "_kernel" in r["Kernel_Name"]), None)
                    if k is None:
                        continue
                    c = tot[p].setdefault(k, {})
                    c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    print("| kernel | VALU instr | MFMA instr | exp/rcp instr | LDS instr | SALU instr | VALU busy (x4 cyc) "
          "| MFMA busy (cyc) | LDS wait (x4 cyc) | wave life (x4 cyc) | LDS bank conflicts (cyc) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for k in SQ_KERNELS:
        if not all(k in t for t in tot):
            continue
        a, b, c = (t[k] for t in tot)
        w1, w2, w3 = a["SQ_WAVES"], b["SQ_WAVES"], c["SQ_WAVES"]
        vals = (b["SQ_INSTS_VALU"] / w2, b["SQ_INSTS_MFMA"] / w2, b["SQ_INSTS_VALU_TRANS_F32"] / w2,
                b["SQ_INSTS_LDS"] / w2, b["SQ_INSTS_SALU"] / w2, a["SQ_ACTIVE_INST_VALU"] / w1,
                c["SQ_VALU_MFMA_BUSY_CYCLES"] / w3, b["SQ_WAIT_INST_LDS"] / w2, a["SQ_WAVE_CYCLES"] / w1,
                b["SQ_LDS_BANK_CONFLICT"] / w2)
        print(f"| {k}_kernel | " + " | ".join(f"{v:.0f}" for v in vals) + " |")


def summarise_trace(trace_dir):
    rows = _read_csvs(trace_dir, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    labels = _stage_labels(names)
    acc = {}
    for r, lab in zip(rows, labels):
        if lab:
            acc.setdefault(lab, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"kernel source hash {kernel_source_hash()}")
    print("| stage (workload:kernel) | launches | avg us | median us | min us |")
    print("|---|---|---|---|---|")
    for lab, v in acc.items():
        v = sorted(v)
        print(f"| {lab} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} | {v[0]:.2f} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 512 MiB device copy first (calibrates HBM counters in profiler runs)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload timings")
    ap.add_argument("--summarise-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarise-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarise-sq", nargs=3, metavar=("PASS1_DIR", "PASS2_DIR", "PASS3_DIR"))
    ap.add_argument("--workload", choices=sorted(WORKLOADS), help="time one workload alone, stage by stage")
    ap.add_argument("--calib-kernels", action="store_true",
                    help="run the known-traffic kernel calls (for a per-kernel check of the HBM counters) and exit")
    ap.add_argument("--summarise-calibration", nargs="+", metavar="PMC_DIR")
    args = ap.parse_args()
    if args.summarise_counters:
        summarise_counters(*args.summarise_counters)
        return
    if args.summarise_trace:
        summarise_trace(args.summarise_trace)
        return
    if args.summarise_sq:
        summarise_sq(args.summarise_sq)
        return
    if args.summarise_calibration:
        summarise_calibration(args.summarise_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs on one GPU and has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = Hip()
    if args.workload:
        print(json.dumps(time_stages(hip, dev, args.workload, args.steps, args.warmup)), flush=True)
        return
    if args.calib_kernels:
        run_calib_kernels(dev)
        print(json.dumps({"calib_kernels": [r[0] for r in calib_expected()]}), flush=True)
        return
    ops = [Op("bidir_bf16_4k", dev), Op("causal_bf16_8k", dev)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    tokens_per_step = sum(op.w.tokens for op in ops)

    if args.calib_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        for op in ops:
            op.run(stream)
    torch.cuda.synchronize()

    # timed region: exactly K steps
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(e0, stream)
    for _ in range(args.steps):
        for op in ops:
            op.run(stream)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = hip.elapsed_ms(e0, e1)
    ms_per_step = ms_total / args.steps

    # each op alone, back to back without events between kernels (for the
    # whole-op roofline fraction)
    op_ms_plain = {}
    for op in ops:
        for _ in range(3):
            op.run(stream)
        hip.record(e0, stream)
        for _ in range(args.steps):
            op.run(stream)
        hip.record(e1, stream)
        op_ms_plain[op.w.name] = hip.elapsed_ms(e0, e1) / args.steps

    # stage-timed region: the same K steps with events between kernels
    n_ev = _lib.FAVOR_N_STAGES + 1
    evs = [[[hip.event() for _ in range(n_ev)] for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, op in enumerate(ops):
            op.run_profiled(stream, evs[s][i])
    torch.cuda.synchronize()
    stage_ms = {}
    op_ms = {}
    for i, op in enumerate(ops):
        per_stage = np.zeros(_lib.FAVOR_N_STAGES)
        for s in range(args.steps):
            for j in range(_lib.FAVOR_N_STAGES):
                per_stage[j] += hip.elapsed_ms(evs[s][i][j], evs[s][i][j + 1])
        per_stage /= args.steps
        for j, name in enumerate(STAGES[op.w.op]):
            stage_ms[f"{op.w.name}:{name}"] = float(per_stage[j])
        op_ms[op.w.name] = float(per_stage.sum())

    # dominant kernel and its roofline (HBM-bound: m = 256 < the bf16 ridge)
    dom = max(stage_ms, key=stage_ms.get)
    dom_op = next(op for op in ops if dom.startswith(op.w.name + ":"))
    kname = dom.split(":")[1]
    elem = 2
    per_token = {"causal_tile": 4 * dom_op.w.d * elem,    # q, k, v read + out written
                 "bidir_out": 2 * dom_op.w.d * elem,      # q read + out written
                 "kv_partial": 2 * dom_op.w.d * elem}.get(kname, 0)  # k, v read
    alg_bytes = per_token * dom_op.w.tokens
    dom_s = stage_ms[dom] * 1e-3
    achieved = alg_bytes / dom_s / 1e9 if dom_s > 0 else 0.0
    src_hash = kernel_source_hash()

    result = {
        "metric": "FAVOR+ tokens/s (B*H*L/s), bidir L=4096 + causal L=8192, one step each",
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V, seeded orthogonal projection)",
        "config": {"workload": "bidir B4 H8 L4096 d64 m256 (shared omega) + causal B2 H8 L8192 d64 m256 (omega per head)",
                   "tokens_per_step": tokens_per_step, "causal_chunk": 64},
        "roofline": {"bound": "hbm", "kernel": kname, "op": dom_op.w.name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_for(dom), "kernel_hash": traffic_kernel_hash(kname),
                     "alg_bytes_per_launch": alg_bytes,
                     "avg_launch_ms": stage_ms[dom],
                     # the whole operation of that kernel (all its kernels): its
                     # algorithmic bytes over the step's per-op time
                     "op_frac": alg_work(dom_op.w)[1] / (op_ms_plain[dom_op.w.name] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "op_us_per_call": op_ms_plain[dom_op.w.name] * 1e3},
        "per_op_tokens_per_s": {name: WORKLOADS[name].tokens / (ms * 1e-3) for name, ms in op_ms.items()},
        "stage_ms": stage_ms,
        "wall_s_timed_region": wall,
        "kernel_source_hash": src_hash,
    }
    if not args.no_configs:
        result["configs"] = time_configs(hip, dev, stream)
        result["streaming"] = time_streaming(hip, dev, stream)
        result["decode"] = time_decode(hip, dev, stream)
        result["hadamard_projection"] = time_hadamard(hip, dev, stream)
        result["givens_projection"] = time_givens(hip, dev, stream)
        result["structured_features"] = time_structured_features(hip, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ops, dev, stream)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
