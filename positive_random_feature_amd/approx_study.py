"""Approximation error of FAVOR+ attention against exact softmax attention as
the number of random features m grows.

This re-creates the pages' approximation study (paperlayer.ai summary of
arXiv:2009.14794v4, section 3: L = 4096, d = 16, m swept; orthogonal against
i.i.d. projections, positive against trigonometric features; the digest,
Theoretical bounds: positive features stay accurate where the softmax kernel
is small, trigonometric ones do not).  The pages' plotted values did not
survive extraction, so the study reports its own numbers and nothing is
compared with the pages' figure.

The FAVOR+ outputs come from the library (positive features with a
Gaussian orthogonal, a Hadamard or an i.i.d. projection; ReLU features as a
further kernel).  Exact softmax attention, and attention through the
trigonometric features exp(|x|^2/2) [sin(omega x), cos(omega x)] / sqrt(m)
that the pages compare against, are evaluated here in float64 with plain
PyTorch: they are the study's references, not part of the library.

Usage: python -m positive_random_feature_amd.approx_study [--L 4096] [--seeds 8]
prints one JSON line: mean squared error of the attention output per method
and m, averaged over seeds.
"""

from __future__ import annotations

import argparse
import json

import numpy as np
import torch

import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import Workload, make_inputs

METHODS = ("positive_orf", "positive_hadamard", "positive_iid", "trig_orf", "trig_iid", "relu_orf")


def exact_softmax(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    """softmax(q k^T) v row by row, float64, no temperature (q, k pre-scaled)."""
    s = q @ k.T
    s = s - s.max(dim=1, keepdim=True).values
    p = torch.exp(s)
    return (p @ v) / p.sum(dim=1, keepdim=True)


def trig_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, omega: torch.Tensor) -> torch.Tensor:
    """Attention through trigonometric random features
    phi(x) = exp(|x|^2/2) [sin(omega x), cos(omega x)] / sqrt(m), float64."""
    m = omega.shape[0]

    def phi(x):
        p = x @ omega.T
        return torch.exp(0.5 * (x * x).sum(dim=1, keepdim=True)) * torch.cat([torch.sin(p), torch.cos(p)], 1) / m ** 0.5

    pq, pk = phi(q), phi(k)
    return (pq @ (pk.T @ v)) / (pq @ pk.sum(dim=0))[:, None]


def run(L: int = 4096, d: int = 16, ms=(32, 64, 128, 256, 512), seeds: int = 8, device: str = "cuda:0") -> dict:
    dev = torch.device(device)
    w = Workload("approx_study", "bidir", 1, 1, L, d, max(ms), "f32", 1.0, False)
    inp = make_inputs(w)
    q, k, v = (torch.from_numpy(a).to(dev) for a in (inp.q, inp.k, inp.v))
    q64, k64, v64 = (t[0, 0].double() for t in (q, k, v))
    exact = exact_softmax(q64, k64, v64)
    res = {meth: {} for meth in METHODS}
    for m in ms:
        errs = {meth: [] for meth in METHODS}
        for seed in range(seeds):
            om_orf = favor.orf_omega(seed, 1, m, d)[0].to(dev)
            om_had = favor.hadamard_omega(seed, 1, m, d, device=dev)[0].contiguous()
            gen = torch.Generator(device=dev)
            gen.manual_seed(1000 + seed)
            om_iid = torch.randn((m, d), generator=gen, device=dev, dtype=torch.float32)
            outs = {
                "positive_orf": favor.bidir(q, k, v, om_orf),
                "positive_hadamard": favor.bidir(q, k, v, om_had),
                "positive_iid": favor.bidir(q, k, v, om_iid),
                "relu_orf": favor.bidir(q, k, v, om_orf, feature="relu"),
            }
            outs = {key: o[0, 0].double() for key, o in outs.items()}
            outs["trig_orf"] = trig_attention(q64, k64, v64, om_orf.double())
            outs["trig_iid"] = trig_attention(q64, k64, v64, om_iid.double())
            for meth in METHODS:
                errs[meth].append(float(((outs[meth] - exact) ** 2).mean()))
        for meth in METHODS:
            res[meth][m] = float(np.mean(errs[meth]))
    return {"study": "attention output MSE against exact softmax", "L": L, "d": d, "seeds": seeds,
            "inputs": "Q, K ~ N(0, d^-1/2), V ~ N(0, 1), seed 0, fp32", "mse": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--L", type=int, default=4096)
    ap.add_argument("--seeds", type=int, default=8)
    args = ap.parse_args()
    print(json.dumps(run(L=args.L, seeds=args.seeds)), flush=True)


if __name__ == "__main__":
    main()
