"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph):
every entry point only enqueues kernels on the given stream (no allocation,
no synchronisation, no memset), so a bidirectional and a causal call can be
captured once and replayed.  Each replay, with eager work and a
synchronisation between replays, must equal the eager result bit for bit."""

import numpy as np
import pytest
import torch

import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd import _lib
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _inputs(name, B, H, L):
    w = WORKLOADS[name]
    inp = make_inputs(w, B=B, H=H, L=L)
    om = ref.orf_omega(w.seed, H if w.omega_per_head else 1, w.m, w.d)
    om = om if w.omega_per_head else om[0]
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0") for b in (inp.q_bits, inp.k_bits, inp.v_bits))
    return q, k, v, torch.from_numpy(om).to("cuda:0")


def test_captured_graph_replays_equal_eager():
    bq, bk, bv, bom = _inputs("bidir_bf16_4k", 2, 4, 1500)
    cq, ck, cv, com = _inputs("causal_bf16_8k", 1, 4, 2100)
    ws_b = torch.empty(favor.workspace_bytes(_lib.FAVOR_OP_BIDIR, favor._shape(bq, bom)), dtype=torch.uint8, device="cuda:0")
    ws_c = torch.empty(favor.workspace_bytes(_lib.FAVOR_OP_CAUSAL, favor._shape(cq, com)), dtype=torch.uint8, device="cuda:0")
    want_b = favor.bidir(bq, bk, bv, bom, workspace=ws_b).clone()
    want_c = favor.causal(cq, ck, cv, com, workspace=ws_c).clone()
    out_b, out_c = torch.empty_like(bq), torch.empty_like(cq)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        favor.bidir(bq, bk, bv, bom, out=out_b, workspace=ws_b)
        favor.causal(cq, ck, cv, com, out=out_c, workspace=ws_c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        favor.bidir(bq, bk, bv, bom, out=out_b, workspace=ws_b)
        favor.causal(cq, ck, cv, com, out=out_c, workspace=ws_c)
    for rep in range(4):
        out_b.fill_(float("nan"))  # eager work between replays
        out_c.fill_(float("nan"))
        ws_b.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_b, want_b), f"bidirectional replay {rep}"
        assert torch.equal(out_c, want_c), f"causal replay {rep}"
        print(f"[graph] replay {rep} equal", flush=True)
