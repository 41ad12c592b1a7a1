"""The benchmarked call pattern on library-built indexes under other seeds.

For seeds 1-3 (new keys, values, surprisal, routing projections, gates,
queries and randomized-SVD test matrices) and five shapes (the 8B-shaped
3-layer stack at 16K with its cap, the 70B-shaped batch of two at 8K with
sigmoid gates, G = 1, G = 2 with d = 64, and the tiny case), the library
builds the index (gate_eps 0.5 on odd seeds), calibrates tau, and runs
bench.py's loop: sekv_route(l, 1, ..., cap) then sekv_decode_attend(l, 1, ...)
for every layer, with no cap, a 10% cap and a cap of one span, on the HBM
tier, and without a cap on the pinned tier.  Each layer is held to the oracle
routing and decoding the library's own exported index: masks bit-exact
outside the score windows (at most 0.1% of pairs excluded), outputs within
5e-3 relative L2."""
import math

import numpy as np
import pytest
import torch

from compressed_kv_cache_sekv_amd import synth
from tests import test_gpu_parity as TP

pytestmark = pytest.mark.gpu

W8 = synth.WORKLOADS
SHAPES = {
    "8b_l3_16k_cap": dict(base="llama8b_l32_128k", L=3, T=16384),
    "70b_b2_8k": dict(base="llama70b_b32_64k", B=2, L=2, T=8192),
    "g1_4k": dict(base="llama8b_l1_32k", T=4096, Hq=8, Hkv=8, L=2),
    "g2_d64_4k": dict(base="llama8b_l1_32k", T=4096, Hq=16, Hkv=8, d=64, L=2),
    "tiny": dict(base="tiny_2k", L=2, B=2),
}


@pytest.fixture(scope="module")
def sl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from compressed_kv_cache_sekv_amd import lib
    return lib


@pytest.fixture(scope="module")
def ctx(sl):
    c = sl.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_benchmarked_path_other_seeds(ctx, sl, shape, seed):
    spec = dict(SHAPES[shape])
    w = W8[spec.pop("base")].scaled(seed=seed, **spec)
    H, K, V = synth.kv_cache(w, device="cuda")
    W = torch.stack([synth.routing_w(w, l, "cuda") for l in range(w.L)])
    S_max = synth.max_spans(w.T, w.l_min)
    gl = [[synth.gates(w, b, l, S_max, "cuda") for l in range(w.L)] for b in range(w.B)]
    gates = None if gl[0][0] is None else torch.stack([torch.stack(x) for x in gl])
    q = synth.query(w, 7 + seed)
    for tier in (sl.TIER_HBM, sl.TIER_PINNED_HOST):
        idx = ctx.build_index(sl.build_params(w, tier=tier, gate_eps=0.5 if seed % 2 else 0.0), K, V, H, W, gates)
        tau = torch.zeros(w.L, w.Hq, device="cuda")
        if w.tau is not None:
            tau.fill_(w.tau)
        else:
            idx.calibrate_tau(0, w.L, synth.calibration_query(w, "cuda"), w.frac, tau)
        tau_h = tau.cpu().numpy()
        caps = [0, int(math.floor(0.1 * int(idx.n_spans.min()))), 1] if tier == sl.TIER_HBM else [0]
        for cap in caps:
            words, out = TP._bench_loop(idx, w, q, tau_h, cap)
            TP.check_layers_against_export(idx, w, W, q, tau_h, cap, words, out, range(w.L),
                                           f"{shape} seed {seed} tier {tier} cap {cap}")
        idx.free()
