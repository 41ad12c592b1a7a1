"""Seeded synthetic inputs for the SeKV decode path.

This module is the only code shared by the CPU oracle and the HIP library: it
draws the *inputs* both sides consume and holds none of the method's
arithmetic (no span split, no summaries, no SVD, no routing, no attention).

Workloads stand in for the long-context evaluations of the SeKV article
(aitrends.kr/articles/75020, sections "주요 결과" / Main results and
"핵심 기여" / Key contributions: long-document benchmarks on ~8B-class models
up to 128K tokens).  None of those benchmarks' items is used; every array is
drawn from the laws below.

Recipe (per batch element b, layer l, KV head g):
  * surprisal H_t ~ N(3, 1.5^2) i.i.d., clipped at 0, fp32.
  * the K and V generators plant a fresh low-rank block after every token whose
    surprisal exceeds CUT = 6.0, the population mean + 2 population std of the
    *unclipped* law.  This is a fixed constant of the data law, not the sample
    statistic the method thresholds on, so planted blocks line up with the
    method's spans almost everywhere but not by construction.
  * rows of a planted block of n tokens: A (n x r) @ B (r x d) with A, B ~ N(0,1)
    plus N(0, 0.05^2) noise; rows of cut tokens: N(0, r) i.i.d. (same variance).
  * routing projection W ~ N(0, 1/d), fp32; decode and calibration queries
    q ~ N(0, 1) rounded to bf16.
  * component gates m = sigmoid(N(mu_g, 1)) per (b, l, kv head, K|V, span slot,
    component), or absent (m = 1).

Every array comes from its own torch.Generator, seeded from a SHA-256 of the
array's name and indices, so any slice can be regenerated on its own, on the
CPU (tests) or on the GPU (full-size runs).  CPU and GPU streams differ; a test
always draws both sides' inputs from the same device's stream.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence

import torch

CUT = 6.0          # planted-block cut of the generating law (3 + 2 * 1.5)
NOISE = 0.05       # std of the additive noise on planted-block rows


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and law of one synthetic workload."""
    name: str
    L: int                 # layers
    Hq: int                # query heads
    Hkv: int               # KV heads
    d: int                 # head dim
    B: int                 # batch (independent sequences)
    T: int                 # context tokens per sequence
    R: int                 # max SVD rank
    dprime: int            # summary-key dimension d'
    rank: int              # rank of the planted K/V blocks
    gate_mu: Optional[float]   # None -> m = 1, else m = sigmoid(N(gate_mu, 1))
    tau: Optional[float]       # fixed threshold, or None -> calibrated to `frac`
    frac: Optional[float]      # target expand fraction for calibration
    cap_frac: Optional[float]  # per-(layer, head) expansion cap as a fraction of N_S
    steps: int                 # decode steps
    tier: str = "hbm"          # factor tier: "hbm" or "pinned"
    alpha_sp: float = 2.0      # surprisal sensitivity of the span split
    l_min: int = 8             # runs shorter than this stay raw
    oversample: int = 8        # randomized-SVD oversampling
    power_iters: int = 2       # randomized-SVD power iterations
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1 layer, 4 query / 1 KV head, d=64, 2K context, tau fixed at 0.5.
    "tiny_2k": Workload("tiny_2k", L=1, Hq=4, Hkv=1, d=64, B=1, T=2048, R=16,
                        dprime=32, rank=8, gate_mu=None, tau=0.5, frac=None,
                        cap_frac=None, steps=1),
    # Llama-3.1-8B-shaped single layer at 32K, ~10% of span-head pairs expand.
    "llama8b_l1_32k": Workload("llama8b_l1_32k", L=1, Hq=32, Hkv=8, d=128, B=1,
                               T=32768, R=32, dprime=64, rank=8, gate_mu=2.0,
                               tau=None, frac=0.10, cap_frac=None, steps=256),
    # Llama-3.1-8B-shaped 32-layer stack at 128K, 10% budget, pinned-host factors.
    "llama8b_l32_128k": Workload("llama8b_l32_128k", L=32, Hq=32, Hkv=8, d=128,
                                 B=1, T=131072, R=16, dprime=64, rank=16,
                                 gate_mu=None, tau=None, frac=0.10,
                                 cap_frac=0.10, steps=64, tier="pinned"),
    # Prefill index build of one 8B-shaped layer at 128K, R=32.
    "prefill_8b_128k": Workload("prefill_8b_128k", L=1, Hq=32, Hkv=8, d=128,
                                B=1, T=131072, R=32, dprime=64, rank=16,
                                gate_mu=None, tau=None, frac=0.10,
                                cap_frac=None, steps=0),
    # Llama-3-70B-shaped single layer, 32 sequences of 64K, ~30% expand.
    "llama70b_b32_64k": Workload("llama70b_b32_64k", L=1, Hq=64, Hkv=8, d=128,
                                 B=32, T=65536, R=64, dprime=64, rank=8,
                                 gate_mu=1.0, tau=None, frac=0.30,
                                 cap_frac=None, steps=128),
}


def _seed(*keys) -> int:
    h = hashlib.sha256(repr(keys).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 62) - 1)


def _gen(device, *keys) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*keys))
    return g


def surprisal(w: Workload, b: int, device="cpu") -> torch.Tensor:
    """H[b, :] as fp32 [T]: N(3, 1.5^2) clipped at 0."""
    g = _gen(device, w.seed, "H", b)
    h = torch.randn(w.T, generator=g, device=device, dtype=torch.float32)
    return (3.0 + 1.5 * h).clamp_min_(0.0)


def _planted_blocks(h: torch.Tensor):
    """Block id per token (-1 for cut tokens) and the block count."""
    cut = h > CUT
    # a new block starts at every non-cut token that follows a cut token or t=0
    noncut = ~cut
    prev_cut = torch.ones_like(cut)
    prev_cut[1:] = cut[:-1]
    starts = noncut & prev_cut
    bid = torch.cumsum(starts.to(torch.int64), 0) - 1
    bid = torch.where(noncut, bid, torch.full_like(bid, -1))
    nblk = int(starts.sum().item())
    return bid, nblk


def kv_rows(w: Workload, h: torch.Tensor, b: int, l: int, g: int, which: str,
            device="cpu") -> torch.Tensor:
    """K (which='K') or V (which='V') rows of (b, l, KV head g): bf16 [T, d]."""
    assert which in ("K", "V")
    T, d, r = w.T, w.d, w.rank
    gen = _gen(device, w.seed, "KV", which, b, l, g)
    bid, nblk = _planted_blocks(h)
    a = torch.randn(T, r, generator=gen, device=device)
    bmat = torch.randn(max(nblk, 1), r, d, generator=gen, device=device)
    noise = torch.randn(T, d, generator=gen, device=device)
    out = torch.randn(T, d, generator=gen, device=device) * math.sqrt(r)
    sel = bid >= 0
    if nblk > 0:
        # block-diagonal product A_blk @ B_blk, done as a padded batched product
        tok = torch.nonzero(sel).squeeze(1)
        blk = bid[tok]
        first = torch.zeros(nblk, dtype=torch.int64, device=device)
        first.scatter_reduce_(0, blk, tok, reduce="amin", include_self=False)
        pos = tok - first[blk]
        plen = int(pos.max().item()) + 1
        apad = torch.zeros(nblk, plen, r, device=device)
        apad[blk, pos] = a[tok]
        prod = torch.bmm(apad, bmat)
        out[tok] = prod[blk, pos] + NOISE * noise[tok]
    return out.to(torch.bfloat16)


def routing_w(w: Workload, l: int, device="cpu") -> torch.Tensor:
    """W^(l,h) for every query head: fp32 [Hq, d', d], N(0, 1/d)."""
    g = _gen(device, w.seed, "W", l)
    return torch.randn(w.Hq, w.dprime, w.d, generator=g, device=device) / math.sqrt(w.d)


def gates(w: Workload, b: int, l: int, s_max: int, device="cpu") -> Optional[torch.Tensor]:
    """Gates m for (b, l): fp32 [Hkv, 2 (K|V), s_max, R], or None when m = 1."""
    if w.gate_mu is None:
        return None
    g = _gen(device, w.seed, "gates", b, l)
    z = torch.randn(w.Hkv, 2, s_max, w.R, generator=g, device=device)
    return torch.sigmoid(z + w.gate_mu)


def query(w: Workload, step: int, device="cpu", layers: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Decode query of one step: bf16 [B, L, Hq, d] (or only `layers`)."""
    ls = range(w.L) if layers is None else layers
    out = []
    for l in ls:
        g = _gen(device, w.seed, "q", step, l)
        out.append(torch.randn(w.B, w.Hq, w.d, generator=g, device=device))
    return torch.stack(out, 1).to(torch.bfloat16)


def calibration_query(w: Workload, device="cpu", layers: Optional[Sequence[int]] = None) -> torch.Tensor:
    """A separate query stream used only to place tau: bf16 [B, L, Hq, d]."""
    ls = range(w.L) if layers is None else layers
    out = []
    for l in ls:
        g = _gen(device, w.seed, "q_cal", l)
        out.append(torch.randn(w.B, w.Hq, w.d, generator=g, device=device))
    return torch.stack(out, 1).to(torch.bfloat16)


def max_spans(T: int, l_min: int) -> int:
    """Upper bound on the number of compressed spans of a T-token context.

    k spans of >= l_min tokens need k * l_min tokens plus k - 1 separating
    tokens, so k <= (T + 1) // (l_min + 1).  Used only to size gate arrays.
    """
    return (T + 1) // (l_min + 1)


def kv_cache(w: Workload, device="cpu", layers: Optional[Sequence[int]] = None,
             batches: Optional[Sequence[int]] = None):
    """Full K, V caches as bf16 [B, L, Hkv, T, d] plus H [B, T] fp32."""
    bs = range(w.B) if batches is None else batches
    ls = range(w.L) if layers is None else layers
    H = torch.stack([surprisal(w, b, device) for b in bs])
    K = torch.empty(len(bs), len(ls), w.Hkv, w.T, w.d, dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    for i, b in enumerate(bs):
        for j, l in enumerate(ls):
            for g in range(w.Hkv):
                K[i, j, g] = kv_rows(w, H[i], b, l, g, "K", device)
                V[i, j, g] = kv_rows(w, H[i], b, l, g, "V", device)
    return H, K, V
