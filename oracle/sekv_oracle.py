"""Plain fp64 CPU oracle of the SeKV decode path (and of its prefill index build).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or run this module.  The HIP library never calls it,
and the two share no code: this file imports only numpy and the standard
library.

Citations name the SeKV article "SeKV: 계층적 시맨틱 메모리를 통한 해상도 적응형
KV 캐시로 장문 컨텍스트 LLM 추론 효율화" (aitrends.kr/articles/75020) and a section
of it:
  [Contrib]  핵심 기여 (Key contributions)
  [Method]   방법론 (Method), including the Fig. 2 architecture caption
  [Tech]     기술 상세 (Technical details), including the reconstruction sum
             that the Method section calls Eq. 8
Where the article leaves a step open, the reading taken is stated at the
function that takes it.

Everything is fp64 numpy; inputs arrive in their storage precision (bf16 K, V,
q; fp32 H, W, gates) and are widened exactly.  No blocking, fusion or
reordering beyond the stated definitions.

Parity pins (tests/test_oracle_pins.py): full-rank + tau=-inf equals full
attention; tau=+inf equals full attention over span-mean-replaced rows; brute
force span split on tiny inputs; SVD against an eigen-decomposition of A^T A;
routing against the (W^T W) identity and a sign test at tau=0.5; the
summary keys of a built index against numpy's weighted average; the cap rule
against brute force; the pooled budget against brute force and against the
per-head cap on a one-head pool; calibration by counting; dropped components
(gate below eps) against the Eckart-Young error of the kept set, against a
reconstruction that leaves them out, and, all dropped, against the closed
form of attention over zero rows; decode at truncated rank with a mixed
per-head z against attention over rows projected onto their top-R
eigenvectors of A^T A (numpy eigh) and mean copies.  The pages print no
worked example, so no pin holds an absolute output value from them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

f64 = np.float64


# ----------------------------------------------------------------------------
# storage rounding (the build's storage formats; the pages fix none)
# ----------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (8 significant bits), ties to
    even, in one rounding step.  Returns fp64 holding bf16-representable values.
    Normal-range values only (|x| >= 2^-126 or 0), which covers every array here."""
    x = np.asarray(x, dtype=f64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    y = np.rint(m * 256.0) / 256.0          # 8 significant bits, ties to even
    return np.ldexp(y, e)


def round_f32(x) -> np.ndarray:
    """Round to fp32 (IEEE round-to-nearest-even), returned as fp64."""
    return np.asarray(x, dtype=f64).astype(np.float32).astype(f64)


# ----------------------------------------------------------------------------
# O1. span split  [Method] boundaries where H_t exceeds mu + alpha*sigma, the
# boundary tokens pinned as anchors; [Method] anchors and very short spans are
# kept raw on the GPU; [Contrib] span length adapts to content density.
# ----------------------------------------------------------------------------

@dataclass
class SpanSplit:
    thr: float
    anchor: np.ndarray        # bool [T]
    spans: np.ndarray         # int64 [N_S, 2]: (start, length), in position order
    raw: np.ndarray           # int64 [N_raw]: raw token positions, ascending


def span_split(H, alpha_sp: float, l_min: int) -> SpanSplit:
    """Readings: mu and sigma are the mean and population std of the whole
    sequence's surprisal (R1); "exceeds" is strict (R2); an anchor is not part
    of any span, spans are the maximal anchor-free runs (R3); runs shorter than
    l_min tokens stay raw (R4)."""
    h = [float(x) for x in np.asarray(H, dtype=f64)]
    T = len(h)
    mu = math.fsum(h) / T
    sigma = math.sqrt(math.fsum((x - mu) ** 2 for x in h) / T)
    thr = mu + alpha_sp * sigma
    anchor = np.array([x > thr for x in h], dtype=bool)
    spans, raw = [], []
    t = 0
    while t < T:
        if anchor[t]:
            raw.append(t)
            t += 1
            continue
        a = t
        while t < T and not anchor[t]:
            t += 1
        if t - a >= l_min:
            spans.append((a, t - a))
        else:
            raw.extend(range(a, t))
    return SpanSplit(thr, anchor,
                     np.array(spans, dtype=np.int64).reshape(-1, 2),
                     np.array(raw, dtype=np.int64))


# ----------------------------------------------------------------------------
# O2. summaries  [Contrib] surprisal-weighted mean key and value per span and a
# low-dim summary key; [Method] / [Tech] the summary key is projected to d'
# dimensions by the per-(layer, head) projection W^(l,h).
# ----------------------------------------------------------------------------

def weighted_mean(X, w) -> np.ndarray:
    """sum_t w_t x_t / sum_t w_t over the rows of X; uniform weights when the
    weights sum to zero (R6: surprisal weights are the raw H_t >= 0)."""
    X = np.asarray(X, dtype=f64)
    w = np.asarray(w, dtype=f64)
    if w.sum() == 0.0:
        w = np.ones_like(w)
    return (w[:, None] * X).sum(0) / w.sum()


def summary_key(W_h, kbar) -> np.ndarray:
    """s = W^(l,h) kbar (R7: the same W that routing applies to q, no 1/sqrt(d')
    scale)."""
    return np.asarray(W_h, dtype=f64) @ np.asarray(kbar, dtype=f64)


# ----------------------------------------------------------------------------
# O3 / O6. truncated SVD  [Contrib] / [Method] / [Tech]: each span's key and
# value matrix is stored as a truncated SVD U Sigma V^T per layer and head.
# ----------------------------------------------------------------------------

def truncated_svd(A, R: int):
    """Exact SVD (LAPACK), the R_eff = min(R, n, d) leading triplets, zero-padded
    to R columns (R14).  Returns U [n, R], sigma [R], Vt [R, d].  Uncentred
    (R13)."""
    A = np.asarray(A, dtype=f64)
    n, d = A.shape
    U_, s_, Vt_ = np.linalg.svd(A, full_matrices=False)
    r = min(R, n, d)
    U = np.zeros((n, R))
    s = np.zeros(R)
    Vt = np.zeros((R, d))
    U[:, :r] = U_[:, :r]
    s[:r] = s_[:r]
    Vt[:r] = Vt_[:r]
    return U, s, Vt


def svd_optimum_error(A, R: int) -> float:
    """Eckart-Young-Mirsky: the least Frobenius error of any rank-R
    approximation is the root sum of squares of the trailing singular values."""
    s_ = np.linalg.svd(np.asarray(A, dtype=f64), compute_uv=False)
    r = min(R, len(s_))
    return float(math.sqrt(math.fsum(float(x) ** 2 for x in s_[r:])))


def kept_components(m, n: int, R: int, eps: Optional[float]) -> np.ndarray:
    """Which of a span's R stored components survive (R28).  [Contrib] (the
    dual-resolution item) and [Tech] (the low-rank paragraph): the component
    gates set each span's effective rank, and components are dropped when
    stored and transferred.  Reading: component i is kept iff it is one of the
    R_eff = min(R, n) components the truncation holds (R14) and, when eps > 0,
    its gate m_i >= eps; eps None or <= 0 drops no gated component.  A dropped
    component is absent from the reconstruction sum, which is the same as
    giving it sigma_i * m_i = 0.  Returns bool [R]."""
    m = np.asarray(m, dtype=f64)
    keep = np.arange(R) < min(R, n)
    if eps is not None and eps > 0:
        keep &= m >= eps        # a NaN gate compares false: dropped
    return keep


def reconstruct(U, sm, Vt) -> np.ndarray:
    """[Tech] reconstruction sum: Khat = sum_i m_i sigma_i u_i v_i^T, with the
    gate already folded into sm = sigma * m (R15)."""
    return np.asarray(U, f64) @ np.diag(np.asarray(sm, f64)) @ np.asarray(Vt, f64)


# ----------------------------------------------------------------------------
# Index build: O1 + O2 + O3 over a whole batch, in the logical layout the
# library's import/export calls document (include/sekv.h, sekv_host_index).
# ----------------------------------------------------------------------------

@dataclass
class BatchIndex:
    """One sequence's index.  Rows are ordered raw tokens (ascending position)
    then one pseudo row per compressed span (span order)."""
    split: SpanSplit
    kres: np.ndarray          # [L, Hkv, N_raw + N_S, d]
    vres: np.ndarray
    s: np.ndarray             # [L, Hq, d', N_S]
    uk: np.ndarray            # [L, Hkv, sum n_S, R]
    uv: np.ndarray
    vkt: np.ndarray           # [L, Hkv, N_S, R, d]
    vvt: np.ndarray
    smk: np.ndarray           # [L, Hkv, N_S, R]
    smv: np.ndarray
    sig_k: np.ndarray         # [L, Hkv, N_S, R] singular values (ungated)
    sig_v: np.ndarray
    rank_k: Optional[np.ndarray] = None   # [L, Hkv, N_S] kept components (R28)
    rank_v: Optional[np.ndarray] = None

    @property
    def n_spans(self) -> int:
        return len(self.split.spans)

    @property
    def n_raw(self) -> int:
        return len(self.split.raw)

    def tok_off(self) -> np.ndarray:
        """Row offset of each span in the concatenated U arrays."""
        lens = self.split.spans[:, 1]
        return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64) if len(lens) else np.zeros(0, np.int64)


def build_index_b(H_b, K_b, V_b, W, gates_b, *, R: int, alpha_sp: float,
                  l_min: int, Hq: int, store: bool = True,
                  layers: Optional[List[int]] = None,
                  kv_heads: Optional[List[int]] = None,
                  gate_eps: Optional[float] = None) -> BatchIndex:
    """Index of one sequence.

    H_b [T] fp32; K_b, V_b [L, Hkv, T, d] (bf16 values); W [L, Hq, d', d] fp32;
    gates_b [L, Hkv, 2, S_max, R] or None (m = 1).  Span ordinal j uses gate
    slot j.  gate_eps > 0 drops the components whose gate is below it
    (kept_components); the dropped ones are stored with sigma * m = 0 and
    rank_k / rank_v count the kept ones.  With store=True the stored arrays are rounded to the storage
    formats (bf16 rows and factors, fp32 s and sigma*m); with store=False they
    stay fp64 (used by the full-rank pin).  `layers` / `kv_heads` restrict the
    work to a subset (the rest stays zero), for sampled checks at full size.
    """
    K_b = np.asarray(K_b, dtype=f64)
    V_b = np.asarray(V_b, dtype=f64)
    W = np.asarray(W, dtype=f64)
    L, Hkv, T, d = K_b.shape
    G = Hq // Hkv
    dp = W.shape[2]
    sp = span_split(H_b, alpha_sp, l_min)
    NS, NR = len(sp.spans), len(sp.raw)
    ntok = int(sp.spans[:, 1].sum()) if NS else 0
    h = np.asarray(H_b, dtype=f64)
    rb = round_bf16 if store else (lambda x: np.asarray(x, f64))
    rf = round_f32 if store else (lambda x: np.asarray(x, f64))
    idx = BatchIndex(sp,
                     kres=np.zeros((L, Hkv, NR + NS, d)), vres=np.zeros((L, Hkv, NR + NS, d)),
                     s=np.zeros((L, Hq, dp, NS)),
                     uk=np.zeros((L, Hkv, ntok, R)), uv=np.zeros((L, Hkv, ntok, R)),
                     vkt=np.zeros((L, Hkv, NS, R, d)), vvt=np.zeros((L, Hkv, NS, R, d)),
                     smk=np.zeros((L, Hkv, NS, R)), smv=np.zeros((L, Hkv, NS, R)),
                     sig_k=np.zeros((L, Hkv, NS, R)), sig_v=np.zeros((L, Hkv, NS, R)),
                     rank_k=np.zeros((L, Hkv, NS), np.int64), rank_v=np.zeros((L, Hkv, NS), np.int64))
    off = idx.tok_off()
    for l in (range(L) if layers is None else layers):
        for g in (range(Hkv) if kv_heads is None else kv_heads):
            K, V = K_b[l, g], V_b[l, g]
            idx.kres[l, g, :NR] = K[sp.raw]          # raw rows are stored as given
            idx.vres[l, g, :NR] = V[sp.raw]
            for j, (a, n) in enumerate(sp.spans):
                kbar = weighted_mean(K[a:a + n], h[a:a + n])
                vbar = weighted_mean(V[a:a + n], h[a:a + n])
                idx.kres[l, g, NR + j] = rb(kbar)
                idx.vres[l, g, NR + j] = rb(vbar)
                for hh in range(g * G, (g + 1) * G):
                    idx.s[l, hh, :, j] = rf(summary_key(W[l, hh], kbar))
                for which, X in ((0, K), (1, V)):
                    U, sig, Vt = truncated_svd(X[a:a + n], R)
                    m = np.ones(R) if gates_b is None else np.asarray(gates_b[l, g, which, j], f64)
                    keep = kept_components(m, n, R, gate_eps)
                    sm = np.where(keep, sig * m, 0.0)
                    if which == 0:
                        idx.uk[l, g, off[j]:off[j] + n] = rb(U)
                        idx.vkt[l, g, j] = rb(Vt)
                        idx.smk[l, g, j] = rf(sm)
                        idx.sig_k[l, g, j] = sig
                        idx.rank_k[l, g, j] = int(keep.sum())
                    else:
                        idx.uv[l, g, off[j]:off[j] + n] = rb(U)
                        idx.vvt[l, g, j] = rb(Vt)
                        idx.smv[l, g, j] = rf(sm)
                        idx.sig_v[l, g, j] = sig
                        idx.rank_v[l, g, j] = int(keep.sum())
    return idx


# ----------------------------------------------------------------------------
# O4. routing  [Method] Stage 1: q^(l,h) through W^(l,h), dot with each span's
# summary key, sigmoid -> alpha_S, compared with the per-(layer, head) tau;
# [Tech] on budget overflow, spans are taken in descending alpha until the
# budget holds.
# ----------------------------------------------------------------------------

def logit_threshold(tau: float) -> float:
    """The routing-score threshold equivalent to alpha > tau (R27).  alpha =
    sigmoid(a) is strictly increasing and lies in (0, 1), so alpha > tau
    exactly when a > log(tau / (1 - tau)) for 0 < tau < 1; every score passes
    a tau <= 0 and none passes a tau >= 1.  A NaN tau passes nothing."""
    tau = float(tau)
    if tau != tau:
        return math.nan
    if tau <= 0.0:
        return -math.inf
    if tau >= 1.0:
        return math.inf
    return math.log(tau) - math.log1p(-tau)


def routing_score(W_h, q_h, s_h) -> np.ndarray:
    """a_S = (W^(l,h) q) . s_S for every span: the argument of the sigmoid."""
    u = np.asarray(W_h, f64) @ np.asarray(q_h, f64)
    return u @ np.asarray(s_h, f64)


def route_head(W_h, q_h, s_h, tau: float, cap: int = 0):
    """One (layer, query head).  W_h [d', d], q_h [d], s_h [d', N_S].
    Returns (alpha [N_S] fp64, z bool [N_S]).  Per query head (R8).  z_S =
    [alpha_S > tau] is decided on the score a_S against logit(tau) and the
    budget cap keeps the cap largest a_S (R27: the same decisions as alpha in
    exact arithmetic, and still ordered where alpha rounds to 1); alpha~ of the
    budget rule read as alpha (R10); the cap is per (layer, head), ties broken
    toward the lower span index (R11)."""
    a = routing_score(W_h, q_h, s_h)
    with np.errstate(over="ignore"):
        alpha = 1.0 / (1.0 + np.exp(-a))
    z = a > logit_threshold(tau)
    if cap > 0 and int(z.sum()) > cap:
        cand = np.nonzero(z)[0]
        order = sorted(cand, key=lambda j: (-a[j], j))
        keep = np.zeros_like(z)
        keep[order[:cap]] = True
        z = keep
    return alpha, z


def pool_budget(score, z, budget: int):
    """The budget rule of [Tech] (expand in descending alpha until the budget
    holds) read over a pool instead of one (layer, head): every (layer, head,
    span) triple of one sequence that a routing call covers.  score, z: dicts
    keyed (b, l, h) -> [N_S(b)] arrays: the routing scores a_S (ordered as
    alpha, R27) and the pre-budget routing.  For each b, keep the `budget`
    largest scores among the routed triples, ties broken toward the lower
    (l, h, span) position (R26); budget 0 = no budget.  Returns the new z
    dict."""
    out = {k: np.array(v, bool) for k, v in z.items()}
    if budget <= 0:
        return out
    for b in sorted({k[0] for k in z}):
        keys = sorted(k for k in z if k[0] == b)
        cand = [(-float(score[k][S]), k[1], k[2], int(S)) for k in keys for S in np.nonzero(z[k])[0]]
        if len(cand) <= budget:
            continue
        cand.sort()
        kept = {(l, h, S) for _, l, h, S in cand[:budget]}
        for k in keys:
            m = np.zeros(len(z[k]), bool)
            for S in np.nonzero(z[k])[0]:
                m[S] = (k[1], k[2], int(S)) in kept
            out[k] = m
    return out


def calibrate_tau(alphas, frac: float) -> float:
    """tau placed so that round(frac * N) of the given alphas exceed it: the
    midpoint of the k-th and (k+1)-th largest (R12), k clipped to [1, N-1]."""
    a = np.sort(np.asarray(alphas, f64).ravel())[::-1]
    N = len(a)
    k = int(math.floor(frac * N + 0.5))
    k = min(max(k, 1), N - 1)
    return float(0.5 * (a[k - 1] + a[k]))


# ----------------------------------------------------------------------------
# O5. decode attention  [Method] Stage 2: selected spans are rebuilt to token
# level through the gated factors (Eq. 8, printed in [Tech]) and merged into
# the final attention output (Fig. 2); [Contrib] unexpanded spans contribute
# through their surprisal-weighted mean key/value.
# ----------------------------------------------------------------------------

def decode_head(q_h, idx: BatchIndex, l: int, g: int, z_h) -> np.ndarray:
    """One (sequence, layer, query head) of KV head g.  Attention set: every raw
    row; for span S with z=1 the n_S materialised rows of Khat, Vhat (bias 0);
    otherwise the pseudo row (kbar, vbar) with logit bias ln n_S (R16).  Scale
    1/sqrt(d) (R17).  No causal mask, no self token (R18)."""
    q = np.asarray(q_h, f64)
    d = q.shape[0]
    NR = idx.n_raw
    off = idx.tok_off()
    keys, vals, bias = [idx.kres[l, g, :NR]], [idx.vres[l, g, :NR]], [np.zeros(NR)]
    for j, (a, n) in enumerate(idx.split.spans):
        if z_h[j]:
            keys.append(reconstruct(idx.uk[l, g, off[j]:off[j] + n], idx.smk[l, g, j], idx.vkt[l, g, j]))
            vals.append(reconstruct(idx.uv[l, g, off[j]:off[j] + n], idx.smv[l, g, j], idx.vvt[l, g, j]))
            bias.append(np.zeros(n))
        else:
            keys.append(idx.kres[l, g, NR + j][None])
            vals.append(idx.vres[l, g, NR + j][None])
            bias.append(np.array([math.log(n)]))
    Kall = np.concatenate(keys)
    Vall = np.concatenate(vals)
    logit = Kall @ q / math.sqrt(d) + np.concatenate(bias)
    p = np.exp(logit - logit.max())
    p /= p.sum()
    return p @ Vall


def full_attention(q_h, K, V) -> np.ndarray:
    """Exact softmax(q K^T / sqrt(d)) V over every context row."""
    q = np.asarray(q_h, f64)
    K = np.asarray(K, f64)
    V = np.asarray(V, f64)
    logit = K @ q / math.sqrt(q.shape[0])
    p = np.exp(logit - logit.max())
    return (p / p.sum()) @ V


# ----------------------------------------------------------------------------
# Whole-step drivers (loops over the per-head definitions above)
# ----------------------------------------------------------------------------

def route_step(idxs: List[BatchIndex], W, q, tau, cap: int = 0, layers=None, heads=None):
    """alpha, z per (b, l, h): dicts keyed by (b, l, h)."""
    W = np.asarray(W, f64)
    q = np.asarray(q, f64)
    tau = np.asarray(tau, f64)
    B = len(idxs)
    L, Hq = tau.shape
    alpha, z = {}, {}
    for b in range(B):
        for l in (range(L) if layers is None else layers):
            for h in (range(Hq) if heads is None else heads):
                alpha[b, l, h], z[b, l, h] = route_head(W[l, h], q[b, l, h], idxs[b].s[l, h], tau[l, h], cap)
    return alpha, z


def score_step(idxs: List[BatchIndex], W, q, layers=None, heads=None):
    """Routing scores a_S per (b, l, h): dict keyed by (b, l, h)."""
    W = np.asarray(W, f64)
    q = np.asarray(q, f64)
    L, Hq = W.shape[0], W.shape[1]
    return {(b, l, h): routing_score(W[l, h], q[b, l, h], idxs[b].s[l, h])
            for b in range(len(idxs)) for l in (range(L) if layers is None else layers)
            for h in (range(Hq) if heads is None else heads)}


def decode_step(idxs: List[BatchIndex], q, z, Hkv: int, keys=None):
    """out[(b, l, h)] for the (b, l, h) in `keys` (default: every key of z)."""
    q = np.asarray(q, f64)
    Hq = q.shape[2]
    G = Hq // Hkv
    out = {}
    for (b, l, h) in (z.keys() if keys is None else keys):
        out[b, l, h] = decode_head(q[b, l, h], idxs[b], l, h // G, z[b, l, h])
    return out
