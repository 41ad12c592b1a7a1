"""Variable effective rank on the GPU: components whose gate is below the
build's gate_eps are not stored, so each blob holds a ragged rank (reading
R28 of the oracle: SeKV article, sections 핵심 기여 / Key contributions, the
dual-resolution item, and 기술 상세 / Technical details, the low-rank
paragraph).

Bars: stored ranks bit-exact against the oracle's kept counts (rounded up to
the 16-wide tile); factor-pool bytes equal to the sum of the blob sizes;
masks bit-exact outside the score windows and decode outputs within 5e-3 of
the oracle decoding the library's exported index, on both tiers and with
layer ranges that start past 0; the kept components of a ragged build
bit-identical to the same components of a build that keeps every component
with the dropped gates set to zero.
"""
import numpy as np
import pytest
import torch

from compressed_kv_cache_sekv_amd import synth
from oracle import sekv_oracle as O
from tests import sekv_cases as SC

pytestmark = pytest.mark.gpu

EPS = 0.5
# R = 64, G = 8, gates sigmoid(N(1, 1)): the 70B-shaped batch, two sequences
W70 = synth.WORKLOADS["llama70b_b32_64k"].scaled(B=2, T=8192)
# two layers (layouts that differ per layer), R = 64, gates sigmoid(N(1, 1))
W2L = synth.WORKLOADS["llama8b_l1_32k"].scaled(L=2, T=8192, R=64, gate_mu=1.0)

_INPUTS = {}


def inputs(w):
    if w.name + str(w.L) not in _INPUTS:
        _INPUTS[w.name + str(w.L)] = SC.make_inputs(w)
    return _INPUTS[w.name + str(w.L)]


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


def build(ctx, sl, w, eps, tier=0, gates=None, ring_bytes=0):
    H, K, V, W, g = inputs(w)
    g = g if gates is None else gates
    print(f"[rank] build {w.name} L={w.L} B={w.B} T={w.T} R={w.R} eps={eps} tier={tier}", flush=True)
    return ctx.build_index(sl.build_params(w, tier=tier, ring_bytes=ring_bytes, gate_eps=eps),
                           K.cuda(), V.cuda(), H.cuda(), W.cuda(), None if g is None else g.cuda())


def oracle_stored_ranks(w, idx, gates, eps):
    """[L][Hkv][N_S][2] per sequence, concatenated: the oracle's kept counts
    (kept_components) rounded up to the 16-wide tile, at least 16."""
    lens = idx.span_lengths()
    out, off = [], 0
    for b in range(w.B):
        ns = int(idx.n_spans[b])
        rb = np.zeros((w.L, w.Hkv, ns, 2), np.int64)
        for l in range(w.L):
            for g in range(w.Hkv):
                for S in range(ns):
                    n = int(lens[off + S])
                    for which in range(2):
                        m = np.ones(w.R) if gates is None else gates[b, l, g, which, S].double().numpy()
                        k = int(O.kept_components(m, n, w.R, eps).sum())
                        rb[l, g, S, which] = 16 if k <= 16 else 16 * ((k + 15) // 16)
        out.append(rb.ravel())
        off += ns
    return np.concatenate(out)


def blob_bytes(rk, rv, d, n):
    npad = (n + 15) // 16 * 16
    return (2 * (rk + rv) * d + 4 * (rk + rv) + 2 * npad * (rk + rv) + 255) // 256 * 256


def calibrated_tau(idx, w):
    tau = torch.zeros(w.L, w.Hq, dtype=torch.float32, device="cuda")
    idx.calibrate_tau(0, w.L, synth.calibration_query(w).cuda(), w.frac, tau)
    torch.cuda.synchronize()
    return tau.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_stored_ranks_follow_the_gates(ctx, sl, eps):
    w = W70
    gates = inputs(w)[4]
    idx = build(ctx, sl, w, eps)
    ex = idx.export(fields=["rank"])
    ref = oracle_stored_ranks(w, idx, gates, eps)
    assert np.array_equal(ex["rank"].astype(np.int64), ref)
    # the pool holds exactly the blobs at those ranks, 256-byte aligned
    lens = idx.span_lengths()
    rk = ref.reshape(-1, 2)
    tot, off, r0 = 0, 0, 0
    for b in range(w.B):
        ns = int(idx.n_spans[b])
        rr = rk[r0:r0 + w.L * w.Hkv * ns].reshape(w.L, w.Hkv, ns, 2)
        n = np.broadcast_to(lens[off:off + ns], (w.L, w.Hkv, ns))
        tot += int(blob_bytes(rr[..., 0], rr[..., 1], w.d, n).sum())
        off += ns
        r0 += w.L * w.Hkv * ns
    assert idx.info.factor_bytes == tot
    full = int(sum(blob_bytes(w.R, w.R, w.d, int(n)) for n in lens)) * w.L * w.Hkv
    mean_rank = float(rk.mean())
    print(f"[rank] eps={eps}: mean stored rank {mean_rank:.1f} of R={w.R}; factor bytes {tot / 2**20:.1f} MiB "
          f"({tot / full:.3f} of rank R everywhere)")
    assert tot < full
    idx.free()


def _route(idx, w, q, tau, lb, lc):
    mask = torch.zeros(w.B, lc, w.Hq, idx.mask_words, dtype=torch.int64, device="cuda")
    idx.route(lb, lc, q[:, lb:lb + lc].contiguous().cuda(),
              torch.as_tensor(tau[lb:lb + lc], dtype=torch.float32).contiguous().cuda(), 0, mask, None)
    return mask


def _decode(idx, w, q, mask, lb, lc, stats=False):
    out = torch.zeros(w.B, lc, w.Hq, w.d, dtype=torch.float32, device="cuda")
    st = idx.decode_attend(lb, lc, q[:, lb:lb + lc].contiguous().cuda(), mask, out, stats=stats)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), st


def _check_against_export(idx, w, q, tau, words, out, lb, lc, label):
    """Masks of layers [lb, lb + lc) and outputs against the oracle routing
    and decoding the library's export of those layers."""
    ex = idx.export(layer_begin=lb, layer_count=lc)
    ix = SC.index_from_export(ex, idx.n_spans, idx.n_raw, lc, w.Hq, w.Hkv, w.d, w.R, w.dprime)
    W = inputs(w)[3][lb:lb + lc]
    ref = SC.route_ref(ix, W, q[:, lb:lb + lc], tau[lb:lb + lc])
    SC.check_masks(lambda k: words[k], ref, label)
    worst = 0.0
    qn = q[:, lb:lb + lc].double().numpy()
    for (b, l, h) in ref.z:
        zg = SC.unpack_mask(words[b, l, h], ix[b].n_spans)
        o = O.decode_head(qn[b, l, h], ix[b], l, h // w.G, zg)
        worst = max(worst, SC.rel_l2(out[b, l, h], o))
    print(f"[rank] {label}: worst rel-L2 {worst:.2e}")
    assert worst <= SC.REL_L2


def _union_blob_bytes(idx, w, words, lb, lc):
    """Bytes the gather must move for these masks: the padded blobs of each
    (b, l, g) union, from the exported ranks and span lengths."""
    rk = idx.export(layer_begin=lb, layer_count=lc, fields=["rank"])["rank"]
    lens = idx.span_lengths()
    tot, so, ro = 0, 0, 0
    for b in range(w.B):
        ns = int(idx.n_spans[b])
        r = rk[ro:ro + lc * w.Hkv * ns * 2].reshape(lc, w.Hkv, ns, 2)
        for l in range(lc):
            for g in range(w.Hkv):
                u = np.zeros(ns, bool)
                for h in range(g * w.G, (g + 1) * w.G):
                    u |= SC.unpack_mask(words[b, l, h], ns)
                n = lens[so:so + ns][u].astype(np.int64)
                tot += int(blob_bytes(r[l, g, u, 0], r[l, g, u, 1], w.d, n).sum())
        so += ns
        ro += lc * w.Hkv * ns * 2
    return tot


@pytest.mark.parametrize("tier,slots", [(0, 0), (1, 2), (1, 1)], ids=["hbm", "pinned-2slots", "pinned-1slot"])
def test_ragged_decode_against_oracle_per_layer_calls(ctx, sl, tier, slots):
    """Two layers whose blob layouts differ, decoded one layer per call (the
    second call starts at layer 1) and both layers in one call: on the pinned
    tier with two ring slots (the second layer gathered while the first is
    attended) and with one (gather and attend in turn)."""
    w = W2L
    idx = build(ctx, sl, w, EPS, tier=tier)
    if slots == 1:
        one = idx.info.ring_bytes // 2     # the default ring holds two slots
        idx.free()
        idx = build(ctx, sl, w, EPS, tier=tier, ring_bytes=one)
    q = synth.query(w, 0)
    tau = calibrated_tau(idx, w)
    for lb, lc in ((0, 1), (1, 1), (0, 2)):
        mask = _route(idx, w, q, tau, lb, lc)
        out, st = _decode(idx, w, q, mask, lb, lc, stats=tier == 1)
        words = mask.cpu().numpy().view(np.uint64)
        _check_against_export(idx, w, q, tau, words, out, lb, lc, f"tier {tier} slots {slots} layers [{lb}, {lb + lc})")
        if tier == 1:
            assert st.pcie_copies == lc
            assert st.pcie_bytes == _union_blob_bytes(idx, w, words, lb, lc)
            print(f"[rank] gather of layers [{lb}, {lb + lc}): {st.pcie_bytes} bytes in {st.pcie_ms:.3f} ms")
    idx.free()


@pytest.mark.parametrize("eps", [EPS, 2.0])
def test_ragged_decode_against_oracle_batch(ctx, sl, eps):
    """The 70B-shaped pair of sequences at gate_eps 0.5, and at 2.0, where
    every gate is below eps: each blob then stores one tile of zero
    components, every expanded span contributes rows of key 0 and value 0."""
    w = W70
    idx = build(ctx, sl, w, eps)
    if eps > 1:
        ex = idx.export(fields=["rank", "smk", "smv"])
        assert (ex["rank"] == 16).all() and not ex["smk"].any() and not ex["smv"].any()
    q = synth.query(w, 0)
    tau = calibrated_tau(idx, w)
    mask = _route(idx, w, q, tau, 0, 1)
    out, _ = _decode(idx, w, q, mask, 0, 1)
    _check_against_export(idx, w, q, tau, mask.cpu().numpy().view(np.uint64), out, 0, 1,
                          f"70B-shaped batch, gate_eps {eps}")
    idx.free()


def test_kept_components_are_compacted_bit_exactly(ctx, sl):
    """A ragged build keeps, in slots 0..k-1 of each blob, exactly the
    components (bitwise: same randomized SVD) that a build keeping every
    component stores at the indices whose gate reaches eps, there with the
    other gates set to zero; both decode the same masks alike."""
    w = W2L
    H, K, V, W, gates = inputs(w)
    zeroed = torch.where(gates >= EPS, gates, torch.zeros_like(gates))
    rag = build(ctx, sl, w, EPS)
    ful = build(ctx, sl, w, 0.0, gates=zeroed)
    er, ef = rag.export(), ful.export()
    R, d, L, Hkv = w.R, w.d, w.L, w.Hkv
    lens = rag.span_lengths()
    so = to = 0
    checked = 0
    for b in range(w.B):
        ns = int(rag.n_spans[b])
        ln = lens[so:so + ns]
        nt = int(ln.sum())
        toff = np.concatenate([[0], np.cumsum(ln)[:-1]]).astype(np.int64)
        sp = lambda a: a.reshape(L, Hkv, ns, R) if a.size == L * Hkv * ns * R else None
        base_sp = sum(L * Hkv * int(rag.n_spans[bb]) for bb in range(b))
        for which, sm_k, u_k, v_k in ((0, "smk", "uk", "vkt"), (1, "smv", "uv", "vvt")):
            smr = er[sm_k][base_sp * R:(base_sp + L * Hkv * ns) * R].reshape(L, Hkv, ns, R)
            smf = ef[sm_k][base_sp * R:(base_sp + L * Hkv * ns) * R].reshape(L, Hkv, ns, R)
            ur = er[u_k][to * R:(to + L * Hkv * nt) * R].reshape(L, Hkv, nt, R)
            uf = ef[u_k][to * R:(to + L * Hkv * nt) * R].reshape(L, Hkv, nt, R)
            vr = er[v_k][base_sp * R * d:(base_sp + L * Hkv * ns) * R * d].reshape(L, Hkv, ns, R, d)
            vf = ef[v_k][base_sp * R * d:(base_sp + L * Hkv * ns) * R * d].reshape(L, Hkv, ns, R, d)
            for l in range(L):
                for g in range(Hkv):
                    for S in range(ns):
                        n = int(ln[S])
                        m = gates[b, l, g, which, S].double().numpy()
                        keep = np.flatnonzero(O.kept_components(m, n, R, EPS))
                        k = len(keep)
                        assert np.array_equal(smr[l, g, S, :k], smf[l, g, S, keep])
                        assert not smr[l, g, S, k:].any()
                        rows = slice(int(toff[S]), int(toff[S]) + n)
                        assert np.array_equal(ur[l, g, rows, :k], uf[l, g, rows][:, keep])
                        assert np.array_equal(vr[l, g, S, :k], vf[l, g, S, keep])
                        checked += 1
        so += ns
        to += L * Hkv * nt
    assert checked > 100
    q = synth.query(w, 1)
    tau = calibrated_tau(rag, w)
    m1 = _route(rag, w, q, tau, 0, w.L)
    m2 = _route(ful, w, q, tau, 0, w.L)
    assert torch.equal(m1, m2)
    o1, _ = _decode(rag, w, q, m1, 0, w.L)
    o2, _ = _decode(ful, w, q, m1, 0, w.L)
    worst = max(SC.rel_l2(o1[k], o2[k]) for k in np.ndindex(o1.shape[:3]))
    print(f"[rank] ragged vs zero-gated full build: worst rel-L2 {worst:.2e}")
    assert worst <= 1e-5
    assert rag.info.factor_bytes < ful.info.factor_bytes
    rag.free()
    ful.free()


def test_ragged_import_export_roundtrip(ctx, sl):
    """Export of a ragged build, imported and exported again: every array and
    rank equal, and the imported index decodes bit-identically."""
    w = W2L
    idx = build(ctx, sl, w, EPS)
    ex = idx.export()
    arr = dict(ex)
    arr["n_spans"] = idx.n_spans.copy()
    arr["n_raw"] = idx.n_raw.copy()
    arr["W"] = inputs(w)[3].numpy().astype(np.float32).ravel()
    imp = ctx.import_index(sl.build_params(w, gate_eps=EPS), arr)
    ex2 = imp.export()
    for k in ex:
        assert np.array_equal(ex[k], ex2[k]), k
    assert imp.info.factor_bytes == idx.info.factor_bytes
    q = synth.query(w, 2)
    tau = calibrated_tau(idx, w)
    mask = _route(idx, w, q, tau, 0, w.L)
    o1, _ = _decode(idx, w, q, mask, 0, w.L)
    o2, _ = _decode(imp, w, q, mask, 0, w.L)
    assert np.array_equal(o1, o2)
    imp.free()
    idx.free()
