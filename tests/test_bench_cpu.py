"""Host logic of bench.py, on the CPU: the algorithmic bytes every roofline
figure rests on, the source-keyed traffic lookup, and the one-GPU refusal."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pack(bits):
    """bool [..., Wd*64] -> uint64 [..., Wd] with bit j of word w = entry 64w + j."""
    b = np.asarray(bits, np.uint8)
    shp = b.shape[:-1] + (b.shape[-1] // 64, 64)
    return np.packbits(b.reshape(shp)[..., ::-1], axis=-1).view(">u8")[..., 0].astype(np.uint64)


def test_union_bytes_against_brute_force():
    rng = np.random.default_rng(3)
    B, Hq, G, R, d, Wd = 2, 8, 4, 16, 128, 2
    n_spans = np.array([100, 77])
    span_len = rng.integers(8, 300, int(n_spans.sum())).astype(np.int32)
    z = rng.random((B, Hq, Wd * 64)) < 0.2
    for b in range(B):
        z[b, :, n_spans[b]:] = False
    # stored ranks (K, V) per (b, g, span): R everywhere, then ragged
    for ragged in (False, True):
        ranks = [np.full((Hq // G, int(n), 2), R, np.int64) if not ragged else
                 16 * rng.integers(1, 5, (Hq // G, int(n), 2)) for n in n_spans]
        got, unions = bench.union_alg_bytes(_pack(z), n_spans, span_len, G, ranks, d)
        want, cnt, off = 0, 0, 0
        for b in range(B):
            for g in range(Hq // G):
                for S in range(int(n_spans[b])):
                    if any(z[b, h, S] for h in range(g * G, (g + 1) * G)):
                        n = int(span_len[off + S])
                        rk, rv = (int(x) for x in ranks[b][g, S])
                        # U (n x r) and V (d x r) in bf16, sigma m (r) in fp32, for K and for V
                        want += 2 * rk * (n + d) + 4 * rk + 2 * rv * (n + d) + 4 * rv
                        if not ragged:
                            assert 2 * rk * (n + d) + 4 * rk + 2 * rv * (n + d) + 4 * rv == 4 * R * (n + d) + 8 * R
                        cnt += 1
            off += int(n_spans[b])
        assert (got, unions) == (want, cnt)


def test_traffic_lookup_is_keyed_to_the_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "bytes_per_launch": 123}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.traffic_from_profile(0) == 123
    rec["kernel_source_sha256_16"] = "0" * 16
    p.write_text(json.dumps(rec))
    assert bench.traffic_from_profile(0) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.traffic_from_profile(0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
