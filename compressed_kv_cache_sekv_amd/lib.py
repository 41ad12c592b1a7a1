"""ctypes binding of libsekv.so (include/sekv.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch tensors supply device pointers and the HIP stream; nothing
here computes any part of the method.  Importing this module loads the
library and raises if it has not been built (python -m
compressed_kv_cache_sekv_amd.build).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SEKV_LIB overrides the library path (e.g. to compare builds).
LIB_PATH = os.environ.get("SEKV_LIB") or os.path.join(HERE, "libsekv.so")

TIER_HBM = 0
TIER_PINNED_HOST = 1

STATUS = {0: "SEKV_OK", 1: "SEKV_EINVAL", 2: "SEKV_ENOMEM", 3: "SEKV_EHIP",
          4: "SEKV_ECAPACITY", 5: "SEKV_ESTATE", 6: "SEKV_EUNSUPPORTED"}

# Every entry point declared in include/sekv.h.
EXPORTS = ("sekv_create", "sekv_destroy", "sekv_last_error", "sekv_max_spans",
           "sekv_validate_params", "sekv_rsvd_batched", "sekv_build_index", "sekv_index_import", "sekv_index_export",
           "sekv_index_export_part",
           "sekv_index_get_info", "sekv_index_counts", "sekv_index_free",
           "sekv_route", "sekv_route_pooled", "sekv_calibrate_tau", "sekv_decode_attend",
           "sekv_decode_attend_noalloc",
           "sekv_timing_enable", "sekv_timing_read")


class SekvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class BuildParams(C.Structure):
    _fields_ = [("B", C.c_int32), ("L", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("d", C.c_int32), ("T", C.c_int32), ("R", C.c_int32), ("dprime", C.c_int32),
                ("alpha_sp", C.c_float), ("l_min", C.c_int32), ("oversample", C.c_int32),
                ("power_iters", C.c_int32), ("seed", C.c_uint64), ("tier", C.c_int32),
                ("ring_bytes", C.c_int64), ("gate_eps", C.c_float)]


class IndexInfo(C.Structure):
    _fields_ = [("B", C.c_int32), ("L", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("d", C.c_int32), ("R", C.c_int32), ("dprime", C.c_int32), ("tier", C.c_int32),
                ("max_spans", C.c_int32), ("mask_words", C.c_int32),
                ("total_spans", C.c_int64), ("total_raw", C.c_int64),
                ("total_span_tokens", C.c_int64), ("resident_bytes", C.c_int64),
                ("factor_bytes", C.c_int64), ("ring_bytes", C.c_int64)]


_HOST_FIELDS = ("span_start", "span_len", "raw_pos", "k_res", "v_res", "s", "uk", "uv",
                "vkt", "vvt", "smk", "smv")


class HostIndex(C.Structure):
    _fields_ = [("n_spans", C.c_void_p), ("n_raw", C.c_void_p)] + \
               [(f, C.c_void_p) for f in _HOST_FIELDS] + [("W", C.c_void_p)]


class HostIndexOut(C.Structure):
    _fields_ = [(f, C.c_void_p) for f in _HOST_FIELDS] + [("rank", C.c_void_p)]


class Stats(C.Structure):
    _fields_ = [("union_spans", C.c_uint64), ("pcie_bytes", C.c_uint64),
                ("pcie_copies", C.c_uint64), ("pcie_ms", C.c_double)]


def load(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m compressed_kv_cache_sekv_amd.build`")
    lib = C.CDLL(path)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    lib.sekv_create.argtypes = [i32, vp, C.POINTER(vp)]
    lib.sekv_destroy.argtypes = [vp]
    lib.sekv_destroy.restype = None
    lib.sekv_last_error.restype = C.c_char_p
    lib.sekv_max_spans.argtypes = [i32, i32]
    lib.sekv_max_spans.restype = i32
    lib.sekv_validate_params.argtypes = [C.POINTER(BuildParams)]
    lib.sekv_rsvd_batched.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, C.c_uint64, vp, vp, vp]
    lib.sekv_build_index.argtypes = [vp, C.POINTER(BuildParams), vp, vp, vp, vp, vp, C.POINTER(vp)]
    lib.sekv_index_import.argtypes = [vp, C.POINTER(BuildParams), C.POINTER(HostIndex), C.POINTER(vp)]
    lib.sekv_index_export.argtypes = [vp, vp, C.POINTER(HostIndexOut)]
    lib.sekv_index_export_part.argtypes = [vp, vp, i32, i32, i32, i32, C.POINTER(HostIndexOut)]
    lib.sekv_index_get_info.argtypes = [vp, C.POINTER(IndexInfo)]
    lib.sekv_index_counts.argtypes = [vp, vp, vp]
    lib.sekv_index_free.argtypes = [vp]
    lib.sekv_index_free.restype = None
    lib.sekv_route.argtypes = [vp, vp, i32, i32, vp, vp, i32, vp, vp]
    lib.sekv_route_pooled.argtypes = [vp, vp, i32, i32, vp, vp, i32, vp, vp]
    lib.sekv_calibrate_tau.argtypes = [vp, vp, i32, i32, vp, f32, vp]
    lib.sekv_decode_attend.argtypes = [vp, vp, i32, i32, vp, vp, vp, C.POINTER(Stats)]
    lib.sekv_decode_attend_noalloc.argtypes = [vp, vp, i32, i32, vp, vp, vp, C.POINTER(Stats)]
    lib.sekv_timing_enable.argtypes = [vp, i32]
    lib.sekv_timing_read.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(i64),
                                     C.POINTER(C.c_double), C.POINTER(i64)]
    return lib


_LIB: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(status: int):
    if status != 0:
        raise SekvError(status, lib().sekv_last_error().decode(errors="replace"))


def _ptr(t) -> Optional[int]:
    """Device or host address of a torch tensor / numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.is_contiguous(), "tensors passed to libsekv must be contiguous"
    return t.data_ptr()


def validate_params(p: BuildParams) -> int:
    """Status of the host-only parameter check (0 = valid)."""
    return lib().sekv_validate_params(C.byref(p))


def build_params(w, tier: Optional[int] = None, ring_bytes: int = 0, gate_eps: float = 0.0) -> BuildParams:
    """BuildParams from a synth.Workload-like object."""
    t = {"hbm": TIER_HBM, "pinned": TIER_PINNED_HOST}[w.tier] if tier is None else tier
    return BuildParams(B=w.B, L=w.L, Hq=w.Hq, Hkv=w.Hkv, d=w.d, T=w.T, R=w.R, dprime=w.dprime,
                       alpha_sp=w.alpha_sp, l_min=w.l_min, oversample=w.oversample,
                       power_iters=w.power_iters, seed=w.seed, tier=t, ring_bytes=ring_bytes,
                       gate_eps=gate_eps)


class Context:
    """A library context bound to a HIP device and stream (default: torch's
    current stream on that device)."""

    def __init__(self, device: int = 0, stream=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream(device)
        self._stream = stream
        h = C.c_void_p()
        check(lib().sekv_create(device, C.c_void_p(stream.cuda_stream), C.byref(h)))
        self.h = h
        self.device = device

    def close(self):
        if self.h:
            lib().sekv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- instrumentation ------------------------------------------------------
    def timing(self, enable: bool):
        check(lib().sekv_timing_enable(self.h, 1 if enable else 0))

    def timing_read(self):
        """(route_ms, route_launches, attend_ms, attend_launches) since the last read."""
        rm, rn = C.c_double(), C.c_int64()
        am, an = C.c_double(), C.c_int64()
        check(lib().sekv_timing_read(self.h, C.byref(rm), C.byref(rn), C.byref(am), C.byref(an)))
        return rm.value, rn.value, am.value, an.value

    # -- prefill --------------------------------------------------------------
    def rsvd_batched(self, A, row_off, rows, max_rows, d, R, oversample, power_iters, seed, U, sigma, Vt):
        check(lib().sekv_rsvd_batched(self.h, int(rows.numel()), _ptr(A), _ptr(row_off), _ptr(rows),
                                      int(max_rows), int(d), int(R), int(oversample), int(power_iters),
                                      int(seed), _ptr(U), _ptr(sigma), _ptr(Vt)))

    def build_index(self, p: BuildParams, K, V, H, W, gates=None) -> "Index":
        h = C.c_void_p()
        check(lib().sekv_build_index(self.h, C.byref(p), _ptr(K), _ptr(V), _ptr(H), _ptr(W),
                                     _ptr(gates), C.byref(h)))
        return Index(self, h)

    def import_index(self, p: BuildParams, arrays: dict) -> "Index":
        """arrays: numpy arrays in the logical layout of sekv_host_index."""
        keep = {k: np.ascontiguousarray(v) for k, v in arrays.items()
                if k in _HOST_FIELDS or k in ("n_spans", "n_raw", "W")}
        hi = HostIndex(**{k: (v.ctypes.data if v.size else None) for k, v in keep.items()})
        h = C.c_void_p()
        check(lib().sekv_index_import(self.h, C.byref(p), C.byref(hi), C.byref(h)))
        return Index(self, h)


class Index:
    def __init__(self, ctx: Context, h):
        self.ctx = ctx
        self.h = h
        info = IndexInfo()
        check(lib().sekv_index_get_info(self.h, C.byref(info)))
        self.info = info
        B = info.B
        self.n_spans = np.zeros(B, np.int32)
        self.n_raw = np.zeros(B, np.int32)
        check(lib().sekv_index_counts(self.h, self.n_spans.ctypes.data, self.n_raw.ctypes.data))

    def free(self):
        if self.h:
            lib().sekv_index_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    @property
    def mask_words(self) -> int:
        return self.info.mask_words

    def route(self, layer_begin, layer_count, q, tau, cap, mask, alpha=None):
        check(lib().sekv_route(self.ctx.h, self.h, layer_begin, layer_count, _ptr(q), _ptr(tau),
                               int(cap), _ptr(mask), _ptr(alpha)))

    def route_pooled(self, layer_begin, layer_count, q, tau, budget, mask, alpha=None):
        check(lib().sekv_route_pooled(self.ctx.h, self.h, layer_begin, layer_count, _ptr(q), _ptr(tau),
                                      int(budget), _ptr(mask), _ptr(alpha)))

    def calibrate_tau(self, layer_begin, layer_count, q_cal, frac, tau_out):
        check(lib().sekv_calibrate_tau(self.ctx.h, self.h, layer_begin, layer_count, _ptr(q_cal),
                                       float(frac), _ptr(tau_out)))

    def decode_attend(self, layer_begin, layer_count, q, mask, out, stats: bool = False):
        st = Stats() if stats else None
        check(lib().sekv_decode_attend(self.ctx.h, self.h, layer_begin, layer_count, _ptr(q),
                                       _ptr(mask), _ptr(out), C.byref(st) if st is not None else None))
        return st

    def decode_attend_noalloc(self, layer_begin, layer_count, q, mask, out):
        check(lib().sekv_decode_attend_noalloc(self.ctx.h, self.h, layer_begin, layer_count, _ptr(q),
                                               _ptr(mask), _ptr(out), None))

    def spans(self):
        """(span_start, span_len, raw_pos) of every sequence, concatenated over b."""
        i = self.info
        out = dict(span_start=np.zeros(int(i.total_spans), np.int32),
                   span_len=np.zeros(int(i.total_spans), np.int32),
                   raw_pos=np.zeros(int(i.total_raw), np.int32))
        ho = HostIndexOut(**{k: (v.ctypes.data if v.size else None) for k, v in out.items()})
        check(lib().sekv_index_export(self.ctx.h, self.h, C.byref(ho)))
        return out["span_start"], out["span_len"], out["raw_pos"]

    def export(self, layer_begin: int = 0, layer_count: Optional[int] = None, fields=None,
               seq_begin: int = 0, seq_count: Optional[int] = None) -> dict:
        """Logical-layout numpy arrays of layers [layer_begin, layer_begin +
        layer_count) of sequences [seq_begin, seq_begin + seq_count) (default:
        everything); `fields` limits which arrays are copied back."""
        i = self.info
        lc = i.L - layer_begin if layer_count is None else layer_count
        bc = i.B - seq_begin if seq_count is None else seq_count
        Hkv, Hq, d, R, dp = i.Hkv, i.Hq, i.d, i.R, i.dprime
        sl = slice(seq_begin, seq_begin + bc)
        NS, NR = int(self.n_spans[sl].sum()), int(self.n_raw[sl].sum())
        lens = self.span_lengths()[int(self.n_spans[:seq_begin].sum()):][:NS]
        NT = int(lens.sum())
        nres = NS + NR
        u16 = np.uint16
        shapes = dict(span_start=(NS, np.int32), span_len=(NS, np.int32), raw_pos=(NR, np.int32),
                      k_res=(lc * Hkv * nres * d, u16), v_res=(lc * Hkv * nres * d, u16),
                      s=(lc * Hq * dp * NS, np.float32),
                      uk=(lc * Hkv * NT * R, u16), uv=(lc * Hkv * NT * R, u16),
                      vkt=(lc * Hkv * NS * R * d, u16), vvt=(lc * Hkv * NS * R * d, u16),
                      smk=(lc * Hkv * NS * R, np.float32), smv=(lc * Hkv * NS * R, np.float32),
                      rank=(lc * Hkv * NS * 2, np.int32))
        out = {k: np.zeros(n, t) for k, (n, t) in shapes.items() if fields is None or k in fields}
        ho = HostIndexOut(**{k: (v.ctypes.data if v.size else None) for k, v in out.items()})
        check(lib().sekv_index_export_part(self.ctx.h, self.h, int(seq_begin), int(bc), int(layer_begin), int(lc),
                                           C.byref(ho)))
        return out

    def span_lengths(self) -> np.ndarray:
        """Span lengths of every sequence, concatenated over b (cached)."""
        if getattr(self, "_lens", None) is None:
            self._lens = self.spans()[1]
        return self._lens
