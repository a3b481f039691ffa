"""ORACLE — test infrastructure only (see oracle/oracle.c for the sources it follows).

A ctypes wrapper over the plain C F32 oracle.  Only tests/, the smoke entry and the benchmark's
CPU-baseline leg may import this package; the GPU library never does.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


class OCfg(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_int32), ("g", ctypes.c_int32), ("half", ctypes.c_int32), ("f", ctypes.c_int32),
                ("layers", ctypes.c_int32), ("vocab", ctypes.c_int32), ("eps", ctypes.c_float),
                ("theta", ctypes.c_float), ("llama3", ctypes.c_int32), ("factor", ctypes.c_float),
                ("low_freq_factor", ctypes.c_float), ("high_freq_factor", ctypes.c_float),
                ("original_max_pos", ctypes.c_float), ("tied", ctypes.c_int32), ("wdt", ctypes.c_int32),
                ("kvdt", ctypes.c_int32)]


class OLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd")]


class OModel(ctypes.Structure):
    _fields_ = [("emb", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("lnf", ctypes.c_void_p),
                ("layers", ctypes.POINTER(OLayer))]


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    pc = ctypes.POINTER(OCfg)
    L.oracle_tree_sum.argtypes = [i32, vp]
    L.oracle_tree_sum.restype = f32
    L.oracle_rmsnorm.argtypes = [i32, vp, vp, i32, f32, vp]
    L.oracle_matvec.argtypes = [i32, i32, vp, i32, vp, vp]
    L.oracle_silu.argtypes = [f32]
    L.oracle_silu.restype = f32
    L.oracle_inv_freq.argtypes = [pc, vp]
    L.oracle_rope_cs.argtypes = [pc, i32, vp, vp]
    L.oracle_rope_head.argtypes = [i32, vp, vp, vp, vp]
    L.oracle_argmax.argtypes = [i32, vp, vp]
    L.oracle_argmax.restype = i32
    L.oracle_head_attention.argtypes = [i32, i32, f32, vp, vp, vp, i32, vp]
    L.oracle_trace_floats.argtypes = [pc]
    L.oracle_trace_floats.restype = ctypes.c_int64
    L.oracle_decode_row.argtypes = [pc, ctypes.POINTER(OModel), vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    L.oracle_decode_row.restype = i32
    L.oracle_lm_head.argtypes = [pc, ctypes.POINTER(OModel), vp, vp]
    L.oracle_lm_head.restype = i32
    L.oracle_prefill_row.argtypes = [pc, ctypes.POINTER(OModel), vp, vp, i32, i32, i32, vp, i32, i32, vp]
    L.oracle_prefill_row.restype = i32
    L.oracle_bf16.argtypes = [f32]
    L.oracle_bf16.restype = ctypes.c_uint16
    L.oracle_hash32.argtypes = [ctypes.c_uint32]
    L.oracle_hash32.restype = ctypes.c_uint32
    L.oracle_uniform.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    L.oracle_uniform.restype = f32
    L.oracle_topk.argtypes = [i32, vp, i32, vp, vp]
    L.oracle_topk.restype = i32
    L.oracle_sample.argtypes = [i32, vp, f32, i32, f32, f32, vp, vp, vp]
    L.oracle_sample.restype = i32
    _lib = L
    return L


def ocfg(cfg) -> OCfg:
    """The oracle's config record from a synth Cfg."""
    return OCfg(cfg.kv, cfg.g, cfg.half, cfg.f, cfg.layers, cfg.vocab, np.float32(cfg.eps), np.float32(cfg.theta),
                int(cfg.rope_llama3), cfg.rope_factor, cfg.rope_low_freq_factor, cfg.rope_high_freq_factor,
                float(cfg.rope_original_max_pos), int(cfg.tied), F32 if cfg.wdtype == "f32" else BF16,
                F32 if cfg.kvdtype == "f32" else BF16)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- elementwise pieces ----

def tree_sum(xs) -> np.float32:
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    return np.float32(lib().oracle_tree_sum(xs.size, _p(xs)))


def rmsnorm(x, g, eps: float, gdt: int = F32) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g)
    out = np.empty_like(x)
    lib().oracle_rmsnorm(x.size, _p(x), _p(g), gdt, np.float32(eps), _p(out))
    return out


def matvec(W, x, wdt: int = F32) -> np.ndarray:
    W = np.ascontiguousarray(W)
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(W.shape[0], dtype=np.float32)
    lib().oracle_matvec(W.shape[0], W.shape[1], _p(W), wdt, _p(x), _p(y))
    return y


def silu(x: float) -> np.float32:
    return np.float32(lib().oracle_silu(np.float32(x)))


def inv_freq(cfg) -> np.ndarray:
    out = np.empty(cfg.half, dtype=np.float32)
    c = ocfg(cfg)
    lib().oracle_inv_freq(ctypes.byref(c), _p(out))
    return out


def rope_cs(cfg, t: int):
    cs = np.empty(cfg.half, dtype=np.float32)
    sn = np.empty(cfg.half, dtype=np.float32)
    c = ocfg(cfg)
    lib().oracle_rope_cs(ctypes.byref(c), t, _p(cs), _p(sn))
    return cs, sn


def rope_head(x, cs, sn) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    cs = np.ascontiguousarray(cs, dtype=np.float32)
    sn = np.ascontiguousarray(sn, dtype=np.float32)
    out = np.empty_like(x)
    lib().oracle_rope_head(x.size // 2, _p(x), _p(cs), _p(sn), _p(out))
    return out


def argmax(xs):
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    v = ctypes.c_float()
    i = lib().oracle_argmax(xs.size, _p(xs), ctypes.byref(v))
    return int(i), float(v.value)


def head_attention(q, K, V, t: int, scale: float, kvdt: int = F32) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    out = np.empty(q.size, dtype=np.float32)
    lib().oracle_head_attention(q.size, t, np.float32(scale), _p(q), _p(K), _p(V), kvdt, _p(out))
    return out


def bf16(x: float) -> int:
    return int(lib().oracle_bf16(np.float32(x)))


# ------------------------------------------------------------------------ sampling ----

def hash32(x: int) -> int:
    return int(lib().oracle_hash32(int(x) & 0xFFFFFFFF))


def uniform(seed: int, n: int) -> np.float32:
    return np.float32(lib().oracle_uniform(int(seed) & 0xFFFFFFFF, int(n) & 0xFFFFFFFF))


def topk(xs, k: int):
    """(ids, values) of the min(k, n) largest, largest first, equal values in id order."""
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    kk = max(0, min(int(k), xs.size))
    ids = np.empty(max(kk, 1), dtype=np.int32)
    vals = np.empty(max(kk, 1), dtype=np.float32)
    m = lib().oracle_topk(xs.size, _p(xs), int(k), _p(ids), _p(vals))
    return ids[:m], vals[:m]


def sample(xs, temp: float, k: int, p: float, u: float):
    """One draw: (id, logit, kept count, kept weight z)."""
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    v = ctypes.c_float()
    nk = ctypes.c_int32()
    z = ctypes.c_float()
    i = lib().oracle_sample(xs.size, _p(xs), np.float32(temp), int(k), np.float32(p), np.float32(u),
                            ctypes.byref(v), ctypes.byref(nk), ctypes.byref(z))
    return int(i), np.float32(v.value), int(nk.value), np.float32(z.value)


# ----------------------------------------------------------------------- the model ----

TRACE_NAMES = ("n1", "q", "k", "v", "qr", "kr", "attn", "a", "n2", "m", "y")


class Model:
    """Weights (numpy arrays from synth.make_weights) bound for the oracle, plus host caches."""

    def __init__(self, cfg, weights: Dict[str, object], rows: int = 1, max_seq: Optional[int] = None,
                 alloc_cache: bool = True):
        self.cfg = cfg
        self.w = weights
        self.c = ocfg(cfg)
        nl = len(weights["layers"])
        assert nl == cfg.layers, "weights hold %d layers, cfg says %d" % (nl, cfg.layers)
        self._layers = (OLayer * nl)()
        for l, lw in enumerate(weights["layers"]):
            for name in ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd"):
                assert lw[name].flags["C_CONTIGUOUS"]
                setattr(self._layers[l], name, lw[name].ctypes.data)
        self.m = OModel(weights["emb"].ctypes.data,
                        weights["lm_head"].ctypes.data if weights["lm_head"] is not None else None,
                        weights["lnf"].ctypes.data, self._layers)
        self.rows = rows
        self.max_seq = max_seq or cfg.max_seq
        kvt = np.float32 if cfg.kvdtype == "f32" else np.uint16
        shape = (cfg.layers, rows, cfg.kv, self.max_seq, cfg.head)
        if alloc_cache:
            self.kc = np.zeros(shape, dtype=kvt)
            self.vc = np.zeros(shape, dtype=kvt)
        else:
            self.kc = self.vc = None

    def trace_floats(self) -> int:
        return int(lib().oracle_trace_floats(ctypes.byref(self.c)))

    def decode(self, tok: int, pos: int, row: int = 0, logits: bool = True, trace: bool = False,
               hidden: bool = False):
        """One position; returns (argmax or -1, logits or None, trace dict or None, hidden or None)."""
        cfg = self.cfg
        lg = np.empty(cfg.vocab, dtype=np.float32) if logits else None
        tr = np.empty(cfg.layers * self.trace_floats(), dtype=np.float32) if trace else None
        hd = np.empty(cfg.dim, dtype=np.float32) if hidden else None
        r = lib().oracle_decode_row(ctypes.byref(self.c), ctypes.byref(self.m), _p(self.kc), _p(self.vc),
                                    self.rows, self.max_seq, row, int(tok), int(pos), _p(lg), _p(tr), _p(hd))
        if r < -1:
            raise ValueError("oracle_decode_row error %d" % r)
        return r, lg, (self.split_trace(tr) if trace else None), hd

    def prefill(self, toks, pos0: int = 0, row: int = 0):
        toks = np.ascontiguousarray(toks, dtype=np.int32)
        lg = np.empty(self.cfg.vocab, dtype=np.float32)
        r = lib().oracle_prefill_row(ctypes.byref(self.c), ctypes.byref(self.m), _p(self.kc), _p(self.vc),
                                     self.rows, self.max_seq, row, _p(toks), toks.size, pos0, _p(lg))
        if r < -1:
            raise ValueError("oracle_prefill_row error %d" % r)
        return r, lg

    def lm_head(self, hidden):
        hidden = np.ascontiguousarray(hidden, dtype=np.float32)
        lg = np.empty(self.cfg.vocab, dtype=np.float32)
        r = lib().oracle_lm_head(ctypes.byref(self.c), ctypes.byref(self.m), _p(hidden), _p(lg))
        return r, lg

    def split_trace(self, tr: np.ndarray):
        cfg = self.cfg
        H, KW, F = cfg.dim, cfg.kvw, cfg.f
        widths = (H, H, KW, KW, H, KW, H, H, H, F, H)
        per = self.trace_floats()
        out = []
        for l in range(cfg.layers):
            seg = tr[l * per:(l + 1) * per]
            d, o = {}, 0
            for name, wdt in zip(TRACE_NAMES, widths):
                d[name] = seg[o:o + wdt]
                o += wdt
            out.append(d)
        return out
