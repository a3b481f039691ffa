"""Seeded synthetic inputs for the Llama decoder step (weights, gains, token ids, pre-filled caches).

This module draws numbers and nothing else: it holds none of the decoder's arithmetic.  The GPU
harness and the CPU oracle's tests both read what it produces, so the two sides see the same bytes.

Recipe (the reading of the configs' "random init" stated once):
  * every tensor has its own stream, seeded by hash32(base_seed ^ fnv1a(key)), key = "<family>/<tensor>"
    or "<family>/L<layer>/<tensor>";
  * matrices and the embedding: N(0, 0.02) (0.02 read as the standard deviation);
  * RMSNorm gains: 1 + N(0, 0.02);
  * bf16 tensors: the F32 value rounded to bf16 with round-to-nearest-even (kept as uint16 bits);
  * token ids: uniform over the vocabulary;
  * pre-filled cache positions: integer-exact uniform U(-a, a), a = sqrt(3) * 0.02 * sqrt(dim).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional

import numpy as np

from . import configs
from .configs import Cfg

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

WEIGHT_STD = 0.02
GAIN_MEAN = 1.0


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u32, u64, i32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
    vp = ctypes.c_void_p
    lib.synth_hash32.argtypes = [u32]
    lib.synth_hash32.restype = u32
    lib.synth_uniform.argtypes = [u32, u32]
    lib.synth_uniform.restype = ctypes.c_float
    for name in ("synth_normal_f32", "synth_normal_bf16"):
        getattr(lib, name).argtypes = [u32, u64, u64, ctypes.c_double, ctypes.c_double, vp]
        getattr(lib, name).restype = None
    lib.synth_tokens.argtypes = [u32, u64, u64, u32, vp]
    lib.synth_int_range.argtypes = [u32, u64, u64, i32, i32, vp]
    for name in ("synth_uniform_kv_f32", "synth_uniform_kv_bf16"):
        getattr(lib, name).argtypes = [u32, u64, u64, ctypes.c_float, vp]
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def hash32(x: int) -> int:
    return int(_load().synth_hash32(x & 0xFFFFFFFF))


def uniform(seed: int, n: int) -> float:
    return float(_load().synth_uniform(seed & 0xFFFFFFFF, n & 0xFFFFFFFF))


def _fnv1a(key: str) -> int:
    h = 0x811C9DC5
    for b in key.encode():
        h ^= b
        h = (h * 0x01000193) & 0xFFFFFFFF
    return h


def stream_seed(key: str, base_seed: int = 0) -> int:
    return hash32((base_seed & 0xFFFFFFFF) ^ _fnv1a(key))


def normal(key: str, shape, mean: float, std: float, dtype: str, base_seed: int = 0,
           out: Optional[np.ndarray] = None) -> np.ndarray:
    n = int(np.prod(shape))
    if 2 * ((n + 1) // 2) > (1 << 32):
        raise ValueError("a stream holds at most 2^32 draws")
    lib = _load()
    if dtype == "f32":
        arr = out if out is not None else np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(stream_seed(key, base_seed), 0, n, mean, std, arr.ctypes.data)
    elif dtype == "bf16":
        arr = out if out is not None else np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(stream_seed(key, base_seed), 0, n, mean, std, arr.ctypes.data)
    else:
        raise ValueError(dtype)
    return arr


LAYER_TENSORS = ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd")


def layer_shapes(cfg: Cfg) -> Dict[str, tuple]:
    """Row = output, as PyTorch stores linear weights (main.bend, type LW)."""
    d, kw, f = cfg.dim, cfg.kvw, cfg.f
    return {"ln1": (d,), "wq": (d, d), "wk": (kw, d), "wv": (kw, d), "wo": (d, d), "ln2": (d,),
            "wg": (f, d), "wu": (f, d), "wd": (d, f)}


def make_layer(cfg: Cfg, layer: int, base_seed: int = 0) -> Dict[str, np.ndarray]:
    fam = cfg.weights_key
    out = {}
    for name, shape in layer_shapes(cfg).items():
        is_gain = name.startswith("ln")
        out[name] = normal(f"{fam}/L{layer}/{name}", shape, GAIN_MEAN if is_gain else 0.0, WEIGHT_STD,
                           cfg.wdtype, base_seed)
    return out


def make_weights(cfg: Cfg, base_seed: int = 0, layers: Optional[int] = None) -> Dict[str, object]:
    """All weights of a model as numpy arrays (float32, or uint16 bf16 bits)."""
    fam = cfg.weights_key
    nl = cfg.layers if layers is None else layers
    w: Dict[str, object] = {
        "emb": normal(f"{fam}/emb", (cfg.vocab, cfg.dim), 0.0, WEIGHT_STD, cfg.wdtype, base_seed),
        "lnf": normal(f"{fam}/lnf", (cfg.dim,), GAIN_MEAN, WEIGHT_STD, cfg.wdtype, base_seed),
        "lm_head": None,
        "layers": [make_layer(cfg, l, base_seed) for l in range(nl)],
    }
    if not cfg.tied:
        w["lm_head"] = normal(f"{fam}/lm_head", (cfg.vocab, cfg.dim), 0.0, WEIGHT_STD, cfg.wdtype, base_seed)
    return w


def tokens(cfg: Cfg, key: str, n: int, base_seed: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_tokens(stream_seed(f"{cfg.weights_key}/tokens/{key}", base_seed), 0, n, cfg.vocab,
                         out.ctypes.data)
    return out


def int_range(key: str, n: int, lo: int, hi: int, base_seed: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_int_range(stream_seed(key, base_seed), 0, n, lo, hi, out.ctypes.data)
    return out


def row_lengths(cfg: Cfg, base_seed: int = 0) -> np.ndarray:
    """Batched-decode row lengths, uniform integers in [len_lo, len_hi]."""
    return int_range(f"{cfg.weights_key}/rowlen/{cfg.name}", cfg.batch, cfg.len_lo, cfg.len_hi, base_seed)


def kv_step(cfg: Cfg) -> float:
    """F32 step of the integer-exact uniform cache fill: amplitude * 2^-23."""
    return float(np.float32(cfg.kv_random_amplitude() * 2.0 ** -23))


def kv_fill_head(cfg: Cfg, layer: int, row: int, which: str, j: int, p0: int, p1: int,
                 base_seed: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Random K ("k") or V ("v") rows of positions p0..p1-1 for kv head j of one cache row/layer,
    shape [p1 - p0, head], float32 or uint16 bf16 bits per cfg.kvdtype."""
    lib = _load()
    D = cfg.head
    n = (p1 - p0) * D
    seed = stream_seed(f"{cfg.weights_key}/kvfill/r{row}/L{layer}/{which}/h{j}", base_seed)
    step = ctypes.c_float(kv_step(cfg))
    if cfg.kvdtype == "f32":
        arr = out if out is not None else np.empty((p1 - p0, D), dtype=np.float32)
        lib.synth_uniform_kv_f32(seed, p0 * D, n, step, arr.ctypes.data)
    else:
        arr = out if out is not None else np.empty((p1 - p0, D), dtype=np.uint16)
        lib.synth_uniform_kv_bf16(seed, p0 * D, n, step, arr.ctypes.data)
    return arr


def np_kv_dtype(cfg: Cfg):
    return np.float32 if cfg.kvdtype == "f32" else np.uint16


def fill_cache_rows(cfg: Cfg, kc: np.ndarray, vc: np.ndarray, row: int, length: int, layers=None,
                    base_seed: int = 0, cache_row: Optional[int] = None) -> None:
    """Fill positions 0..length-1 of one cache row (all layers, all kv heads) of host caches laid out
    [layers][rows][kv][max_seq][head]. `row` keys the streams; `cache_row` is where it is written."""
    cr = row if cache_row is None else cache_row
    for l in range(cfg.layers if layers is None else layers):
        for j in range(cfg.kv):
            kv_fill_head(cfg, l, row, "k", j, 0, length, base_seed, out=kc[l, cr, j, :length])
            kv_fill_head(cfg, l, row, "v", j, 0, length, base_seed, out=vc[l, cr, j, :length])


_dev_lib = None


def _load_dev():
    global _dev_lib
    if _dev_lib is not None:
        return _dev_lib
    from . import build as _b
    if not os.path.exists(_b.DEV_LIB):
        raise RuntimeError(f"{_b.DEV_LIB} is not built (python synth/build.py)")
    lib = ctypes.CDLL(_b.DEV_LIB)
    lib.synth_dev_fill_kv.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.synth_dev_fill_kv.restype = ctypes.c_int
    _dev_lib = lib
    return lib


def fill_cache_device(cfg: Cfg, k_ptr: int, v_ptr: int, rows: int, max_seq: int, lengths, layers=None,
                      base_seed: int = 0, stream: int = 0, row_keys=None) -> None:
    """Device-side fill of device caches laid out [layers][rows][kv][max_seq][head]: positions
    0..lengths[r]-1 of cache row r get the bytes fill_cache_rows writes for row key row_keys[r]
    (default r).  Asynchronous on `stream` (a hipStream_t as an int, 0 = the null stream)."""
    lib = _load_dev()
    D, kv = cfg.head, cfg.kv
    esize = 4 if cfg.kvdtype == "f32" else 2
    step = kv_step(cfg)
    nl = cfg.layers if layers is None else layers
    seeds = (ctypes.c_uint32 * kv)()
    for l in range(nl):
        for r in range(rows):
            key = r if row_keys is None else int(row_keys[r])
            n = int(lengths[r]) * D
            if n == 0:
                continue
            off = ((l * rows + r) * kv) * max_seq * D * esize
            for which, base in (("k", k_ptr), ("v", v_ptr)):
                for j in range(kv):
                    seeds[j] = hash32(stream_seed(f"{cfg.weights_key}/kvfill/r{key}/L{l}/{which}/h{j}", base_seed))
                rc = lib.synth_dev_fill_kv(seeds, kv, base + off, max_seq * D, n, step, int(cfg.kvdtype != "f32"),
                                           stream)
                if rc != 0:
                    raise RuntimeError(f"synth_dev_fill_kv failed ({rc}) at layer {l} row {r} {which}")


__all__ = ["configs", "Cfg", "make_weights", "make_layer", "tokens", "row_lengths", "kv_fill_head",
           "fill_cache_rows", "normal", "stream_seed", "hash32", "uniform", "LAYER_TENSORS", "layer_shapes",
           "np_kv_dtype", "kv_step", "int_range", "fill_cache_device"]
