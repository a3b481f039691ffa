"""Shared pieces of the GPU parity tests: tolerances, a paired (oracle, GPU) model, cache filling."""
from __future__ import annotations

import functools
import sys
import time

import numpy as np

import oracle
import synth

# Tolerances on logits: F32 models max|d| <= 1e-3 and max|d| / max|ref| <= 1e-4; bf16 weights max|d| <= 2e-2.
F32_ABS, F32_REL, BF16_ABS = 1e-3, 1e-4, 2e-2


def log(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


def tol_abs(cfg) -> float:
    return F32_ABS if cfg.wdtype == "f32" else BF16_ABS


def check_logits(cfg, got: np.ndarray, ref: np.ndarray, what: str = ""):
    d = float(np.abs(got.astype(np.float64) - ref).max())
    scale = float(np.abs(ref).max())
    rel = d / scale
    if cfg.wdtype == "f32":
        assert d <= F32_ABS and rel <= F32_REL, f"{what}: max|d| {d:.3g} rel {rel:.3g}"
    else:
        assert d <= BF16_ABS, f"{what}: max|d| {d:.3g} (rel {rel:.3g})"
    return d, rel


def check_argmax(cfg, got_id: int, ref: np.ndarray, what: str = ""):
    """Equal argmax wherever the oracle's top-2 gap exceeds the tolerance; otherwise either near-tied id."""
    order = np.argsort(-ref, kind="stable")
    top1, top2 = float(ref[order[0]]), float(ref[order[1]])
    if top1 - top2 > tol_abs(cfg):
        assert got_id == int(order[0]), f"{what}: argmax {got_id} != {order[0]} (gap {top1 - top2:.3g})"
    else:
        assert ref[got_id] >= top1 - tol_abs(cfg), f"{what}: argmax {got_id} not among the near-tied"


@functools.lru_cache(maxsize=2)
def weights(cfg):
    t = time.time()
    w = synth.make_weights(cfg)
    log(f"weights {cfg.name}: {time.time() - t:.1f}s")
    return w


def fill_random(cfg, om: oracle.Model, dec, rows, length: int):
    """Positions 0..length-1 of the given cache rows get the seeded integer-exact random K/V, the same
    bytes on both sides (host fill, then a copy to the device)."""
    import torch
    for r in rows:
        synth.fill_cache_rows(cfg, om.kc, om.vc, r, length, cache_row=r)
    kt = torch.from_numpy(om.kc.view(np.int16) if om.kc.dtype == np.uint16 else om.kc)
    vt = torch.from_numpy(om.vc.view(np.int16) if om.vc.dtype == np.uint16 else om.vc)
    dk = dec.kv.k.view(torch.int16) if om.kc.dtype == np.uint16 else dec.kv.k
    dv = dec.kv.v.view(torch.int16) if om.vc.dtype == np.uint16 else dec.kv.v
    dk.copy_(kt)
    dv.copy_(vt)
    torch.cuda.synchronize()


def gpu_cache(dec):
    import torch
    torch.cuda.synchronize()
    k = dec.kv.k.view(torch.int16).cpu().numpy().view(np.uint16) if dec.kv.k.dtype == torch.bfloat16 else \
        dec.kv.k.cpu().numpy()
    v = dec.kv.v.view(torch.int16).cpu().numpy().view(np.uint16) if dec.kv.v.dtype == torch.bfloat16 else \
        dec.kv.v.cpu().numpy()
    return k, v


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a
