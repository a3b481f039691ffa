"""GPU parity of sampling (temperature, top-k, top-p) against the CPU oracle.

Sampling decides integers (the candidates and the drawn id) from F32 arithmetic that both sides do in
the same precision and order (weights from the correctly rounded exponential, one running sum in
candidate order, the page's strict comparisons), so the drawn ids, their logits and the top-k lists
must be identical, element by element.  Logits are seeded and synthetic: normal rows with the scale of
an LM head's output and a few outliers, rows with heavy ties (few distinct values, both zeros), rows of
one value, and two patterns that push the kernels' candidate bound onto its slow paths.  Sizes: the 128256-token vocabulary at 1, 4 and 64 rows, ragged chunk edges, the largest
vocabulary allowed for k = 256, strided rows, k above V.
"""
import numpy as np
import pytest

import oracle
from parity_util import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32 = np.float32


def _logits(rng, B, V, kind):
    if kind == "normal":
        x = (rng.standard_normal((B, V)) * 3.0).astype(F32)
        hot = rng.integers(0, V, size=(B, 3))
        for b in range(B):
            x[b, hot[b]] += F32(12.0)
        return x
    if kind == "ties":
        x = (rng.integers(-4, 5, size=(B, V)).astype(F32) * F32(0.75))
        x[rng.random((B, V)) < 0.05] = F32(-0.0)
        return x
    if kind == "flat":
        return np.full((B, V), 0.37, dtype=F32)
    # the two below defeat the kernel's first-pass bound (per-wavefront maxima of threads that take
    # every 256th logit): in "lopsided" three of four wavefronts see only large values, so far more
    # keys pass the bound than its buffer holds and the bound is raised; in "sparse" 1152 of every
    # 8192 logits are large, so the survivors are sorted by the bitonic network
    t = np.arange(V) % 256
    if kind == "lopsided":
        x = rng.standard_normal((B, V)).astype(F32)
        x[:, t < 192] += F32(100.0)
        return x
    if kind == "sparse":
        x = rng.standard_normal((B, V)).astype(F32)
        x[:, (t < 192) & (t % 64 < 12)] += F32(100.0)
        return x
    raise ValueError(kind)


def _run(x, temp, k, p, seeds=None, draw=0, u=None, ld=None):
    import llama_architecture_decoder_amd as lm
    B, V = x.shape
    ld = ld or V
    buf = torch.full((B, ld), float("nan"), dtype=torch.float32, device="cuda")
    buf[:, :V] = torch.from_numpy(x).cuda()
    view = buf[:, :V]
    ids = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    vals = torch.empty(B, dtype=torch.float32, device="cuda")
    tk = torch.full((B, k), -9, dtype=torch.int32, device="cuda")
    sd = torch.from_numpy(np.asarray(seeds, dtype=np.uint32).view(np.int32)).cuda() if seeds is not None else None
    ut = torch.from_numpy(np.asarray(u, dtype=F32)).cuda() if u is not None else None
    lm.sample(view, temp, k, p, seeds=sd, draw=draw, u=ut, ids=ids, vals=vals, topk_ids=tk)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy(), tk.cpu().numpy()


def _check(x, temp, k, p, got, us):
    ids, vals, tk = got
    B, V = x.shape
    for b in range(B):
        oid, ov = oracle.topk(x[b], k)
        want_tk = np.full(k, -1, dtype=np.int64)
        want_tk[:oid.size] = oid
        assert np.array_equal(tk[b].astype(np.int64), want_tk), f"row {b}: top-k lists differ"
        i, v, nk, z = oracle.sample(x[b], temp, k, p, float(us[b]))
        assert ids[b] == i, f"row {b}: drew {ids[b]}, oracle {i} (kept {nk}, u {us[b]})"
        assert vals[b].view(np.uint32) == F32(x[b, i]).view(np.uint32)


CASES = [
    # rows, vocabulary, logits, temp, k, p
    (1, 128256, "normal", 0.6, 50, 0.9),
    (1, 128256, "normal", 1.0, 256, 1.0),
    (4, 128256, "ties", 0.8, 256, 0.95),
    (4, 128256, "normal", 0.3, 1, 0.5),
    (64, 128256, "normal", 1.7, 200, 0.95),
    (64, 128256, "normal", 0.6, 7, 0.0),
    (3, 49152, "normal", 0.9, 40, 0.8),
    (2, 1, "normal", 1.0, 5, 0.9),
    (2, 7, "ties", 1.0, 3, 1.0),
    (3, 300, "normal", 0.7, 256, 0.9),
    (2, 4095, "ties", 1.2, 100, 0.7),
    (2, 4096, "normal", 1.0, 64, 0.9),
    (2, 4097, "normal", 1.0, 64, 0.9),
    (2, 262144, "normal", 0.9, 256, 0.99),
    (3, 1000, "flat", 0.8, 64, 0.5),
    (2, 100, "normal", 2.0, 256, 1.0),
    (2, 128256, "lopsided", 1.0, 256, 0.9),
    (2, 128256, "sparse", 1.0, 200, 0.9),
    (2, 128256, "lopsided", 1.0, 100, 0.9),
    (2, 128256, "sparse", 1.0, 64, 0.9),
]


@pytest.mark.parametrize("B,V,kind,temp,k,p", CASES, ids=[f"B{c[0]}-V{c[1]}-{c[2]}-k{c[4]}" for c in CASES])
def test_sample_parity_seeded(B, V, kind, temp, k, p):
    log(f"sample B={B} V={V} {kind} temp={temp} k={k} p={p}")
    rng = np.random.default_rng(V * 7 + B * 131 + k)
    x = _logits(rng, B, V, kind)
    seeds = rng.integers(0, 2 ** 32, size=B, dtype=np.uint64).astype(np.uint32)
    draw = int(rng.integers(0, 1000))
    got = _run(x, temp, k, p, seeds=seeds, draw=draw)
    us = [oracle.uniform(int(s), draw) for s in seeds]
    _check(x, temp, k, p, got, us)


def test_sample_parity_given_uniforms_and_strided_rows():
    # u given directly, at the ends of [0, 1) and on the grid of every kept count; rows 160 floats apart
    log("sample: given u, strided rows")
    rng = np.random.default_rng(5)
    B, V, k = 12, 150, 16
    x = _logits(rng, B, V, "ties")
    x[6:] = _logits(rng, 6, V, "flat")
    us = np.array([0.0, 1.0 - 2 ** -24, 0.5, 0.25, 0.125, 0.875, 0.0, 0.5, 0.75, 1.0 - 2 ** -24, 0.3125, 0.5],
                  dtype=F32)
    for p in (0.0, 0.5, 1.0):
        got = _run(x, 0.9, k, p, u=us, ld=160)
        _check(x, 0.9, k, p, got, us)


def test_sample_draws_follow_the_seed_counter():
    # the same seeds and draw give the same ids; successive draws are the oracle's successive uniforms
    log("sample: seed counter")
    rng = np.random.default_rng(6)
    B, V, k, temp, p = 8, 32000, 40, 1.0, 0.95
    x = _logits(rng, B, V, "normal") / F32(3.0)
    seeds = np.arange(B, dtype=np.uint32) * np.uint32(2654435761)
    first = _run(x, temp, k, p, seeds=seeds, draw=0)
    again = _run(x, temp, k, p, seeds=seeds, draw=0)
    assert np.array_equal(first[0], again[0])
    for draw in (0, 1, 2, 77):
        got = _run(x, temp, k, p, seeds=seeds, draw=draw)
        _check(x, temp, k, p, got, [oracle.uniform(int(s), draw) for s in seeds])
