"""Pins of the oracle's sampling step (bend-ml-llama main.bend, "Sampling") against what the page and
the mathematics fix (no GPU).

The draw picks among the k largest logits (equal values in id order) with probability proportional to
exp(v / temp), restricted by top-p to a prefix, using one uniform u.  The pins: a stable sort for the
top-k, the argmax for k = 1, exact closed forms when every weight is 1, frequencies over a fine grid of
u against the softmax in float64, exact invariances, the law sample_below, and properties of the
generator (range, grid, moments, inverse of the bijection).
"""
import numpy as np
import pytest

import oracle

F32 = np.float32


def _tied_logits(rng, n):
    # few distinct values, so ties are everywhere, with both zeros present
    x = rng.integers(-3, 4, size=n).astype(F32) * F32(0.5)
    x[rng.random(n) < 0.1] = F32(-0.0)
    return x


# ---------------------------------------------------------------------------- top-k ----

@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (50, 50), (50, 64), (300, 17), (1000, 256), (40, 0)])
def test_topk_is_a_stable_descending_sort(n, k):
    # [bend] topk: the k largest, largest first, equal values with the lower id first
    rng = np.random.default_rng(100 + n + k)
    for x in (_tied_logits(rng, n), rng.standard_normal(n).astype(F32)):
        ids, vals = oracle.topk(x, k)
        want = np.argsort(-x, kind="stable")[:k]
        assert ids.tolist() == want.tolist()
        assert np.array_equal(vals, x[want])


def test_topk_boundary_tie_keeps_lower_ids():
    # a value equal to the smallest held one does not enter, so the earliest of a run of ties stays
    x = np.array([5, 1, 1, 1, 1, 0, 1], dtype=F32)
    ids, _ = oracle.topk(x, 3)
    assert ids.tolist() == [0, 1, 2]


def test_topk_k1_is_argmax():
    # [bend] argmax keeps the first of equal maxima, as a one-candidate top-k does
    rng = np.random.default_rng(7)
    for n in (1, 5, 333):
        x = _tied_logits(rng, n)
        i, v = oracle.argmax(x)
        ids, vals = oracle.topk(x, 1)
        assert ids.tolist() == [i] and float(vals[0]) == v


# ------------------------------------------------------------------------- the draw ----

def test_u0_and_p0_draw_the_top_candidate():
    # target = 0 stops at the first candidate (its weight is 1 > 0); p = 0 keeps only the first
    rng = np.random.default_rng(11)
    for trial in range(20):
        x = (rng.standard_normal(500) * 3).astype(F32)
        top = int(np.argmax(x))
        temp = float(rng.uniform(0.2, 2.0))
        k = int(rng.integers(1, 300))
        assert oracle.sample(x, temp, k, float(rng.uniform(0, 1)), 0.0)[0] == top
        i, v, nk, z = oracle.sample(x, temp, k, 0.0, float(rng.uniform(0, 1)))
        assert (i, nk, float(z)) == (top, 1, 1.0)


def test_k1_draws_the_argmax():
    rng = np.random.default_rng(12)
    for trial in range(20):
        x = _tied_logits(rng, 200)
        i, _ = oracle.argmax(x)
        assert oracle.sample(x, float(rng.uniform(0.1, 3)), 1, float(rng.uniform(0, 1)),
                             float(rng.uniform(0, 1)))[0] == i


@pytest.mark.parametrize("n,k", [(50, 1), (50, 4), (50, 7), (50, 50), (50, 64), (3, 8)])
def test_all_equal_logits_closed_form(n, k):
    # every weight is exp(0) = 1, so the running weights are the integers 1, 2, ...: the kept count is
    # 1 + #{m in 1..k-1 : m < p*k} and the draw is the candidate floor(u * kept), at most the last kept;
    # candidates are ids 0..k-1 (ties in id order)
    x = np.full(n, 0.37, dtype=F32)
    kk = min(n, k)
    for p in (0.0, 0.25, 0.5, 0.9, 1.0):
        lim = F32(p) * F32(kk)
        kept = 1 + sum(1 for m in range(1, kk) if F32(m) < lim)
        for u in (0.0, 0.5, 0.25, 0.999999, 1.0 / 3.0, 0.75):
            target = F32(u) * F32(kept)
            want = min(int(np.floor(target)), kept - 1)
            i, v, nk, z = oracle.sample(x, 0.8, k, p, u)
            assert (i, nk, float(z)) == (want, kept, float(kept)), (p, u)
            assert v == x[i]


def test_strict_comparisons_at_exact_boundaries():
    # k = 4 equal weights, p = 0.5: lim = 2 and the running weight 2 is not below it, so two are kept;
    # u = 0.5 gives target 1.0, which is not below the first running weight 1, so the second is drawn
    x = np.zeros(4, dtype=F32)
    i, _, nk, _ = oracle.sample(x, 1.0, 4, 0.5, 0.5)
    assert (i, nk) == (1, 2)


def _softmax64(v, temp):
    a = np.asarray(v, dtype=np.float64) / temp
    e = np.exp(a - a.max())
    return e / e.sum()


@pytest.mark.parametrize("temp", [1.0, 0.5, 2.0])
@pytest.mark.parametrize("k,p", [(6, 1.0), (3, 1.0), (6, 0.55), (4, 0.8)])
def test_draw_frequencies_follow_the_tempered_softmax(temp, k, p):
    # over u on a fine grid, each candidate is drawn with probability w_j / z: the softmax of v/temp over
    # the top-k, restricted to the top-p prefix (the first candidates whose mass before them is below p)
    x = np.array([0.3, 1.9, -0.7, 1.2, 0.9, -1.6], dtype=F32)
    order = np.argsort(-x, kind="stable")[:k]
    prob = _softmax64(x[order], temp)
    before = np.concatenate([[0.0], np.cumsum(prob)[:-1]])
    keep = int(np.sum(before < p))
    assert np.all(np.abs(before - p) > 1e-5), "grid case sits on a top-p boundary"
    want = np.zeros(x.size)
    want[order[:keep]] = prob[:keep] / prob[:keep].sum()
    M = 20000
    got = np.zeros(x.size)
    for j in range(M):
        got[oracle.sample(x, temp, k, p, (j + 0.5) / M)[0]] += 1
    got /= M
    assert np.max(np.abs(got - want)) < 2.0 / M


def test_temperature_enters_only_through_v_over_temp():
    # doubling the logits and the temperature leaves every quotient v/temp unchanged (exact in F32)
    rng = np.random.default_rng(13)
    for trial in range(30):
        x = (rng.standard_normal(400) * 2).astype(F32)
        temp, k, p, u = float(rng.uniform(0.2, 2)), int(rng.integers(1, 400)), float(rng.uniform()), float(
            rng.uniform())
        a = oracle.sample(x, temp, k, p, u)
        b = oracle.sample(x * F32(2), F32(temp) * F32(2), k, p, u)
        assert (a[0], a[2], float(a[3])) == (b[0], b[2], float(b[3]))


def test_law_sample_below():
    # [bend] LAW sample_below: the drawn id is an id of the logits, and it is one of the top-k
    rng = np.random.default_rng(14)
    for trial in range(60):
        n = int(rng.integers(1, 600))
        x = _tied_logits(rng, n) if trial % 2 else (rng.standard_normal(n) * 4).astype(F32)
        k = int(rng.integers(1, 300))
        i, v, nk, z = oracle.sample(x, float(rng.uniform(0.05, 4)), k, float(rng.uniform(-0.1, 1.1)),
                                    float(rng.uniform()))
        assert 0 <= i < n and v == x[i]
        assert i in oracle.topk(x, k)[0].tolist()
        assert 1 <= nk <= min(n, k)


# ------------------------------------------------------------------------ generator ----

def test_uniform_is_on_the_2_pow_minus_24_grid_in_0_1():
    # [bend] uniform: 24 bits scaled by 2^-24
    for seed in (0, 1, 12345, 0xFFFFFFFF):
        for n in range(0, 4000, 7):
            u = oracle.uniform(seed, n)
            assert 0.0 <= u < 1.0
            s = float(u) * 2 ** 24
            assert s == int(s)


def test_uniform_moments_and_bins():
    us = np.array([oracle.uniform(2024, n) for n in range(40000)], dtype=np.float64)
    assert abs(us.mean() - 0.5) < 0.01
    assert abs(us.var() - 1.0 / 12.0) < 0.003
    counts = np.bincount((us * 32).astype(int), minlength=32)
    chi2 = float(np.sum((counts - 1250.0) ** 2 / 1250.0))
    assert chi2 < 70.0  # 31 degrees of freedom: p < 1e-4 above this


def _unshift(y, s):
    # inverse of x ^= x >> s on 32-bit words
    x = y
    for _ in range(32 // s + 1):
        x = y ^ (x >> s)
    return x & 0xFFFFFFFF


def test_hash32_is_the_stated_bijection():
    # [bend] hash32: x ^= x>>16; x *= 0x7feb352d; x ^= x>>15; x *= 0x846ca68b; x ^= x>>16.  Undo each step
    # (multiplicative inverses mod 2^32) and recover the input.
    inv1 = pow(0x7FEB352D, -1, 2 ** 32)
    inv2 = pow(0x846CA68B, -1, 2 ** 32)
    rng = np.random.default_rng(15)
    xs = [0, 1, 2, 0xFFFFFFFF, 0x80000000] + [int(v) for v in rng.integers(0, 2 ** 32, size=2000)]
    seen = set()
    for x in xs:
        h = oracle.hash32(x)
        y = _unshift(h, 16)
        y = (y * inv2) & 0xFFFFFFFF
        y = _unshift(y, 15)
        y = (y * inv1) & 0xFFFFFFFF
        y = _unshift(y, 16)
        assert y == x
        seen.add(h)
    assert oracle.hash32(0) == 0 and len(seen) == len(set(xs))
