"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test names the passage it follows.  None of them re-types the oracle's formula: they use
printed values (tests/golden/), closed forms, invariants, special cases that reduce to exact
results, an independent float64 brute force with full-sequence masked attention, and two library
routines (transformers' LlamaForCausalLM and rotary init, torch's bf16 conversion).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import configs
from conftest import read_golden

F32 = np.float32


# ---------------------------------------------------------------- shapes and layout laws ----

def test_layout_totals_match_pages():
    # bend-ml-llama main.bend "The configuration", layout laws; nest 8B card README ("8.03B")
    for name, total in read_golden("layout_totals.txt"):
        cfg = configs.get(name)
        assert cfg.model_values() == int(total), name
        # the shapes synth generates add up to the same count
        shapes = synth.layer_shapes(cfg)
        n = cfg.vocab * cfg.dim + cfg.dim + cfg.layers * sum(int(np.prod(s)) for s in shapes.values())
        if not cfg.tied:
            n += cfg.vocab * cfg.dim
        assert n == int(total), name


def test_config_sizes_match_pages():
    # bend-ml-llama main.bend, laws smollm2_*_sizes; nest 8B card README
    for name, dim, heads, head, kvw in read_golden("config_sizes.txt"):
        cfg = configs.get(name)
        assert (cfg.dim, cfg.heads, cfg.head, cfg.kvw) == (int(dim), int(heads), int(head), int(kvw))


def test_kv_cache_bytes_8b():
    # nest 8B card README "Loading": about 1 GiB of bf16 caches at MaxSeq 8192
    (ms, nbytes), = read_golden("kv_cache_bytes.txt")
    cfg = configs.LLAMA31_8B
    assert int(ms) == cfg.max_seq
    assert 2 * cfg.layers * cfg.kv * cfg.max_seq * cfg.head * cfg.kvbytes == int(nbytes)


# ------------------------------------------------------------------------- RMSNorm ----

def test_tree_sum_exact_cases_and_pairing():
    # main.bend "The numeric pieces": pair_sums / tree_sum; [a,b,c,d,e] -> [a+b, c+d, e]
    assert oracle.tree_sum([]) == 0.0
    assert oracle.tree_sum([3.5]) == F32(3.5)
    assert oracle.tree_sum([1, 2, 3, 4, 5]) == F32(15)
    # pairing is visible in rounding: 2^24 + 1 + 1 left to right loses both ones; pairs (1+1) keep them
    big = float(2 ** 24)
    assert oracle.tree_sum([1.0, 1.0, big]) == F32(big + 2)       # (1+1)+2^24
    assert oracle.tree_sum([big, 1.0, 1.0, 0.0]) == F32(big)      # (2^24+1)+(1+0): each +1 rounds away (ties to even)
    # pairwise error bound: |S - exact| <= ceil(log2 n) * u * sum|x|
    rng = np.random.default_rng(1)
    for n in (2, 7, 64, 576, 2048, 4097):
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, n)).astype(F32)
        exact = math.fsum(float(v) for v in x)
        bound = math.ceil(math.log2(n)) * 2.0 ** -24 * float(np.abs(x.astype(np.float64)).sum())
        assert abs(float(oracle.tree_sum(x)) - exact) <= bound + 1e-30


def test_rmsnorm_closed_forms():
    # main.bend rmsnorm: g * (x * (1 / sqrt(sum(x^2)/dim + eps)))
    n, eps = 576, 1e-5
    for c in (0.5, 1.0, 3.0, -2.25):
        x = np.full(n, c, dtype=F32)
        g = np.linspace(0.5, 1.5, n).astype(F32)
        out = oracle.rmsnorm(x, g, eps)
        ref = g.astype(np.float64) * c / math.sqrt(c * c + eps)
        np.testing.assert_allclose(out, ref, rtol=4e-7, atol=0)
    # scale invariance: x -> 4x with eps -> 16 eps scales every intermediate by a power of two, so
    # the result is bit-identical; and agreement with a float64 evaluation
    rng = np.random.default_rng(2)
    x = rng.standard_normal(2048).astype(F32)
    g = (1 + 0.02 * rng.standard_normal(2048)).astype(F32)
    a = oracle.rmsnorm(x, g, 1e-5)
    b = oracle.rmsnorm((x * F32(4.0)).astype(F32), g, float(F32(1e-5) * F32(16.0)))
    np.testing.assert_array_equal(a, b)
    x64 = x.astype(np.float64)
    ref = g * (x64 / np.sqrt((x64 * x64).mean() + 1e-5))
    np.testing.assert_allclose(a, ref, rtol=1e-6, atol=1e-7)


def test_rmsnorm_bf16_gain_widening_is_exact():
    # main.bend BF16 loading: bf16 is the upper half of an F32, so widening is exact
    rng = np.random.default_rng(3)
    g32 = (1 + 0.02 * rng.standard_normal(128)).astype(F32)
    g16 = (g32.view(np.uint32) >> 16).astype(np.uint16)
    gw = (g16.astype(np.uint32) << 16).view(F32)
    x = rng.standard_normal(128).astype(F32)
    np.testing.assert_array_equal(oracle.rmsnorm(x, g16, 1e-5, gdt=oracle.BF16), oracle.rmsnorm(x, gw, 1e-5))


# ------------------------------------------------------------------------ matvec ----

def test_matvec_brute_force_and_bf16():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((37, 129)).astype(F32)
    x = rng.standard_normal(129).astype(F32)
    y = oracle.matvec(W, x)
    ref = W.astype(np.float64) @ x.astype(np.float64)
    bound = 129 * 2.0 ** -24 * (np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64)))
    assert np.all(np.abs(y - ref) <= bound)
    # transposed operand is caught: row r = output r
    assert not np.allclose(oracle.matvec(W[:, :37].T.copy(), x[:37]), oracle.matvec(W[:, :37], x[:37]))
    # identity rows pick single inputs exactly
    I = np.eye(16, dtype=F32)
    v = rng.standard_normal(16).astype(F32)
    np.testing.assert_array_equal(oracle.matvec(I, v), v)
    Wb = (W.view(np.uint32) >> 16).astype(np.uint16)
    Wbw = (Wb.astype(np.uint32) << 16).view(F32)
    np.testing.assert_array_equal(oracle.matvec(Wb, x, wdt=oracle.BF16), oracle.matvec(Wbw, x))


# ----------------------------------------------------------------------- SwiGLU ----

def test_silu_limits_and_definition():
    # main.bend silu(x) = x / (1 + exp(-x))
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(50.0) == F32(50.0)
    assert abs(float(oracle.silu(-50.0))) < 1e-20
    for x in np.linspace(-8, 8, 33):
        ref = x / (1 + math.exp(-x))
        assert abs(float(oracle.silu(x)) - ref) <= 3e-7 * max(1.0, abs(ref))


# ----------------------------------------------------------------------- argmax ----

def test_argmax_first_index():
    # main.bend argmax: first index of the largest value (strict >); empty -> (0, 0.0)
    assert oracle.argmax(np.array([], dtype=F32)) == (0, 0.0)
    assert oracle.argmax(np.array([1, 3, 3, 2], dtype=F32))[0] == 1
    assert oracle.argmax(np.array([-5, -1, -1, -7], dtype=F32))[0] == 1
    x = np.zeros(49152, dtype=F32)
    x[[7, 100, 40000]] = 2.0
    assert oracle.argmax(x)[0] == 7


# ------------------------------------------------------------------------- RoPE ----

def _hf_inv_freq(cfg):
    import torch
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    rp = {"rope_type": "default", "rope_theta": cfg.theta}
    if cfg.rope_llama3:
        rp = dict(rope_type="llama3", rope_theta=cfg.theta, factor=cfg.rope_factor,
                  low_freq_factor=cfg.rope_low_freq_factor, high_freq_factor=cfg.rope_high_freq_factor,
                  original_max_position_embeddings=cfg.rope_original_max_pos)
    hc = LlamaConfig(hidden_size=cfg.dim, num_attention_heads=cfg.heads, num_key_value_heads=cfg.kv,
                     head_dim=cfg.head, max_position_embeddings=131072, rope_parameters=rp)
    fn = ROPE_INIT_FUNCTIONS[rp["rope_type"]] if cfg.rope_llama3 else None
    if fn is None:
        from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
        inv, _ = LlamaRotaryEmbedding.compute_default_rope_parameters(hc, device=torch.device("cpu"))
    else:
        inv, _ = fn(hc, torch.device("cpu"))
    return inv.float().numpy()


@pytest.mark.parametrize("name", ["smollm2_135m", "smollm2_360m", "smollm2_1_7b", "llama31_8b"])
def test_inv_freq_matches_transformers(name):
    # main.bend inv_freq (LlamaRotaryEmbedding default); nest rope.linnet `tables` (llama3).  The nest
    # card reports its table matching transformers to 5.96e-8; the same bound holds here.
    cfg = configs.get(name)
    ours = oracle.inv_freq(cfg)
    ref = _hf_inv_freq(cfg)
    assert ours.shape == ref.shape == (cfg.half,)
    rel = np.abs(ours.astype(np.float64) - ref) / np.abs(ref)
    assert rel.max() <= 1.2e-7
    # closed form in float64 for the unscaled table
    if not cfg.rope_llama3:
        exact = 1.0 / cfg.theta ** (2.0 * np.arange(cfg.half) / cfg.head)
        assert (np.abs(ours - exact) / exact).max() <= 2.4e-7


def test_llama3_bands_match_pages():
    # nest 8B card README "Validation": indices 29-34 blended, the rest unchanged or divided by 8
    cfg = configs.LLAMA31_8B
    scaled = oracle.inv_freq(cfg)
    plain = oracle.inv_freq(cfg.replace(rope_llama3=False))
    for band, lo, hi in read_golden("llama3_bands.txt"):
        for i in range(int(lo), int(hi) + 1):
            if band == "unchanged":
                assert scaled[i] == plain[i], i
            elif band == "divided":
                assert scaled[i] == F32(plain[i] / F32(8.0)), i
            else:
                assert plain[i] / 8 < scaled[i] < plain[i], i
    # blend weights: continuity at both edges (smooth = 1 at wavelength 2048 -> unscaled, 0 at 8192 -> /8)
    wl = 2 * math.pi / plain.astype(np.float64)
    s = (8192.0 / wl - 1.0) / 3.0
    mid = np.arange(29, 35)
    ref = (1 - s[mid]) * plain[mid] / 8 + s[mid] * plain[mid]
    np.testing.assert_allclose(scaled[mid], ref, rtol=3e-7)
    assert np.all(np.diff(scaled) < 0)  # still monotone in i


def test_rope_identity_at_zero_and_rotation_laws():
    # main.bend rot_lo / rot_hi: lo' = lo*c - hi*s, hi' = hi*c + lo*s, pairs (i, i + half)
    cfg = configs.SMOLLM2_135M
    cs, sn = oracle.rope_cs(cfg, 0)
    assert np.all(cs == 1) and np.all(sn == 0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(cfg.head).astype(F32)
    np.testing.assert_array_equal(oracle.rope_head(x, cs, sn), x)  # head_split: nothing lost or moved
    # pairing: a single nonzero at i lands only on i and i + half
    for i in (0, 5, cfg.half - 1):
        e = np.zeros(cfg.head, dtype=F32)
        e[i] = 1.0
        cs, sn = oracle.rope_cs(cfg, 7)
        r = oracle.rope_head(e, cs, sn)
        nz = set(np.nonzero(r)[0].tolist())
        assert nz <= {i, i + cfg.half}
        assert r[i] == cs[i] and r[i + cfg.half] == sn[i]
    # norm of every pair preserved; q(m).k(n) depends only on m - n
    q = rng.standard_normal(cfg.head).astype(F32)
    k = rng.standard_normal(cfg.head).astype(F32)
    for t in (1, 17, 1000):
        cs, sn = oracle.rope_cs(cfg, t)
        r = oracle.rope_head(q, cs, sn).astype(np.float64)
        h = cfg.half
        np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, q[:h].astype(np.float64) ** 2 + q[h:].astype(np.float64) ** 2,
                                   rtol=2e-6, atol=1e-7)

    def dot(m, n):
        a = oracle.rope_head(q, *oracle.rope_cs(cfg, m)).astype(np.float64)
        b = oracle.rope_head(k, *oracle.rope_cs(cfg, n)).astype(np.float64)
        return a @ b
    assert abs(dot(10, 3) - dot(107, 100)) < 1e-4
    assert abs(dot(10, 3) - dot(10, 4)) > 1e-3


def test_rope_cos_sin_match_transformers_at_long_positions():
    # nest card README: cos/sin tables agree to ~4.7e-7 at short positions; the angle is rounded to F32
    import torch
    cfg = configs.LLAMA31_8B
    inv = torch.from_numpy(_hf_inv_freq(cfg))
    for t in (0, 1, 100, 7936, 8191, 32127):
        cs, sn = oracle.rope_cs(cfg, t)
        ang = (inv * torch.tensor(float(t), dtype=torch.float32)).float()
        np.testing.assert_allclose(cs, torch.cos(ang).numpy(), atol=3e-7, rtol=0)
        np.testing.assert_allclose(sn, torch.sin(ang).numpy(), atol=3e-7, rtol=0)


# -------------------------------------------------------------------- attention ----

def test_attention_special_cases():
    # main.bend head_att: softmax(scale * K q) . V over positions 0..t
    rng = np.random.default_rng(6)
    D = 64
    K = rng.standard_normal((10, D)).astype(F32)
    V = rng.standard_normal((10, D)).astype(F32)
    q = rng.standard_normal(D).astype(F32)
    # t = 0: one weight exp(0)/exp(0) = 1, so the output is V[0] exactly
    np.testing.assert_array_equal(oracle.head_attention(q, K, V, 0, 0.125), V[0])
    # identical keys: uniform weights, the mean of the value rows
    Kc = np.repeat(K[:1], 10, axis=0)
    out = oracle.head_attention(q, Kc, V, 6, 0.125)
    np.testing.assert_allclose(out, V[:7].astype(np.float64).mean(0), rtol=1e-5, atol=1e-6)
    # float64 brute force
    s = (K[:8].astype(np.float64) @ q.astype(np.float64)) * 0.125
    w = np.exp(s - s.max())
    w /= w.sum()
    np.testing.assert_allclose(oracle.head_attention(q, K, V, 7, 0.125), w @ V[:8].astype(np.float64), rtol=2e-6,
                               atol=2e-7)
    # causality: rows after t are never read (NaN there changes nothing)
    K2, V2 = K.copy(), V.copy()
    K2[8:] = np.nan
    V2[8:] = np.nan
    np.testing.assert_array_equal(oracle.head_attention(q, K2, V2, 7, 0.125), oracle.head_attention(q, K, V, 7, 0.125))


# ----------------------------------------------------------------- whole model ----

def _brute_force_f64(cfg, w, toks):
    """Float64 full-sequence forward with a causal mask (no cache), written from the pages' layer
    description: an independent formulation of the same model."""
    def W(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            a = (a.astype(np.uint32) << 16).view(np.float32)
        return a.astype(np.float64)

    S, D, h = len(toks), cfg.head, cfg.half
    x = W(w["emb"])[toks]
    inv = 1.0 / cfg.theta ** (2.0 * np.arange(h) / D)
    assert not cfg.rope_llama3
    ang = np.arange(S)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)

    def rope(t):  # t [S, n, D]
        lo, hi = t[..., :h], t[..., h:]
        return np.concatenate([lo * c[:, None] - hi * s[:, None], hi * c[:, None] + lo * s[:, None]], -1)

    def rms(v, g):
        return W(g) * (v / np.sqrt((v * v).mean(-1, keepdims=True) + cfg.eps))

    mask = np.triu(np.full((S, S), -np.inf), 1)
    for lw in w["layers"]:
        n1 = rms(x, lw["ln1"])
        q = rope((n1 @ W(lw["wq"]).T).reshape(S, cfg.heads, D))
        k = rope((n1 @ W(lw["wk"]).T).reshape(S, cfg.kv, D))
        v = (n1 @ W(lw["wv"]).T).reshape(S, cfg.kv, D)
        out = np.empty((S, cfg.heads, D))
        for hh in range(cfg.heads):
            j = hh // cfg.g
            sc = q[:, hh] @ k[:, j].T / math.sqrt(D) + mask
            p = np.exp(sc - sc.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
            out[:, hh] = p @ v[:, j]
        x = x + out.reshape(S, -1) @ W(lw["wo"]).T
        n2 = rms(x, lw["ln2"])
        gt, up = n2 @ W(lw["wg"]).T, n2 @ W(lw["wu"]).T
        x = x + (gt / (1 + np.exp(-gt)) * up) @ W(lw["wd"]).T
    head = W(w["emb"] if cfg.tied else w["lm_head"])
    return rms(x, w["lnf"]) @ head.T


@pytest.mark.parametrize("name", ["tiny", "tiny_f32_untied_bf16w"])
def test_whole_model_vs_float64_brute_force(name):
    if name == "tiny":
        cfg = configs.TINY
    else:
        cfg = configs.TINY.replace(name=name, tied=False, wdtype="bf16", kvdtype="f32")
    w = synth.make_weights(cfg)
    toks = synth.tokens(cfg, "bf", 20)
    ref = _brute_force_f64(cfg, w, toks)
    om = oracle.Model(cfg, w)
    for p, tk in enumerate(toks):
        r, lg, _, _ = om.decode(int(tk), p)
        np.testing.assert_allclose(lg, ref[p], rtol=0, atol=1e-5 * np.abs(ref[p]).max())
        gap = np.sort(ref[p])[-1] - np.sort(ref[p])[-2]
        if gap > 1e-4:
            assert r == int(np.argmax(ref[p]))


def test_gqa_mapping_and_first_position_exact():
    # main.bend gqa_head: query head j*g+i reads key/value head j; at t = 0 the output of head h is the
    # value row of head h // g exactly (one softmax weight of 1)
    cfg = configs.SMOLLM2_135M.replace(layers=2)
    w = synth.make_weights(cfg, layers=2)
    om = oracle.Model(cfg, w, max_seq=16)
    _, _, tr, _ = om.decode(123, 0, trace=True)
    D = cfg.head
    for layer in tr:
        for h in range(cfg.heads):
            j = h // cfg.g
            np.testing.assert_array_equal(layer["attn"][h * D:(h + 1) * D], layer["v"][j * D:(j + 1) * D])
        # and a wrong mapping (h % kv) would differ
        h = 1
        assert not np.array_equal(layer["attn"][h * D:(h + 1) * D], layer["v"][(h % cfg.kv) * D:(h % cfg.kv + 1) * D])


def test_cache_write_touches_exactly_one_slot_per_kv_head():
    # main.bend KV.push / kv_heads: one key array and one value array per kv head; position t at t*head
    cfg = configs.TINY
    w = synth.make_weights(cfg)
    om = oracle.Model(cfg, w, rows=3, max_seq=16)
    om.kc[:] = 7.0
    om.vc[:] = 7.0
    om.decode(5, 4, row=1)
    changed = np.argwhere(np.any(om.kc != 7.0, axis=-1))
    assert {tuple(c) for c in changed} == {(l, 1, j, 4) for l in range(cfg.layers) for j in range(cfg.kv)}
    changed = np.argwhere(np.any(om.vc != 7.0, axis=-1))
    assert {tuple(c) for c in changed} == {(l, 1, j, 4) for l in range(cfg.layers) for j in range(cfg.kv)}
    # the written keys are the rotated keys of the trace, the values the unrotated values
    om2 = oracle.Model(cfg, w, rows=1, max_seq=16)
    for p, tk in enumerate([3, 9, 5]):
        _, _, tr, _ = om2.decode(tk, p, trace=True)
    for l in range(cfg.layers):
        np.testing.assert_array_equal(om2.kc[l, 0, :, 2].ravel(), tr[l]["kr"])
        np.testing.assert_array_equal(om2.vc[l, 0, :, 2].ravel(), tr[l]["v"])


def test_causality_perturbation():
    # main.bend law causal / read_len: attention at t reads exactly positions 0..t
    cfg = configs.TINY
    w = synth.make_weights(cfg)
    om = oracle.Model(cfg, w, max_seq=32)
    toks = synth.tokens(cfg, "causal", 6)
    for p, tk in enumerate(toks[:-1]):
        om.decode(int(tk), p)
    snap_k, snap_v = om.kc.copy(), om.vc.copy()
    _, ref, _, _ = om.decode(int(toks[-1]), 5)
    om.kc[:] = snap_k
    om.vc[:] = snap_v
    om.kc[:, :, :, 6:] = np.nan
    om.vc[:, :, :, 6:] = 1e30
    _, got, _, _ = om.decode(int(toks[-1]), 5)
    np.testing.assert_array_equal(got, ref)


def test_position_and_token_errors_write_nothing():
    # main.bend kv_room: a push at t >= cap is rejected; needle's checks for token range
    cfg = configs.TINY
    w = synth.make_weights(cfg)
    om = oracle.Model(cfg, w, max_seq=8)
    before = om.kc.copy()
    for tok, pos in ((1, 8), (1, -1), (-1, 0), (cfg.vocab, 0)):
        with pytest.raises(ValueError):
            om.decode(tok, pos)
    with pytest.raises(ValueError):
        om.prefill(np.array([1, 2, 3], dtype=np.int32), pos0=6)
    with pytest.raises(ValueError):
        om.prefill(np.array([], dtype=np.int32), pos0=0)
    np.testing.assert_array_equal(om.kc, before)


def test_prefill_equals_sequential_decode():
    # main.bend forward_pre: prompt positions skip the final norm and LM head; nest `prefill`
    # continues at pos + S
    cfg = configs.TINY
    w = synth.make_weights(cfg)
    toks = synth.tokens(cfg, "pf", 9)
    a = oracle.Model(cfg, w, max_seq=16)
    ra, la = a.prefill(toks[:5])
    ra2, la2 = a.prefill(toks[5:], pos0=5)
    b = oracle.Model(cfg, w, max_seq=16)
    for p, tk in enumerate(toks):
        rb, lb, _, _ = b.decode(int(tk), p)
        if p == 4:
            np.testing.assert_array_equal(la, lb)
            assert ra == rb
    np.testing.assert_array_equal(la2, lb)
    np.testing.assert_array_equal(a.kc, b.kc)
    np.testing.assert_array_equal(a.vc, b.vc)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000).astype(F32) * 10.0 ** rng.uniform(-20, 20, 20000).astype(F32),
                        # exact ties: low 16 bits = 0x8000
                        ((rng.integers(0, 0x7F80, 1000, dtype=np.uint32) << 16) | 0x8000).view(F32),  # finite only
                        np.array([0.0, -0.0, np.inf, -np.inf], dtype=F32)]).astype(F32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16(float(v)) for v in x], dtype=np.uint16)
    np.testing.assert_array_equal(ours, ref)


# -------------------------------------------------- against transformers (library) ----

def hf_model(cfg, w):
    import torch
    from transformers import LlamaConfig, LlamaForCausalLM
    rp = {"rope_type": "default", "rope_theta": cfg.theta}
    if cfg.rope_llama3:
        rp = dict(rope_type="llama3", rope_theta=cfg.theta, factor=cfg.rope_factor,
                  low_freq_factor=cfg.rope_low_freq_factor, high_freq_factor=cfg.rope_high_freq_factor,
                  original_max_position_embeddings=cfg.rope_original_max_pos)
    hc = LlamaConfig(vocab_size=cfg.vocab, hidden_size=cfg.dim, intermediate_size=cfg.f,
                     num_hidden_layers=cfg.layers, num_attention_heads=cfg.heads, num_key_value_heads=cfg.kv,
                     head_dim=cfg.head, rms_norm_eps=cfg.eps, tie_word_embeddings=cfg.tied,
                     attn_implementation="eager", max_position_embeddings=131072, rope_parameters=rp)
    m = LlamaForCausalLM(hc).float().eval()

    def t(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            a = (a.astype(np.uint32) << 16).view(np.float32)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))

    sd = {"model.embed_tokens.weight": t(w["emb"]), "model.norm.weight": t(w["lnf"])}
    names = {"ln1": "input_layernorm", "ln2": "post_attention_layernorm", "wq": "self_attn.q_proj",
             "wk": "self_attn.k_proj", "wv": "self_attn.v_proj", "wo": "self_attn.o_proj", "wg": "mlp.gate_proj",
             "wu": "mlp.up_proj", "wd": "mlp.down_proj"}
    for l, lw in enumerate(w["layers"]):
        for k, v in names.items():
            sd[f"model.layers.{l}.{v}.weight"] = t(lw[k])
    sd["lm_head.weight"] = t(w["emb"] if cfg.tied else w["lm_head"])
    m.load_state_dict(sd, strict=True)
    return m


@pytest.mark.parametrize("name,layers,n", [("tiny", None, 24), ("smollm2_135m", None, 10),
                                           ("llama31_8b", 1, 6)])
def test_oracle_matches_transformers(name, layers, n):
    # The pages check their decoder against transformers' LlamaForCausalLM in F32 with eager attention
    # (llama.bend post: worst max|d|/max|ref| 2.1e-5 .. 8.3e-5; nest card: 6.68e-6 on 2 layers).
    # Same synthetic weights here, F32 cache so both sides keep the same K/V values.
    import torch
    cfg = configs.get(name)
    if layers:
        # full layer width, one layer and a cut vocabulary (the library's random init of two
        # 128256 x 4096 tables alone takes a minute on the CPU)
        cfg = configs.truncated(cfg, layers, vocab=8192)
    cfg = cfg.replace(kvdtype="f32")
    w = synth.make_weights(cfg)
    toks = synth.tokens(cfg, "hf", n)
    m = hf_model(cfg, w)
    with torch.no_grad():
        ref = m(torch.from_numpy(toks[None].astype(np.int64))).logits[0].numpy()
    del m
    om = oracle.Model(cfg, w, max_seq=max(n, 8))
    for p, tk in enumerate(toks):
        r, lg, _, _ = om.decode(int(tk), p)
        assert np.abs(lg - ref[p]).max() <= 1e-5 * np.abs(ref[p]).max(), p
        top2 = np.sort(ref[p])[-2:]
        if top2[1] - top2[0] > 1e-4:
            assert r == int(np.argmax(ref[p]))


@pytest.mark.parametrize("name,layers,vocab", [("tiny", None, None), ("smollm2_135m", 1, None),
                                               ("llama31_8b", 1, 8192)])
def test_lm_head_matches_decode_and_transformers(name, layers, vocab):
    # main.bend "The model": head_of = the LM head (the embedding when tied, the separate head matrix of
    # the nest card otherwise) over rmsnorm(x, final norm), then argmax.  The oracle's standalone head
    # (the reference for the GPU lm_head_argmax) must give the decode's own logits bit for bit from the
    # decode's hidden state, and match transformers' model.norm + lm_head on that state; the untied case
    # uses a head matrix unlike the embedding, so a swapped head, the wrong gain or a skipped norm fails.
    import torch
    cfg = configs.get(name)
    if layers:
        cfg = configs.truncated(cfg, layers, **({"vocab": vocab} if vocab else {}))
    cfg = cfg.replace(kvdtype="f32")
    w = synth.make_weights(cfg)
    if not cfg.tied:
        assert not np.array_equal(w["lm_head"], w["emb"])
    om = oracle.Model(cfg, w, max_seq=8)
    toks = synth.tokens(cfg, "lmhead", 3)
    m = hf_model(cfg, w)
    for p, tk in enumerate(toks):
        r, lg, _, hd = om.decode(int(tk), p, hidden=True)
        r2, lg2 = om.lm_head(hd)
        np.testing.assert_array_equal(lg2, lg)
        assert r2 == r
        with torch.no_grad():
            h = torch.from_numpy(hd[None].copy())
            ref = m.lm_head(m.model.norm(h))[0].numpy()
        assert np.abs(lg2 - ref).max() <= 1e-5 * np.abs(ref).max(), p
        top2 = np.sort(ref)[-2:]
        if top2[1] - top2[0] > 1e-4:
            assert r2 == int(np.argmax(ref))
    # a hidden state that is not a decode's
    rng = np.random.default_rng(5)
    hid = rng.standard_normal(cfg.dim).astype(F32)
    r3, lg3 = om.lm_head(hid)
    with torch.no_grad():
        ref = m.lm_head(m.model.norm(torch.from_numpy(hid[None].copy())))[0].numpy()
    assert np.abs(lg3 - ref).max() <= 1e-5 * np.abs(ref).max()
    del m
