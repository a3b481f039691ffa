"""GPU parity of the decode step through the C ABI against the CPU oracle (same seeded inputs).

Teacher forcing: both sides take the oracle's chosen token at every step, so a legitimate near-tie
cannot cascade.  Coverage of the workloads' steps: 135M and 360M all of them (prompt and every decode
step); 1.7B the 512-token prompt, the first and the last 32 of its 512 steps; 8B the first and the last
32 of its 256 steps.  Logits: F32 models within max|d| 1e-3 and max|d|/max|ref| 1e-4, bf16-weight models
within max|d| 2e-2; argmax equal wherever the oracle's top-2 gap exceeds that tolerance.  Cache
indexing and the RoPE + append arithmetic are bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import configs
from parity_util import (check_argmax, check_logits, fill_random, gpu_cache, log, weights, widen)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lm():
    import llama_architecture_decoder_amd as lm
    return lm


def _dev_tok(t):
    return torch.tensor([int(t)], dtype=torch.int32, device="cuda")


def _pair(cfg, max_seq, rows=1):
    lm = _lm()
    w = weights(cfg)
    om = oracle.Model(cfg, w, rows=rows, max_seq=max_seq)
    dec = lm.Decoder(cfg, w, rows=rows, max_seq=max_seq)
    return om, dec


def _step(cfg, om, dec, tok, pos, row=0):
    """One teacher-forced step on both sides; returns (oracle id, oracle logits, gpu id, gpu logits)."""
    r, ref, _, _ = om.decode(int(tok), pos, row=row)
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.decode(_dev_tok(tok), [pos], logits, nxt)
    torch.cuda.synchronize()
    return r, ref, int(nxt.item()), logits[0].cpu().numpy()


def _check_written_slots(cfg, om, dec, p0, p1, row=0):
    gk, gv = gpu_cache(dec)
    for name, g, o in (("K", gk, om.kc), ("V", gv, om.vc)):
        a = widen(np.ascontiguousarray(g[:, row, :, p0:p1]))
        b = widen(np.ascontiguousarray(o[:, row, :, p0:p1]))
        scale = float(np.abs(b).max())
        tol = (1e-4 if cfg.kvdtype == "f32" else 1.6e-2) * scale
        assert float(np.abs(a - b).max()) <= tol, f"{name} slots {p0}..{p1 - 1}"


CASES = [
    # name, layers (None = all), prompt length, random fill before the prompt, decode steps, max_seq
    ("smollm2_135m", None, 8, 0, 16, 2048),        # the whole workload: prompt 8, 16 decode steps
    ("smollm2_360m", None, 128, 0, 256, 2048),     # the whole workload: prompt 128, 256 decode steps
    ("smollm2_1_7b", None, 512, 0, 32, 8192),      # the workload's 512-token prompt and its first 32 steps
    ("smollm2_1_7b", None, 0, 992, 32, 8192),      # its last 32 decode positions (992..1023)
    ("llama31_8b", None, 0, 7936, 32, 8192),       # the workload's first 32 steps (7936..7967)
    ("llama31_8b", None, 0, 8160, 32, 8192),       # its last 32 steps, up to max_seq - 1
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers,prompt,fill,steps,max_seq", CASES,
                         ids=[f"{c[0]}-p{c[2]}-f{c[3]}-d{c[4]}" for c in CASES])
def test_decode_parity(name, layers, prompt, fill, steps, max_seq):
    cfg = configs.get(name)
    log(f"case {name} prompt={prompt} fill={fill} steps={steps} max_seq={max_seq}")
    om, dec = _pair(cfg, max_seq)
    if fill:
        fill_random(cfg, om, dec, [0], fill)
    pos = fill
    tok = int(synth.tokens(cfg, f"first/{fill}", 1)[0])
    worst = 0.0
    if prompt:
        toks = synth.tokens(cfg, "prompt", prompt)
        r, ref = om.prefill(toks, pos0=pos)
        logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        dec.prefill(torch.from_numpy(toks).cuda(), pos0=pos, logits=logits[0], next_tok=nxt)
        torch.cuda.synchronize()
        got = logits[0].cpu().numpy()
        d, rel = check_logits(cfg, got, ref, "prefill")
        check_argmax(cfg, int(nxt.item()), ref, "prefill")
        worst = max(worst, rel)
        pos += prompt
        tok = r
    for s in range(steps):
        r, ref, gid, got = _step(cfg, om, dec, tok, pos)
        d, rel = check_logits(cfg, got, ref, f"step {s} pos {pos}")
        check_argmax(cfg, gid, ref, f"step {s} pos {pos}")
        worst = max(worst, rel)
        pos += 1
        tok = r  # teacher forcing: the oracle's token
        if s % 32 == 31:
            log(f"{name}: {s + 1}/{steps} steps, worst max|d|/max|ref| {worst:.3g}")
    _check_written_slots(cfg, om, dec, fill, pos)
    assert dec.status() == 0
    log(f"{name}: worst max|d|/max|ref| {worst:.3g} over {steps} steps")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,pos", [("smollm2_135m", 0), ("smollm2_135m", 37), ("smollm2_1_7b", 511),
                                      ("llama31_8b", 7936), ("llama31_8b", 8191)])
def test_rope_append_bit_exact_and_indexing(name, pos):
    """The slot written is (layer, row, kv head, pos) and nothing else; its bits are exactly the F32
    RoPE of the GPU's own pre-RoPE key (oracle rotation, same cos/sin table), rounded as the cache type,
    and the value is the pre-RoPE value itself, rounded."""
    cfg = configs.truncated(configs.get(name), 2)
    lm = _lm()
    w = weights(cfg)
    dec = lm.Decoder(cfg, w, rows=2, max_seq=pos + 8)
    om = oracle.Model(cfg, w, rows=2, max_seq=pos + 8)
    fill_random(cfg, om, dec, [1], pos + 8)  # row 1 is a neighbour that must stay untouched
    fill_random(cfg, om, dec, [0], pos)
    # a sentinel pattern in row 0 beyond pos
    sentinel = 0x5A5A if cfg.kvdtype == "bf16" else np.float32(-7.25)
    kk, vv = gpu_cache(dec)
    kk[:, 0, :, pos:] = sentinel
    vv[:, 0, :, pos:] = sentinel
    _upload(dec, kk, vv)
    before_k, before_v = kk.copy(), vv.copy()
    tok = int(synth.tokens(cfg, "bitexact", 1)[0])
    trace = dec.decode_traced(_dev_tok(tok), pos)
    tr = dec.split_trace(trace)
    after_k, after_v = gpu_cache(dec)
    cs, sn = oracle.rope_cs(cfg, pos)
    D = cfg.head
    for l in range(cfg.layers):
        for j in range(cfg.kv):
            kr = oracle.rope_head(tr[l]["k"][j * D:(j + 1) * D], cs, sn)
            vr = tr[l]["v"][j * D:(j + 1) * D]
            if cfg.kvdtype == "bf16":
                ek = np.array([oracle.bf16(x) for x in kr], dtype=np.uint16)
                ev = np.array([oracle.bf16(x) for x in vr], dtype=np.uint16)
            else:
                ek, ev = kr, vr
            np.testing.assert_array_equal(after_k[l, 0, j, pos].view(np.uint16 if cfg.kvdtype == "bf16" else np.uint32),
                                          ek.view(np.uint16 if cfg.kvdtype == "bf16" else np.uint32))
            np.testing.assert_array_equal(after_v[l, 0, j, pos].view(np.uint16 if cfg.kvdtype == "bf16" else np.uint32),
                                          ev.view(np.uint16 if cfg.kvdtype == "bf16" else np.uint32))
    # everything else is bitwise unchanged
    mask = np.ones(after_k.shape[:4], dtype=bool)
    mask[:, 0, :, pos] = False
    for a, b in ((after_k, before_k), (after_v, before_v)):
        assert np.array_equal(a[mask].view(np.uint8), b[mask].view(np.uint8))


def _upload(dec, k, v):
    if k.dtype == np.uint16:
        dec.kv.k.view(torch.int16).copy_(torch.from_numpy(k.view(np.int16)))
        dec.kv.v.view(torch.int16).copy_(torch.from_numpy(v.view(np.int16)))
    else:
        dec.kv.k.copy_(torch.from_numpy(k))
        dec.kv.v.copy_(torch.from_numpy(v))
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,pos", [("smollm2_135m", 100), ("llama31_8b", 5000)])
def test_causality_and_determinism(name, pos):
    """Rows after t are never read (NaN there changes no bit), and two runs give the same bits."""
    cfg = configs.truncated(configs.get(name), 2)
    lm = _lm()
    w = weights(cfg)
    dec = lm.Decoder(cfg, w, rows=1, max_seq=pos + 64)
    om = oracle.Model(cfg, w, rows=1, max_seq=pos + 64, alloc_cache=True)
    fill_random(cfg, om, dec, [0], pos + 64)
    k0, v0 = gpu_cache(dec)
    tok = _dev_tok(3)

    def run():
        logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
        dec.decode(tok, [pos], logits, None)
        torch.cuda.synchronize()
        return logits.cpu().numpy()

    a = run()
    _upload(dec, k0, v0)
    b = run()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "not deterministic"
    k1, v1 = k0.copy(), v0.copy()
    nan = 0x7FC0 if cfg.kvdtype == "bf16" else np.float32(np.nan)
    k1[:, :, :, pos + 1:] = nan
    v1[:, :, :, pos + 1:] = nan
    _upload(dec, k1, v1)
    c = run()
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32)), "read past position t"


@pytest.mark.timeout(600)
def test_batched_rows_each_at_own_position():
    """decode_rows: B rows, each at its own position of its own cache row (nest decode_rows)."""
    cfg = configs.truncated(configs.SMOLLM2_135M, 3)
    lm = _lm()
    w = weights(cfg)
    rows = 3
    om = oracle.Model(cfg, w, rows=rows, max_seq=256)
    dec = lm.Decoder(cfg, w, rows=rows, max_seq=256)
    lens = [0, 31, 200]
    for r, n in enumerate(lens):
        if n:
            fill_random(cfg, om, dec, [r], n)
    toks = synth.tokens(cfg, "rows", rows)
    logits = torch.empty((rows, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    dec.decode(torch.from_numpy(toks).cuda(), lens, logits, nxt)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    for r in range(rows):
        rid, ref, _, _ = om.decode(int(toks[r]), lens[r], row=r)
        check_logits(cfg, got[r], ref, f"row {r}")
        check_argmax(cfg, int(nxt[r].item()), ref, f"row {r}")


@pytest.mark.timeout(300)
def test_token_out_of_range_sets_status():
    cfg = configs.truncated(configs.SMOLLM2_135M, 2)
    lm = _lm()
    dec = lm.Decoder(cfg, weights(cfg), rows=1, max_seq=16)
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    dec.decode(_dev_tok(cfg.vocab), [0], logits, None)
    assert dec.status() == lm.E_TOKEN
    assert dec.status() == 0  # cleared
    dec.decode(_dev_tok(5), [1], logits, None)
    assert dec.status() == 0


def _set_status(dec, value):
    """Write the workspace's status word from the host (it is the first word of the workspace)."""
    base = dec.ws.mem.data_ptr()
    off = (-base) % 256
    dec.ws.mem[off:off + 4].copy_(torch.tensor(np.array([value], dtype=np.int32).view(np.uint8)))
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,fill", [("smollm2_135m", 300), ("smollm2_1_7b", 600), ("llama31_8b", 1000)])
def test_wait_give_up_ends_the_step(name, fill):
    """A device-side wait that gives up (status bit 3, forced here from the host before the step: with the
    bit set every wait of the launch that runs the q/k/v product with the attention ends at its first
    unsuccessful poll) still lets every launch of the step finish; llama_status reports LLAMA_E_WAIT once
    and clears it, and the same step run again equals the oracle.  Covers the query wait, the in-launch
    merge (F32 caches) and the O role's input wait (SmolLM2-135M shape)."""
    cfg = configs.truncated(configs.get(name), 2)
    lm = _lm()
    om, dec = _pair(cfg, fill + 8)
    fill_random(cfg, om, dec, [0], fill)
    tok = int(synth.tokens(cfg, f"first/{fill}", 1)[0])
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    _set_status(dec, 8)
    dec.decode(_dev_tok(tok), [fill], logits, nxt)
    torch.cuda.synchronize()
    assert 0 <= int(nxt.item()) < cfg.vocab
    assert dec.status() == lm.E_WAIT
    assert dec.status() == 0  # cleared by the read
    r, ref, gid, got = _step(cfg, om, dec, tok, fill)  # the same position again: it rewrites slot fill
    check_logits(cfg, got, ref, "after a wait that gave up")
    check_argmax(cfg, gid, ref, "after a wait that gave up")
    assert dec.status() == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["smollm2_135m", "llama31_8b"])
def test_lm_head_argmax(name):
    cfg = configs.truncated(configs.get(name), 1)
    lm = _lm()
    w = weights(cfg)
    dec = lm.Decoder(cfg, w, rows=2, max_seq=16)
    om = oracle.Model(cfg, w, rows=1, max_seq=16, alloc_cache=False)
    rng = np.random.default_rng(11)
    hid = rng.standard_normal((2, cfg.dim)).astype(np.float32)
    logits = torch.empty((2, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(2, dtype=torch.int32, device="cuda")
    dec.lm_head_argmax(torch.from_numpy(hid).cuda(), logits, am)
    torch.cuda.synchronize()
    for b in range(2):
        rid, ref = om.lm_head(hid[b])
        check_logits(cfg, logits[b].cpu().numpy(), ref, f"row {b}")
        check_argmax(cfg, int(am[b].item()), ref, f"row {b}")
    # duplicated maxima: the first index wins (main.bend argmax)
    x = torch.zeros((1, cfg.dim), dtype=torch.float32, device="cuda")
    dec.lm_head_argmax(x, None, am[:1])
    torch.cuda.synchronize()
    assert int(am[0].item()) == 0  # all logits 0: index 0


# LM-head rows that tie for the largest logit, in different blocks of both LM-head kernels (the batch-1
# GEMV's grid-strided row groups of 8 and the batched product's 128-output blocks), the same block and
# the same 16-lane row too.  The final norm keeps one coordinate only (gain 1 at c0, 0 elsewhere), so
# every logit is W[r][c0] * n[c0] exactly and rows with equal W[r][c0] tie whatever the hidden state.
TIE_POS = (120000, 4072, 1001, 1000)   # W[r][c0] = +1: the largest logits when n[c0] > 0
TIE_NEG = (121000, 5072, 2001, 2000)   # W[r][c0] = -1: the largest logits when n[c0] < 0


def _tie_weights(cfg, c0=7):
    w = dict(weights(cfg))
    lnf = np.zeros_like(w["lnf"])
    lnf[c0] = 0x3F80  # bf16 1.0
    head = w["lm_head"].copy()
    head[list(TIE_POS), c0] = 0x3F80
    head[list(TIE_NEG), c0] = 0xBF80  # bf16 -1.0
    w["lnf"], w["lm_head"] = lnf, head
    return w


def _check_ties(lg, got, what):
    # main.bend argmax: the first index of the largest value
    for rows in (TIE_POS, TIE_NEG):
        vals = lg[list(rows)]
        assert np.all(vals == vals[0]), f"{what}: tied rows differ {vals}"
    want = min(TIE_POS) if lg[TIE_POS[0]] > lg[TIE_NEG[0]] else min(TIE_NEG)
    assert lg[want] == lg.max(), f"{what}: tie rows are not the maximum"
    assert got == want, f"{what}: argmax {got}, the first of the tied maxima is {want}"
    return want


@pytest.mark.timeout(600)
def test_lm_head_argmax_cross_block_ties():
    lm = _lm()
    cfg = configs.truncated(configs.LLAMA31_8B, 1)
    w = _tie_weights(cfg)
    om = oracle.Model(cfg, w, rows=1, max_seq=16, alloc_cache=False)
    # batch 1 and 2 through lm_head_argmax (the GEMV with its block winners and the final reduce)
    dec = lm.Decoder(cfg, w, rows=2, max_seq=16)
    rng = np.random.default_rng(3)
    hid = rng.standard_normal((2, cfg.dim)).astype(np.float32)
    hid[1, 7] = -abs(hid[1, 7])
    hid[0, 7] = abs(hid[0, 7])
    logits = torch.empty((2, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(2, dtype=torch.int32, device="cuda")
    dec.lm_head_argmax(torch.from_numpy(hid).cuda(), logits, am)
    torch.cuda.synchronize()
    wants = []
    for b in range(2):
        lg = logits[b].cpu().numpy()
        wants.append(_check_ties(lg, int(am[b].item()), f"lm_head_argmax row {b}"))
        rid, _ = om.lm_head(hid[b])
        assert rid == wants[-1]
    assert wants == [1000, 2000]
    # argmax alone (no logits written)
    dec.lm_head_argmax(torch.from_numpy(hid).cuda(), None, am)
    torch.cuda.synchronize()
    assert am.cpu().tolist() == wants
    del dec
    # 32 rows through a decode step (the batched matrix-core LM head and its per-row reduce)
    B = 32
    dec = lm.Decoder(cfg, w, rows=B, max_seq=16)
    toks = synth.tokens(cfg, "ties", B)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    dec.decode(torch.from_numpy(toks).cuda(), [0] * B, logits, nxt)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    seen = set()
    for b in range(B):
        seen.add(_check_ties(got[b], int(nxt[b].item()), f"decode row {b}"))
    log(f"cross-block ties: batch-32 winners {sorted(seen)}")
