"""GPU parity of the matrix-core prefill (bf16 weights and cache) against the CPU oracle.

The prompt's positions go through each layer together: tiled MFMA products over all rows, RoPE + append
of every position, causal attention over the cache.  Compared with the oracle's position-by-position
prefill: last-position logits within max|d| 2e-2, argmax equal outside near-ties, every appended K/V
slot within bf16 rounding.  Cases cover ragged row tiles (S not a multiple of 128 or 32), a prompt that
continues a filled cache (pos0 > 0), prompts longer than the workspace's chunk, g = 3 / head 64, and a
2800-position prompt whose products take the 256x256-tile kernel (every epilogue, K split in slices).
At the full 8B size the prefill is checked against the GPU's own decode path (prefill of S positions
equals S decode steps), which the decode tests tie to the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import configs
from parity_util import check_argmax, check_logits, fill_random, gpu_cache, log, weights, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cfg(name, layers):
    if name == "smollm2_135m_bf16":
        return configs.truncated(configs.SMOLLM2_135M, layers, wdtype="bf16", kvdtype="bf16")
    return configs.truncated(configs.get(name), layers)


def _check_slots(cfg, dec, om, p0, p1, what):
    gk, gv = gpu_cache(dec)
    for nm, g, o in (("K", gk, om.kc), ("V", gv, om.vc)):
        a = widen(np.ascontiguousarray(g[:, 0, :, p0:p1]))
        b = widen(np.ascontiguousarray(o[:, 0, :, p0:p1]))
        tol = 1.6e-2 * float(np.abs(b).max())
        d = float(np.abs(a - b).max())
        assert d <= tol, f"{what}: {nm} slots {p0}..{p1 - 1}: max|d| {d:.3g} > {tol:.3g}"


CASES = [
    # model, layers, prompt length, filled positions before it, workspace chunk, max_seq
    ("llama31_8b", 2, 300, 0, 512, 1024),          # ragged row tile and query tile
    ("llama31_8b", 2, 200, 1000, 256, 2048),       # continues a filled cache
    ("llama31_8b", 2, 300, 0, 128, 1024),          # three chunks: 128, 128, 44
    ("smollm2_135m_bf16", 3, 257, 0, 512, 1024),   # g = 3, head 64
    ("llama31_8b", 1, 2, 5, 64, 256),              # the smallest prompt that takes this path
    ("llama31_8b", 2, 2800, 0, 2800, 3072),        # large tiles (11 row tiles, the last ragged), split K
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers,S,fill,chunk,max_seq", CASES,
                         ids=[f"{c[0]}-L{c[1]}-S{c[2]}-f{c[3]}-c{c[4]}" for c in CASES])
def test_prefill_parity(name, layers, S, fill, chunk, max_seq):
    import llama_architecture_decoder_amd as lm
    cfg = _cfg(name, layers)
    log(f"case {name} layers={layers} S={S} fill={fill} chunk={chunk}")
    w = weights(cfg)
    om = oracle.Model(cfg, w, rows=1, max_seq=max_seq)
    dec = lm.Decoder(cfg, w, rows=1, max_seq=max_seq, max_prefill=chunk)
    if fill:
        fill_random(cfg, om, dec, [0], fill)
    toks = synth.tokens(cfg, f"prefill/{S}/{fill}", S)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.prefill(torch.from_numpy(toks).cuda(), pos0=fill, logits=logits, next_tok=nxt)
    torch.cuda.synchronize()
    assert dec.status() == 0
    rid, ref = om.prefill(toks, pos0=fill)
    d, rel = check_logits(cfg, logits.cpu().numpy(), ref, "prefill")
    check_argmax(cfg, int(nxt.item()), ref, "prefill")
    _check_slots(cfg, dec, om, fill, fill + S, "prefill")
    # one decode step after the prompt reads what the prefill appended
    tok = torch.tensor([rid], dtype=torch.int32, device="cuda")
    lg2 = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    dec.decode(tok, [fill + S], lg2, None)
    torch.cuda.synchronize()
    _, ref2, _, _ = om.decode(rid, fill + S)
    check_logits(cfg, lg2[0].cpu().numpy(), ref2, "decode after prefill")
    log(f"{name} S={S}: max|d| {d:.3g} rel {rel:.3g}")


@pytest.mark.timeout(900)
def test_prefill_4096_equals_decode_steps_8b():
    """The 4096-position prompt at the full 8B size: prefill (one pass per layer, in chunks of the
    workspace) equals 4096 decode steps, logits of the last position and every appended K/V slot."""
    import llama_architecture_decoder_amd as lm
    cfg = configs.LLAMA31_8B_LONG
    S = cfg.prompt_len
    w = weights(configs.LLAMA31_8B)
    max_seq = S + 64
    a = lm.Decoder(cfg, w, rows=1, max_seq=max_seq, max_prefill=S)
    b = lm.Decoder(cfg, None, rows=1, max_seq=max_seq, weights=a.w)
    toks = torch.from_numpy(synth.tokens(cfg, "bench/prompt", S)).cuda()
    la = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    a.prefill(toks, pos0=0, logits=la)
    lb = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    for i in range(S):
        b.decode(toks[i:i + 1], [i], lb if i == S - 1 else None, None)
    torch.cuda.synchronize()
    assert a.status() == 0 and b.status() == 0
    ref = lb[0].double().cpu().numpy()
    d, rel = check_logits(cfg, la.cpu().numpy(), ref, "prefill vs decode")
    ka, va = gpu_cache(a)
    kb, vb = gpu_cache(b)
    for nm, x, y in (("K", ka, kb), ("V", va, vb)):
        xa = widen(np.ascontiguousarray(x[:, 0, :, :S]))
        ya = widen(np.ascontiguousarray(y[:, 0, :, :S]))
        tol = 1.6e-2 * float(np.abs(ya).max())
        assert float(np.abs(xa - ya).max()) <= tol, nm
    log(f"prefill 4096 vs decode: max|d| {d:.3g} rel {rel:.3g}")


@pytest.mark.timeout(1200)
def test_prefill_4096_oracle_parity_8b_width():
    """The 4096-position prompt of the long-context workload, at the full 8B width and in the benchmark's
    launch configuration (one pass: max_prefill 4096, a MaxSeq-32768 cache row), on a 2-layer truncation
    so the oracle finishes: last-position logits within 2e-2, the argmax outside near-ties and every
    appended K/V slot of both layers (the second layer's slots depend on every position's first-layer
    output) within bf16 rounding.  The oracle runs position after position (its prefill is sequential
    decode), in pieces of 256 positions with a progress line after each."""
    import llama_architecture_decoder_amd as lm
    cfg = configs.truncated(configs.LLAMA31_8B_LONG, 2)
    S, max_seq = cfg.prompt_len, cfg.max_seq
    assert (S, max_seq) == (4096, 32768)
    w = weights(cfg)
    dec = lm.Decoder(cfg, w, rows=1, max_seq=max_seq, max_prefill=S)
    toks = synth.tokens(cfg, "bench/prompt", S)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.prefill(torch.from_numpy(toks).cuda(), pos0=0, logits=logits, next_tok=nxt)
    torch.cuda.synchronize()
    assert dec.status() == 0
    got, gid = logits.cpu().numpy(), int(nxt.item())
    om = oracle.Model(cfg, w, rows=1, max_seq=max_seq)
    piece = 256
    for p0 in range(0, S, piece):
        rid, ref = om.prefill(toks[p0:p0 + piece], pos0=p0)
        log(f"oracle prefill {p0 + piece}/{S}")
    d, rel = check_logits(cfg, got, ref, "prefill 4096")
    check_argmax(cfg, gid, ref, "prefill 4096")
    _check_slots(cfg, dec, om, 0, S, "prefill 4096")
    log(f"prefill 4096 (2 layers, 8B width) vs oracle: max|d| {d:.3g} rel {rel:.3g}")
