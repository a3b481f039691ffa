"""GPU parity of batched decode rows against the CPU oracle.

Several cache rows each take one token at their own position in one step; with bf16 weights (widths a
multiple of 128) the projections run as matrix-core products over all rows (operands split into bf16
hi + lo), so this covers tile counts 1..4 of 16 token rows and ragged last tiles; narrower models take
the per-row path.  Every row is compared with an oracle
decode of that row alone: logits within max|d| 2e-2, argmax equal outside near-ties, the appended K/V
slot within bf16 rounding.  Two teacher-forced steps, so the second reads what the first appended.
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


CASES = [
    # model, layers, rows, max_seq
    ("smollm2_135m_bf16", 3, 64, 512),   # widths not a multiple of 128: the per-row path, largest batch
    ("smollm2_135m_bf16", 3, 17, 512),
    ("llama31_8b", 2, 2, 256),           # matrix-core rows: one ragged 16-row tile
    ("llama31_8b", 2, 20, 512),          # two tiles, the second ragged
    ("llama31_8b", 2, 33, 4096),         # three tiles, lengths across several attention chunks (spans of 2)
    ("llama31_8b", 2, 64, 512),          # the largest batch: four full tiles
    ("llama31_8b", 2, 40, 8192),         # attention in spans of 4 chunks, ragged last spans and chunks
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers,rows,max_seq", CASES, ids=[f"{c[0]}-L{c[1]}-B{c[2]}" for c in CASES])
def test_batched_rows_parity(name, layers, rows, max_seq):
    import llama_architecture_decoder_amd as lm
    cfg = _cfg(name, layers)
    log(f"case {name} layers={layers} rows={rows} max_seq={max_seq}")
    w = weights(cfg)
    om = oracle.Model(cfg, w, rows=rows, max_seq=max_seq)
    dec = lm.Decoder(cfg, w, rows=rows, max_seq=max_seq)
    lens = synth.int_range(f"batched/{name}/{rows}", rows, 0, max_seq - 2).astype(np.int64)
    lens[0] = 0                      # one row with an empty cache
    lens[-1] = max_seq - 2           # one row that ends at the last slot
    fill_random(cfg, om, dec, list(range(rows)), int(lens.max()))
    toks = synth.tokens(cfg, f"batched/{rows}", rows)
    logits = torch.empty((rows, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    worst = 0.0
    for step in range(2):
        pos = [int(p) + step for p in lens]
        dec.decode(torch.from_numpy(toks).cuda(), pos, logits, nxt)
        torch.cuda.synchronize()
        got = logits.cpu().numpy()
        gid = nxt.cpu().numpy()
        new = np.empty(rows, dtype=np.int32)
        for r in range(rows):
            rid, ref, _, _ = om.decode(int(toks[r]), pos[r], row=r)
            d, _ = check_logits(cfg, got[r], ref, f"step {step} row {r} pos {pos[r]}")
            check_argmax(cfg, int(gid[r]), ref, f"step {step} row {r} pos {pos[r]}")
            worst = max(worst, d)
            new[r] = rid
        gk, gv = gpu_cache(dec)
        for r in range(rows):
            p = pos[r]
            for nm, g, o in (("K", gk, om.kc), ("V", gv, om.vc)):
                a = widen(np.ascontiguousarray(g[:, r, :, p:p + 1]))
                b = widen(np.ascontiguousarray(o[:, r, :, p:p + 1]))
                tol = (1e-4 if cfg.kvdtype == "f32" else 1.6e-2) * float(np.abs(b).max())
                assert float(np.abs(a - b).max()) <= tol, f"{nm} row {r} slot {p}"
        toks = new  # teacher forcing
    assert dec.status() == 0
    log(f"{name} B={rows}: worst max|d| {worst:.3g}")


@pytest.mark.timeout(300)
def test_device_fill_matches_host_fill():
    """The device cache filler writes the host generator's bytes (sampled layers, rows and heads)."""
    cfg = configs.truncated(configs.LLAMA31_8B_LONG, 2)
    rows, max_seq = 3, 1024
    lens = [1000, 0, 17]
    k = torch.full((cfg.layers, rows, cfg.kv, max_seq, cfg.head), 7.0, dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, -3.0)
    synth.fill_cache_device(cfg, k.data_ptr(), v.data_ptr(), rows, max_seq, lens, row_keys=[5, 6, 7])
    torch.cuda.synchronize()
    gk = k.view(torch.int16).cpu().numpy().view(np.uint16)
    gv = v.view(torch.int16).cpu().numpy().view(np.uint16)
    for l in range(cfg.layers):
        for r, n in enumerate(lens):
            for j in (0, cfg.kv - 1):
                hk = synth.kv_fill_head(cfg, l, 5 + r, "k", j, 0, n)
                hv = synth.kv_fill_head(cfg, l, 5 + r, "v", j, 0, n)
                assert np.array_equal(gk[l, r, j, :n], hk), (l, r, j)
                assert np.array_equal(gv[l, r, j, :n], hv), (l, r, j)
                # positions past the length are untouched
                assert (gk[l, r, j, n:] == 0x40E0).all() and (gv[l, r, j, n:] == 0xC040).all()


@pytest.mark.timeout(900)
def test_long_context_batch32_sampled_rows():
    """The batch-32 long-context workload at its full size (32 layers, MaxSeq 32768, lengths uniform in
    [8192, 32000]) in the launch configuration the benchmark times; sampled rows are recomputed alone by
    the oracle (rows are independent)."""
    import llama_architecture_decoder_amd as lm
    cfg = configs.LLAMA31_8B_LONG
    B = cfg.batch
    lens = synth.row_lengths(cfg).astype(np.int64)
    w = weights(configs.LLAMA31_8B)  # the same weight streams (one family)
    dec = lm.Decoder(cfg, w, rows=B, max_seq=cfg.max_seq)
    log(f"long batch: lengths {int(lens.min())}..{int(lens.max())}")
    synth.fill_cache_device(cfg, dec.kv.k.data_ptr(), dec.kv.v.data_ptr(), B, cfg.max_seq, lens,
                            stream=torch.cuda.current_stream().cuda_stream)
    toks = synth.tokens(cfg, "bench/rows", B)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    dec.decode(torch.from_numpy(toks).cuda(), [int(p) for p in lens], logits, nxt)
    torch.cuda.synchronize()
    assert dec.status() == 0
    got = logits.cpu().numpy()
    gid = nxt.cpu().numpy()
    sample = [int(np.argmax(lens)), int(np.argmin(lens))]
    for r in sample:
        n = int(lens[r])
        om = oracle.Model(cfg, w, rows=1, max_seq=n + 1)
        synth.fill_cache_rows(cfg, om.kc, om.vc, r, n, cache_row=0)
        rid, ref, _, _ = om.decode(int(toks[r]), n, row=0)
        d, rel = check_logits(cfg, got[r], ref, f"row {r} pos {n}")
        check_argmax(cfg, int(gid[r]), ref, f"row {r} pos {n}")
        log(f"long batch row {r} at {n}: max|d| {d:.3g} rel {rel:.3g}")
        del om
    del dec
    torch.cuda.empty_cache()
