"""GPU parity at the full rope-scaled context of the Llama-3.1-8B shape (MaxSeq 131072; nest card: the
caches alone are ~16 GiB at 32 layers), two layers at full width.

Positions up to 131071 stress what grows with the context: the split attention merges up to 512 chunks,
and the F32 rope angles position x frequency lose the most bits there (the same F32 tables on both sides,
r2).  Cache positions 0..t-1 hold the seeded random keys and values (host fill for the oracle, device fill
with the same bytes for the GPU); both sides decode at t and t+1 (teacher forced), logits within the bf16
tolerance, argmax equal outside near-ties, the appended keys and values within bf16 rounding.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import configs
from parity_util import check_argmax, check_logits, gpu_cache, log, weights, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAXSEQ = 131072


@pytest.mark.timeout(900)
@pytest.mark.parametrize("t", [65536, 131070])
def test_long_context_decode_parity(t):
    import llama_architecture_decoder_amd as lm
    cfg = configs.truncated(configs.LLAMA31_8B, 2)
    w = weights(cfg)
    log(f"long context t={t}")
    om = oracle.Model(cfg, w, rows=1, max_seq=MAXSEQ)
    synth.fill_cache_rows(cfg, om.kc, om.vc, 0, t, cache_row=0)
    dec = lm.Decoder(cfg, w, rows=1, max_seq=MAXSEQ)
    synth.fill_cache_device(cfg, dec.kv.k.data_ptr(), dec.kv.v.data_ptr(), 1, MAXSEQ, [t])
    torch.cuda.synchronize()
    tok = int(synth.tokens(cfg, f"long/{t}", 1)[0])
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for step in range(2):
        p = t + step
        dec.decode(torch.tensor([tok], dtype=torch.int32, device="cuda"), [p], logits, nxt)
        rid, ref, _, _ = om.decode(tok, p, row=0)
        check_logits(cfg, logits.cpu().numpy()[0], ref, f"t={p}")
        check_argmax(cfg, int(nxt.item()), ref, f"t={p}")
        tok = rid
    assert dec.status() == 0
    gk, gv = gpu_cache(dec)
    for nm, g, o in (("K", gk, om.kc), ("V", gv, om.vc)):
        # the pre-filled positions are the generator's bytes on both sides; the appended ones agree to rounding
        assert np.array_equal(g[:, 0, :, t - 64:t], o[:, 0, :, t - 64:t]), nm
        a = widen(np.ascontiguousarray(g[:, 0, :, t:t + 2]))
        b = widen(np.ascontiguousarray(o[:, 0, :, t:t + 2]))
        assert float(np.abs(a - b).max()) <= 1.6e-2 * float(np.abs(b).max()), nm
