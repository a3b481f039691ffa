"""GPU generation loop `llama_generate_until` (nest card `generate_until`: greedy steps until every row
produces eos, at most max_new) against greedy chains of the CPU oracle.

The F32 SmolLM2-135M shape (4 layers) keeps the logits within 1e-3 of the oracle's; the chains below were
checked to have a top-2 gap above twice that at every step, so the greedy tokens must agree exactly.  One
row stops early on an eos its chain reaches; two rows at different positions run to max_new (an eos
neither produces), and the steps' tokens fill the step-major output with zeros after the count.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import configs
from parity_util import log, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MIN_GAP = 2.5e-3  # above twice the F32 logit tolerance (1e-3)


def _cfg():
    return configs.truncated(configs.SMOLLM2_135M, 4)


def _chain(om, tok, pos, row, n):
    out = []
    for i in range(n):
        tok, lg, _, _ = om.decode(int(tok), pos + i, row=row)
        top2 = np.sort(lg)[-2:]
        assert top2[1] - top2[0] > MIN_GAP, f"near tie at step {i}: the chain is not a safe check"
        out.append(int(tok))
    return out


@pytest.mark.timeout(600)
def test_generate_until_stops_on_eos():
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    w = weights(cfg)
    prompt = synth.tokens(cfg, "generate/prompt", 8)
    om = oracle.Model(cfg, w, rows=1, max_seq=64)
    first, _ = om.prefill(prompt, pos0=0, row=0)
    chain = _chain(om, first, 8, 0, 12)
    k = next(i for i in range(4, 12) if chain[i] not in chain[:i])  # an eos the chain meets first at step k
    log(f"chain {chain}, eos {chain[k]} at step {k}")
    dec = lm.Decoder(cfg, w, rows=1, max_seq=64)
    nt = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.prefill(torch.from_numpy(prompt).cuda(), pos0=0, next_tok=nt)
    assert int(nt.item()) == int(first)
    produced, n = dec.generate_until(nt, [8], 12, chain[k])
    got = produced.cpu().numpy()
    assert n == k + 1
    assert got[:n, 0].tolist() == chain[:n]
    assert (got[n:] == 0).all()


@pytest.mark.timeout(600)
def test_generate_until_two_rows_to_max_new():
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    w = weights(cfg)
    om = oracle.Model(cfg, w, rows=2, max_seq=64)
    dec = lm.Decoder(cfg, w, rows=2, max_seq=64)
    starts, toks = [5, 17], [101, 3030]
    # the rows' earlier positions: the same synthetic cache contents on both sides
    from parity_util import fill_random
    fill_random(cfg, om, dec, [0, 1], 17)
    chains = [_chain(om, toks[r], starts[r], r, 9) for r in range(2)]
    produced, n = dec.generate_until(torch.tensor(toks, dtype=torch.int32, device="cuda"), starts, 9, -7)
    got = produced.cpu().numpy()
    assert n == 9
    for r in range(2):
        assert got[:, r].tolist() == chains[r]
