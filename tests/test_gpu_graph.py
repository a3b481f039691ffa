"""HIP-graph replay of decode steps (torch graph capture): every replay equals the eager step.

The batch-1 q/k/v + attention launch synchronises through tagged words whose tag is derived from a step
counter in device memory, advanced by each step's embedding launch, so a replayed step must never take a
word left behind by an earlier launch.  Two steps at the same position with different tokens are
captured as two graphs and replayed alternately, with eager steps in between; every replay's logits, next
token and appended K/V slot must equal the eager run of the same step bit for bit (the kernels are
deterministic).  Were the tags of two launches ever equal, a replay could read the other graph's queries
or key/value words, and its logits would differ.  Cases: the bf16 plan (8B shape: matrix-core attention
role, separate merge) and the F32 plan (1.7B shape: vector-unit role, merge inside the launch).
"""
import numpy as np
import pytest

import synth
from synth import configs
from parity_util import log, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # name, layers, position of the captured steps (cache filled before it), max_seq
    ("llama31_8b", 2, 4000, 8192),
    ("smollm2_1_7b", 2, 700, 2048),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,layers,p,max_seq", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, layers, p, max_seq):
    import llama_architecture_decoder_amd as lm
    cfg = configs.truncated(configs.get(name), layers)
    log(f"case {name} layers={layers} position={p}")
    dec = lm.Decoder(cfg, weights(cfg), rows=1, max_seq=max_seq)
    synth.fill_cache_device(cfg, dec.kv.k.data_ptr(), dec.kv.v.data_ptr(), 1, max_seq, [p])
    torch.cuda.synchronize()
    dev = "cuda"
    toks = {"a": torch.tensor([11], dtype=torch.int32, device=dev),
            "b": torch.tensor([int(cfg.vocab) - 17], dtype=torch.int32, device=dev)}
    logits = {k: torch.empty((1, cfg.vocab), dtype=torch.float32, device=dev) for k in toks}
    nxt = {k: torch.empty(1, dtype=torch.int32, device=dev) for k in toks}
    other = torch.tensor([5], dtype=torch.int32, device=dev)
    other_next = torch.empty(1, dtype=torch.int32, device=dev)

    def slot():
        return (dec.kv.k[:, 0, :, p, :].clone(), dec.kv.v[:, 0, :, p, :].clone())

    s = torch.cuda.Stream()
    ref = {}
    with torch.cuda.stream(s):
        for k in toks:  # the eager steps (b's runs last, so its slot is what the cache holds now)
            dec.decode(toks[k], [p], logits[k], nxt[k], stream=s)
            s.synchronize()
            ref[k] = (logits[k].cpu().clone(), int(nxt[k].item()), slot())
        assert not torch.equal(ref["a"][0], ref["b"][0])
        graphs = {}
        for k in toks:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                dec.decode(toks[k], [p], logits[k], nxt[k], stream=s)
            graphs[k] = g
        s.synchronize()
        for rep in range(4):
            for k in toks:
                logits[k].fill_(float("nan"))
                nxt[k].fill_(-1)
                graphs[k].replay()
                s.synchronize()
                got = logits[k].cpu()
                assert torch.equal(got, ref[k][0]), f"replay {rep} of step {k}: logits differ from the eager step"
                assert int(nxt[k].item()) == ref[k][1], f"replay {rep} of step {k}: next token"
                gk, gv = slot()
                assert torch.equal(gk, ref[k][2][0]) and torch.equal(gv, ref[k][2][1]), f"replay {rep} of {k}: K/V slot"
                # eager work between the replays: a step at p + 1 (a slot the replayed steps do not read)
                dec.decode(other, [p + 1], None, other_next, stream=s)
                s.synchronize()
    assert dec.status() == 0
    log(f"{name}: 8 replays of two captured steps equal their eager runs")
