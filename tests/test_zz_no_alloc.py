"""llama_sample_noalloc (the sampling entry point that allocates nothing: its candidate keys live in a
static device buffer of the library) against llama_sample with a caller scratch buffer, through the C
ABI: identical drawn ids, logits and top-k lists.  Two calls in a row, the second on a smaller input
(fewer rows, a narrower vocabulary, another k), so stale candidates of the first call in the shared
buffer would show; a request beyond the buffer is rejected before anything runs.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _pair(x, temp, k, p, seed0):
    import llama_architecture_decoder_amd as lm
    B, V = x.shape
    logits = torch.from_numpy(x).cuda()
    seeds = torch.arange(seed0, seed0 + B, dtype=torch.int32, device="cuda")
    out = {}
    for name in ("scratch", "noalloc"):
        ids = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        vals = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
        topk = torch.full((B, k), -9, dtype=torch.int32, device="cuda")
        if name == "scratch":
            lm.sample(logits, temp, k, p, seeds=seeds, draw=3, ids=ids, vals=vals, topk_ids=topk)
        else:
            lm.sample_noalloc(logits, temp, k, p, ids, seeds=seeds, draw=3, vals=vals, topk_ids=topk)
        torch.cuda.synchronize()
        out[name] = (ids.cpu().numpy(), vals.cpu().numpy(), topk.cpu().numpy())
    for a, b in zip(out["scratch"], out["noalloc"]):
        np.testing.assert_array_equal(a, b)
    assert (out["noalloc"][0] >= 0).all() and (out["noalloc"][0] < V).all()
    return out["noalloc"]


@pytest.mark.timeout(300)
def test_sample_noalloc_matches_scratch_entry_point():
    import llama_architecture_decoder_amd as lm
    rng = np.random.default_rng(2024)
    # the largest request the static buffer holds: 64 rows of the 128256-token vocabulary, k = 256
    x1 = (rng.standard_normal((64, 128256)) * 3.0).astype(np.float32)
    r1 = _pair(x1, 0.7, 256, 0.95, 100)
    # then a smaller one on the same buffer: 3 rows, 20000 logits, k = 40
    x2 = (rng.standard_normal((3, 20000)) * 2.0).astype(np.float32)
    x2[:, 777] += 30.0
    r2 = _pair(x2, 0.9, 40, 0.8, 7)
    assert (r2[2][:, 0] == 777).all()  # the outlier leads every top-k list
    # beyond the buffer: more rows than it holds at this size, rejected before any launch
    big = torch.zeros((65, 128256), dtype=torch.float32, device="cuda")
    ids = torch.zeros(65, dtype=torch.int32, device="cuda")
    seeds = torch.zeros(65, dtype=torch.int32, device="cuda")
    rc = lm.lib().llama_sample_noalloc(big.data_ptr(), 128256, 65, 128256, 1.0, 256, 0.9, seeds.data_ptr(), 0, None,
                                       ids.data_ptr(), None, None, None)
    assert rc == lm.E_UNSUPPORTED
    assert int(ids.abs().sum().item()) == 0
