"""GPU parity of the packed prefill (nest cards `prefill_packed` / `prefill_paged`) against the CPU oracle.

Several requests' prompts go end to end into one call; the oracle runs each segment as its own prefill of
its own cache row.  Each segment's last-position logits must match within the bf16 tolerance (argmax equal
outside near-ties), the appended keys and values must sit at exactly the segment's slots within bf16
rounding of the oracle's, and every other cache position must keep its bytes.  The cases cover a segment
that continues in the next pass (the workspace's max_prefill is 128 here), a pass of one position, one-
position segments, segments that start after positions already cached, and the page pool with a shared
prefix.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import configs
from parity_util import check_argmax, check_logits, log, weights, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PAGE = 64
MARK_K, MARK_V = 0x3F80, 0xBF80  # 1.0 / -1.0 in bf16: never a written value here


def _cfg():
    return configs.truncated(configs.LLAMA31_8B, 2)


def _upload(dst, src):
    dst.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.int16)))


def _download(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _close_bf16(got, ref, what):
    a, r = widen(np.ascontiguousarray(got)), widen(np.ascontiguousarray(ref))
    assert float(np.abs(a - r).max()) <= 1.6e-2 * float(np.abs(r).max()), what


ROW_CASES = [
    # (cache row, positions already cached, segment length) per segment, packed in this order
    ("split_across_passes", [(0, 0, 50), (1, 0, 77), (2, 64, 33)]),
    ("one_position_last_pass", [(0, 0, 100), (1, 0, 29)]),
    ("one_position_segments", [(2, 5, 1), (0, 0, 1), (1, 130, 2)]),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,segs", ROW_CASES, ids=[c[0] for c in ROW_CASES])
def test_packed_rows_parity(name, segs):
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    w = weights(cfg)
    rows, max_seq = 3, 256
    log(f"packed rows {name}: segments {segs}")
    om = oracle.Model(cfg, w, rows=rows, max_seq=max_seq)
    sentinel_k = np.full(om.kc.shape, MARK_K, dtype=np.uint16)
    sentinel_v = np.full(om.vc.shape, MARK_V, dtype=np.uint16)
    for r, p0, _ in segs:
        if p0:
            synth.fill_cache_rows(cfg, om.kc, om.vc, r, p0, cache_row=r)
            sentinel_k[:, r, :, :p0] = om.kc[:, r, :, :p0]
            sentinel_v[:, r, :, :p0] = om.vc[:, r, :, :p0]
    dec = lm.Decoder(cfg, w, rows=rows, max_seq=max_seq, max_prefill=128)
    _upload(dec.kv.k, sentinel_k)
    _upload(dec.kv.v, sentinel_v)
    toks = [synth.tokens(cfg, f"packed/{name}/{i}", n) for i, (_, _, n) in enumerate(segs)]
    packed = torch.from_numpy(np.concatenate(toks)).cuda()
    logits = torch.empty((len(segs), cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(segs), dtype=torch.int32, device="cuda")
    dec.prefill_packed(packed, segs, logits=logits, next_tok=nxt)
    got, gid = logits.cpu().numpy(), nxt.cpu().numpy()
    assert dec.status() == 0
    for i, (r, p0, n) in enumerate(segs):
        _, ref = om.prefill(toks[i], pos0=p0, row=r)
        check_logits(cfg, got[i], ref, f"{name} segment {i}")
        check_argmax(cfg, int(gid[i]), ref, f"{name} segment {i}")
    gk, gv = _download(dec.kv.k), _download(dec.kv.v)
    written = np.zeros((rows, max_seq), dtype=bool)
    for r, p0, n in segs:
        _close_bf16(gk[:, r, :, p0:p0 + n], om.kc[:, r, :, p0:p0 + n], f"K row {r}")
        _close_bf16(gv[:, r, :, p0:p0 + n], om.vc[:, r, :, p0:p0 + n], f"V row {r}")
        written[r, p0:p0 + n] = True
    # the cached prefixes kept their bytes, every position no segment wrote kept its marker
    keep = ~written
    assert np.array_equal(gk.transpose(1, 3, 0, 2, 4)[keep], sentinel_k.transpose(1, 3, 0, 2, 4)[keep])
    assert np.array_equal(gv.transpose(1, 3, 0, 2, 4)[keep], sentinel_v.transpose(1, 3, 0, 2, 4)[keep])


@pytest.mark.timeout(900)
def test_packed_paged_shared_prefix_parity():
    """Three requests of the page pool in one call: two continue after a shared 128-position prefix (the
    same two pool pages in both table rows), one starts fresh; 200 positions, so two passes."""
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    w = weights(cfg)
    npool, prefix = 16, 128
    # (positions cached before the call, segment length) of requests A, B, C
    segs = [(prefix, 40), (prefix, 70), (0, 90)]
    table = np.array([[3, 11, 5, 0, 0],
                      [3, 11, 7, 14, 0],
                      [9, 2, 0, 0, 0]], dtype=np.int32)
    pages = table.shape[1]
    max_seq = pages * PAGE
    om = oracle.Model(cfg, w, rows=3, max_seq=max_seq)
    for r in (0, 1):
        synth.fill_cache_rows(cfg, om.kc, om.vc, 0, prefix, cache_row=r)  # the same prefix bytes
    pool_k = np.full((cfg.layers, 1, cfg.kv, npool * PAGE, cfg.head), MARK_K, dtype=np.uint16)
    pool_v = np.full(pool_k.shape, MARK_V, dtype=np.uint16)
    slots = lambda tr, lo, hi: np.asarray(tr)[np.arange(lo, hi) // PAGE] * PAGE + np.arange(lo, hi) % PAGE
    s = slots(table[0], 0, prefix)
    pool_k[:, 0, :, s, :] = om.kc[:, 0, :, :prefix, :].transpose(2, 0, 1, 3)
    pool_v[:, 0, :, s, :] = om.vc[:, 0, :, :prefix, :].transpose(2, 0, 1, 3)
    before_k, before_v = pool_k.copy(), pool_v.copy()
    dec = lm.Decoder(cfg, w, rows=1, max_seq=npool * PAGE, max_prefill=128, ws_rows=1, ws_seq=max_seq)
    _upload(dec.kv.k, pool_k)
    _upload(dec.kv.v, pool_v)
    toks = [synth.tokens(cfg, f"packed/paged/{i}", n) for i, (_, n) in enumerate(segs)]
    logits = torch.empty((3, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(3, dtype=torch.int32, device="cuda")
    dec.prefill_packed(torch.from_numpy(np.concatenate(toks)).cuda(), [(0, p0, n) for p0, n in segs],
                       table=torch.from_numpy(table).cuda(), logits=logits, next_tok=nxt)
    got, gid = logits.cpu().numpy(), nxt.cpu().numpy()
    assert dec.status() == 0
    for i, (p0, n) in enumerate(segs):
        _, ref = om.prefill(toks[i], pos0=p0, row=i)
        check_logits(cfg, got[i], ref, f"paged segment {i}")
        check_argmax(cfg, int(gid[i]), ref, f"paged segment {i}")
    gk, gv = _download(dec.kv.k), _download(dec.kv.v)
    written = np.zeros(npool * PAGE, dtype=bool)
    for i, (p0, n) in enumerate(segs):
        s = slots(table[i], p0, p0 + n)
        _close_bf16(gk[:, 0, :, s, :], om.kc[:, i, :, p0:p0 + n, :].transpose(2, 0, 1, 3), f"K request {i}")
        _close_bf16(gv[:, 0, :, s, :], om.vc[:, i, :, p0:p0 + n, :].transpose(2, 0, 1, 3), f"V request {i}")
        written[s] = True
    assert np.array_equal(gk[:, 0, :, ~written, :], before_k[:, 0, :, ~written, :])
    assert np.array_equal(gv[:, 0, :, ~written, :], before_v[:, 0, :, ~written, :])


@pytest.mark.timeout(600)
def test_packed_f32_model_runs_segment_by_segment():
    """An F32 model (no matrix-core prefill): the packed call runs each segment as its own prefill; logits
    within the F32 tolerance, each segment's appended K/V within F32 rounding of the oracle's."""
    import llama_architecture_decoder_amd as lm
    cfg = configs.truncated(configs.SMOLLM2_135M, 3)
    w = weights(cfg)
    segs = [(1, 0, 9), (0, 4, 5), (2, 0, 1)]
    rows, max_seq = 3, 64
    om = oracle.Model(cfg, w, rows=rows, max_seq=max_seq)
    synth.fill_cache_rows(cfg, om.kc, om.vc, 0, 4, cache_row=0)
    dec = lm.Decoder(cfg, w, rows=rows, max_seq=max_seq)
    dec.kv.k.copy_(torch.from_numpy(om.kc))
    dec.kv.v.copy_(torch.from_numpy(om.vc))
    toks = [synth.tokens(cfg, f"packed/f32/{i}", n) for i, (_, _, n) in enumerate(segs)]
    logits = torch.empty((len(segs), cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(segs), dtype=torch.int32, device="cuda")
    dec.prefill_packed(torch.from_numpy(np.concatenate(toks)).cuda(), segs, logits=logits, next_tok=nxt)
    got, gid = logits.cpu().numpy(), nxt.cpu().numpy()
    assert dec.status() == 0
    for i, (r, p0, n) in enumerate(segs):
        _, ref = om.prefill(toks[i], pos0=p0, row=r)
        check_logits(cfg, got[i], ref, f"f32 segment {i}")
        check_argmax(cfg, int(gid[i]), ref, f"f32 segment {i}")
    torch.cuda.synchronize()
    gk, gv = dec.kv.k.cpu().numpy(), dec.kv.v.cpu().numpy()
    for r, p0, n in segs:
        for nm, g, o in (("K", gk, om.kc), ("V", gv, om.vc)):
            d = float(np.abs(g[:, r, :, p0:p0 + n] - o[:, r, :, p0:p0 + n]).max())
            assert d <= 1e-4 * max(1.0, float(np.abs(o[:, r, :, p0:p0 + n]).max())), f"{nm} row {r}: {d}"
