"""GPU parity of the paged cache (nest card `decode_paged` / `prefill_paged`) against the CPU oracle.

The oracle keeps every request in its own contiguous cache row; the GPU keeps them in one pool of
64-position pages, request b's positions in the pages its table row lists (scattered, out of order,
some shared).  The pool is filled with the same bytes the oracle's rows hold, then both sides run the
same teacher-forced steps: logits within the bf16 tolerance, argmax equal outside near-ties, the
appended keys and values at their pool slots within bf16 rounding of the oracle's, and every other
pool position untouched.  A table entry outside the pool must write nothing and raise the page flag.
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


def _cfg(layers=2):
    return configs.truncated(configs.LLAMA31_8B, layers)


def _pool_upload(dec, pool_k, pool_v):
    dec.kv.k.view(torch.int16).copy_(torch.from_numpy(pool_k.view(np.int16)))
    dec.kv.v.view(torch.int16).copy_(torch.from_numpy(pool_v.view(np.int16)))
    torch.cuda.synchronize()


def _pool_download(dec):
    torch.cuda.synchronize()
    k = dec.kv.k.view(torch.int16).cpu().numpy().view(np.uint16)
    v = dec.kv.v.view(torch.int16).cpu().numpy().view(np.uint16)
    return k, v


def _slots(table_row, n):
    p = np.arange(n)
    return np.asarray(table_row)[p // PAGE] * PAGE + p % PAGE


def _scatter(om, table, lens, npool):
    """Pool arrays [layers][1][kv][npool*64][head] holding each oracle row's positions 0..len-1 at their
    slots; the rest a fixed marker."""
    cfg = om.cfg
    shape = (cfg.layers, 1, cfg.kv, npool * PAGE, cfg.head)
    pk = np.full(shape, 0x3F80, dtype=np.uint16)  # 1.0: never part of a row
    pv = np.full(shape, 0xBF80, dtype=np.uint16)
    for b, n in enumerate(lens):
        s = _slots(table[b], n)
        pk[:, 0, :, s, :] = om.kc[:, b, :, :n, :].transpose(2, 0, 1, 3)
        pv[:, 0, :, s, :] = om.vc[:, b, :, :n, :].transpose(2, 0, 1, 3)
    return pk, pv


CASES = [
    # requests, their lengths before the steps, pool pages
    ([200], 16),
    ([0, 63, 64, 300, 1000], 48),
    ([130, 130, 700, 5, 64, 129, 1], 64),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("lens,npool", CASES, ids=[f"B{len(c[0])}" for c in CASES])
def test_paged_decode_parity(lens, npool):
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    B = len(lens)
    steps = 2
    need = [(n + steps + PAGE - 1) // PAGE for n in lens]
    pages = max(need)
    log(f"paged decode B={B} lens={lens} pool={npool} pages/row={pages}")
    rng = np.random.default_rng(sum(lens) + npool)
    perm = rng.permutation(npool)
    table = np.zeros((B, pages), dtype=np.int32)
    used = 0
    for b in range(B):
        table[b, :need[b]] = perm[used:used + need[b]]
        used += need[b]
        table[b, need[b]:] = perm[(used + b) % npool]  # entries past the row's length: never reached
    assert used <= npool
    w = weights(cfg)
    max_seq = pages * PAGE
    om = oracle.Model(cfg, w, rows=B, max_seq=max_seq)
    for b, n in enumerate(lens):
        synth.fill_cache_rows(cfg, om.kc, om.vc, b, n, cache_row=b)
    dec = lm.Decoder(cfg, w, rows=1, max_seq=npool * PAGE, ws_rows=B, ws_seq=max_seq)
    pk, pv = _scatter(om, table, lens, npool)
    _pool_upload(dec, pk, pv)
    tdev = torch.from_numpy(table).cuda()
    toks = synth.tokens(cfg, f"paged/{B}", B)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(steps):
        pos = [n + step for n in lens]
        dec.decode_paged(torch.from_numpy(toks).cuda(), pos, tdev, logits, nxt)
        got, gid = logits.cpu().numpy(), nxt.cpu().numpy()
        new = np.empty(B, dtype=np.int32)
        for b in range(B):
            rid, ref, _, _ = om.decode(int(toks[b]), pos[b], row=b)
            check_logits(cfg, got[b], ref, f"step {step} request {b} pos {pos[b]}")
            check_argmax(cfg, int(gid[b]), ref, f"step {step} request {b} pos {pos[b]}")
            new[b] = rid
        toks = new
    assert dec.status() == 0
    gk, gv = _pool_download(dec)
    written = np.zeros(npool * PAGE, dtype=bool)
    for b, n in enumerate(lens):
        s = _slots(table[b], n + steps)
        # the filled positions are the uploaded bytes; the appended ones within bf16 rounding
        for nm, g, o in (("K", gk, om.kc), ("V", gv, om.vc)):
            assert np.array_equal(g[:, 0, :, s[:n], :], o[:, b, :, :n, :].transpose(2, 0, 1, 3)), f"{nm} {b}"
            a = widen(np.ascontiguousarray(g[:, 0, :, s[n:], :]))
            r = widen(np.ascontiguousarray(o[:, b, :, n:n + steps, :].transpose(2, 0, 1, 3)))
            assert float(np.abs(a - r).max()) <= 1.6e-2 * float(np.abs(r).max()), f"{nm} request {b} appended"
        written[s] = True
    # no other slot of the pool changed
    assert (gk[:, 0, :, ~written, :] == 0x3F80).all() and (gv[:, 0, :, ~written, :] == 0xBF80).all()


@pytest.mark.timeout(600)
def test_paged_shared_prefix_pages():
    """Two requests read the same prefix pages and write their own: each matches an oracle row holding
    the prefix."""
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    prefix, npool = 192, 12  # three shared pages
    lens = [prefix, prefix]
    om = oracle.Model(cfg, weights(cfg), rows=2, max_seq=8 * PAGE)
    synth.fill_cache_rows(cfg, om.kc, om.vc, 0, prefix, cache_row=0)
    om.kc[:, 1] = om.kc[:, 0]
    om.vc[:, 1] = om.vc[:, 0]
    table = np.array([[7, 2, 9, 4, 0, 0, 0, 0], [7, 2, 9, 11, 0, 0, 0, 0]], dtype=np.int32)
    dec = lm.Decoder(cfg, weights(cfg), rows=1, max_seq=npool * PAGE, ws_rows=2, ws_seq=8 * PAGE)
    pk, pv = _scatter(om, table[:1], lens[:1], npool)
    _pool_upload(dec, pk, pv)
    toks = np.array([11, 4242], dtype=np.int32)
    logits = torch.empty((2, cfg.vocab), dtype=torch.float32, device="cuda")
    dec.decode_paged(torch.from_numpy(toks).cuda(), lens, torch.from_numpy(table).cuda(), logits)
    got = logits.cpu().numpy()
    for b in range(2):
        _, ref, _, _ = om.decode(int(toks[b]), prefix, row=b)
        check_logits(cfg, got[b], ref, f"request {b}")
    assert dec.status() == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("S,pos0", [(300, 0), (77, 128), (200, 65)])
def test_paged_prefill_parity(S, pos0):
    """One request's prompt into scattered pages (chunked matrix-core prefill), after pos0 positions that
    already sit in its first pages: last-position logits against the oracle, and the pool slots equal
    those a contiguous prefill of the same request writes to its row (the same kernels on other
    addresses), with nothing else touched."""
    import llama_architecture_decoder_amd as lm
    cfg = _cfg()
    w = weights(cfg)
    npool = 16
    pages = (pos0 + S + PAGE - 1) // PAGE
    rng = np.random.default_rng(S * 7 + pos0)
    table = rng.permutation(npool)[:pages].astype(np.int32)
    log(f"paged prefill S={S} pos0={pos0} table={table.tolist()}")
    max_seq = pages * PAGE
    om = oracle.Model(cfg, w, rows=1, max_seq=max_seq)
    synth.fill_cache_rows(cfg, om.kc, om.vc, 0, pos0, cache_row=0)
    toks = synth.tokens(cfg, f"paged/prompt/{S}/{pos0}", S)
    rid, ref = om.prefill(toks, pos0=pos0, row=0)
    dec = lm.Decoder(cfg, w, rows=1, max_seq=npool * PAGE, max_prefill=128, ws_rows=1, ws_seq=max_seq)
    pk, pv = _scatter(om, table[None, :], [pos0], npool)
    _pool_upload(dec, pk, pv)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.prefill_paged(torch.from_numpy(toks).cuda(), torch.from_numpy(table).cuda(), pos0=pos0, logits=logits,
                      next_tok=nxt)
    check_logits(cfg, logits.cpu().numpy(), ref, "paged prefill")
    check_argmax(cfg, int(nxt.item()), ref, "paged prefill")
    assert dec.status() == 0
    gk, gv = _pool_download(dec)
    # a contiguous prefill of the same request
    flat = lm.Decoder(cfg, None, rows=1, max_seq=max_seq, max_prefill=128, weights=dec.w)
    for dst, src in ((flat.kv.k, om.kc), (flat.kv.v, om.vc)):
        dst.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.int16)))
    flat.prefill(torch.from_numpy(toks).cuda(), pos0=pos0)
    fk = flat.kv.k.view(torch.int16).cpu().numpy().view(np.uint16)
    fv = flat.kv.v.view(torch.int16).cpu().numpy().view(np.uint16)
    s = _slots(table, pos0 + S)
    assert np.array_equal(gk[:, 0, :, s, :], fk[:, 0, :, :pos0 + S, :].transpose(2, 0, 1, 3))
    assert np.array_equal(gv[:, 0, :, s, :], fv[:, 0, :, :pos0 + S, :].transpose(2, 0, 1, 3))
    rest = np.ones(npool * PAGE, dtype=bool)
    rest[s] = False
    assert (gk[:, 0, :, rest, :] == 0x3F80).all() and (gv[:, 0, :, rest, :] == 0xBF80).all()


@pytest.mark.timeout(300)
def test_page_entry_outside_pool_sets_flag_and_writes_nothing():
    import llama_architecture_decoder_amd as lm
    cfg = _cfg(1)
    npool = 4
    dec = lm.Decoder(cfg, weights(cfg), rows=1, max_seq=npool * PAGE, ws_rows=1, ws_seq=2 * PAGE)
    pk = np.full((cfg.layers, 1, cfg.kv, npool * PAGE, cfg.head), 0x3F80, dtype=np.uint16)
    _pool_upload(dec, pk, pk)
    table = torch.tensor([[1, npool]], dtype=torch.int32, device="cuda")  # position 70 lies in page 1: outside
    dec.decode_paged(torch.tensor([3], dtype=torch.int32, device="cuda"), [70], table)
    assert dec.status() == lm.E_PAGE
    assert dec.status() == 0  # cleared
    gk, gv = _pool_download(dec)
    assert (gk == 0x3F80).all() and (gv == 0x3F80).all()
