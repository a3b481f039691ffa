"""The C ABI on a machine without a GPU: the library loads, exports every function the header declares,
and rejects invalid arguments with the documented codes before any device work (no compute call)."""
import ctypes
import subprocess

import numpy as np
import pytest

import llama_architecture_decoder_amd as lm
from synth import configs


@pytest.fixture(scope="module")
def L():
    return lm.lib()


def test_header_declares_the_boundary():
    names = set(lm.header_functions())
    for need in ("llama_decode_step", "llama_prefill", "kv_cache_alloc", "lm_head_argmax", "llama_kv_cache_bytes",
                 "llama_workspace_bytes", "llama_workspace_init", "llama_status", "llama_strerror",
                 "llama_decode_step_traced", "llama_trace_floats", "llama_abi_version", "llama_sample",
                 "llama_sample_scratch_bytes", "llama_decode_step_paged", "llama_prefill_paged",
                 "llama_generate_until", "llama_prefill_packed"):
        assert need in names, need


def test_library_exports_every_header_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", lm.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in lm.header_functions() if n not in exported]
    assert not missing, missing
    for n in lm.header_functions():
        assert hasattr(L, n)
    assert L.llama_abi_version() == 1


def test_strerror_covers_codes(L):
    for code in range(0, -9, -1):
        assert L.llama_strerror(code).decode() not in ("", "unknown error")
    assert L.llama_strerror(-100).decode() == "unknown error"


def _c(cfg, **kw):
    c = lm.make_cfg(cfg)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_kv_cache_bytes_and_config_checks(L):
    c = _c(configs.LLAMA31_8B)
    # nest 8B card: 1 GiB of bf16 caches (both) at MaxSeq 8192
    assert L.llama_kv_cache_bytes(ctypes.byref(c), 1, 8192) == (1 << 30) // 2
    assert L.llama_kv_cache_bytes(ctypes.byref(c), 0, 8192) == lm.E_SHAPE
    assert L.llama_kv_cache_bytes(None, 1, 8192) == lm.E_NULL
    for field, bad in (("kv", 0), ("g", -1), ("half", 0), ("f", 0), ("layers", 0), ("vocab", 0), ("eps", 0.0),
                       ("theta", -1.0), ("weight_dtype", 7), ("kv_dtype", 2), ("rope_llama3", 2),
                       ("rope_factor", 0.0), ("tied_lm_head", 3)):
        assert L.llama_kv_cache_bytes(ctypes.byref(_c(configs.LLAMA31_8B, **{field: bad})), 1, 16) == lm.E_CONFIG, field
    c = _c(configs.LLAMA31_8B, rope_high_freq_factor=0.5)
    assert L.llama_kv_cache_bytes(ctypes.byref(c), 1, 16) == lm.E_CONFIG
    # valid but not built: head 32, g = 5, dim not a multiple of 8
    assert L.llama_kv_cache_bytes(ctypes.byref(_c(configs.TINY)), 1, 16) == lm.E_UNSUPPORTED
    assert L.llama_kv_cache_bytes(ctypes.byref(_c(configs.SMOLLM2_135M, g=5)), 1, 16) == lm.E_UNSUPPORTED
    for name in configs.CONFIGS:
        assert L.llama_kv_cache_bytes(ctypes.byref(_c(configs.get(name))), 1, 64) > 0, name


def test_workspace_bytes(L):
    c = _c(configs.LLAMA31_8B)
    n1 = L.llama_workspace_bytes(ctypes.byref(c), 1, 8192, 0)
    n32 = L.llama_workspace_bytes(ctypes.byref(c), 32, 32768, 0)
    assert 0 < n1 < n32
    assert L.llama_workspace_bytes(ctypes.byref(c), 0, 8192, 0) == lm.E_SHAPE
    assert L.llama_workspace_bytes(ctypes.byref(c), 65, 8192, 0) == lm.E_SHAPE
    assert L.llama_workspace_bytes(ctypes.byref(c), 1, 1 << 20, 0) == lm.E_UNSUPPORTED


def test_workspace_prefill_rows(L):
    # A prompt chunk of the matrix-core prefill needs, per row: the F32 residual, q|k|v and attention rows,
    # one bf16 hi/lo operand pair of width max(dim, f) and the down product's pair of width f; its SwiGLU
    # output is never F32, so no [max_prefill][f] F32 buffer.  F32 models prefill through the decode
    # kernels and need nothing per prompt row.
    c = _c(configs.LLAMA31_8B)
    d = configs.LLAMA31_8B
    n2 = L.llama_workspace_bytes(ctypes.byref(c), 1, 32768, 2048)
    n4 = L.llama_workspace_bytes(ctypes.byref(c), 1, 32768, 4096)
    per_row = (n4 - n2) / 2048
    rows = 4 * (2 * d.dim + d.dim + 2 * d.kvw) + 4 * max(d.dim, d.f) + 4 * d.f
    assert rows <= per_row < rows + 2 * d.f, per_row  # (+ split-K partial sums, far below a row of f F32)
    cf = _c(configs.SMOLLM2_1_7B)
    assert L.llama_workspace_bytes(ctypes.byref(cf), 1, 8192, 4096) == L.llama_workspace_bytes(ctypes.byref(cf), 1,
                                                                                              8192, 0)


def test_kv_cache_alloc_binds_without_touching_memory(L):
    cfg = configs.SMOLLM2_135M
    c = _c(cfg)
    need = L.llama_kv_cache_bytes(ctypes.byref(c), 2, 32)
    k = np.zeros(need + 16, dtype=np.uint8)
    v = np.zeros(need + 16, dtype=np.uint8)
    kp = k.ctypes.data + ((-k.ctypes.data) % 16)
    vp = v.ctypes.data + ((-v.ctypes.data) % 16)
    rec = lm.llama_kv()
    assert L.kv_cache_alloc(ctypes.byref(c), 2, 32, kp, vp, need, ctypes.byref(rec)) == lm.OK
    assert (rec.rows, rec.max_seq, rec.layers, rec.kv, rec.head, rec.dtype) == (2, 32, cfg.layers, cfg.kv, 64, lm.F32)
    assert not k.any() and not v.any()
    assert L.kv_cache_alloc(ctypes.byref(c), 2, 32, kp, vp, need - 1, ctypes.byref(rec)) == lm.E_WORKSPACE
    assert L.kv_cache_alloc(ctypes.byref(c), 2, 32, None, vp, need, ctypes.byref(rec)) == lm.E_NULL
    assert L.kv_cache_alloc(ctypes.byref(c), 2, 32, kp + 4, vp, need, ctypes.byref(rec)) == lm.E_SHAPE


def test_decode_and_prefill_reject_before_any_device_work(L):
    """Argument errors come back before the library touches the workspace or a GPU: the fake device
    pointers below are never dereferenced."""
    cfg = configs.SMOLLM2_135M
    c = _c(cfg)
    fake = 1 << 40
    kv = lm.llama_kv(fake, fake, 2, 16, cfg.layers, cfg.kv, 64, lm.F32)
    lw = (lm.llama_layer_w * cfg.layers)()
    for l in range(cfg.layers):
        for f in ("ln1", "wq", "wk", "wv", "wo", "ln2", "w_gate", "w_up", "w_down"):
            setattr(lw[l], f, fake)
    w = lm.llama_weights(fake, None, fake, lw)
    ws = lm.llama_ws(fake, 1 << 30, 2, 16, 0, 0, 0)  # never initialised: reached only after the checks
    pos = (ctypes.c_int32 * 3)(0, 0, 0)

    def dec(B, p, cc=c, kvr=kv, tokens=fake):
        for i, v in enumerate(p):
            pos[i] = v
        return L.llama_decode_step(ctypes.byref(cc), ctypes.byref(w), ctypes.byref(kvr), tokens, pos, B, None, None,
                                   ctypes.byref(ws), None)

    assert dec(1, [16]) == lm.E_POS
    assert dec(1, [-1]) == lm.E_POS
    assert dec(2, [3, 16]) == lm.E_POS
    assert dec(0, [0]) == lm.E_SHAPE
    assert dec(3, [0, 0, 0]) == lm.E_SHAPE  # more rows than the cache holds
    assert dec(1, [0], tokens=None) == lm.E_NULL
    assert dec(1, [0], cc=_c(cfg, eps=-1.0)) == lm.E_CONFIG
    bad_kv = lm.llama_kv(fake, fake, 2, 16, cfg.layers, cfg.kv + 1, 64, lm.F32)
    assert dec(1, [0], kvr=bad_kv) == lm.E_SHAPE
    # valid arguments, uninitialised workspace record
    assert dec(1, [0]) == lm.E_WORKSPACE
    # prefill: S <= 0, row outside, pos0 + S > max_seq
    pf = lambda row, S, p0: L.llama_prefill(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), row, fake, S, p0,
                                            None, None, ctypes.byref(ws), None)
    assert pf(0, 0, 0) == lm.E_SHAPE
    assert pf(2, 4, 0) == lm.E_SHAPE
    assert pf(0, 4, 13) == lm.E_POS
    assert pf(0, 4, -1) == lm.E_POS
    assert pf(0, 4, 12) == lm.E_WORKSPACE
    # lm_head_argmax: NULL outputs
    assert L.lm_head_argmax(ctypes.byref(c), ctypes.byref(w), fake, 1, None, None, ctypes.byref(ws), None) == lm.E_NULL
    # a misaligned weight pointer is refused
    lw[3].wq = fake + 2
    assert dec(1, [0]) == lm.E_SHAPE


def test_sample_scratch_bytes_and_argument_checks(L):
    """Sampling's size query and its argument errors, all decided on the host (the fake device pointers
    are never dereferenced)."""
    V = 128256
    # 16 chunks of 8192 logits, k = 50 rounds up to 64 candidates per chunk, 8-byte keys
    assert L.llama_sample_scratch_bytes(3, V, 50) == 3 * 16 * 64 * 8
    assert L.llama_sample_scratch_bytes(1, 1, 1) == 8
    assert L.llama_sample_scratch_bytes(0, V, 1) == 0
    assert L.llama_sample_scratch_bytes(-1, V, 1) == lm.E_SHAPE
    assert L.llama_sample_scratch_bytes(1, 0, 1) == lm.E_SHAPE
    assert L.llama_sample_scratch_bytes(1, V, 0) == lm.E_CONFIG
    assert L.llama_sample_scratch_bytes(1, V, 257) == lm.E_UNSUPPORTED
    assert L.llama_sample_scratch_bytes(1, 262144, 256) == 32 * 256 * 8
    assert L.llama_sample_scratch_bytes(1, 262145, 256) == lm.E_UNSUPPORTED
    assert L.llama_sample_scratch_bytes(1, 524288, 128) == 64 * 128 * 8
    fake = 1 << 40
    big = 1 << 30

    def smp(B=1, V=V, ld=V, temp=0.8, k=50, p=0.9, seeds=fake, u=None, ids=fake, scratch=fake, nbytes=big,
            logits=fake):
        return L.llama_sample(logits, ld, B, V, temp, k, p, seeds, 0, u, ids, None, None, scratch, nbytes, None)

    assert smp(ld=V - 1) == lm.E_SHAPE
    assert smp(B=-1) == lm.E_SHAPE
    assert smp(temp=0.0) == lm.E_CONFIG
    assert smp(temp=-1.0) == lm.E_CONFIG
    assert smp(temp=float("inf")) == lm.E_CONFIG
    assert smp(temp=float("nan")) == lm.E_CONFIG
    assert smp(p=float("nan")) == lm.E_CONFIG
    assert smp(k=0) == lm.E_CONFIG
    assert smp(k=300) == lm.E_UNSUPPORTED
    assert smp(logits=None) == lm.E_NULL
    assert smp(ids=None) == lm.E_NULL
    assert smp(seeds=None) == lm.E_NULL
    assert smp(scratch=None) == lm.E_NULL
    assert smp(nbytes=16 * 64 * 8 - 1) == lm.E_WORKSPACE
    assert smp(scratch=fake + 4) == lm.E_WORKSPACE
    assert smp(B=0, logits=None, ids=None, scratch=None) == lm.OK


def test_paged_calls_reject_before_any_device_work(L):
    """The paged entry points' argument errors, decided on the host (fake device pointers are never read)."""
    fake = 1 << 40
    ws = lm.llama_ws(fake, 1 << 30, 4, 1024, 0, 0, 0)  # never initialised: reached only after the checks
    pos = (ctypes.c_int32 * 3)(0, 0, 0)

    def setup(cfg, max_seq=1024, dtype=None):
        c = _c(cfg)
        kvd = lm.BF16 if cfg.kvdtype == "bf16" else lm.F32
        kv = lm.llama_kv(fake, fake, 1, max_seq, cfg.layers, cfg.kv, 2 * cfg.half, kvd if dtype is None else dtype)
        lw = (lm.llama_layer_w * cfg.layers)()
        for l in range(cfg.layers):
            for f in ("ln1", "wq", "wk", "wv", "wo", "ln2", "w_gate", "w_up", "w_down"):
                setattr(lw[l], f, fake)
        return c, kv, lm.llama_weights(fake, fake, fake, lw), lw

    cfg = configs.truncated(configs.LLAMA31_8B, 1)
    c, kv, w, lw = setup(cfg)

    def dec(B, p, pages=4, table=fake, kvr=kv):
        for i, v in enumerate(p):
            pos[i] = v
        return L.llama_decode_step_paged(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kvr), fake, pos, B, table,
                                         pages, None, None, ctypes.byref(ws), None)

    assert dec(1, [0], table=None) == lm.E_NULL
    assert dec(1, [0], pages=0) == lm.E_SHAPE
    assert dec(0, [0]) == lm.E_SHAPE
    assert dec(1, [256]) == lm.E_POS          # 4 pages hold positions 0..255
    assert dec(2, [3, -1]) == lm.E_POS
    _, odd_pool, _, _ = setup(cfg, max_seq=1000)
    assert dec(1, [0], kvr=odd_pool) == lm.E_SHAPE   # the pool is not whole pages
    assert dec(1, [255]) == lm.E_WORKSPACE           # valid arguments, uninitialised workspace
    f32 = configs.SMOLLM2_135M                       # F32 cache: the paged attention needs bf16
    c2, kv2, w2, _ = setup(f32)
    assert L.llama_decode_step_paged(ctypes.byref(c2), ctypes.byref(w2), ctypes.byref(kv2), fake, pos, 1, fake, 4,
                                     None, None, ctypes.byref(ws), None) == lm.E_UNSUPPORTED

    def pf(S, p0, pages=4, table=fake):
        return L.llama_prefill_paged(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), table, pages, fake, S, p0,
                                     None, None, ctypes.byref(ws), None)

    assert pf(4, 0, table=None) == lm.E_NULL
    assert pf(0, 0) == lm.E_SHAPE
    assert pf(4, 253) == lm.E_POS
    assert pf(4, -1) == lm.E_POS
    assert pf(4, 252) == lm.E_WORKSPACE
    assert L.llama_strerror(lm.E_PAGE)


def test_packed_prefill_rejects_before_any_device_work(L):
    """llama_prefill_packed's argument errors, decided on the host from the segment lists (fake device
    pointers are never read)."""
    fake = 1 << 40
    ws = lm.llama_ws(fake, 1 << 30, 4, 1024, 256, 0, 0)  # never initialised: reached only after the checks
    cfg = configs.truncated(configs.LLAMA31_8B, 1)
    c = _c(cfg)
    kv = lm.llama_kv(fake, fake, 3, 1024, cfg.layers, cfg.kv, 2 * cfg.half, lm.BF16)
    lw = (lm.llama_layer_w * cfg.layers)()
    for l in range(cfg.layers):
        for f in ("ln1", "wq", "wk", "wv", "wo", "ln2", "w_gate", "w_up", "w_down"):
            setattr(lw[l], f, fake)
    w = lm.llama_weights(fake, fake, fake, lw)

    def pk(segs, table=None, pages=0, rows=True, logits=None):
        n = len(segs)
        arr = lambda k: (ctypes.c_int32 * max(n, 1))(*[int(s[k]) for s in segs])
        return L.llama_prefill_packed(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), table, pages, fake, n,
                                      arr(0) if rows else None, arr(1), arr(2), logits, None, ctypes.byref(ws), None)

    assert pk([(0, 0, 4)], rows=False) == lm.E_NULL           # contiguous rows need seg_row
    assert pk([]) == lm.E_SHAPE
    assert pk([(0, 0, 1)] * 65) == lm.E_SHAPE                 # at most 64 segments
    assert pk([(0, 0, 4), (1, 0, 0)]) == lm.E_SHAPE           # empty segment
    assert pk([(0, 0, 4), (3, 0, 4)]) == lm.E_SHAPE           # row outside the cache
    assert pk([(0, 0, 4), (1, -1, 4)]) == lm.E_POS
    assert pk([(0, 0, 4), (2, 1021, 4)]) == lm.E_POS          # past max_seq 1024
    assert pk([(0, 0, 4)], logits=fake + 2) == lm.E_SHAPE     # misaligned logits
    assert pk([(0, 0, 4), (1, 1020, 4), (0, 4, 9)]) == lm.E_WORKSPACE  # valid; uninitialised workspace
    # paged: segment s is table row s, seg_row unread; room = pages * 64
    assert pk([(0, 0, 4)], table=fake, pages=0, rows=False) == lm.E_SHAPE
    assert pk([(0, 250, 7)], table=fake, pages=4, rows=False) == lm.E_POS
    assert pk([(0, 250, 6), (9, 0, 5)], table=fake, pages=4, rows=False) == lm.E_WORKSPACE
