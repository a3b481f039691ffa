"""Python binding of libllama_mi355x (include/llama_mi355x.h): argument marshalling only.

Every step of the decoder runs in the library's HIP kernels; PyTorch only provides device memory and
the stream.  Importing works anywhere, but `lib()` raises if the built library is missing, and the
entry points need an MI355X (gfx950) GPU.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libllama_mi355x.so")  # the in-tree build, never another
HEADER = os.path.join(os.path.dirname(_HERE), "include", "llama_mi355x.h")

F32, BF16 = 0, 1
OK = 0
E_CONFIG, E_POS, E_TOKEN, E_SHAPE, E_NULL, E_WORKSPACE, E_HIP, E_UNSUPPORTED, E_PAGE, E_WAIT = range(-1, -11, -1)
ERROR_NAMES = {0: "OK", -1: "E_CONFIG", -2: "E_POS", -3: "E_TOKEN", -4: "E_SHAPE", -5: "E_NULL",
               -6: "E_WORKSPACE", -7: "E_HIP", -8: "E_UNSUPPORTED", -9: "E_PAGE",
               -10: "E_WAIT"}
PAGE_SIZE = 64


class LlamaError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {ERROR_NAMES.get(code, code)} ({_strerror(code)})")


class llama_cfg(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_int32), ("g", ctypes.c_int32), ("half", ctypes.c_int32), ("f", ctypes.c_int32),
                ("layers", ctypes.c_int32), ("vocab", ctypes.c_int32), ("eps", ctypes.c_float),
                ("theta", ctypes.c_float), ("rope_llama3", ctypes.c_int32), ("rope_factor", ctypes.c_float),
                ("rope_low_freq_factor", ctypes.c_float), ("rope_high_freq_factor", ctypes.c_float),
                ("rope_original_max_pos", ctypes.c_int32), ("tied_lm_head", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class llama_layer_w(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln1", "wq", "wk", "wv", "wo", "ln2", "w_gate", "w_up", "w_down")]


class llama_weights(ctypes.Structure):
    _fields_ = [("emb", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(llama_layer_w))]


class llama_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("layers", ctypes.c_int32), ("kv", ctypes.c_int32),
                ("head", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class llama_ws(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("bytes", ctypes.c_size_t), ("max_batch", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("max_prefill", ctypes.c_int32), ("cfg_key", ctypes.c_uint32),
                ("magic", ctypes.c_uint32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with llama_architecture_decoder_amd/build.py "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pc, pw, pk, ps = (ctypes.POINTER(llama_cfg), ctypes.POINTER(llama_weights), ctypes.POINTER(llama_kv),
                      ctypes.POINTER(llama_ws))
    L.llama_abi_version.restype = ctypes.c_int
    L.llama_strerror.argtypes = [ctypes.c_int]
    L.llama_strerror.restype = ctypes.c_char_p
    L.llama_kv_cache_bytes.argtypes = [pc, i32, i32]
    L.llama_kv_cache_bytes.restype = i64
    L.kv_cache_alloc.argtypes = [pc, i32, i32, vp, vp, sz, pk]
    L.llama_workspace_bytes.argtypes = [pc, i32, i32, i32]
    L.llama_workspace_bytes.restype = i64
    L.llama_workspace_init.argtypes = [pc, i32, i32, i32, vp, sz, vp, ps]
    L.llama_decode_step.argtypes = [pc, pw, pk, vp, ctypes.POINTER(i32), i32, vp, vp, ps, vp]
    L.llama_trace_floats.argtypes = [pc]
    L.llama_trace_floats.restype = i64
    L.llama_decode_step_traced.argtypes = [pc, pw, pk, vp, ctypes.POINTER(i32), vp, vp, ps, vp, i64, vp]
    L.llama_prefill.argtypes = [pc, pw, pk, i32, vp, i32, i32, vp, vp, ps, vp]
    L.lm_head_argmax.argtypes = [pc, pw, vp, i32, vp, vp, ps, vp]
    L.llama_decode_step_paged.argtypes = [pc, pw, pk, vp, ctypes.POINTER(i32), i32, vp, i32, vp, vp, ps, vp]
    L.llama_generate_until.argtypes = [pc, pw, pk, vp, ctypes.POINTER(i32), i32, i32, i32, vp,
                                       ctypes.POINTER(i32), ps, vp]
    L.llama_prefill_paged.argtypes = [pc, pw, pk, vp, i32, vp, i32, i32, vp, vp, ps, vp]
    L.llama_prefill_packed.argtypes = [pc, pw, pk, vp, i32, vp, i32, vp, vp, vp, vp, vp, ps, vp]
    L.llama_status.argtypes = [ps, vp]
    L.llama_sample_scratch_bytes.argtypes = [i32, i32, i32]
    L.llama_sample_scratch_bytes.restype = i64
    L.llama_sample.argtypes = [vp, i64, i32, i32, ctypes.c_float, i32, ctypes.c_float, vp, ctypes.c_uint32, vp, vp,
                               vp, vp, vp, sz, vp]
    L.llama_sample_noalloc.argtypes = [vp, i64, i32, i32, ctypes.c_float, i32, ctypes.c_float, vp, ctypes.c_uint32,
                                       vp, vp, vp, vp, vp]
    L.llama_profile_enable.argtypes = [ctypes.c_int]
    L.llama_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
    _lib = L
    return L


def _strerror(code: int) -> str:
    try:
        return lib().llama_strerror(code).decode()
    except Exception:  # library missing: still format the error
        return "?"


def _check(rc: int, what: str):
    if rc != OK:
        raise LlamaError(rc, what)


def make_cfg(c) -> llama_cfg:
    """llama_cfg from any object with the Cfg fields (kv, g, half, f, layers, vocab, eps, theta, tied,
    wdtype, kvdtype, rope_llama3, rope_factor, rope_low_freq_factor, rope_high_freq_factor,
    rope_original_max_pos)."""
    return llama_cfg(c.kv, c.g, c.half, c.f, c.layers, c.vocab, float(np.float32(c.eps)), float(np.float32(c.theta)),
                     int(c.rope_llama3), c.rope_factor, c.rope_low_freq_factor, c.rope_high_freq_factor,
                     int(c.rope_original_max_pos), int(c.tied), F32 if c.wdtype == "f32" else BF16,
                     F32 if c.kvdtype == "f32" else BF16)


def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def to_device(a: np.ndarray, device="cuda"):
    """Host array (float32, or uint16 bf16 bits) -> device tensor (float32 / bfloat16)."""
    torch = _torch()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceWeights:
    """Weights in device memory (torch tensors) and the llama_weights record pointing at them."""

    def __init__(self, cfg, host: Dict[str, object], device="cuda"):
        self.cfg = cfg
        self.t: Dict[str, object] = {}
        self.t["emb"] = to_device(host["emb"], device)
        self.t["lnf"] = to_device(host["lnf"], device)
        self.t["lm_head"] = to_device(host["lm_head"], device) if host.get("lm_head") is not None else None
        self.layers: List[Dict[str, object]] = []
        for lw in host["layers"]:
            self.layers.append({k: to_device(v, device) for k, v in lw.items()})
        self._bind()

    def _bind(self):
        n = len(self.layers)
        self._lw = (llama_layer_w * n)()
        names = {"ln1": "ln1", "wq": "wq", "wk": "wk", "wv": "wv", "wo": "wo", "ln2": "ln2", "wg": "w_gate",
                 "wu": "w_up", "wd": "w_down"}
        for l, lw in enumerate(self.layers):
            for k, field in names.items():
                setattr(self._lw[l], field, lw[k].data_ptr())
        self.rec = llama_weights(self.t["emb"].data_ptr(),
                                 self.t["lm_head"].data_ptr() if self.t["lm_head"] is not None else None,
                                 self.t["lnf"].data_ptr(), self._lw)

    def nbytes(self) -> int:
        n = sum(t.numel() * t.element_size() for t in self.t.values() if t is not None)
        for lw in self.layers:
            n += sum(t.numel() * t.element_size() for t in lw.values())
        return n


class KVCache:
    """K and V caches [layers][rows][kv][max_seq][head] in device memory, bound by kv_cache_alloc."""

    def __init__(self, cfg, rows: int, max_seq: int, device="cuda"):
        torch = _torch()
        self.c = make_cfg(cfg)
        nbytes = lib().llama_kv_cache_bytes(ctypes.byref(self.c), rows, max_seq)
        if nbytes < 0:
            raise LlamaError(int(nbytes), "llama_kv_cache_bytes")
        dt = torch.float32 if cfg.kvdtype == "f32" else torch.bfloat16
        shape = (cfg.layers, rows, cfg.kv, max_seq, cfg.head)
        self.k = torch.empty(shape, dtype=dt, device=device)
        self.v = torch.empty(shape, dtype=dt, device=device)
        self.rec = llama_kv()
        _check(lib().kv_cache_alloc(ctypes.byref(self.c), rows, max_seq, self.k.data_ptr(), self.v.data_ptr(),
                                    nbytes, ctypes.byref(self.rec)), "kv_cache_alloc")
        self.rows, self.max_seq = rows, max_seq


class Workspace:
    def __init__(self, cfg, max_batch: int, max_seq: int, max_prefill: int = 0, device="cuda", stream=None):
        torch = _torch()
        self.c = make_cfg(cfg)
        nbytes = lib().llama_workspace_bytes(ctypes.byref(self.c), max_batch, max_seq, max_prefill)
        if nbytes < 0:
            raise LlamaError(int(nbytes), "llama_workspace_bytes")
        self.mem = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
        base = self.mem.data_ptr()
        off = (-base) % 256
        self.rec = llama_ws()
        _check(lib().llama_workspace_init(ctypes.byref(self.c), max_batch, max_seq, max_prefill, base + off,
                                          int(nbytes), _stream_handle(stream), ctypes.byref(self.rec)),
               "llama_workspace_init")


class Decoder:
    """One model on one GPU: weights, a cache of `rows` rows and a workspace, with the C ABI's calls."""

    def __init__(self, cfg, host_weights: Dict[str, object], rows: int = 1, max_seq: Optional[int] = None,
                 max_prefill: int = 0, device="cuda", weights: Optional[DeviceWeights] = None,
                 ws_rows: Optional[int] = None, ws_seq: Optional[int] = None):
        """rows x max_seq: the cache (for a paged cache: rows=1 and max_seq = pool positions); ws_rows and
        ws_seq size the workspace (default: the cache's), e.g. requests per step and their longest
        position + 1 over a page pool."""
        self.cfg = cfg
        self.c = make_cfg(cfg)
        self.max_seq = max_seq or cfg.max_seq
        self.w = weights if weights is not None else DeviceWeights(cfg, host_weights, device)
        self.kv = KVCache(cfg, rows, self.max_seq, device)
        self.ws = Workspace(cfg, ws_rows or rows, ws_seq or self.max_seq, max_prefill, device)
        self.device = device

    # --- calls -----------------------------------------------------------------------------
    def decode(self, tokens, pos: Sequence[int], logits=None, next_tok=None, stream=None) -> None:
        """tokens: device int32 [B]; pos: host ints [B]; logits: device f32 [B][vocab] or None;
        next_tok: device int32 [B] or None (may be `tokens`)."""
        B = len(pos)
        parr = (ctypes.c_int32 * B)(*[int(p) for p in pos])
        rc = lib().llama_decode_step(ctypes.byref(self.c), ctypes.byref(self.w.rec), ctypes.byref(self.kv.rec),
                                     tokens.data_ptr(), parr, B, _ptr(logits), _ptr(next_tok),
                                     ctypes.byref(self.ws.rec), _stream_handle(stream))
        _check(rc, "llama_decode_step")

    def decode_traced(self, tokens, pos: int, logits=None, next_tok=None, stream=None):
        torch = _torch()
        n = int(lib().llama_trace_floats(ctypes.byref(self.c)))
        trace = torch.empty(n, dtype=torch.float32, device=self.device)
        parr = (ctypes.c_int32 * 1)(int(pos))
        rc = lib().llama_decode_step_traced(ctypes.byref(self.c), ctypes.byref(self.w.rec),
                                            ctypes.byref(self.kv.rec), tokens.data_ptr(), parr, _ptr(logits),
                                            _ptr(next_tok), ctypes.byref(self.ws.rec), trace.data_ptr(), n,
                                            _stream_handle(stream))
        _check(rc, "llama_decode_step_traced")
        return trace

    def split_trace(self, trace) -> List[Dict[str, np.ndarray]]:
        cfg = self.cfg
        H, KW, F = cfg.dim, cfg.kvw, cfg.f
        per = 4 * H + 2 * KW + F
        t = trace.cpu().numpy()
        out = []
        for l in range(cfg.layers):
            s = t[l * per:(l + 1) * per]
            o = 0
            d = {}
            for name, w in (("q", H), ("k", KW), ("v", KW), ("attn", H), ("x1", H), ("m", F), ("y", H)):
                d[name] = s[o:o + w]
                o += w
            out.append(d)
        return out

    def prefill(self, tokens, pos0: int = 0, row: int = 0, logits=None, next_tok=None, stream=None) -> None:
        rc = lib().llama_prefill(ctypes.byref(self.c), ctypes.byref(self.w.rec), ctypes.byref(self.kv.rec), row,
                                 tokens.data_ptr(), int(tokens.numel()), pos0, _ptr(logits), _ptr(next_tok),
                                 ctypes.byref(self.ws.rec), _stream_handle(stream))
        _check(rc, "llama_prefill")

    def generate_until(self, token, pos: Sequence[int], max_new: int, eos: int, produced=None, stream=None):
        """Greedy steps from token (device int32 [B]) at positions pos until every row produces eos or max_new
        steps; returns (produced device int32 [max_new][B], steps taken)."""
        torch = _torch()
        B = len(pos)
        if produced is None:
            produced = torch.empty((max_new, B), dtype=torch.int32, device=self.device)
        parr = (ctypes.c_int32 * B)(*[int(p) for p in pos])
        n = ctypes.c_int32(0)
        rc = lib().llama_generate_until(ctypes.byref(self.c), ctypes.byref(self.w.rec), ctypes.byref(self.kv.rec),
                                        token.data_ptr(), parr, B, int(max_new), int(eos), produced.data_ptr(),
                                        ctypes.byref(n), ctypes.byref(self.ws.rec), _stream_handle(stream))
        _check(rc, "llama_generate_until")
        return produced, int(n.value)

    def decode_paged(self, tokens, pos: Sequence[int], table, logits=None, next_tok=None, stream=None) -> None:
        """A step of B requests in a paged cache: cache row 0 is the page pool, request b's positions lie
        in the pages of table[b] (device int32 [B][pages])."""
        B = len(pos)
        parr = (ctypes.c_int32 * B)(*[int(p) for p in pos])
        rc = lib().llama_decode_step_paged(ctypes.byref(self.c), ctypes.byref(self.w.rec), ctypes.byref(self.kv.rec),
                                           tokens.data_ptr(), parr, B, table.data_ptr(), int(table.shape[-1]),
                                           _ptr(logits), _ptr(next_tok), ctypes.byref(self.ws.rec),
                                           _stream_handle(stream))
        _check(rc, "llama_decode_step_paged")

    def prefill_paged(self, tokens, table_row, pos0: int = 0, logits=None, next_tok=None, stream=None) -> None:
        """One request's prompt into the page pool, its pages listed in table_row (device int32 [pages])."""
        rc = lib().llama_prefill_paged(ctypes.byref(self.c), ctypes.byref(self.w.rec), ctypes.byref(self.kv.rec),
                                       table_row.data_ptr(), int(table_row.shape[-1]), tokens.data_ptr(),
                                       int(tokens.numel()), pos0, _ptr(logits), _ptr(next_tok),
                                       ctypes.byref(self.ws.rec), _stream_handle(stream))
        _check(rc, "llama_prefill_paged")

    def prefill_packed(self, tokens, segments, table=None, logits=None, next_tok=None, stream=None) -> None:
        """Several prompts packed end to end in tokens (device int32), segments = [(row, pos0, length)] in
        that order: each writes its own request's cache and attends only over that request.  With table
        (device int32 [len(segments)][pages]) segment s is the paged request of table row s and its row is
        not read.  logits [len(segments)][vocab] / next_tok [len(segments)] get each segment's last-position
        logits and argmax."""
        n = len(segments)
        rows = (ctypes.c_int32 * n)(*[int(r) for r, _, _ in segments])
        pos0 = (ctypes.c_int32 * n)(*[int(p) for _, p, _ in segments])
        lens = (ctypes.c_int32 * n)(*[int(m) for _, _, m in segments])
        rc = lib().llama_prefill_packed(ctypes.byref(self.c), ctypes.byref(self.w.rec), ctypes.byref(self.kv.rec),
                                        _ptr(table), int(table.shape[-1]) if table is not None else 0,
                                        tokens.data_ptr(), n, rows, pos0, lens, _ptr(logits), _ptr(next_tok),
                                        ctypes.byref(self.ws.rec), _stream_handle(stream))
        _check(rc, "llama_prefill_packed")

    def lm_head_argmax(self, hidden, logits=None, argmax=None, stream=None):
        B = hidden.shape[0]
        rc = lib().lm_head_argmax(ctypes.byref(self.c), ctypes.byref(self.w.rec), hidden.data_ptr(), B,
                                  _ptr(logits), _ptr(argmax), ctypes.byref(self.ws.rec), _stream_handle(stream))
        _check(rc, "lm_head_argmax")

    def status(self, stream=None) -> int:
        return int(lib().llama_status(ctypes.byref(self.ws.rec), _stream_handle(stream)))


K_EMBED, K_QKV, K_ATTN, K_O, K_GATE_UP, K_DOWN, K_LM_HEAD, K_SAMPLE, K_QKV_ATTN = range(9)
KERNEL_CLASSES = {"embed": K_EMBED, "qkv": K_QKV, "attention": K_ATTN, "o_proj": K_O, "gate_up": K_GATE_UP,
                  "down": K_DOWN, "lm_head": K_LM_HEAD, "sample": K_SAMPLE, "qkv_attention": K_QKV_ATTN}


def sample_scratch_bytes(B: int, V: int, k: int) -> int:
    n = int(lib().llama_sample_scratch_bytes(B, V, k))
    if n < 0:
        raise LlamaError(n, "llama_sample_scratch_bytes")
    return n


def sample(logits, temp: float, k: int, p: float, seeds=None, draw: int = 0, u=None, ids=None, vals=None,
           topk_ids=None, scratch=None, stream=None):
    """Draw one token per row of `logits` (device F32 [B][V], rows may be strided) with temperature,
    top-k and top-p.  u: device F32 [B] uniforms, or None to draw `draw` of each row's seed (device
    uint32 [B], as int32 tensors).  Returns the ids tensor (device int32 [B]); vals and topk_ids are
    filled when given.  scratch: a device uint8 tensor of sample_scratch_bytes(B, V, k) bytes, or None
    to allocate one."""
    torch = _torch()
    B, V = int(logits.shape[0]), int(logits.shape[1])
    assert logits.dtype == torch.float32 and logits.stride(1) == 1
    if ids is None:
        ids = torch.empty(B, dtype=torch.int32, device=logits.device)
    if scratch is None:
        scratch = torch.empty(max(8, sample_scratch_bytes(B, V, k)), dtype=torch.uint8, device=logits.device)
    rc = lib().llama_sample(logits.data_ptr(), int(logits.stride(0)), B, V, float(temp), int(k), float(p),
                            _ptr(seeds), int(draw) & 0xFFFFFFFF, _ptr(u), ids.data_ptr(), _ptr(vals), _ptr(topk_ids),
                            scratch.data_ptr(), int(scratch.numel()), _stream_handle(stream))
    _check(rc, "llama_sample")
    return ids


def sample_noalloc(logits, temp: float, k: int, p: float, ids, seeds=None, draw: int = 0, u=None, vals=None,
                   topk_ids=None, stream=None):
    """As sample(), through llama_sample_noalloc: the candidates stay in the library's static device
    buffer, so nothing is allocated here or in the library; `ids` (device int32 [B]) is required."""
    B, V = int(logits.shape[0]), int(logits.shape[1])
    rc = lib().llama_sample_noalloc(logits.data_ptr(), int(logits.stride(0)), B, V, float(temp), int(k), float(p),
                                    _ptr(seeds), int(draw) & 0xFFFFFFFF, _ptr(u), ids.data_ptr(), _ptr(vals),
                                    _ptr(topk_ids), _stream_handle(stream))
    _check(rc, "llama_sample_noalloc")
    return ids


def profile_enable(on: bool = True) -> None:
    _check(lib().llama_profile_enable(1 if on else 0), "llama_profile_enable")


def profile_read(kernel_class: int):
    """(launches, summed milliseconds) of one kernel class since profile_enable."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check(lib().llama_profile_read(kernel_class, ctypes.byref(n), ctypes.byref(ms)), "llama_profile_read")
    return int(n.value), float(ms.value)


def _ptr(t):
    return None if t is None else t.data_ptr()


def header_functions() -> List[str]:
    """Names of the functions include/llama_mi355x.h declares."""
    import re
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|int64_t|char\s*\*|const char\s*\*|void)\s*\*?\s*(\w+)\s*\(", txt,
                      flags=re.M)
