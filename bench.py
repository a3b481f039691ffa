#!/usr/bin/env python3
"""Batch-1 decode throughput of the Llama-architecture decoder step on one MI355X, plus roofline.

Workload (the metric's main line): the Llama-3.1-8B-shaped decoder (random-init bf16 weights, F32
arithmetic, bf16 KV cache, MaxSeq 8192) with positions 0..7935 pre-filled with seeded random K/V, then
K greedy decode steps at positions 7936, 7937, ... (K = 256 covers the whole cache).  A step is one
call of llama_decode_step: embedding, 32 layers, final norm, LM head, argmax; the argmax feeds the next
step on the device.  The 1.7B shape (F32, 512-token prompt, 512 decode steps) is measured alongside.

Timing: W untimed warm-up steps, then K steps between two HIP events on the library's stream (with a
device synchronisation on both sides).  A second, profiled pass of the same steps has every kernel
launch record a pair of HIP events from its own dispatch packet (llama_profile_*), which gives the
dominant kernel's (the gate/up GEMV's) average duration for the roofline; `traffic` is the HBM bytes
per launch that rocprofv3 counters measured for the same sources (profiles/decode_8b_hbm_traffic.*).
The CPU oracle is timed on the host on a bounded sample of the same workload.
Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
METRIC = "decode tokens/sec at batch 1 (1.7B & 8B shapes) + % of HBM roofline"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_weight_bytes(cfg):
    d, kw, f = cfg.dim, cfg.kvw, cfg.f
    return (2 * d + 2 * d * d + 2 * kw * d + 3 * f * d) * cfg.wbytes


def token_bytes(cfg, t):
    """Algorithmic HBM bytes of one decode step at position t: every layer matrix and gain, the final
    norm, the LM head (the embedding when tied), one embedding row, K/V rows 0..t-1 read of every layer
    and the K/V row written at t.  Activations are not counted."""
    b = cfg.layers * layer_weight_bytes(cfg) + cfg.dim * cfg.wbytes
    b += cfg.vocab * cfg.dim * cfg.wbytes  # LM head
    b += cfg.dim * cfg.wbytes  # one embedding row
    kvrow = cfg.kvw * cfg.kvbytes
    b += cfg.layers * 2 * kvrow * t  # positions 0..t-1 read (t itself comes from the append)
    b += cfg.layers * 2 * kvrow  # the append at t
    return b


def kernel_bytes(cfg, cls, t=None):
    """Algorithmic bytes of one launch of a kernel class (weights + gains + input + output vectors)."""
    d, kw, f, wb = cfg.dim, cfg.kvw, cfg.f, cfg.wbytes
    if cls == "gate_up":
        return 2 * f * d * wb + d * wb + d * 4 + f * 4
    if cls == "down":
        return d * f * wb + f * 4 + 2 * d * 4
    if cls == "qkv":
        return (d + 2 * kw) * d * wb + d * wb + d * 4 + (d + 2 * kw) * 4
    if cls == "o_proj":
        return d * d * wb + d * 4 + 2 * d * 4
    if cls == "lm_head":
        return cfg.vocab * d * wb + d * wb + d * 4 + cfg.vocab * 4
    if cls == "attention":
        return 2 * kw * cfg.kvbytes * (t + 1) + (d + 2 * kw) * 4 + d * 4
    if cls == "qkv_attention":  # the q/k/v product and the attention in one launch (+ its merge)
        return kernel_bytes(cfg, "qkv", t) + 2 * kw * cfg.kvbytes * t + d * 4
    raise KeyError(cls)


def class_bytes(cfg, name, t, prof):
    """Algorithmic bytes of one launch of a profiled kernel class; the q/k/v + attention launch also carries
    the O product's bytes where the step launched no separate O product (small F32 shapes)."""
    if name == "embed":
        return None
    b = kernel_bytes(cfg, name, t)
    if name == "qkv_attention" and prof.get("o_proj", (0, 0.0))[0] == 0:
        b += kernel_bytes(cfg, "o_proj", t)
    return b


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_8b_hbm_traffic.json")


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, scaled
    by a plain copy of known size; None when the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = hashlib.sha256()
        for p in rec["sources"]:
            h.update(open(os.path.join(ROOT, p), "rb").read())
        if h.hexdigest()[:16] != rec["sources_sha256_16"]:
            return None
        return int(rec["per_launch"][kernel]["traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def build_model(cfg, lm, synth, max_seq, fill, keep_host):
    import numpy as np
    import torch
    t0 = time.time()
    w = synth.make_weights(cfg)
    log(f"{cfg.name}: weights generated in {time.time() - t0:.1f}s")
    dec = lm.Decoder(cfg, w, rows=1, max_seq=max_seq)
    log(f"{cfg.name}: weights on device ({dec.w.nbytes() / 1e9:.2f} GB)")
    kc = vc = None
    if fill:
        kt = np.float32 if cfg.kvdtype == "f32" else np.uint16
        shape = (cfg.layers, 1, cfg.kv, max_seq, cfg.head)
        kc = np.zeros(shape, dtype=kt)
        vc = np.zeros(shape, dtype=kt)
        synth.fill_cache_rows(cfg, kc, vc, 0, fill)
        for host, devt in ((kc, dec.kv.k), (vc, dec.kv.v)):
            if host.dtype == np.uint16:
                devt.view(torch.int16).copy_(torch.from_numpy(host.view(np.int16)))
            else:
                devt.copy_(torch.from_numpy(host))
        torch.cuda.synchronize()
        log(f"{cfg.name}: cache rows 0..{fill - 1} filled")
    if not keep_host:
        w = None
    return dec, w, kc, vc


def time_decode(dec, cfg, p0, steps, warmup, first_tok, profile=False):
    import torch
    lm = sys.modules["llama_architecture_decoder_amd"]
    tok = torch.tensor([first_tok], dtype=torch.int32, device="cuda")
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    for i in range(warmup):
        dec.decode(tok, [p0 + i], logits, tok)
    torch.cuda.synchronize()
    tok.fill_(first_tok)
    torch.cuda.synchronize()
    if profile:
        lm.profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        dec.decode(tok, [p0 + i], logits, tok)
    e1.record()
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    if dec.status() != 0:
        raise RuntimeError("device status flag set during the timed steps")
    prof = {}
    if profile:
        for name, cls in lm.KERNEL_CLASSES.items():
            n, ms = lm.profile_read(cls)
            prof[name] = (n, ms)
        lm.profile_enable(False)
    return e0.elapsed_time(e1), (h1 - h0) * 1e3, prof


def batched_step_bytes(cfg, positions):
    """Algorithmic HBM bytes of one batched decode step: the weights once, one embedding row per row,
    and every row's K/V reads (positions 0..t-1) and append."""
    b = token_bytes(cfg, 0) - cfg.dim * cfg.wbytes - cfg.layers * 2 * cfg.kvw * cfg.kvbytes
    kvrow = cfg.kvw * cfg.kvbytes
    for t in positions:
        b += cfg.dim * cfg.wbytes + cfg.layers * 2 * kvrow * (int(t) + 1)
    return b


def time_batched(cfg, lm, synth, dev_weights, steps, warmup):
    """Batch-`cfg.batch` decode: every row pre-filled (on the device) to its own random length, then
    `steps` greedy steps of all rows together."""
    import numpy as np
    import torch
    B = cfg.batch
    lens = synth.row_lengths(cfg).astype(np.int64)
    dec = lm.Decoder(cfg, None, rows=B, max_seq=cfg.max_seq, weights=dev_weights)
    log(f"{cfg.name}: cache {2 * dec.kv.k.numel() * dec.kv.k.element_size() / 1e9:.1f} GB; filling rows to "
        f"lengths {int(lens.min())}..{int(lens.max())}")
    t0 = time.time()
    synth.fill_cache_device(cfg, dec.kv.k.data_ptr(), dec.kv.v.data_ptr(), B, cfg.max_seq, lens,
                            stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    log(f"{cfg.name}: filled in {time.time() - t0:.1f}s")
    first = torch.from_numpy(synth.tokens(cfg, "bench/rows", B)).cuda()
    tok = first.clone()
    for i in range(warmup):
        dec.decode(tok, [int(p) + i for p in lens], None, tok)
    torch.cuda.synchronize()
    tok.copy_(first)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        dec.decode(tok, [int(p) + i for p in lens], None, tok)
    e1.record()
    torch.cuda.synchronize()
    if dec.status() != 0:
        raise RuntimeError("device status flag set during the batched steps")
    ms = e0.elapsed_time(e1) / steps
    bytes_step = sum(batched_step_bytes(cfg, lens + i) for i in range(steps)) / steps
    out = {"workload": f"{cfg.name}: llama31_8b-shaped decode, batch {B} rows, bf16 weights and KV, MaxSeq "
                       f"{cfg.max_seq}, row lengths uniform in [{cfg.len_lo}, {cfg.len_hi}] (pre-filled random), "
                       f"{steps} steps", "value": round(B * 1e3 / ms, 2), "unit": "tokens/s",
           "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
           "dtype": "bf16 matrix-core products (f32 activations as hi + lo), f32 accumulation",
           "hbm_fraction": round(bytes_step / (ms * 1e-3) / HBM_PEAK, 4), "bytes_per_step": int(bytes_step),
           "row_lengths": [int(lens.min()), int(lens.max())]}
    del dec
    torch.cuda.empty_cache()
    return out


def prefill_flops(cfg, S, pos0=0):
    """Algorithmic FLOPs of a prefill of S positions: 2 per multiply-add of every layer product for every
    position, causal attention (scores and weighted sum, 4 * head per visible key per query head), and
    the LM head of the last position."""
    d, kw, f = cfg.dim, cfg.kvw, cfg.f
    mats = 2 * d * d + 2 * kw * d + 3 * f * d
    keys = sum(pos0 + i + 1 for i in range(S))
    att = 4 * cfg.head * cfg.heads * keys
    return cfg.layers * (2 * S * mats + att) + 2 * cfg.vocab * d


MFMA_BF16_PEAK = 2.5e15  # MI355X dense bf16 matrix-core peak, FLOP/s


def time_prefill(cfg, lm, synth, dev_weights, reps, warmup):
    """Prefill of a `cfg.prompt_len`-position random prompt into a fresh cache row (MaxSeq cfg.max_seq)."""
    import torch
    S = cfg.prompt_len
    dec = lm.Decoder(cfg, None, rows=1, max_seq=cfg.max_seq, max_prefill=S, weights=dev_weights)
    toks = torch.from_numpy(synth.tokens(cfg, "bench/prompt", S)).cuda()
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        dec.prefill(toks, pos0=0, next_tok=nxt)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dec.prefill(toks, pos0=0, next_tok=nxt)
    e1.record()
    torch.cuda.synchronize()
    if dec.status() != 0:
        raise RuntimeError("device status flag set during the prefill")
    ms = e0.elapsed_time(e1) / reps
    lm.profile_enable(True)
    dec.prefill(toks, pos0=0, next_tok=nxt)
    torch.cuda.synchronize()
    kernels = {}
    for name, cls in lm.KERNEL_CLASSES.items():
        n, kms = lm.profile_read(cls)
        if n:
            kernels[name] = {"launches": n, "ms": round(kms, 3)}
    lm.profile_enable(False)
    ksum = sum(k["ms"] for k in kernels.values())
    for k in kernels.values():
        k["share"] = round(k["ms"] / ksum, 4)  # of the summed launch time of the profiled prefill
    fl = prefill_flops(cfg, S)
    # the products: the largest share of the time; matrix-core work per launch counted algorithmically
    d, kw, f = cfg.dim, cfg.kvw, cfg.f
    gu = kernels.get("gate_up")
    gu_flops = 2 * S * 2 * f * d
    out = {"workload": f"{cfg.name}: prefill of a {S}-position random prompt at positions 0..{S - 1} of a fresh "
                       f"cache row (MaxSeq {cfg.max_seq}), bf16 weights and KV, F32 activations",
           "value": round(S * 1e3 / ms, 1), "unit": "tokens/s", "ms_per_prefill": round(ms, 3), "reps": reps,
           "warmup": warmup, "dtype": "bf16 matrix-core products (f32 activations as hi + lo), f32 accumulation",
           "flops": fl, "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
           "mfma_fraction": round(fl / (ms * 1e-3) / MFMA_BF16_PEAK, 4), "kernels": kernels}
    if gu:
        per = gu["ms"] / gu["launches"] * 1e-3
        out["roofline"] = {"bound": "mfma", "kernel": "split + k_gemm_big<SwiGLU> (gate+up, 256x256 tiles)",
                           "achieved": round(gu_flops / per / 1e12, 1), "peak": MFMA_BF16_PEAK / 1e12,
                           "unit": "TFLOP/s", "frac": round(gu_flops / per / MFMA_BF16_PEAK, 4),
                           "flops_per_launch": gu_flops, "avg_launch_us": round(per * 1e6, 1),
                           "note": "algorithmic FLOPs; the products run twice (bf16 hi and lo of the F32 "
                                   "activations), so executed matrix-core work is 2x; a register-only "
                                   "probe of this instruction sustains 2.0-2.2 PFLOP/s on this GPU"}
    del dec
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def omp_threads(n):
    """Set the OpenMP thread count of the oracle's parallel loops (libgomp, loaded with the oracle)."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def cpu_baseline(cfg, w, kc, vc, p0, first_tok, budget_s):
    """The oracle's greedy decode on the host, on all usable cores and then on one (the pages' table has
    a 1-thread and a 16-thread column), each for about budget_s seconds of wall clock."""
    import oracle
    om = oracle.Model(cfg, w, rows=1, max_seq=kc.shape[3], alloc_cache=False)
    om.kc, om.vc = kc, vc
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))

    def run(threads, start_pos):
        omp_threads(threads)
        tok, n, t0 = first_tok, 0, time.perf_counter()
        while True:
            tok, _, _, _ = om.decode(tok, start_pos + n)
            n += 1
            el = time.perf_counter() - t0
            log(f"oracle ({threads} threads) step {n} at position {start_pos + n - 1}: {el:.1f}s")
            if el >= budget_s:
                return n, el

    n, el = run(cores, p0)
    # the one-core leg starts where the first left off in the cache, at the same positions' depth
    n1, el1 = run(1, p0)
    omp_threads(cores)
    return {"value": n / el, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{cfg.name}: first {n} greedy decode steps at positions {p0}..{p0 + n - 1} "
                      f"(same weights and pre-filled cache as the GPU run), {el:.1f}s wall",
            "one_core": {"value": n1 / el1, "unit": "tokens/s", "cores": 1,
                         "sample": f"first {n1} greedy decode steps at positions {p0}..{p0 + n1 - 1}, "
                                   f"{el1:.1f}s wall"}}


def time_secondary(args, lm, synth, configs, c3=None):
    """A batch-1 F32 workload (default the 1.7B shape): its prompt, then its timed greedy steps, then a
    profiled pass."""
    import torch
    c3 = c3 or configs.SMOLLM2_1_7B
    dec3, _, _, _ = build_model(c3, lm, synth, c3.max_seq, 0, keep_host=False)
    prompt = torch.from_numpy(synth.tokens(c3, "bench/prompt", c3.prompt_len)).cuda()
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    dec3.prefill(prompt, pos0=0, next_tok=nxt)
    torch.cuda.synchronize()
    s3 = min(c3.decode_steps, args.secondary_steps or c3.decode_steps)
    ev3, _, _ = time_decode(dec3, c3, c3.prompt_len, s3, args.warmup, int(nxt.item()))
    ms3 = ev3 / s3
    pev3, _, prof3 = time_decode(dec3, c3, c3.prompt_len, s3, 0, int(nxt.item()), profile=True)
    b3 = sum(token_bytes(c3, c3.prompt_len + i) for i in range(s3)) / s3
    mean3 = c3.prompt_len + (s3 - 1) // 2
    k3 = {}
    ksum3 = sum(kms for n, kms in prof3.values() if n)
    for name, (n, kms) in prof3.items():
        if n:
            per = kms / n
            kb = class_bytes(c3, name, mean3, prof3)
            k3[name] = {"launches": n, "avg_us": round(per * 1e3, 3), "share": round(kms / ksum3, 4),
                        "GBps": round(kb / (per * 1e-3) / 1e9, 1) if kb else None}
    res3 = {"workload": f"{c3.name}-shaped decode, batch 1, F32, {c3.prompt_len}-token prompt "
                                       f"then {s3} steps at positions {c3.prompt_len}..{c3.prompt_len + s3 - 1}",
                           "value": round(1e3 / ms3, 2), "unit": "tokens/s", "ms_per_step": round(ms3, 4),
                           "dtype": "f32", "hbm_fraction": round(b3 / (ms3 * 1e-3) / HBM_PEAK, 4),
                           "bytes_per_token": int(b3), "kernels": k3}
    log(f"{c3.name}: {1e3 / ms3:.1f} tok/s")
    del dec3
    torch.cuda.empty_cache()
    return res3


def time_serving(cfg, lm, synth, dev_weights, n_req=256, conc=64, pmin=128, pmax=512, new=128, pass_tokens=2048):
    """Continuous batching over a paged cache (the pages' serving workload): n_req requests with prompts of
    uniform random length in [pmin, pmax] and `new` greedy tokens each, at most `conc` in flight.  Each
    request gets a slot; the prompts of all requests admitted at one step (every free slot takes the next
    request) run as one llama_prefill_packed call over the page pool, packed end to end (the argmax after
    each prompt is its first new token, scattered into the slots' entries of the device token array); then
    every step runs llama_decode_step_paged over all slots (idle ones at position 0 of a scratch page).
    Pages (64 positions) come from a free list when a prompt is admitted and when a row reaches a new page,
    and go back when its request finishes; page tables and slot lists reach the device from rings of
    pinned host buffers, so the host never waits for the GPU.  Tokens/s = n_req * new / (time from the
    first admission to the last step)."""
    import numpy as np
    import torch
    PAGE = lm.PAGE_SIZE
    per_req = (pmax + new + PAGE - 1) // PAGE
    npool = conc * per_req + 1  # page 0: the idle slots' scratch page
    dec = lm.Decoder(cfg, None, rows=1, max_seq=npool * PAGE, max_prefill=pass_tokens, weights=dev_weights,
                     ws_rows=conc, ws_seq=per_req * PAGE)
    lens = synth.int_range("serve/prompt_lens", n_req, pmin, pmax).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)])
    prompts = torch.from_numpy(np.concatenate([synth.tokens(cfg, f"serve/prompt/{r}", int(lens[r]))
                                               for r in range(n_req)])).cuda()
    tokens = torch.zeros(conc, dtype=torch.int32, device="cuda")
    first = torch.zeros(conc, dtype=torch.int32, device="cuda")
    table = np.zeros((conc, per_req), dtype=np.int32)
    table_dev = torch.zeros((conc, per_req), dtype=torch.int32, device="cuda")
    ptable_dev = torch.zeros((conc, per_req), dtype=torch.int32, device="cuda")  # admitted requests' rows
    slots_dev = torch.zeros(conc, dtype=torch.int64, device="cuda")

    class Ring:
        """Pinned host buffers for host-to-device copies that never make the host wait for the GPU."""

        def __init__(self, shape, dtype, n=8):
            self.buf = [torch.empty(shape, dtype=dtype, pin_memory=True) for _ in range(n)]
            self.ev = [None] * n
            self.i = 0

        def put(self, dst, src):
            i = self.i % len(self.buf)
            self.i += 1
            if self.ev[i] is not None:
                self.ev[i].synchronize()
            b = self.buf[i].numpy()
            b[...] = 0
            b[:src.shape[0]] = src
            dst.copy_(self.buf[i], non_blocking=True)
            self.ev[i] = torch.cuda.Event()
            self.ev[i].record()

    tables, ptables, slot_lists = (Ring((conc, per_req), torch.int32), Ring((conc, per_req), torch.int32),
                                   Ring(conc, torch.int64))

    def upload():
        tables.put(table_dev, table)

    free = list(range(1, npool))
    req = [-1] * conc
    pos = [0] * conc
    gen = [0] * conc
    pages = [[] for _ in range(conc)]
    nxt, done, steps, prefills = 0, 0, 0, 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    e0.record()
    while done < n_req:
        changed = False
        adm = []
        for s in range(conc):
            if req[s] < 0 and nxt < n_req:
                r, L = nxt, int(lens[nxt])
                nxt += 1
                need = (L + PAGE - 1) // PAGE
                pages[s] = [free.pop() for _ in range(need)]
                table[s, :] = 0
                table[s, :need] = pages[s]
                req[s], pos[s], gen[s] = r, L, 1
                adm.append(s)
        if adm:
            # the admitted requests are consecutive, so their prompts are one range of the packed array
            upload()
            ptables.put(ptable_dev, table[adm])
            slot_lists.put(slots_dev, np.asarray(adm, dtype=np.int64))
            r0, r1 = req[adm[0]], req[adm[-1]] + 1
            dec.prefill_packed(prompts[offs[r0]:offs[r1]], [(0, 0, int(lens[req[s]])) for s in adm],
                               table=ptable_dev[:len(adm)], next_tok=first)
            tokens.index_copy_(0, slots_dev[:len(adm)], first[:len(adm)])
            prefills += 1
        for s in range(conc):
            if req[s] >= 0 and pos[s] // PAGE >= len(pages[s]):
                pages[s].append(free.pop())
                table[s, len(pages[s]) - 1] = pages[s][-1]
                changed = True
        if changed:
            upload()
        dec.decode_paged(tokens, [pos[s] if req[s] >= 0 else 0 for s in range(conc)], table_dev, None, tokens)
        steps += 1
        for s in range(conc):
            if req[s] < 0:
                continue
            pos[s] += 1
            gen[s] += 1
            if gen[s] == new:
                free.extend(pages[s])
                pages[s] = []
                table[s, :] = 0
                req[s] = -1
                done += 1
    e1.record()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    if dec.status() != 0:
        raise RuntimeError("device status flag set during the serving run")
    gpu_s = e0.elapsed_time(e1) * 1e-3
    out = {"workload": f"{n_req} requests, prompts uniform in [{pmin}, {pmax}] tokens, {new} greedy new tokens each, "
                       f"at most {conc} in flight; paged bf16 cache ({npool} pages of {PAGE}); {cfg.name} shape",
           "value": round(n_req * new / gpu_s, 1), "unit": "tokens/s", "seconds": round(gpu_s, 3),
           "host_seconds": round(host_s, 3), "decode_steps": steps, "prefill_calls": prefills,
           "prefill_pass_tokens": pass_tokens,
           "prompt_tokens": int(lens.sum())}
    log(f"serving: {out['value']} tok/s ({gpu_s:.2f} s, {steps} steps)")
    del dec, prompts
    torch.cuda.empty_cache()
    return out


def time_long_context(cfg, lm, synth, dev_weights, steps=8, max_seq=131072):
    """Batch-1 decode at the end of the full rope-scaled context: positions max_seq - steps .. max_seq - 1
    of a max_seq cache whose earlier positions hold seeded random keys and values (filled on the device).
    Bytes per token: all weights, the LM head and the K/V rows read (~33 GB at the 8B shape)."""
    import torch
    dec = lm.Decoder(cfg, None, rows=1, max_seq=max_seq, weights=dev_weights)
    p0 = max_seq - steps
    synth.fill_cache_device(cfg, dec.kv.k.data_ptr(), dec.kv.v.data_ptr(), 1, max_seq, [p0])
    torch.cuda.synchronize()
    first = int(synth.tokens(cfg, "bench/long", 1)[0])
    ev_ms, _, _ = time_decode(dec, cfg, p0, steps, 1, first)
    # the warm-up step wrote position p0; the timed steps rewrite p0 .. max_seq - 1
    ms = ev_ms / steps
    b = sum(token_bytes(cfg, p0 + i) for i in range(steps)) / steps
    out = {"workload": f"{cfg.name}-shaped decode, batch 1, bf16, positions {p0}..{max_seq - 1} of MaxSeq {max_seq} "
                       f"(0..{p0 - 1} pre-filled random)", "value": round(1e3 / ms, 2), "unit": "tokens/s",
           "ms_per_step": round(ms, 4), "bytes_per_token": int(b),
           "hbm_fraction": round(b / (ms * 1e-3) / HBM_PEAK, 4)}
    log(f"long context: {out['value']} tok/s, hbm {out['hbm_fraction']}")
    del dec
    torch.cuda.empty_cache()
    return out


def time_sample(lm, vocab, reps=200):
    """Sampling (temperature 0.6, top-k 50, top-p 0.9) over synthetic F32 logits resident in HBM, for 1
    and 64 rows of the vocabulary.  The time per call is the span from the start of its first kernel to
    the end of its second, from HIP events recorded in the dispatch packets (llama_profile), so host
    launch overhead between calls is not counted."""
    import torch
    out = {"workload": f"sampling over [B][{vocab}] F32 logits: temperature 0.6, top-k 50, top-p 0.9, "
                       f"seeded draws", "rows": {}}
    for B in (1, 64):
        g = torch.Generator(device="cuda").manual_seed(1234 + B)
        logits = torch.randn((B, vocab), generator=g, device="cuda") * 3.0
        seeds = torch.arange(B, dtype=torch.int32, device="cuda")
        ids = torch.empty(B, dtype=torch.int32, device="cuda")
        scratch = torch.empty(lm.sample_scratch_bytes(B, vocab, 50), dtype=torch.uint8, device="cuda")
        for i in range(5):
            lm.sample(logits, 0.6, 50, 0.9, seeds=seeds, draw=i, ids=ids, scratch=scratch)
        torch.cuda.synchronize()
        lm.profile_enable(True)
        for i in range(reps):
            lm.sample(logits, 0.6, 50, 0.9, seeds=seeds, draw=i, ids=ids, scratch=scratch)
        torch.cuda.synchronize()
        n, ms = lm.profile_read(lm.K_SAMPLE)
        lm.profile_enable(False)
        us = ms * 1e3 / n
        nbytes = B * vocab * 4
        out["rows"][str(B)] = {"us_per_call": round(us, 2), "logit_bytes": nbytes,
                               "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                               "hbm_fraction": round(nbytes / (us * 1e-6) / HBM_PEAK, 4)}
        log(f"sampling B={B}: {us:.2f} us per call (GPU)")
        del logits, scratch
    torch.cuda.empty_cache()
    return out


def copy_probe():
    """Three copies of a 1 GiB buffer (a plain copy kernel of known size, for calibrating HBM counters)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    return n


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the 4096-position prefill (for profiling its kernels)")
    ap.add_argument("--batched-only", action="store_true",
                    help="time only the batch-32 long-context decode (for profiling its kernels)")
    ap.add_argument("--small-only", nargs="?", const="both", choices=["both", "135m", "360m"],
                    help="only the small shapes (135M and 360M decode, or the one named)")
    ap.add_argument("--secondary-only", action="store_true",
                    help="time only the 1.7B-shaped decode (for profiling its kernels)")
    ap.add_argument("--long-only", action="store_true",
                    help="time only the batch-1 decode at the end of a 131072-position cache")
    ap.add_argument("--serving-only", action="store_true",
                    help="time only the paged continuous-batching workload (for profiling its kernels)")
    ap.add_argument("--sample-only", action="store_true",
                    help="time only sampling over the 8B vocabulary (for profiling its kernels)")
    ap.add_argument("--secondary-steps", type=int, default=0,
                    help="decode steps of the F32 workloads (default: each workload's own count)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the decode steps, copy a 1 GiB buffer 3 times (counter calibration: a plain "
                         "copy kernel of known size)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: it measures the single-GPU decode step "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    import llama_architecture_decoder_amd as lm
    import synth
    from synth import configs

    torch.cuda.set_device(0)
    cfg = configs.LLAMA31_8B
    p0 = cfg.kv_fill
    steps = max(1, min(args.steps, cfg.max_seq - p0))
    want_cpu = not args.no_cpu_baseline
    def emit(d):
        if args.copy_probe:
            d["copy_probe_bytes"] = copy_probe()
        print(json.dumps(d), flush=True)

    if args.secondary_only:
        emit({"secondary": time_secondary(args, lm, synth, configs)})
        return
    if args.small_only:
        shapes = {"135m": [configs.SMOLLM2_135M], "360m": [configs.SMOLLM2_360M],
                  "both": [configs.SMOLLM2_135M, configs.SMOLLM2_360M]}[args.small_only]
        emit({"small_shapes": [time_secondary(args, lm, synth, configs, c) for c in shapes]})
        return
    if args.sample_only:
        emit({"sampling": time_sample(lm, cfg.vocab)})
        return
    if args.long_only:
        dec, _, _, _ = build_model(cfg, lm, synth, 16, 0, keep_host=False)
        emit({"long_context": time_long_context(cfg, lm, synth, dec.w)})
        return
    if args.serving_only:
        dec, _, _, _ = build_model(cfg, lm, synth, 16, 0, keep_host=False)
        emit({"serving": time_serving(cfg, lm, synth, dec.w)})
        return
    if args.prefill_only or args.batched_only:
        dec, _, _, _ = build_model(cfg, lm, synth, 16, 0, keep_host=False)
        c5 = configs.LLAMA31_8B_LONG
        if args.prefill_only:
            emit({"prefill": time_prefill(c5, lm, synth, dec.w, 2, 1)})
        else:
            emit({"batched": time_batched(c5, lm, synth, dec.w, min(args.steps, c5.decode_steps), args.warmup)})
        return
    dec, w, kc, vc = build_model(cfg, lm, synth, cfg.max_seq, p0, keep_host=want_cpu)
    first = int(synth.tokens(cfg, "bench/first", 1)[0])

    log(f"timed: {steps} steps at positions {p0}..{p0 + steps - 1} after {args.warmup} warm-up steps")
    ev_ms, host_ms, _ = time_decode(dec, cfg, p0, steps, args.warmup, first)
    ms_step = ev_ms / steps
    tok_s = 1e3 / ms_step
    log(f"{tok_s:.1f} tok/s ({ms_step:.3f} ms/step; host clock {host_ms / steps:.3f} ms/step)")
    log("profiled pass (events around every launch)")
    pev_ms, _, prof = time_decode(dec, cfg, p0, steps, 0, first, profile=True)
    mean_t = p0 + (steps - 1) / 2.0
    bytes_tok = sum(token_bytes(cfg, p0 + i) for i in range(steps)) / steps
    hbm_frac = bytes_tok / (ms_step * 1e-3) / HBM_PEAK

    kernels = {}
    ksum = sum(ms for n, ms in prof.values() if n)
    for name, (n, ms) in prof.items():
        if n == 0:
            continue
        per = ms / n
        kb = class_bytes(cfg, name, int(mean_t), prof)
        kernels[name] = {"launches": n, "avg_us": round(per * 1e3, 3), "share": round(ms / ksum, 4),
                         "GBps": round(kb / (per * 1e-3) / 1e9, 1) if kb else None}
    dom = "gate_up"
    n, ms = prof[dom]
    avg_s = ms / n * 1e-3
    ach = kernel_bytes(cfg, dom) / avg_s
    roofline = {"bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK, 4), "traffic": measured_traffic("gate_up"),
                "kernel": "k_gemv<bf16, SwiGLU> (gate+up)",
                "scope": "the dominant kernel alone; the whole step's fraction of the HBM peak is hbm_fraction",
                "bytes_per_launch": kernel_bytes(cfg, dom), "avg_launch_us": round(avg_s * 1e6, 3)}

    result = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "storage_dtype": "bf16 weights and KV cache", "data": "synthetic",
        "config": {"workload": f"llama31_8b-shaped decode, batch 1, bf16 weights and KV, F32 arithmetic, "
                               f"positions {p0}..{p0 + steps - 1} of MaxSeq {cfg.max_seq} (0..{p0 - 1} "
                               f"pre-filled random)", "batch": 1, "positions": [p0, p0 + steps - 1],
                   "max_seq": cfg.max_seq, "hidden": cfg.dim, "layers": cfg.layers, "vocab": cfg.vocab},
        "hbm_fraction": round(hbm_frac, 4), "bytes_per_token": int(bytes_tok),
        "host_ms_per_step": round(host_ms / steps, 4),
        "roofline": roofline, "kernels": kernels,
        "kernel_share_basis": "each kernel class's summed launch time over the summed time of all launches, "
                              "from a second pass whose launches record HIP events in their dispatch packets",
        "profiled_ms_per_step": round(pev_ms / steps, 4),
    }
    if not args.no_secondary:
        c5 = configs.LLAMA31_8B_LONG
        result["batched"] = time_batched(c5, lm, synth, dec.w, c5.decode_steps, args.warmup)
        log(f"batch {c5.batch}: {result['batched']['value']:.1f} tok/s, hbm {result['batched']['hbm_fraction']:.3f}")
        result["prefill"] = time_prefill(c5, lm, synth, dec.w, 3, 1)
        log(f"prefill {c5.prompt_len}: {result['prefill']['ms_per_prefill']:.1f} ms, "
            f"{result['prefill']['tflops']:.0f} TFLOP/s")
        result["sampling"] = time_sample(lm, cfg.vocab)
        result["serving"] = time_serving(cfg, lm, synth, dec.w)
        result["long_context"] = time_long_context(cfg, lm, synth, dec.w)
    del dec
    torch.cuda.empty_cache()
    if args.copy_probe:
        result["copy_probe_bytes"] = copy_probe()

    if want_cpu:
        log(f"cpu baseline: oracle on {cfg.name}, ~{args.cpu_seconds:.0f}s sample")
        result["cpu_baseline"] = cpu_baseline(cfg, w, kc, vc, p0, first, args.cpu_seconds)
    w = kc = vc = None

    if not args.no_secondary:
        result["secondary"] = time_secondary(args, lm, synth, configs)
        # the two small shapes of the pages' table, for completeness (launch-bound at these sizes)
        result["small_shapes"] = [time_secondary(args, lm, synth, configs, c)
                                  for c in (configs.SMOLLM2_135M, configs.SMOLLM2_360M)]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
