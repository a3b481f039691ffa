"""Model shapes and workloads of the synthetic Llama-architecture decoders.

Shapes follow the pages' configs: `Cfg{kv, g, half, f, layers, vocab, eps, theta}` from bend-ml-llama
(main.bend, "The configuration": smollm2_135m / smollm2_360m / smollm2_1_7b) and the Llama-3.1-8B
model card (nest, README and `crate.rope` constants).  Workloads (prompt lengths, decode steps, cache
sizes, pre-filled positions) are the synthetic stand-ins for the pages' measurements; the weights are
random-init (N(0, 0.02) matrices, 1 + N(0, 0.02) norm gains), never checkpoints.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional


@dataclasses.dataclass(frozen=True)
class Cfg:
    name: str
    kv: int          # key/value heads
    g: int           # query heads per key/value head
    half: int        # half a head
    f: int           # MLP inner width
    layers: int
    vocab: int
    eps: float
    theta: float
    tied: bool       # LM head = embedding
    wdtype: str      # "f32" | "bf16" (weights, norm gains, embedding, LM head)
    kvdtype: str     # "f32" | "bf16" (KV cache)
    max_seq: int     # cache positions per row
    rope_llama3: bool = False
    rope_factor: float = 8.0
    rope_low_freq_factor: float = 1.0
    rope_high_freq_factor: float = 4.0
    rope_original_max_pos: int = 8192
    # workload
    prompt_len: int = 0          # prompt prefilled from position 0 (random ids)
    decode_steps: int = 0        # greedy decode steps after the prompt / pre-filled positions
    kv_fill: int = 0             # positions 0..kv_fill-1 pre-filled with random K/V (batch-1 rows)
    batch: int = 1               # decode rows
    len_lo: int = 0              # batched decode: row lengths uniform in [len_lo, len_hi]
    len_hi: int = 0
    family: str = ""             # weight streams are keyed by family, so shapes that share weights
                                 # (the 8B batch workload, truncated copies) draw the same numbers

    @property
    def weights_key(self) -> str:
        return self.family or self.name

    # derived sizes (main.bend: head = 2*half, heads = kv*g, dim = heads*head, kvw = kv*head)
    @property
    def head(self) -> int:
        return 2 * self.half

    @property
    def heads(self) -> int:
        return self.kv * self.g

    @property
    def dim(self) -> int:
        return self.heads * self.head

    @property
    def kvw(self) -> int:
        return self.kv * self.head

    @property
    def wbytes(self) -> int:
        return 4 if self.wdtype == "f32" else 2

    @property
    def kvbytes(self) -> int:
        return 4 if self.kvdtype == "f32" else 2

    def layer_values(self) -> int:
        """Values of one layer: two norms, q and o (dim x dim), k and v (kvw x dim), gate/up/down."""
        d, kw, f = self.dim, self.kvw, self.f
        return 2 * d + 2 * d * d + 2 * kw * d + 3 * f * d

    def model_values(self) -> int:
        """Embedding + layers + final norm (+ a separate LM head when untied)."""
        n = self.vocab * self.dim + self.layers * self.layer_values() + self.dim
        if not self.tied:
            n += self.vocab * self.dim
        return n

    def kv_random_amplitude(self) -> float:
        """Half-width a of the uniform fill U(-a, a) for pre-filled cache rows: the standard deviation
        of a fresh projection of a unit-RMS vector by N(0, 0.02) weights is 0.02*sqrt(dim), and
        U(-a, a) has standard deviation a/sqrt(3)."""
        return math.sqrt(3.0) * 0.02 * math.sqrt(self.dim)

    def replace(self, **kw) -> "Cfg":
        return dataclasses.replace(self, **kw)


SMOLLM2_135M = Cfg("smollm2_135m", kv=3, g=3, half=32, f=1536, layers=30, vocab=49152, eps=1e-5,
                   theta=10000.0, tied=True, wdtype="f32", kvdtype="f32", max_seq=2048,
                   prompt_len=8, decode_steps=16)
SMOLLM2_360M = Cfg("smollm2_360m", kv=5, g=3, half=32, f=2560, layers=32, vocab=49152, eps=1e-5,
                   theta=100000.0, tied=True, wdtype="f32", kvdtype="f32", max_seq=2048,
                   prompt_len=128, decode_steps=256)
SMOLLM2_1_7B = Cfg("smollm2_1_7b", kv=32, g=1, half=32, f=8192, layers=24, vocab=49152, eps=1e-5,
                   theta=130000.0, tied=True, wdtype="f32", kvdtype="f32", max_seq=8192,
                   prompt_len=512, decode_steps=512)
LLAMA31_8B = Cfg("llama31_8b", kv=8, g=4, half=64, f=14336, layers=32, vocab=128256, eps=1e-5,
                 theta=500000.0, tied=False, wdtype="bf16", kvdtype="bf16", max_seq=8192,
                 rope_llama3=True, kv_fill=7936, decode_steps=256)
LLAMA31_8B_LONG = LLAMA31_8B.replace(name="llama31_8b_long", family="llama31_8b", max_seq=32768, kv_fill=0, prompt_len=4096,
                                     decode_steps=128, batch=32, len_lo=8192, len_hi=32000)

CONFIGS = {c.name: c for c in (SMOLLM2_135M, SMOLLM2_360M, SMOLLM2_1_7B, LLAMA31_8B, LLAMA31_8B_LONG)}

# small shapes for brute-force checks and ragged-tail tests (not workloads of the pages)
TINY = Cfg("tiny", kv=2, g=2, half=4, f=16, layers=2, vocab=32, eps=1e-5, theta=10000.0, tied=True,
           wdtype="f32", kvdtype="f32", max_seq=64, prompt_len=5, decode_steps=6)
TINY_BF16 = TINY.replace(name="tiny_bf16", tied=False, wdtype="bf16", kvdtype="bf16", rope_llama3=True,
                         theta=500000.0)


def get(name: str) -> Cfg:
    if name in CONFIGS:
        return CONFIGS[name]
    if name == "tiny":
        return TINY
    if name == "tiny_bf16":
        return TINY_BF16
    raise KeyError(name)


def truncated(cfg: Cfg, layers: Optional[int] = None, **kw) -> Cfg:
    """The same shape with fewer layers (for CPU-bounded checks at full width)."""
    c = cfg.replace(name=f"{cfg.name}_L{layers}" if layers else cfg.name, family=cfg.weights_key, **kw)
    if layers is not None:
        c = c.replace(layers=layers)
    return c
