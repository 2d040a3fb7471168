"""The five synthetic workloads the layer is measured and checked on.

Shapes and constants follow the pages' statement of the two models (Muse
Glimmer 30B: 32 query heads, 2 KV heads, head width 128, query multiplier
3.87; Muse Spark Open: 128 query heads, 16 KV heads, head width 64, query
multiplier 5.4730064863875; 2048-token causal window on local layers) as given
in the deep dive's side-by-side table (section 1.2) and its attention section
(3.2). RoPE base 10000 and output-norm eps 1e-6 are the workload settings.

Stream ids name the tensors of a workload for ``synth.normal_*``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

GLIMMER_SCALE = 3.87
SPARK_SCALE = 5.4730064863875

# stream ids
S_Q, S_K, S_V, S_G = 1, 2, 3, 4
S_CACHE_BASE = 1 << 20   # + (b * Hkv + h) * 2 + {0: K, 1: V}
S_LENGTHS = 7
# decoder-block inputs: hidden states and the synthetic weights
S_X, S_IN_NORM, S_W_QKVG, S_W_O, S_POST_NORM, S_RES_GATE = 9, 10, 11, 12, 13, 14


@dataclass(frozen=True)
class Layer:
    """One attention layer's settings (arguments of the C ABI)."""
    hq: int
    hkv: int
    d: int
    window: int          # 0 = global (full causal)
    theta: float         # 0 = NoPE
    scale: float         # query multiplier applied after the weightless norm
    qk_eps: float = 1e-5
    out_norm: bool = False
    out_eps: float = 1e-6

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclass(frozen=True)
class Prefill:
    name: str
    layer: Layer
    batch: int
    seq: int
    seed: int = 0


@dataclass(frozen=True)
class Decode:
    name: str
    layer: Layer
    batch: int
    len_lo: int
    len_hi: int
    page_tokens: int = 32      # 32 tokens x 64 dims x 2 B = 4 KiB per (page, head)
    seed: int = 0


def glimmer(window: int, theta: float) -> Layer:
    return Layer(hq=32, hkv=2, d=128, window=window, theta=theta, scale=GLIMMER_SCALE)


def spark(window: int, theta: float) -> Layer:
    return Layer(hq=128, hkv=16, d=64, window=window, theta=theta, scale=SPARK_SCALE,
                 out_norm=True, out_eps=1e-6)


TINY_LOCAL = Prefill("tiny_glimmer_swa256", Layer(hq=16, hkv=1, d=128, window=256, theta=10000.0,
                                                  scale=GLIMMER_SCALE), 1, 1024)
TINY_GLOBAL = replace(TINY_LOCAL, name="tiny_glimmer_global",
                      layer=replace(TINY_LOCAL.layer, window=0, theta=0.0))
GLIMMER_LOCAL = Prefill("glimmer_local_prefill_32k", glimmer(2048, 10000.0), 1, 32768)
GLIMMER_GLOBAL = Prefill("glimmer_global_prefill_128k", glimmer(0, 0.0), 1, 131072)
SPARK_LOCAL = Prefill("spark_local_prefill_256k", spark(2048, 10000.0), 1, 262144)
SPARK_GLOBAL = Prefill("spark_global_prefill_256k", spark(0, 0.0), 1, 262144)
SPARK_DECODE_GLOBAL = Decode("spark_decode_global_paged", spark(0, 0.0), 16, 131072, 1048576)
SPARK_DECODE_LOCAL = Decode("spark_decode_local_ring", spark(2048, 10000.0), 16, 131072, 1048576)

PREFILL = [TINY_LOCAL, TINY_GLOBAL, GLIMMER_LOCAL, GLIMMER_GLOBAL, SPARK_LOCAL, SPARK_GLOBAL]
DECODE = [SPARK_DECODE_GLOBAL, SPARK_DECODE_LOCAL]


@dataclass(frozen=True)
class Chunk:
    """Chunked prefill: `seq` new tokens per sequence after `start` cached
    positions (paged cache on global layers, ring on local ones)."""
    name: str
    layer: Layer
    batch: int
    seq: int
    start: int
    page_tokens: int = 32
    seed: int = 0


SPARK_CHUNK_GLOBAL = Chunk("spark_global_chunk_2k_at_128k", spark(0, 0.0), 1, 2048, 131072)
SPARK_CHUNK_LOCAL = Chunk("spark_local_chunk_2k_at_128k", spark(2048, 10000.0), 1, 2048, 131072)
CHUNK = [SPARK_CHUNK_GLOBAL, SPARK_CHUNK_LOCAL]

# A block-diffusion drafter's non-causal block (deep dive, section 8.2): the
# Glimmer assistant's attention shape (32 query heads, 8 KV heads, head width
# 128, window 2048, 16-token blocks), 16 sequences each with 131072 context
# positions (its ring keeps the last 2048).  The multiplier and RoPE base
# follow the Glimmer workloads.
GLIMMER_DRAFT_BLOCK = Chunk("glimmer_assistant_block16_at_128k",
                            Layer(hq=32, hkv=8, d=128, window=2048, theta=10000.0, scale=GLIMMER_SCALE),
                            16, 16, 131072)
DRAFT = [GLIMMER_DRAFT_BLOCK]


@dataclass(frozen=True)
class Block:
    """The attention half of a decoder block (input norm, projections, the
    layer, o_proj, post-norm and residual) on `seq` tokens."""
    name: str
    layer: Layer
    hidden: int
    spark: bool      # True: weightless post-norm + residual gate; False: centered post-norm + add
    batch: int
    seq: int
    seed: int = 0


SPARK_BLOCK_LOCAL = Block("spark_attn_block_local_4k", spark(2048, 10000.0), 8192, True, 1, 4096)
BLOCKS = [SPARK_BLOCK_LOCAL]


def decode_lengths(seed: int, batch: int, lo: int, hi: int):
    """KV lengths (new token included), integers uniform in [lo, hi]."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + S_LENGTHS))
    return rng.integers(lo, hi, endpoint=True, size=batch).astype(np.int64)
