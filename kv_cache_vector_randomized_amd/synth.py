"""Seeded synthetic inputs for the five workloads (shared by tests, bench and smoke).

This module only draws random numbers and lays them out: it holds none of the
quantization or attention arithmetic, so both the HIP path and the CPU oracle
can take their inputs from it without sharing any of the method's code.

Random quantities that the method itself draws (the +-1 sign vector of the
randomized Hadamard rotation, the Gaussian QJL projection S) are generated here
and passed to both sides as inputs.

bf16 tensors are produced by round-to-nearest-even from float32 draws and are
returned as their raw uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

HEAD_DIM = 128
BLOCK_TOKENS = 16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round half to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and quantizer settings of one workload (names follow the pages' notation)."""
    name: str
    head_dim: int
    num_kv_heads: int
    num_q_heads: int
    batch: int
    context: int            # tokens attended per sequence in the decode step
    key_bits: int
    key_mode: str           # "lloyd" | "lloyd_nc" | "lloyd_qjl" | "fp8" | "polar"
    val_bits: int
    val_mode: str           # "uniform" | "lloyd"
    dtype: str              # "f32" | "bf16"
    outlier: str            # description of the outlier-channel recipe
    seed: int


# The workloads.  Sizes are the full ones; tests shrink batch/context with
# `shrink()` while keeping the recipe.
WORKLOADS = {
    "toy": Workload("toy", 128, 1, 1, 1, 4096, 4, "lloyd", 4, "lloyd", "f32",
                    "channels {3,17,64,100} x10 on K and V", 1),
    "gqa_decode": Workload("gqa_decode", 128, 8, 32, 16, 8192, 4, "lloyd_nc", 4, "uniform", "bf16",
                           "2% of channels per KV head x8", 2),
    "long_3bit": Workload("long_3bit", 128, 8, 32, 4, 32768, 3, "lloyd_nc", 3, "uniform", "bf16",
                          "none", 3),
    "prefill_append": Workload("prefill_append", 128, 8, 32, 1, 131072, 4, "lloyd_nc", 4, "uniform", "bf16",
                               "5% of channels per KV head Student-t nu=4", 4),
    "qjl": Workload("qjl", 128, 8, 32, 8, 16384, 2, "lloyd_qjl", 4, "uniform", "bf16",
                    "none", 5),
    # asymmetric presets: 3-bit corrected keys with 4-bit values (the serving
    # engine's k3v4_nc), and 3-bit keys + 1-bit QJL residual with 2-bit values
    "k3v4_nc": Workload("k3v4_nc", 128, 8, 32, 16, 8192, 3, "lloyd_nc", 4, "uniform", "bf16",
                        "2% of channels per KV head x8", 6),
    "k3qjl_v2": Workload("k3qjl_v2", 128, 8, 32, 8, 16384, 3, "lloyd_qjl", 2, "uniform", "bf16",
                         "none", 7),
    # FP8 (E4M3) keys with 4-bit uniform values (the serving engine's k8v4)
    "k8v4": Workload("k8v4", 128, 8, 32, 16, 8192, 8, "fp8", 4, "uniform", "bf16",
                     "2% of channels per KV head x8", 8),
    # 8-bit Lloyd-Max keys (corrected norm) with 3-bit uniform values (the MLX default turbo8v3)
    "turbo8v3": Workload("turbo8v3", 128, 8, 32, 16, 8192, 8, "lloyd_nc", 3, "uniform", "bf16",
                         "2% of channels per KV head x8", 9),
    # PolarQuant keys (3-bit angles, fp32 radius) with 4-bit uniform values
    "polar3": Workload("polar3", 128, 8, 32, 16, 8192, 3, "polar", 4, "uniform", "bf16",
                       "2% of channels per KV head x8", 10),
}


def shrink(w: Workload, batch: Optional[int] = None, context: Optional[int] = None) -> Workload:
    return dataclasses.replace(w, batch=batch if batch is not None else w.batch,
                               context=context if context is not None else w.context)


def sign_vector(seed: int, d: int = HEAD_DIM) -> np.ndarray:
    """Seeded +-1 vector (int8) for the randomized Hadamard rotation."""
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    return np.where(rng.integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)


def qjl_matrix(d: int = HEAD_DIM, m: Optional[int] = None) -> np.ndarray:
    """Seeded Gaussian projection S (m x d, float32, entries N(0,1)), shared by all heads."""
    rng = np.random.Generator(np.random.PCG64(2000))
    return rng.standard_normal((m or d, d), dtype=np.float64).astype(np.float32)


def _outlier_channels(rng, num_heads, d, count):
    return np.stack([np.sort(rng.choice(d, size=count, replace=False)) for _ in range(num_heads)])


def kv_tensor(w: Workload, num_tokens: int, which: str, seed_offset: int = 0) -> np.ndarray:
    """K or V activations [num_tokens, num_kv_heads, d] with the workload's outlier recipe.

    Returns float32 for f32 workloads and bf16 bit patterns (uint16) for bf16 ones.
    """
    assert which in ("k", "v")
    d, hk = w.head_dim, w.num_kv_heads
    rng = np.random.Generator(np.random.PCG64([w.seed, 0 if which == "k" else 1, seed_offset]))
    x = rng.standard_normal((num_tokens, hk, d), dtype=np.float32)
    chan_rng = np.random.Generator(np.random.PCG64([w.seed, 7]))
    if w.name == "toy":
        x[:, :, [3, 17, 64, 100]] *= np.float32(10.0)
    elif w.name in ("gqa_decode", "k3v4_nc", "k8v4", "turbo8v3", "polar3"):
        ch = _outlier_channels(chan_rng, hk, d, int(round(0.02 * d)))
        for h in range(hk):
            x[:, h, ch[h]] *= np.float32(8.0)
    elif w.name == "prefill_append":
        ch = _outlier_channels(chan_rng, hk, d, int(round(0.05 * d)))
        t = rng.standard_t(4.0, size=(num_tokens, hk, ch.shape[1])).astype(np.float32)
        for h in range(hk):
            x[:, h, ch[h]] = t[:, h, :]
    if w.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def query_tensor(w: Workload, batch: Optional[int] = None, seed_offset: int = 0) -> np.ndarray:
    """Decode queries [batch, num_q_heads, d] ~ N(0,1) (bf16 bits or float32)."""
    b = batch if batch is not None else w.batch
    rng = np.random.Generator(np.random.PCG64([w.seed, 2, seed_offset]))
    q = rng.standard_normal((b, w.num_q_heads, w.head_dim), dtype=np.float32)
    return f32_to_bf16_bits(q) if w.dtype == "bf16" else q


@dataclasses.dataclass
class PagedLayout:
    """Block tables for a batch of sequences stored in 16-token pages at seeded positions."""
    num_blocks: int
    block_tables: np.ndarray   # int32 [batch, max_blocks]
    seq_lens: np.ndarray       # int32 [batch]

    def slots(self, b: int, start: int, stop: int) -> np.ndarray:
        """Cache slots (block * 16 + offset) of tokens [start, stop) of sequence b (int64)."""
        t = np.arange(start, stop, dtype=np.int64)
        return self.block_tables[b, t // BLOCK_TOKENS].astype(np.int64) * BLOCK_TOKENS + t % BLOCK_TOKENS


def paged_layout(batch: int, seq_lens, seed: int, spare_blocks: int = 0) -> PagedLayout:
    """Give every sequence ceil(len/16) pages; pages are a seeded permutation of all blocks."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(batch)
    need = (seq_lens.astype(np.int64) + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    max_blocks = int(max(1, need.max()))
    total = int(need.sum()) + spare_blocks
    rng = np.random.Generator(np.random.PCG64([seed, 9]))
    perm = rng.permutation(max(total, 1)).astype(np.int32)
    tables = np.zeros((batch, max_blocks), dtype=np.int32)
    pos = 0
    for b in range(batch):
        n = int(need[b])
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    return PagedLayout(num_blocks=max(total, 1), block_tables=tables, seq_lens=seq_lens)
