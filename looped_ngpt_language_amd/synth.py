"""Seeded synthetic inputs for the looped nGPT forward pass.

This module is the single source of inputs for both the GPU path and the CPU
oracle. It holds model shapes and random draws only: no part of the forward
computation lives here.

Recipe (stated once, used everywhere):
  * Weight matrices are stored ``[out, in]``. Matrix ``m`` is drawn from its own
    PCG64 stream ``numpy.random.default_rng([seed, m])`` as standard normals in
    float32, then every row is scaled to unit L2 norm (the unit-norm weight
    constraint of the normalised transformer, applied here as initialisation).
    Matrix ids: 0 = embedding ``E [V, d]``; for physical block ``b`` the ids
    ``1 + 7*b + {0..6}`` are W_q, W_k, W_v, W_o, W_gate, W_up, W_down; the last
    id ``1 + 7*n_blocks`` is the LM head ``[V, d]`` (untied).
  * For bf16 configurations each normalised row is rounded to bfloat16
    (round-to-nearest-even) and the float32 array holds those exact values.
  * The per-dimension residual step sizes alpha_attn and alpha_mlp are the
    constant 0.05 in every block.
  * Prompt token ids come from ``default_rng(1).integers(0, V, T)``; the
    batched-serving prompt lengths from ``default_rng(2).integers(256, 4097, n)``.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shapes of one looped nGPT model (names follow the pages' I/R/O stacks)."""

    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    n_in: int
    n_rec: int
    n_out: int
    window: int
    dtype: str
    full_every: int = 4
    rope_theta: float = 10000.0
    attn_scale: float | None = None  # None -> sqrt(head_dim)
    alpha: float = 0.05
    page_size: int = 16

    @property
    def n_blocks(self) -> int:
        return self.n_in + self.n_rec + self.n_out

    @property
    def scale(self) -> float:
        return math.sqrt(self.head_dim) if self.attn_scale is None else float(self.attn_scale)

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


# Tiny fp32 model: every path exercised, CPU oracle in seconds.
TINY = ModelShape(d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, d_ff=512, vocab=1024,
                  n_in=2, n_rec=4, n_out=2, window=16, dtype=F32)
# Mid-size bf16 model.
MID = ModelShape(d_model=1024, n_heads=8, n_kv_heads=4, head_dim=128, d_ff=4096, vocab=32768,
                 n_in=8, n_rec=20, n_out=8, window=1024, dtype=BF16)
# ~4B-parameter bf16 model (8/20/8 blocks, d=3072, 24/8 heads of 128, FFN 8192, V=131072).
DORY4B = ModelShape(d_model=3072, n_heads=24, n_kv_heads=8, head_dim=128, d_ff=8192, vocab=131072,
                    n_in=8, n_rec=20, n_out=8, window=4096, dtype=BF16)

SHAPES = {"tiny": TINY, "mid": MID, "dory4b": DORY4B}

MATRICES_PER_BLOCK = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def matrix_shapes(s: ModelShape) -> dict:
    q = s.n_heads * s.head_dim
    kv = s.n_kv_heads * s.head_dim
    return {"wq": (q, s.d_model), "wk": (kv, s.d_model), "wv": (kv, s.d_model),
            "wo": (s.d_model, q), "wg": (s.d_ff, s.d_model), "wu": (s.d_ff, s.d_model),
            "wd": (s.d_model, s.d_ff)}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_matrix(seed: int, matrix_id: int, rows: int, cols: int, dtype: str) -> np.ndarray:
    """One weight matrix: N(0,1) float32 draws, rows scaled to unit L2 norm, bf16-rounded if asked."""
    rng = np.random.default_rng([seed, matrix_id])
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    norm = np.sqrt(np.einsum("ij,ij->i", w, w, dtype=np.float64))
    w = (w / norm[:, None]).astype(np.float32)
    if dtype == BF16:
        w = from_bf16_bits(to_bf16_bits(w))
    return w


@dataclasses.dataclass
class Weights:
    shape: ModelShape
    embed: np.ndarray            # [V, d] float32 (bf16-exact values for bf16 shapes)
    lm_head: np.ndarray          # [V, d]
    blocks: list                 # per physical block: dict name -> array, plus alpha_attn/alpha_mlp [d]


def make_weights(s: ModelShape, seed: int = 0, threads: int | None = None) -> Weights:
    """All weights of the model, drawn per matrix (streams are independent, so threads are used)."""
    shp = matrix_shapes(s)
    jobs = [(0, (s.vocab, s.d_model))]
    for b in range(s.n_blocks):
        for i, name in enumerate(MATRICES_PER_BLOCK):
            jobs.append((1 + 7 * b + i, shp[name]))
    jobs.append((1 + 7 * s.n_blocks, (s.vocab, s.d_model)))
    if threads is None:
        import os
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as ex:
        mats = list(ex.map(lambda j: draw_matrix(seed, j[0], j[1][0], j[1][1], s.dtype), jobs))
    alpha = np.full(s.d_model, s.alpha, dtype=np.float32)
    blocks = []
    for b in range(s.n_blocks):
        blk = {name: mats[1 + 7 * b + i] for i, name in enumerate(MATRICES_PER_BLOCK)}
        blk["alpha_attn"] = alpha.copy()
        blk["alpha_mlp"] = alpha.copy()
        blocks.append(blk)
    return Weights(shape=s, embed=mats[0], lm_head=mats[-1], blocks=blocks)


def prompt_tokens(s: ModelShape, n: int, seed: int = 1) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, s.vocab, n).astype(np.int32)


def batch_prompt_lengths(n_seqs: int = 128, lo: int = 256, hi: int = 4096, seed: int = 2) -> np.ndarray:
    return np.random.default_rng(seed).integers(lo, hi + 1, n_seqs).astype(np.int32)


def batch_prompts(s: ModelShape, lengths, seed: int = 1) -> list:
    """One uniform-random prompt per sequence, drawn in order from a single stream."""
    rng = np.random.default_rng(seed)
    return [rng.integers(0, s.vocab, int(n)).astype(np.int32) for n in lengths]
