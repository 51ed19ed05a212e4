"""Temperature / top-p (nucleus) sampling of the oracle -- TEST INFRASTRUCTURE ONLY.

The pages give only the serving recommendation: temperature 1.0 and top-p 0.95
(lucasainews article "NVIDIA, 루프 구조 4B 모델 Dory1.0-4B 4가지 정밀도로 공개",
section "실행 방법"). Everything else is a READING, stated here and mirrored by
the device sampler:

  * probabilities: p_i = exp((l_i - max l) / T) / sum_j exp((l_j - max l) / T);
  * nucleus: the tokens whose logit is at least tau, where tau is the largest
    logit value such that those tokens hold at least top_p of the mass (so all
    tokens tied with the boundary logit are in); top_p >= 1 keeps every token;
  * draw: given a uniform u in [0, 1) supplied by the caller, the first token
    in ascending token-id order whose running nucleus mass exceeds
    u * (nucleus mass) -- an inverse-CDF draw from the renormalised nucleus
    (any fixed order gives the same distribution; id order needs no sort);
  * T <= 0 is greedy decoding: the lowest id among the largest logits.

Plain float64 numpy, one row at a time.
"""
from __future__ import annotations

import numpy as np


def probabilities(logits, temperature: float) -> np.ndarray:
    """Softmax of logits / T in float64 (T > 0)."""
    l = np.asarray(logits, dtype=np.float64)
    z = np.exp((l - l.max()) / float(temperature))
    return z / z.sum()


def nucleus(logits, temperature: float, top_p: float) -> np.ndarray:
    """Boolean mask of the top-p nucleus (all ties at the boundary logit included)."""
    l = np.asarray(logits, dtype=np.float64)
    if top_p >= 1.0:
        return np.ones(l.shape, dtype=bool)
    p = probabilities(l, temperature)
    order = np.argsort(-l, kind="stable")            # largest logits first
    running = np.cumsum(p[order])
    k = int(np.searchsorted(running, top_p, side="left"))   # first position whose running mass reaches top_p
    if k >= l.size:
        return np.ones(l.shape, dtype=bool)          # rounding left the total just below top_p
    return l >= l[order[k]]                          # the boundary logit and every tie of it


def sample_row(logits, temperature: float, top_p: float, u: float) -> int:
    """One draw for one row of logits with the caller's uniform u in [0, 1)."""
    l = np.asarray(logits, dtype=np.float64)
    if temperature <= 0.0:
        return int(np.argmax(l))
    keep = nucleus(l, temperature, top_p)
    p = np.where(keep, probabilities(l, temperature), 0.0)
    target = float(u) * p.sum()
    running = np.cumsum(p)
    hit = np.nonzero((running > target) & keep)[0]
    return int(hit[0]) if hit.size else int(np.nonzero(keep)[0][-1])


def sample(logits, temperature: float, top_p: float, uniforms) -> np.ndarray:
    """Rows of logits [R, V] and uniforms [R] -> token ids [R] (int64)."""
    rows = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    us = np.atleast_1d(np.asarray(uniforms, dtype=np.float64))
    return np.array([sample_row(r, temperature, top_p, u) for r, u in zip(rows, us)], dtype=np.int64)
