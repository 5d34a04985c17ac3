"""Sampler chain on one logits row (test infrastructure: the CPU oracle).

The engine page ("llama.cpp AI LLM Engine - how it works", Steps 14-16,
"Sampler chain") fixes the order of the steps, each acting on the candidate
set the previous one left:

  1. repetition penalty: tokens that already appeared lose probability;
  2. cut-offs: top-k keeps the k largest logits, top-p keeps the tokens whose
     accumulated probability stays within p, min-p drops tokens far below
     the leader;
  3. temperature divides the logits of what is left;
  4. one token is chosen: the largest logit (greedy) or at random with the
     softmax probabilities of the remaining logits.
The chain records the chosen token in its own history.

Readings where the page gives no formula:
  * penalties over the last n history tokens, for each distinct token with
    count c: logit / r if logit > 0 else logit * r (repeat r), then
    logit - c * f - p (frequency f, presence p);
  * candidates are ordered by logit descending, ties by lower token id; top-k
    keeps the first k; top-p keeps the shortest prefix whose softmax mass
    (temperature 1, over the current candidates) reaches p (at least one);
    min-p keeps candidates with probability >= min_p * the largest
    probability; temperature t > 0 divides the logits (t <= 0: the largest
    logit is chosen);
  * the random choice takes a uniform u in [0, 1): the first candidate, in
    the order above, whose accumulated probability exceeds u.
Probabilities are computed in float64 here.
"""
from dataclasses import dataclass
from typing import Sequence

import numpy as np


@dataclass
class SamplerParams:
    top_k: int = 40
    top_p: float = 1.0
    min_p: float = 0.0
    temperature: float = 1.0
    penalty_last_n: int = 0
    penalty_repeat: float = 1.0
    penalty_freq: float = 0.0
    penalty_present: float = 0.0


def apply_penalties(logits: np.ndarray, history: Sequence[int], p: SamplerParams) -> np.ndarray:
    z = np.asarray(logits, np.float64).copy()
    window = list(history)[-p.penalty_last_n:] if p.penalty_last_n > 0 else []
    ids, counts = np.unique(np.asarray(window, np.int64), return_counts=True)
    for t, c in zip(ids, counts):
        v = z[t]
        v = v / p.penalty_repeat if v > 0 else v * p.penalty_repeat
        z[t] = v - c * p.penalty_freq - p.penalty_present
    return z


def ordered(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Candidate ids ordered by value descending, ties by lower id."""
    return ids[np.lexsort((ids, -z[ids]))]


def softmax_of(v: np.ndarray) -> np.ndarray:
    e = np.exp(v - v.max())
    return e / e.sum()


def candidates(logits: np.ndarray, history: Sequence[int], p: SamplerParams):
    """Steps 1-3: (ordered candidate ids, their logits after temperature)."""
    z = apply_penalties(logits, history, p)
    c = ordered(z, np.arange(z.size))
    if p.top_k > 0:
        c = c[:p.top_k]
    if p.top_p < 1.0:
        cum = np.cumsum(softmax_of(z[c]))
        keep = int(np.searchsorted(cum, p.top_p, side="left")) + 1
        c = c[:max(1, min(keep, c.size))]
    if p.min_p > 0.0:
        pr = softmax_of(z[c])
        c = c[pr >= p.min_p * pr.max()]
    v = z[c] / p.temperature if p.temperature > 0 else z[c]
    return c, v


def sample(logits: np.ndarray, history: Sequence[int], p: SamplerParams, u: float):
    """The chosen token and the distance of u from the nearest decision
    boundary of the accumulated probabilities (inf for greedy)."""
    c, v = candidates(logits, history, p)
    if p.temperature <= 0:
        return int(c[0]), float("inf")
    cum = np.cumsum(softmax_of(v))
    i = int(np.searchsorted(cum, u, side="right"))
    i = min(i, c.size - 1)
    margin = float(np.min(np.abs(cum - u)))
    return int(c[i]), margin
