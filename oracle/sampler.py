"""Temperature + Gumbel-max token sampler (test infrastructure, not product code).

What it follows:
  * nano-vllm walkthrough (xingyun3d.csdn.net), section 六 (模型执行), its sampler
    paragraph: the logits are divided by the temperature, noise is added and the
    token is the argmax of the noisy scores (the Gumbel-max trick: a parallel,
    sort-free way to draw from softmax(logits / temperature));
  * deep dive ("万字深度解析 Nano-vLLM"), section 3.3, and the overview's list of
    sampling settings: temperature 0 is greedy search (the plain argmax).

Readings where the pages leave a step open:
  * the noise is one standard Gumbel(0, 1) draw per (row, vocabulary entry); it is
    random input drawn by the caller and passed in, never generated here;
  * a row with temperature 0 takes the argmax of its raw logits and reads no noise;
  * ties go to the lowest index (the first maximum);
  * the argmax is taken on scores rounded the way the kernel rounds them:
    ``score = fl32(fl32(logit / T) + g)``, i.e. an IEEE binary32 division followed
    by a binary32 addition.  ``score_dtype=np.float64`` gives the exact-arithmetic
    version used by the distribution pins.

Inputs: logits as float32 or raw bfloat16 bits (uint16), [batch, vocab];
temperatures float32 [batch] (0 or positive and finite); gumbel float32
[batch, vocab].  Output: int64 token ids [batch].
"""
from __future__ import annotations

import numpy as np

from .paged_oracle import to_f64


def first_argmax(scores: np.ndarray) -> int:
    """Index of the largest score; the lowest index among equal maxima."""
    best = np.max(scores)
    return int(np.flatnonzero(scores == best)[0])


def sample(logits: np.ndarray, temperatures: np.ndarray, gumbel: np.ndarray,
           score_dtype=np.float32) -> np.ndarray:
    """One token per row: greedy where the temperature is 0, otherwise
    argmax_i(logits[b, i] / T_b + gumbel[b, i])."""
    z = to_f64(logits)                      # exact: bf16 and fp32 widen without rounding
    g = np.asarray(gumbel)
    temps = np.asarray(temperatures, dtype=np.float32)
    batch = z.shape[0]
    out = np.empty(batch, dtype=np.int64)
    for b in range(batch):
        t = temps[b]
        if t == 0:
            out[b] = first_argmax(z[b])
            continue
        scaled = z[b].astype(score_dtype) / score_dtype(t)
        scores = scaled + g[b].astype(score_dtype)
        out[b] = first_argmax(scores)
    return out
