"""Oracle for the training-side kernel of SeerAttention-R: causal prefill
attention with the block-level ground truth of the AttnGate's distillation.

TEST INFRASTRUCTURE ONLY.  Plain float64 NumPy, one (sequence, KV head)
group at a time, no tiling and no fusion.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; it imports nothing
from the HIP library or its binding.

Pages cited:
  [CP] chapterpal.com summary page "SeerAttention-R: Sparse Attention
       Adaptation for Long Reasoning":
       Knowl 3 -- the ground truth for decoding sparsity: the full attention
         map of the original model, max-pooled over keys in blocks of b
         (column-wise 1D pooling), then max-pooled over the query heads of
         each GQA group, then normalised to sum to 1 per query row;
       Knowl 4 -- the same values obtained inside a FlashAttention-2 forward
         from each tile's row maximum r_ij rescaled by exp(r_ij - m_i) / l_i.
The fused form reaches exactly (up to rounding) the pooled map of Knowl 3,
because exp is increasing: max_t exp(s_t - m) / l = exp(max_t s_t - m) / l.
So this oracle is that definition written out; the tile form of Knowl 4 is
checked against it in tests/test_oracle.py.

Readings (each listed in the design notes):
  * The forward is causal (a decoder's prefill): the query at position p
    attends the keys at positions 0..p.  Masked keys have probability 0, so
    a block lying wholly after p has ground truth 0.
  * Scores are q.k * scale, scale passed in (1/sqrt(d) for the models).
  * The per-head pooled map is gt_h[p, j] = max over the keys t of block j
    (t <= p) of softmax_t(q_h . k_t * scale); the group's target is
    G[p, j] = max_h gt_h[p, j], normalised as G[p, j] / sum_j G[p, j].

Parity pins: tests/test_oracle.py (torch's scaled_dot_product_attention,
torch's max_pool1d, a tile-by-tile statement of Knowl 4, closed forms).
"""

from __future__ import annotations

import numpy as np

__all__ = ["prefill_group", "prefill_attention", "pooled_attention_map", "group_ground_truth"]


def prefill_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions: np.ndarray,
                      scale: float):
    """Causal attention of queries q [n, d] at `positions` over keys and
    values k, v [L, d] (key t sits at position t).

    Returns (o [n, d], lse [n], prob [n, L]) where prob is the attention map
    (0 at masked keys) and lse the natural log of each row's normaliser.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    L = k.shape[0]
    s = (q @ k.T) * float(scale)
    visible = np.arange(L)[None, :] <= positions[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(visible, np.exp(s - m), 0.0)
    l = e.sum(axis=1, keepdims=True)
    prob = e / l
    return prob @ v, (m + np.log(l))[:, 0], prob


def pooled_attention_map(prob: np.ndarray, block_size: int) -> np.ndarray:
    """[CP Knowl 3]: column-wise max pooling of an attention map [n, L] over
    keys in non-overlapping blocks of block_size (the last block may be
    short): [n, ceil(L/b)]."""
    n, L = prob.shape
    nb = -(-L // block_size)
    out = np.zeros((n, nb))
    for j in range(nb):
        out[:, j] = prob[:, j * block_size:min((j + 1) * block_size, L)].max(axis=1)
    return out


def group_ground_truth(per_head: np.ndarray) -> np.ndarray:
    """[CP Knowl 3]: max over the query heads of a GQA group ([g, n, NB] ->
    [n, NB]), then each row normalised to sum to 1."""
    g = per_head.max(axis=0)
    return g / g.sum(axis=1, keepdims=True)


def prefill_group(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions, scale: float,
                  block_size: int):
    """One (sequence, KV head) group: queries q [g, n, d] of the group's g
    heads at `positions`, keys and values k, v [L, d].

    Returns (o [g, n, d], lse [g, n], gt_head [g, n, NB], gt [n, NB]) with
    NB = ceil(L / block_size): the attention output, its log-normaliser, the
    per-head pooled map and the group's normalised ground truth.
    """
    q = np.asarray(q, dtype=np.float64)
    g = q.shape[0]
    outs, lses, pooled = [], [], []
    for h in range(g):
        o, lse, prob = prefill_attention(q[h], k, v, positions, scale)
        outs.append(o)
        lses.append(lse)
        pooled.append(pooled_attention_map(prob, block_size))
    per_head = np.stack(pooled)
    return np.stack(outs), np.stack(lses), per_head, group_ground_truth(per_head)
