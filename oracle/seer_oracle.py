"""Oracle for the SeerAttention-R decode-time hot path.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, float64 CPU
statement of what the decode path computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and this module imports
nothing from that path.

Pages cited (each is web text about the method):
  [CP]  chapterpal.com summary page "SeerAttention-R: Sparse Attention
        Adaptation for Long Reasoning" -- its numbered "Knowl" sections.
  [PN]  papernotes.org ICLR 2026 notes page "Sparse Attention Adaptation for
        Long Reasoning" -- its "key design" paragraphs.
  [SK]  skillsmp.com page "sparse-attention-reasoning" -- "Step 4: Optimized
        Kernel Implementation" (masked dense attention).

Conventions (readings of the pages, each listed in the design notes):
  * All bf16 inputs are converted exactly to float64 before any arithmetic.
  * One K Compression Cache entry is stored rounded to bf16 (round to
    nearest, ties to even), because the cache is a bf16 tensor.
  * RoPE uses the rotate-half pairing (i, i + D/2) over the gate dimension,
    with frequencies theta^(-2i/D) and angles formed in float64.
  * A compressed block j sits at position j*b (its first token); the decode
    query sits at position L-1, where L counts the current token.
  * Only complete blocks are scored.  Blocks at or beyond the number of cached
    entries (normally just the last partial block) are always selected.
  * Top-k ties go to the lower block index.  Threshold comparison is strict.
  * Selected blocks are reported in ascending order.

Parity pins: every function here is checked in tests/test_oracle.py against
something other than itself (library routines, closed forms, brute force,
invariants the pages state).  The gate numerics with *trained* weights are
parity unpinned: the pages give no weights and no worked example; the
synthetic workloads use seeded random weights instead.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "round_to_bf16",
    "rope",
    "pool_block",
    "compress_block",
    "build_kcomp",
    "update_kcomp",
    "gate_query",
    "gate_logits",
    "select_topk",
    "select_threshold",
    "select_topp",
    "blocks_to_tokens",
    "attention_gathered",
    "attention_masked_dense",
    "dense_decode_pair",
    "decode_pair",
    "memory_ratio",
]


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of raw bf16 bit patterns (uint16) as float64.

    A bf16 number is the upper half of an IEEE binary32 number, so widening
    the 16 bits to the top of a 32-bit word gives the same value exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and binary32's exponent range.  For a
    normal value x = m * 2^e with 0.5 <= |m| < 1 the spacing of bf16 values
    around x is 2^(e-8); below 2^-126 the spacing is fixed at 2^-133
    (subnormals).  Dividing by the spacing is exact, np.round rounds half to
    even, and values past the largest finite bf16 become infinities.  The
    result is returned as float64 holding the bf16 value.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    if np.any(finite):
        xf = x[finite]
        _, e = np.frexp(xf)
        q_exp = np.maximum(e - 8, -133)
        q = np.ldexp(1.0, q_exp)
        r = np.round(xf / q) * q
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, xf), r)
        out[finite] = r
    return out


# ---------------------------------------------------------------------------
# RoPE inside the gate  ([CP Knowl 1]: RoPE is re-applied to the pre-RoPE Q
# and K within the gate; [PN key design 2])
# ---------------------------------------------------------------------------

def rope(v: np.ndarray, pos: float, theta: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of the last axis of v at position pos.

    Rotate-half pairing: for i < D/2 with frequency w_i = theta^(-2i/D) and
    angle a = pos * w_i,
        out[i]       = v[i] cos a - v[i+D/2] sin a
        out[i+D/2]   = v[i+D/2] cos a + v[i] sin a
    """
    v = np.asarray(v, dtype=np.float64)
    D = v.shape[-1]
    if D % 2:
        raise ValueError("RoPE needs an even dimension")
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    w = np.power(float(theta), -2.0 * i / D)
    a = float(pos) * w
    c, s = np.cos(a), np.sin(a)
    lo, hi = v[..., :half], v[..., half:]
    out = np.empty_like(v)
    out[..., :half] = lo * c - hi * s
    out[..., half:] = hi * c + lo * s
    return out


# ---------------------------------------------------------------------------
# K branch of the gate and the K Compression Cache
# ---------------------------------------------------------------------------

def pool_block(keys: np.ndarray) -> np.ndarray:
    """[P_max, P_min, P_avg] of one block of pre-RoPE keys, shape [b, d] -> [3d].

    [CP Knowl 1, Knowl 2]: sequence pooling with kernel = stride = b; the
    max, min and average outputs are concatenated in that order.
    """
    keys = np.asarray(keys, dtype=np.float64)
    b = keys.shape[0]
    return np.concatenate([keys.max(axis=0), keys.min(axis=0), keys.sum(axis=0) / b])


def compress_block(keys: np.ndarray, w_k: np.ndarray, block_index: int,
                   block_size: int, theta: float = 10000.0) -> np.ndarray:
    """One K Compression Cache entry: bf16(RoPE(W_k @ pool(keys), j*b)).

    [CP Knowl 2] K_gate = RoPE(W_k concat[P_max, P_min, P_avg](K_nope)) with
    W_k of shape [d_gate, 3d]; [CP Knowl 1] each compressed block takes the
    position of its first token; [CP Knowl 5] the cache stores K_gate.
    """
    u = pool_block(keys)
    v = np.asarray(w_k, dtype=np.float64) @ u
    return round_to_bf16(rope(v, block_index * block_size, theta))


def build_kcomp(k_nope: np.ndarray, w_k: np.ndarray, seq_len: int,
                block_size: int, theta: float = 10000.0) -> np.ndarray:
    """All cache entries of one (sequence, KV head): one per complete block.

    k_nope: [>= seq_len, d] pre-RoPE keys.  Returns [floor(L/b), d_gate].
    [CP Knowl 5]: only complete blocks have entries.
    """
    nb = seq_len // block_size
    dg = w_k.shape[0]
    out = np.zeros((nb, dg), dtype=np.float64)
    for j in range(nb):
        out[j] = compress_block(k_nope[j * block_size:(j + 1) * block_size], w_k,
                                j, block_size, theta)
    return out


def update_kcomp(cache: list, k_nope: np.ndarray, w_k: np.ndarray, seq_len: int,
                 block_size: int, theta: float = 10000.0,
                 max_new_blocks: Optional[int] = None) -> list:
    """Incremental cache update after the sequence has grown to seq_len.

    [CP Knowl 5]: the cache is updated once every b new tokens by pooling the
    latest b keys.  Entries already written are never touched; entries are
    appended for blocks that have become complete, at most max_new_blocks of
    them per call (None = all).
    """
    nb = seq_len // block_size
    start = len(cache)
    stop = nb if max_new_blocks is None else min(nb, start + max_new_blocks)
    for j in range(start, stop):
        cache.append(compress_block(k_nope[j * block_size:(j + 1) * block_size],
                                    w_k, j, block_size, theta))
    return cache


# ---------------------------------------------------------------------------
# Q branch and block scores  ([CP Knowl 1, Knowl 2]; [PN key design 1])
# ---------------------------------------------------------------------------

def gate_query(q_nope_group: np.ndarray, w_q: np.ndarray, pos: int,
               theta: float = 10000.0) -> np.ndarray:
    """Q_gate = RoPE(W_q @ reshape(q_nope of the g heads of a group, [g*d]), pos).

    q_nope_group: [g, d], the query heads h*g .. h*g+g-1 that share KV head h
    (the reshape of [.., H_q, 1, d] to [.., H_kv, 1, g*d] groups consecutive
    heads).  w_q: [d_gate, g*d] for this KV head.
    """
    x = np.asarray(q_nope_group, dtype=np.float64).reshape(-1)
    y = np.asarray(w_q, dtype=np.float64) @ x
    return rope(y, pos, theta)


def gate_logits(q_gate: np.ndarray, kcomp: np.ndarray) -> np.ndarray:
    """Un-softmaxed block scores z_j = Q_gate . K_gate[j] / sqrt(d_gate).

    [CP Knowl 2]: S = softmax(Q_gate K_gate^T / sqrt(d_gate)); [CP Knowl 5]
    top-k works on the logits before the softmax.
    """
    kcomp = np.asarray(kcomp, dtype=np.float64)
    dg = q_gate.shape[-1]
    if kcomp.shape[0] == 0:
        return np.zeros((0,), dtype=np.float64)
    return (kcomp @ np.asarray(q_gate, dtype=np.float64)) / math.sqrt(dg)


# ---------------------------------------------------------------------------
# Binarisation into active blocks  ([CP Knowl 5])
# ---------------------------------------------------------------------------

def _forced_blocks(n_cached: int, seq_len: int, block_size: int) -> list:
    """Blocks with no cache entry, always active.

    [CP Knowl 5]: when L is not a multiple of b the incomplete last block is
    selected unconditionally.  A block with no cache entry cannot be scored;
    with an up-to-date cache that is exactly the partial block.
    """
    total = -(-seq_len // block_size)
    return list(range(n_cached, total))


def _keep_within_capacity(ranked_scored: list, forced: list,
                          capacity: Optional[int]) -> list:
    """The active set when it may not fit the index row.

    [CP Knowl 5]: the incomplete last block is always selected, so blocks
    without a cache entry (the partial block, plus complete blocks a lagging
    cache has not scored yet) come before scored blocks: with a capacity of
    c, the last min(c, #forced) forced blocks are kept (the partial block is
    the last), and the scored blocks fill what room is left in their given
    order (best first for top-k and top-p).
    """
    if capacity is None:
        return list(ranked_scored) + list(forced)
    cap = max(0, int(capacity))
    kept_forced = list(forced)[max(0, len(forced) - cap):]
    room = cap - len(kept_forced)
    return list(ranked_scored)[:room] + kept_forced


def select_topk(z: np.ndarray, k: int, seq_len: int, block_size: int,
                capacity: Optional[int] = None) -> np.ndarray:
    """Token-budget selection: the k largest logits, plus the forced blocks.

    z holds the logits of the cached complete blocks (len = n_cached).  Order
    is (z descending, index ascending), so ties go to the lower block index.
    Returns ascending block indices.  With a `capacity`, the forced blocks are
    kept first and k shrinks to the room left (_keep_within_capacity).
    """
    z = np.asarray(z, dtype=np.float64)
    n = z.shape[0]
    k_eff = max(0, min(int(k), n))
    order = sorted(range(n), key=lambda j: (-z[j], j))
    chosen = _keep_within_capacity(order[:k_eff], _forced_blocks(n, seq_len, block_size),
                                   capacity)
    return np.asarray(sorted(chosen), dtype=np.int64)


def select_threshold(z: np.ndarray, tau: float, seq_len: int, block_size: int,
                     capacity: Optional[int] = None) -> np.ndarray:
    """Threshold selection: blocks whose softmax score exceeds tau, plus forced.

    softmax_j(z) > tau  <=>  z_j > ln(tau) + LSE(z), evaluated in float64.
    The softmax runs over the scored (complete, cached) blocks only.  With a
    `capacity` too small for the set, the forced blocks are kept first and
    the scored blocks fill the rest in index order (_keep_within_capacity).
    """
    z = np.asarray(z, dtype=np.float64)
    n = z.shape[0]
    chosen = []
    if n > 0:
        m = z.max()
        lse = m + math.log(float(np.sum(np.exp(z - m))))
        thr = (math.log(tau) if tau > 0 else -math.inf) + lse
        chosen = [j for j in range(n) if z[j] > thr]
    chosen = _keep_within_capacity(chosen, _forced_blocks(n, seq_len, block_size), capacity)
    return np.asarray(sorted(chosen), dtype=np.int64)


def select_topp(z: np.ndarray, p: float, seq_len: int, block_size: int,
                capacity: Optional[int] = None) -> np.ndarray:
    """Top-p (nucleus) selection: the smallest set of scored blocks, taken in
    descending score order (equal scores: lower index first), whose softmax
    probability mass reaches p; plus the forced blocks.

    [CP Knowl 14] names top-p sparsity as the adaptive direction beyond the
    fixed budget of [CP Knowl 5]; the set is read as the usual nucleus: walk
    the blocks from the highest score and stop as soon as the mass taken so
    far is at least p (p <= 0 takes none, a p the total never reaches takes
    all).  The softmax runs over the scored blocks, in float64.
    """
    z = np.asarray(z, dtype=np.float64)
    n = z.shape[0]
    chosen = []
    if n > 0:
        m = z.max()
        e = np.exp(z - m)
        prob = e / float(np.sum(e))
        order = sorted(range(n), key=lambda j: (-z[j], j))
        mass = 0.0
        for j in order:
            if mass >= p:
                break
            chosen.append(j)
            mass += float(prob[j])
    chosen = _keep_within_capacity(chosen, _forced_blocks(n, seq_len, block_size), capacity)
    return np.asarray(sorted(chosen), dtype=np.int64)


def topk_budget_blocks(token_budget: int, block_size: int) -> int:
    """[CP Knowl 5]: a token budget B becomes a block budget k = ceil(B/b)."""
    return -(-int(token_budget) // int(block_size))


# ---------------------------------------------------------------------------
# Attention over the gathered tokens  ([CP Knowl 6]; [SK Step 4])
# ---------------------------------------------------------------------------

def blocks_to_tokens(blocks: Iterable[int], seq_len: int, block_size: int) -> np.ndarray:
    """Token positions covered by the active blocks, clipped to the sequence."""
    toks = []
    for j in blocks:
        lo = int(j) * block_size
        hi = min(lo + block_size, seq_len)
        toks.extend(range(lo, hi))
    return np.asarray(toks, dtype=np.int64)


def attention_gathered(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                       tokens: np.ndarray, scale: float):
    """Softmax attention of each query head over the gathered tokens only.

    q: [g, d]; k, v: [>= max(tokens)+1, d].  Returns (o [g, d], lse [g]) with
    lse = ln sum_t exp(s_t).  An empty token set gives o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    g, d = q.shape
    if len(tokens) == 0:
        return np.zeros((g, d)), np.full((g,), -np.inf)
    kt = np.asarray(k, dtype=np.float64)[tokens]
    vt = np.asarray(v, dtype=np.float64)[tokens]
    s = (q @ kt.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ vt) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def attention_masked_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           seq_len: int, active_tokens: np.ndarray, scale: float):
    """Second formulation: dense scores over t < L with -inf outside the set.

    [SK Step 4]: scores = Q K^T / sqrt(d), masked_fill(mask == 0, -inf),
    softmax, then multiply by V.  Must agree with attention_gathered.
    """
    q = np.asarray(q, dtype=np.float64)
    kk = np.asarray(k, dtype=np.float64)[:seq_len]
    vv = np.asarray(v, dtype=np.float64)[:seq_len]
    s = (q @ kk.T) * scale
    mask = np.zeros((seq_len,), dtype=bool)
    mask[np.asarray(active_tokens, dtype=np.int64)] = True
    s = np.where(mask[None, :], s, -np.inf)
    if not mask.any():
        return np.zeros_like(q), np.full((q.shape[0],), -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p / l) @ vv, (m + np.log(l))[:, 0]


def dense_decode_pair(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_len: int,
                      scale: float):
    """Full attention decode of one (sequence, KV head): every token t < L."""
    return attention_gathered(q, k, v, np.arange(seq_len, dtype=np.int64), scale)


def sparse_decode_pair(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_len: int,
                       blocks: Sequence[int], block_size: int, scale: float):
    """Block-sparse decode of one (sequence, KV head) over the given blocks.

    Blocks outside [0, ceil(L/b)) are skipped, as the kernel skips invalid
    index entries ([CP Knowl 6]; [PN key design 4]).
    """
    total = -(-seq_len // block_size)
    valid = [int(j) for j in blocks if 0 <= int(j) < total]
    return attention_gathered(q, k, v, blocks_to_tokens(valid, seq_len, block_size), scale)


# ---------------------------------------------------------------------------
# One whole decode step of one (sequence, KV head)
# ---------------------------------------------------------------------------

def decode_pair(q_nope: np.ndarray, q: np.ndarray, k_nope: np.ndarray,
                k: np.ndarray, v: np.ndarray, w_q: np.ndarray, kcomp: np.ndarray,
                seq_len: int, block_size: int, *, mode: str, topk: int = 0,
                tau: float = 0.0, scale: Optional[float] = None,
                theta: float = 10000.0, capacity: Optional[int] = None):
    """Gate, select and attend for one (sequence, KV head) at length seq_len.

    q_nope, q: [g, d] (pre- and post-RoPE query heads of the group);
    k_nope, k, v: [>= seq_len, d]; kcomp: [n_cached, d_gate] cache entries.
    tau is the threshold (mode "threshold") or the mass p (mode "topp").
    Returns dict(q_gate, logits, blocks, o, lse).
    """
    g, d = np.asarray(q).shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qg = gate_query(q_nope, w_q, seq_len - 1, theta)
    z = gate_logits(qg, kcomp)
    if mode == "topk":
        blocks = select_topk(z, topk, seq_len, block_size, capacity)
    elif mode == "threshold":
        blocks = select_threshold(z, tau, seq_len, block_size, capacity)
    elif mode == "topp":
        blocks = select_topp(z, tau, seq_len, block_size, capacity)
    else:
        raise ValueError(mode)
    o, lse = sparse_decode_pair(q, k, v, seq_len, blocks, block_size, scale)
    return dict(q_gate=qg, logits=z, blocks=blocks, o=o, lse=lse)


def memory_ratio(d_gate: int, head_dim: int, block_size: int) -> float:
    """Bytes of the compression cache over bytes of the K and V caches.

    One d_gate-wide entry per b tokens, against 2*d values per token, both
    in the same element type.  [CP Knowl 5] quotes 1/128 at b = 64.
    """
    return d_gate / (2.0 * block_size * head_dim)
