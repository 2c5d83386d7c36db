"""Seeded synthetic inputs for the decode path.

This module only draws random tensors with the shapes and structure of the
workloads; it holds none of the method's arithmetic (no gate, no pooling, no
selection, no attention).  Both the HIP path's tests and benchmark and the
float64 oracle consume what it produces.

Recipe (shared by every workload):
  * values are drawn in float32 from a torch.Generator seeded per workload,
    then rounded to bf16 (round to nearest even);
  * query, keys and values ~ N(0, 1); the model's own RoPE is taken as the
    identity, so the post-RoPE tensors equal the pre-RoPE ones (q = q_nope,
    K = K_nope).  With separate_nope=True the pre-RoPE query and keys the
    gate reads are drawn on their own instead (after every other draw, so
    the other tensors are unchanged): a model whose RoPE is not the
    identity, in which the gate's inputs and attention's inputs differ;
  * gate weights ~ N(0, 1/fan_in): W_q[h] is [d_gate, g*d], W_k[h] is
    [d_gate, 3d];
  * "planted" blocks: for each (sequence, KV head) a few complete blocks are
    drawn without replacement and every key in them gets +3 * u added, u the
    unit vector of the mean of that group's query heads.  This raises those
    tokens' attention logits by about 3 so that sparse and dense outputs
    differ measurably.  (The random gate does not know about them.)
  * Cache slots past a sequence's length are left as drawn (never read).

Prefill workloads (the training-side forward with the gate's ground truth,
whole sequences of up to 32k tokens as in the distillation):
  * q, K, V ~ N(0, 1) in float32, rounded to bf16;
  * each (sequence, KV head) has a random unit direction u shared by its
    query heads: every query gets +4u, the key of token 0 gets +8u (an
    attention sink) and the keys of `planted` random blocks get +8u, so the
    attention map has the sink and a few heavy blocks instead of being flat.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    d_gate: int
    block_size: int
    max_seq_len: int
    mode: str                 # "topk" | "threshold"
    topk_blocks: int = 0
    tau: float = 0.0
    planted: int = 0          # planted blocks per (sequence, KV head)
    seq_len: Optional[int] = None            # fixed length for every sequence
    seq_len_range: Optional[tuple] = None    # (lo, hi) inclusive, uniform
    avoid_multiple_of_block: bool = False
    steps: int = 1            # decode steps (pipeline workload)
    seed: int = 0
    theta: float = 10000.0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def nb_max(self) -> int:
        return -(-self.max_seq_len // self.block_size)

    def max_selected(self) -> int:
        if self.mode == "threshold":
            return self.nb_max
        return min(self.topk_blocks + 1, self.nb_max)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny parity case, two single-length decode layers
# shaped like Qwen3-8B / Qwen3-14B attention, a block-128 threshold batch of
# mixed lengths, and a 256-step pipeline at up to 128k context.
WORKLOADS = {
    "tiny": Workload("tiny", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                     d_gate=64, block_size=64, max_seq_len=1024, mode="topk",
                     topk_blocks=4, planted=2, seq_len=1024, seed=1001),
    "qwen3_8b_layer": Workload("qwen3_8b_layer", batch=1, num_q_heads=32,
                               num_kv_heads=8, head_dim=128, d_gate=128,
                               block_size=64, max_seq_len=32768, mode="topk",
                               topk_blocks=64, planted=5, seq_len=32768,
                               seed=1002),
    "qwen3_14b_b16": Workload("qwen3_14b_b16", batch=16, num_q_heads=40,
                              num_kv_heads=8, head_dim=128, d_gate=128,
                              block_size=64, max_seq_len=32768, mode="topk",
                              topk_blocks=52, planted=5, seq_len=32768,
                              seed=1003),
    "threshold_b128": Workload("threshold_b128", batch=64, num_q_heads=32,
                               num_kv_heads=8, head_dim=128, d_gate=128,
                               block_size=128, max_seq_len=65536,
                               mode="threshold", tau=0.01,
                               seq_len_range=(8192, 65536),
                               avoid_multiple_of_block=True, seed=1004),
    "pipeline_128k": Workload("pipeline_128k", batch=32, num_q_heads=32,
                              num_kv_heads=8, head_dim=128, d_gate=128,
                              block_size=64, max_seq_len=131072, mode="topk",
                              topk_blocks=64, seq_len_range=(16384, 130816),
                              steps=256, seed=1005),
}


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_seq_len: int
    seq_lens: tuple           # one length per sequence
    planted: int = 0          # heavy blocks per (sequence, KV head)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def nb_max(self) -> int:
        return -(-self.max_seq_len // self.block_size)


PREFILL_WORKLOADS = {
    "prefill_tiny": PrefillWorkload("prefill_tiny", batch=2, num_q_heads=4, num_kv_heads=2,
                                    head_dim=64, block_size=64, max_seq_len=600,
                                    seq_lens=(600, 333), planted=2, seed=2001),
    # one Qwen3-14B-shaped attention layer over a 32k-token training sequence
    "qwen3_14b_prefill_32k": PrefillWorkload("qwen3_14b_prefill_32k", batch=1, num_q_heads=40,
                                             num_kv_heads=8, head_dim=128, block_size=64,
                                             max_seq_len=32768, seq_lens=(32768,), planted=8,
                                             seed=2002),
}


def make_prefill_inputs(w: PrefillWorkload, device: str = "cpu") -> dict:
    """q [B, Hq, Lmax, d], k, v [B, Hkv, Lmax, d] bf16 and seq_lens [B] int32
    on `device`, by the prefill recipe above."""
    cpu_gen = torch.Generator(device="cpu").manual_seed(w.seed)
    dev_gen = cpu_gen if device == "cpu" else torch.Generator(device=device).manual_seed(w.seed)
    B, Hq, Hkv, d, L, bs = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_seq_len,
                            w.block_size)
    g = w.group
    u = torch.randn((B, Hkv, d), generator=cpu_gen, dtype=torch.float32)
    u = (u / u.norm(dim=-1, keepdim=True)).to(device)
    q = torch.empty((B, Hq, L, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((B, Hkv, L, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, Hkv, L, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        for h in range(Hkv):
            for i in range(g):
                x = torch.randn((L, d), generator=dev_gen, device=device, dtype=torch.float32)
                q[b, h * g + i] = (x + 4.0 * u[b, h]).to(torch.bfloat16)
            x = torch.randn((L, d), generator=dev_gen, device=device, dtype=torch.float32)
            x[0] += 8.0 * u[b, h]
            nb = w.seq_lens[b] // bs
            if nb > 1 and w.planted > 0:
                for j in (torch.randperm(nb - 1, generator=cpu_gen)[:w.planted] + 1).tolist():
                    x[j * bs:(j + 1) * bs] += 8.0 * u[b, h]
            k[b, h] = x.to(torch.bfloat16)
            v[b, h] = torch.randn((L, d), generator=dev_gen, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    seq = torch.tensor(list(w.seq_lens), dtype=torch.int32, device=device)
    return dict(q=q, k=k, v=v, seq_lens=seq)


def draw_seq_lens(w: Workload, gen: torch.Generator) -> torch.Tensor:
    """Per-sequence lengths (int32, CPU) for the workload."""
    if w.seq_len is not None:
        return torch.full((w.batch,), int(w.seq_len), dtype=torch.int32)
    lo, hi = w.seq_len_range
    out = torch.empty((w.batch,), dtype=torch.int32)
    for i in range(w.batch):
        while True:
            v = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
            if not (w.avoid_multiple_of_block and v % w.block_size == 0):
                break
        out[i] = v
    return out


def _normal_bf16(shape, gen, device, std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, device: str = "cpu", seq_lens: Optional[torch.Tensor] = None,
                kv_len: Optional[int] = None, separate_nope: bool = False) -> dict:
    """Draw every input tensor of one decode step of workload w.

    Returns a dict of tensors on `device`:
      q [B, Hq, d] bf16, k, v [B, Hkv, Lmax, d] bf16 (attention's inputs),
      q_nope [B, Hq, d], k_nope [B, Hkv, Lmax, d] bf16 (the gate's pre-RoPE
      inputs: the same tensors as q and k unless separate_nope),
      w_q [Hkv, dg, g*d], w_k [Hkv, dg, 3d] bf16, seq_lens [B] int32,
      planted [B, Hkv, planted] int64 (block ids).
    kv_len overrides the allocated cache length (default w.max_seq_len).
    """
    cpu_gen = torch.Generator(device="cpu").manual_seed(w.seed)
    dev_gen = cpu_gen if device == "cpu" else torch.Generator(device=device).manual_seed(w.seed)
    B, Hq, Hkv, d, dg = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate
    g = w.group
    lmax = int(kv_len or w.max_seq_len)
    if seq_lens is None:
        seq_lens = draw_seq_lens(w, cpu_gen)
    seq_lens = seq_lens.to(torch.int32).cpu()
    q = _normal_bf16((B, Hq, d), dev_gen, device)
    w_q = _normal_bf16((Hkv, dg, g * d), dev_gen, device, std=1.0 / math.sqrt(g * d))
    w_k = _normal_bf16((Hkv, dg, 3 * d), dev_gen, device, std=1.0 / math.sqrt(3 * d))
    k = torch.empty((B, Hkv, lmax, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, Hkv, lmax, d), dtype=torch.bfloat16, device=device)
    for b in range(B):  # per sequence, to bound the float32 temporaries
        k[b] = _normal_bf16((Hkv, lmax, d), dev_gen, device)
        v[b] = _normal_bf16((Hkv, lmax, d), dev_gen, device)
    planted = torch.zeros((B, Hkv, w.planted), dtype=torch.int64)
    if w.planted > 0:
        qf = q.float().view(B, Hkv, g, d).mean(dim=2)
        u = qf / qf.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        for b in range(B):
            nb = int(seq_lens[b]) // w.block_size
            for h in range(Hkv):
                if nb == 0:
                    continue
                n = min(w.planted, nb)
                sel = torch.randperm(nb, generator=cpu_gen)[:n]
                planted[b, h, :n] = sel
                for j in sel.tolist():
                    lo, hi = j * w.block_size, (j + 1) * w.block_size
                    blk = k[b, h, lo:hi].float() + 3.0 * u[b, h][None, :]
                    k[b, h, lo:hi] = blk.to(torch.bfloat16)
    q_nope, k_nope = q, k
    if separate_nope:
        q_nope = _normal_bf16((B, Hq, d), dev_gen, device)
        k_nope = torch.empty((B, Hkv, lmax, d), dtype=torch.bfloat16, device=device)
        for b in range(B):
            k_nope[b] = _normal_bf16((Hkv, lmax, d), dev_gen, device)
    return dict(q=q, k=k, v=v, q_nope=q_nope, k_nope=k_nope, w_q=w_q, w_k=w_k,
                seq_lens=seq_lens.to(device), planted=planted)


def append_token(inputs: dict, gen: torch.Generator) -> None:
    """Pipeline step input: draw the new token's q, K, V at position L_b.

    Writes K[b, :, L_b] and V[b, :, L_b] for every sequence, redraws q, then
    increments seq_lens.  Where the gate's pre-RoPE inputs are tensors of
    their own (make_inputs(separate_nope=True)), K_nope[b, :, L_b] and q_nope
    are drawn too, after the others.  Lengths must stay below the cache
    capacity.
    """
    q, k, v, seq_lens = inputs["q"], inputs["k"], inputs["v"], inputs["seq_lens"]
    B, Hkv, lmax, d = k.shape
    pos = seq_lens.long()
    if int(pos.max()) >= lmax:
        raise ValueError("sequence would exceed the cache capacity")
    dev = k.device
    new_k = _normal_bf16((B, Hkv, d), gen, dev)
    new_v = _normal_bf16((B, Hkv, d), gen, dev)
    bidx = torch.arange(B, device=dev)
    k[bidx, :, pos] = new_k
    v[bidx, :, pos] = new_v
    q.copy_(_normal_bf16(tuple(q.shape), gen, dev))
    k_nope, q_nope = inputs.get("k_nope", k), inputs.get("q_nope", q)
    if k_nope is not k:
        k_nope[bidx, :, pos] = _normal_bf16((B, Hkv, d), gen, dev)
    if q_nope is not q:
        q_nope.copy_(_normal_bf16(tuple(q_nope.shape), gen, dev))
    seq_lens.add_(1)
