"""GPU parity of the causal prefill forward with the fused ground truth
(seer_prefill_attention) against the float64 oracle (oracle/prefill_gt.py).

Tolerances (derived from the arithmetic):
  * out: as the decode output, |d| <= 2e-2 + 1e-2 |ref| (bf16 inputs, P
    rounded to bf16 before the P.V product, bf16 output);
  * lse: |d| <= 1e-3 (float32 scores and normaliser);
  * ground truth: |d| <= 1e-6 + 2e-3 |ref|.  A value is exp2(r - lse) with r
    a float32 dot product of bf16 operands (exact products, float32 sums:
    <= ~5e-5 absolute in log2 units at d = 128) and lse within ~1.5e-4, so
    each per-head value is within ~1.4e-4 relative and the normalised group
    maximum within ~3e-4; blocks after the query are exactly 0.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
from seer_testlib import assert_gt_close, assert_lse_close, assert_out_close, f64
from workloads import PREFILL_WORKLOADS, PrefillWorkload, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_seer_amd as S
    S.lib()
    return S


def run(S, dims, inp, scale, with_gt=True):
    B, Hq, Hkv, d, L = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim, dims.max_seq_len
    ws = torch.empty(S.seer_prefill_workspace_bytes(dims) // 4 + 64, dtype=torch.float32,
                     device=DEV)
    out = torch.full((B, Hq, L, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq, L), float("nan"), dtype=torch.float32, device=DEV)
    gt = (torch.full((B, Hkv, L, dims.nb_max), float("nan"), dtype=torch.float32, device=DEV)
          if with_gt else None)
    S.seer_prefill_attention(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale, ws, out,
                             lse, gt)
    torch.cuda.synchronize()
    return out, lse, gt


def make_case(d, bs, Hq, Hkv, lens, seed):
    lmax = max(lens) + 37
    w = PrefillWorkload("case", batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                        block_size=bs, max_seq_len=lmax, seq_lens=tuple(lens), planted=2,
                        seed=seed)
    inp = make_prefill_inputs(w, device="cpu")
    for b, L in enumerate(lens):  # never-read rows hold NaN
        inp["q"][b, :, L:] = float("nan")
        inp["k"][b, :, L:] = float("nan")
        inp["v"][b, :, L:] = float("nan")
    return w, inp


def check_against_oracle(S, w, inp, out, lse, gt, scale, rows=None, heads=None):
    g, bs = w.group, w.block_size
    og, lg, gg = f64(out), f64(lse), f64(gt)
    for b, L in enumerate(w.seq_lens):
        if L == 0:
            continue
        pos = np.arange(L) if rows is None else np.asarray(rows)
        nb = -(-L // bs)
        for h in (range(w.num_kv_heads) if heads is None else heads):
            qq = f64(inp["q"][b, h * g:(h + 1) * g])[:, pos]
            kk, vv = f64(inp["k"][b, h, :L]), f64(inp["v"][b, h, :L])
            o_ref, l_ref, _, gt_ref = O.prefill_group(qq, kk, vv, pos, scale, bs)
            what = f"b={b} h={h}"
            for i in range(g):
                assert_out_close(og[b, h * g + i, pos], o_ref[i], what)
                assert_lse_close(lg[b, h * g + i, pos], l_ref[i], what)
            assert_gt_close(gg[b, h, pos, :nb], gt_ref, what)
            assert np.all(gg[b, h, pos, nb:] == 0), f"{what}: blocks past the sequence"
    return True


CASES = [
    # d, bs, Hq, Hkv, lens
    (64, 64, 4, 2, [300]),
    (128, 64, 8, 2, [700, 1, 255, 256, 257]),
    (128, 128, 5, 1, [1000, 130]),
    (128, 64, 16, 1, [513]),
    (64, 128, 2, 2, [64, 65, 130]),
]


@pytest.mark.parametrize("d,bs,Hq,Hkv,lens", CASES)
def test_prefill_matches_oracle(S, d, bs, Hq, Hkv, lens):
    say(f"prefill d={d} bs={bs} Hq={Hq} Hkv={Hkv} lens={lens}")
    w, inp = make_case(d, bs, Hq, Hkv, lens, seed=d + bs + Hq)
    dims = S.make_dims(w.batch, Hq, Hkv, d, d, bs, w.max_seq_len)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    scale = 1.0 / math.sqrt(d)
    out, lse, gt = run(S, dims, dinp, scale)
    check_against_oracle(S, w, inp, out, lse, gt, scale)
    # rows past each sequence are left untouched
    for b, L in enumerate(lens):
        assert torch.all(torch.isnan(lse[b, :, L:])) and torch.all(torch.isnan(gt[b, :, L:]))
        assert torch.all(torch.isnan(out[b, :, L:].float()))
    # without the ground truth: the same attention, bit for bit
    out2, lse2, _ = run(S, dims, dinp, scale, with_gt=False)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def _random_prefill_cases(n: int, seed: int):
    """n seeded shapes: d and b in {64, 128}, 1 to 16 query heads per KV
    head, 1 to 3 KV heads and sequences, lengths from 0 to 1200 with block
    edges among them, and softmax scales around 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d, bs = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        hkv, g = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 5, 8, 16]))
        lens = [int(x) for x in rng.integers(1, 1201, size=int(rng.integers(1, 4)))]
        lens[int(rng.integers(0, len(lens)))] = int(rng.choice([0, 1, bs - 1, bs, bs + 1, 4 * bs]))
        scale = float(rng.uniform(0.5, 2.0)) / math.sqrt(d)
        cases.append((i, d, bs, hkv * g, hkv, tuple(lens), scale))
    return cases


@pytest.mark.parametrize("i,d,bs,Hq,Hkv,lens,scale", _random_prefill_cases(8, 4242))
def test_prefill_random_shapes_match_oracle(S, i, d, bs, Hq, Hkv, lens, scale):
    """A seeded sweep of prefill shapes against the oracle, every row of
    every head; rows past each sequence untouched."""
    lens = list(lens)
    say(f"random prefill {i}: d={d} bs={bs} Hq={Hq} Hkv={Hkv} lens={lens} scale={scale:.4f}")
    w, inp = make_case(d, bs, Hq, Hkv, lens, seed=5000 + i)
    dims = S.make_dims(w.batch, Hq, Hkv, d, d, bs, w.max_seq_len)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    out, lse, gt = run(S, dims, dinp, scale)
    check_against_oracle(S, w, inp, out, lse, gt, scale)
    for b, L in enumerate(lens):
        assert torch.all(torch.isnan(lse[b, :, L:])) and torch.all(torch.isnan(gt[b, :, L:]))


def test_prefill_deterministic_and_tiny_workload(S):
    w = PREFILL_WORKLOADS["prefill_tiny"]
    say(f"prefill {w.name}")
    inp = make_prefill_inputs(w, device="cpu")
    dims = S.make_dims(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.head_dim,
                       w.block_size, w.max_seq_len)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    scale = 1.0 / math.sqrt(w.head_dim)
    a = run(S, dims, dinp, scale)
    b = run(S, dims, dinp, scale)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                           y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))
    check_against_oracle(S, w, inp, *a, scale)


def test_prefill_full_size_sampled(S):
    """The 32k-token Qwen3-14B-shaped layer in the launch configuration the
    benchmark times: sampled rows against the oracle, and at every row the
    properties of the target (sums to 1, zero after the query, finite)."""
    w = PREFILL_WORKLOADS["qwen3_14b_prefill_32k"]
    say(f"prefill {w.name} (full size)")
    inp = make_prefill_inputs(w, device=DEV)
    dims = S.make_dims(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.head_dim,
                       w.block_size, w.max_seq_len)
    scale = 1.0 / math.sqrt(w.head_dim)
    out, lse, gt = run(S, dims, inp, scale)
    L, bs, nb = w.seq_lens[0], w.block_size, w.nb_max
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    assert torch.isfinite(gt).all()
    sums = gt.sum(dim=-1, dtype=torch.float64)
    assert float((sums - 1).abs().max()) < 1e-4
    last = torch.arange(L, device=DEV) // bs
    after = torch.arange(nb, device=DEV)[None, :] > last[:, None]
    assert float(gt.masked_select(after[None, None].expand_as(gt)).abs().max()) == 0.0
    rows = [0, 1, 63, 64, 255, 256, 1000, 4095, 16384, 32767]
    cpu = {k: v.cpu() for k, v in inp.items()}
    check_against_oracle(S, w, cpu, out.cpu(), lse.cpu(), gt.cpu(), scale, rows=rows,
                         heads=[0, 3, 7])


def test_prefill_binding_checks(S):
    say("prefill binding checks")
    dims = S.make_dims(1, 4, 2, 64, 64, 64, 128)
    q = torch.zeros((1, 4, 128, 64), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device=DEV)
    seq = torch.full((1,), 128, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((1, 4, 128), dtype=torch.float32, device=DEV)
    small = torch.empty(16, dtype=torch.float32, device=DEV)
    with pytest.raises(S.SeerError):  # workspace too small
        S.seer_prefill_attention(dims, q, kv, kv, seq, 0.1, small, out, lse)
    ws = torch.empty(S.seer_prefill_workspace_bytes(dims) // 4 + 64, dtype=torch.float32,
                     device=DEV)
    with pytest.raises(ValueError):  # gt of the wrong shape
        S.seer_prefill_attention(dims, q, kv, kv, seq, 0.1, ws, out, lse,
                                 torch.empty((1, 2, 128, 3), dtype=torch.float32, device=DEV))
    S.seer_prefill_attention(dims, q, kv, kv, seq, 0.1, ws, out, lse)
    torch.cuda.synchronize()
    # all-zero q and k: uniform attention, lse = ln(t + 1)
    assert torch.allclose(lse[0, 0].double(), torch.log(torch.arange(1, 129, device=DEV).double()),
                          atol=1e-5)
