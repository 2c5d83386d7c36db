"""Helpers shared by the GPU parity tests: tolerance checks and oracle calls.

Tolerances (what the tests require of the HIP path against the float64
oracle on the same inputs):
  * attention outputs: |O_gpu - O_ref| <= 2e-2 + 1e-2 |O_ref| elementwise,
    lse within 1e-3 absolute;
  * compression cache entries: within one bf16 step of the oracle's bf16
    value (a float32 and a float64 evaluation can fall on different sides of
    a rounding boundary);
  * gate query within 1e-5 relative to its norm; logits within 1e-4 absolute
    given the same cache;
  * top-k indices on identical float32 logits: exact;
  * threshold indices: exact wherever |z_j - (ln tau + LSE)| > 1e-3;
  * top-p indices: a top prefix (ties to the lower index) that reaches p,
    exact wherever the cumulative softmax mass at the cut is farther than
    a margin (1e-5 on identical logits, 1e-3 end to end) from p;
  * end-to-end top-k: exact wherever the oracle's k-th / (k+1)-th logit gap
    exceeds 1e-3, otherwise the GPU's set must still be a valid top-k within
    1e-3.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O

OUT_ATOL = 2e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3
GAP = 1e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def assert_out_close(o_gpu: np.ndarray, o_ref: np.ndarray, what: str = "") -> float:
    """Elementwise |o_gpu - o_ref| <= 2e-2 + 1e-2 |o_ref|.  Written as a
    negated <= so that a NaN or infinite output (an element never written,
    or poisoned input that leaked through) fails instead of passing."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, f"{what}: shape {o_gpu.shape} != {o_ref.shape}"
    err = np.abs(o_gpu - o_ref)
    bound = OUT_ATOL + OUT_RTOL * np.abs(o_ref)
    bad = ~(err <= bound)
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} of {bad.size} outputs outside 2e-2 + 1e-2|ref| "
        f"({int((~np.isfinite(o_gpu)).sum())} not finite); max err {np.nanmax(err):.3e}")
    return float(err.max()) if err.size else 0.0


def assert_lse_close(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = "") -> None:
    """|l_gpu - l_ref| <= 1e-3, with -inf matching -inf (empty selections);
    NaN fails."""
    l_gpu = np.asarray(l_gpu, dtype=np.float64)
    l_ref = np.asarray(l_ref, dtype=np.float64)
    assert l_gpu.shape == l_ref.shape, f"{what}: shape {l_gpu.shape} != {l_ref.shape}"
    both_inf = np.isneginf(l_gpu) & np.isneginf(l_ref)
    with np.errstate(invalid="ignore"):
        err = np.abs(np.where(both_inf, 0.0, l_gpu - l_ref))
    assert np.all(err <= LSE_ATOL), f"{what}: lse max err {np.nanmax(err):.3e}"


def assert_gt_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """Prefill ground truth: |got - ref| <= 1e-6 + 2e-3 |ref| elementwise
    (derivation in tests/test_prefill_gpu.py); NaN and inf fail."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    err = np.abs(got - ref)
    bound = 1e-6 + 2e-3 * np.abs(ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} ground-truth values off "
                           f"({int((~np.isfinite(got)).sum())} not finite), worst "
                           f"{float(np.nanmax(err - bound)):.3e} over the bound")


def step_decode_counters(st) -> torch.Tensor:
    """The per-(b, h) split counters of a DecodeStep's fused-step workspace
    (int32 view): they follow the gate workspace, rounded up to 256 bytes."""
    import block_sparse_attention_seer_amd as S
    d = st.dims
    off = -(-S.seer_gate_workspace_bytes(d) // 256) * 256 // 4
    return st.step_ws.view(torch.int32)[off:off + d.batch * d.num_kv_heads]


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(e-8) for x = m 2^e, 0.5 <= m < 1)."""
    _, e = np.frexp(np.where(x == 0, 1.0, x))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def host_inputs(inp: dict, w, b: int, h: int, seq_len: int):
    """Attention's inputs of pair (b, h) in float64: q [g, d], K, V [L, d],
    and the gate weights W_q[h], W_k[h]."""
    g = w.group
    q = f64(inp["q"][b, h * g:(h + 1) * g])
    k = f64(inp["k"][b, h, :seq_len])
    v = f64(inp["v"][b, h, :seq_len])
    wq = f64(inp["w_q"][h])
    wk = f64(inp["w_k"][h])
    return q, k, v, wq, wk


def host_gate_inputs(inp: dict, w, b: int, h: int, seq_len: int):
    """The gate's pre-RoPE inputs of pair (b, h) in float64: q_nope [g, d]
    and K_nope [L, d] (the same values as q and K when the inputs were drawn
    without separate pre-RoPE tensors)."""
    g = w.group
    qn = inp.get("q_nope", inp["q"])
    kn = inp.get("k_nope", inp["k"])
    return f64(qn[b, h * g:(h + 1) * g]), f64(kn[b, h, :seq_len])


def oracle_chain(inp: dict, w, b: int, h: int, seq_len: int, capacity=None):
    """The oracle's whole decode step for pair (b, h): its own cache built
    from K_nope, the gate on q_nope, the selection, and attention of q over
    K and V."""
    q, k, v, wq, wk = host_inputs(inp, w, b, h, seq_len)
    q_nope, k_nope = host_gate_inputs(inp, w, b, h, seq_len)
    kc = O.build_kcomp(k_nope, wk, seq_len, w.block_size, w.theta)
    res = O.decode_pair(q_nope, q, k_nope, k, v, wq, kc, seq_len, w.block_size, mode=w.mode,
                        topk=w.topk_blocks, tau=w.tau, scale=1.0 / math.sqrt(w.head_dim),
                        theta=w.theta, capacity=capacity)
    res["kcomp"] = kc
    return res


def topk_gap(z: np.ndarray, k: int) -> float:
    """Oracle gap between the k-th and (k+1)-th largest logits (inf if k >= n)."""
    n = len(z)
    if k <= 0 or k >= n:
        return math.inf
    s = np.sort(z)[::-1]
    return float(s[k - 1] - s[k])


def check_topk_set(gpu_blocks, ref_blocks, z_ref: np.ndarray, k: int, n_scored: int,
                   forced: list, what: str) -> bool:
    """True if identical; if the oracle gap is small, require a valid top-k within GAP."""
    gpu_blocks = [int(x) for x in gpu_blocks]
    ref_blocks = [int(x) for x in ref_blocks]
    if gpu_blocks == ref_blocks:
        return True
    k_eff = min(k, n_scored)
    gap = topk_gap(z_ref, k_eff)
    assert gap <= GAP, f"{what}: selection differs with oracle gap {gap:.3e} > {GAP}"
    chosen = [j for j in gpu_blocks if j < n_scored]
    assert len(chosen) == k_eff, f"{what}: {len(chosen)} scored blocks chosen, want {k_eff}"
    assert [j for j in gpu_blocks if j >= n_scored] == forced, f"{what}: forced blocks differ"
    assert gpu_blocks == sorted(gpu_blocks)
    rest = [j for j in range(n_scored) if j not in set(chosen)]
    if rest:
        assert min(z_ref[chosen]) >= max(z_ref[rest]) - GAP, f"{what}: invalid top-k"
    return False


def threshold_value(z: np.ndarray, tau: float) -> float:
    m = z.max()
    return math.log(tau) + m + math.log(float(np.sum(np.exp(z - m))))


def check_topp_set(got, z, p, nc, forced, what, eps):
    """A top-p selection `got` (ascending, forced blocks included) against the
    definition on logits z[:nc] (float64): its scored part must be the first s
    blocks of the descending order (equal logits: lower index first), with
    mass(first s) >= p - eps and mass(first s-1) < p + eps.  Returns whether
    it equals the oracle's set exactly."""
    z = np.asarray(z, dtype=np.float64)[:nc]
    scored = [j for j in got if j < nc]
    assert [j for j in got if j >= nc] == list(forced), f"{what}: forced blocks"
    ref = O.select_topp(z, p, nc * 64 + 1, 64).tolist()  # scored part only
    ref = [j for j in ref if j < nc]
    if scored == ref:
        return True
    order = sorted(range(nc), key=lambda j: (-z[j], j))
    s = len(scored)
    assert sorted(scored) == sorted(order[:s]), f"{what}: not a top prefix"
    if nc == 0:
        return True
    e = np.exp(z - z.max())
    prob = e / e.sum()
    cum = np.concatenate([[0.0], np.cumsum(prob[order])])
    reach = cum[s] >= p - eps or s == nc
    short_before = s == 0 or cum[s - 1] < p + eps
    assert reach and short_before, f"{what}: top-p cut at {s} (mass {cum[s]:.9f}, p {p})"
    return False
