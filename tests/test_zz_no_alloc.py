"""seer_decode_step_noalloc: the fused step with the library's static
workspace gives exactly what seer_decode_step gives with a caller's
workspace of seer_decode_step_workspace_bytes (the same kernels on the same
path), call after call, with the array shared between calls of different
sizes; and a step too large for the array is refused before any launch.
"""

from __future__ import annotations

import ctypes
import sys

import pytest
import torch

from workloads import WORKLOADS, make_inputs

DEV = "cuda:0"
MODES = {"topk": 1, "threshold": 2, "topp": 3}


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def S():
    import block_sparse_attention_seer_amd as S
    S.lib()
    return S


def _states(S, w, inp, lag_blocks):
    """Two decode states over the same cache: one for seer_decode_step, one
    for seer_decode_step_noalloc.  The cache lags `lag_blocks` blocks behind
    the sequences, so the step computes those entries itself."""
    dims = S.make_dims(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate,
                       w.block_size, w.max_seq_len)
    kw = dict(mode=MODES[w.mode], topk_blocks=w.topk_blocks, threshold=w.tau, device=DEV)
    a, b = S.DecodeStep(dims, **kw), S.DecodeStep(dims, **kw)
    built = torch.clamp(inp["seq_lens"] - lag_blocks * w.block_size, min=0)
    for st in (a, b):
        st.build_cache(inp["k_nope"], inp["w_k"], built)
    return dims, a, b


def _noalloc(S, st, inp, max_new_blocks=1):
    S.seer_decode_step_noalloc(st.dims, inp["q_nope"], inp["q"], inp["k_nope"], inp["k"],
                               inp["v"], inp["w_q"], inp["w_k"], inp["seq_lens"], st.kcomp_lens,
                               st.kcomp, max_new_blocks, st.rope_theta, st.mode, st.topk_blocks,
                               st.threshold, st.max_selected, st.block_idx, st.num_selected,
                               st.logits, 1.0 / (st.dims.head_dim ** 0.5), st.split_request,
                               st.out, st.lse)


def _assert_same(a, b, what):
    for name in ("kcomp_lens", "kcomp", "num_selected", "block_idx", "logits"):
        assert torch.equal(getattr(a, name), getattr(b, name)), f"{what}: {name}"
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16)), f"{what}: out"
    assert torch.equal(a.lse.view(torch.int32), b.lse.view(torch.int32)), f"{what}: lse"


# the first call: 48 (b, h) pairs under a threshold (uneven selections, so the
# automatic split count takes the stream-K decode and its larger workspace),
# lengths 3000 to 20000 tokens, each sequence one block ahead of its cache;
# the second: a smaller top-k batch of 8 pairs at 16 query heads per KV head
CALLS = [
    ("threshold_b128", dict(batch=6, max_seq_len=20000, seq_len_range=(3000, 20000))),
    ("qwen3_14b_b16", dict(batch=2, num_q_heads=32, num_kv_heads=2, max_seq_len=9000,
                           seq_len=None, seq_len_range=(100, 9000))),
]


@pytest.mark.gpu
def test_noalloc_step_equals_step_with_workspace_two_calls(S):
    sizes = []
    for i, (name, over) in enumerate(CALLS):
        w = WORKLOADS[name].replace(**over)
        say(f"no-alloc step call {i + 1}: {name} {over}")
        inp = make_inputs(w, device=DEV, separate_nope=True)
        dims, a, b = _states(S, w, inp, lag_blocks=1)
        need = S.seer_decode_step_workspace_bytes(dims, a.max_selected, a.split_request)
        assert 0 < need <= S.NOALLOC_SCRATCH_BYTES
        sizes.append(need)
        a.fused_step(inp["q_nope"], inp["q"], inp["k_nope"], inp["k"], inp["v"], inp["w_q"],
                     inp["w_k"], inp["seq_lens"])
        _noalloc(S, b, inp)
        torch.cuda.synchronize()
        assert int(a.kcomp_lens.sum()) > int(torch.clamp(
            inp["seq_lens"] - w.block_size, min=0).div(w.block_size, rounding_mode="floor").sum())
        _assert_same(a, b, f"call {i + 1} ({name})")
        # a second step on the same state (no entries left to compute)
        a.fused_step(inp["q_nope"], inp["q"], inp["k_nope"], inp["k"], inp["v"], inp["w_q"],
                     inp["w_k"], inp["seq_lens"])
        _noalloc(S, b, inp)
        torch.cuda.synchronize()
        _assert_same(a, b, f"call {i + 1} ({name}), repeated")
        del inp, a, b
        torch.cuda.empty_cache()
    assert sizes[1] < sizes[0]  # the second call is the smaller one


@pytest.mark.gpu
def test_noalloc_step_replays_from_a_graph(S):
    """Captured after an eager call, the step replays to the eager result;
    the program's own work and synchronizations run between replays."""
    w = WORKLOADS["tiny"].replace(batch=3, num_q_heads=8, num_kv_heads=2, seq_len=None,
                                  seq_len_range=(500, 1000), max_seq_len=1000)
    say("no-alloc step under graph capture")
    inp = make_inputs(w, device=DEV, separate_nope=True)
    dims, a, b = _states(S, w, inp, lag_blocks=0)
    _noalloc(S, b, inp)  # eager first: the library's set-up happens outside the capture
    a.fused_step(inp["q_nope"], inp["q"], inp["k_nope"], inp["k"], inp["v"], inp["w_q"],
                 inp["w_k"], inp["seq_lens"])
    torch.cuda.synchronize()
    _assert_same(a, b, "eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _noalloc(S, b, inp)
    for r in range(3):
        for name in ("out", "lse", "block_idx", "logits"):
            getattr(b, name).fill_(0)
        a.fused_step(inp["q_nope"], inp["q"], inp["k_nope"], inp["k"], inp["v"], inp["w_q"],
                     inp["w_k"], inp["seq_lens"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(a, b, f"replay {r + 1}")


def test_noalloc_step_refuses_a_workspace_beyond_the_array(S):
    """512 (b, h) pairs at 128 splits need far more than the array holds:
    the call fails with SEER_ERR_WORKSPACE and a message giving both sizes,
    before any pointer is read or any HIP call made (all pointers null; this
    runs without a GPU)."""
    dims = S.make_dims(64, 32, 8, 128, 128, 64, 8192)
    need = S.seer_decode_step_workspace_bytes(dims, 65, 128)
    assert need > S.NOALLOC_SCRATCH_BYTES
    lib = S.lib()
    nul = None
    rc = lib.seer_decode_step_noalloc(ctypes.byref(dims), nul, nul, nul, nul, nul, nul, nul,
                                      nul, nul, nul, 1, 10000.0, 1, 64, 0.0, 65, nul, nul, nul,
                                      0.088, 128, nul, nul, nul)
    assert rc == 3
    msg = lib.seer_last_error_message().decode()
    assert str(need) in msg and str(S.NOALLOC_SCRATCH_BYTES) in msg
