"""Pins of the float64 oracle against things other than itself.

Each test checks one oracle function against a library routine, a closed
form, a brute-force enumeration or an invariant the pages state, chosen so
that a plausible mistake (a dropped term, a wrong sign, index or position, a
transposed operand) fails.  CPU only.
"""

import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- bf16

def test_bf16_bits_match_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint64).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    mine = O.bf16_bits_to_f64(bits)
    both_nan = np.isnan(t) & np.isnan(mine)
    assert np.array_equal(t[~both_nan], mine[~both_nan])


def test_round_to_bf16_matches_torch_on_float32_values():
    # A float32 value rounded straight to bf16 from float64 must equal
    # torch's float32 -> bf16 conversion (round to nearest even).
    rng = np.random.default_rng(1)
    mant = rng.uniform(1.0, 2.0, size=20000)
    expo = rng.integers(-140, 128, size=20000)
    sign = rng.choice([-1.0, 1.0], size=20000)
    x32 = (sign * np.ldexp(mant, expo)).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    mine = O.round_to_bf16(x32.astype(np.float64))
    assert np.array_equal(ref, mine)


def test_round_to_bf16_ties_and_overflow():
    one = 1.0
    # exactly halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert O.round_to_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0
    # halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): goes up
    assert O.round_to_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    assert O.round_to_bf16(np.array([-(one + 2.0 ** -8)]))[0] == -1.0
    # just above halfway goes up
    assert O.round_to_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 2.0 ** -7
    assert np.isinf(O.round_to_bf16(np.array([3.4e38]))[0])
    assert O.round_to_bf16(np.array([0.0]))[0] == 0.0


# --------------------------------------------------------------------- RoPE

def test_rope_identity_at_zero_and_norm():
    rng = np.random.default_rng(2)
    v = rng.normal(size=(5, 64))
    assert np.array_equal(O.rope(v, 0), v)
    r = O.rope(v, 12345)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)


def test_rope_relative_position_property():
    rng = np.random.default_rng(3)
    a, c = rng.normal(size=128), rng.normal(size=128)
    for p1, p2 in [(100, 37), (5000, 4936), (32767, 64)]:
        lhs = O.rope(a, p1) @ O.rope(c, p2)
        rhs = O.rope(a, p1 - p2) @ c
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_rope_matches_complex_rotation():
    # Rotate-half RoPE is a complex rotation of (v_i + i v_{i+D/2}) by
    # exp(i * pos * theta^(-2i/D)); recomputed here element by element.
    rng = np.random.default_rng(4)
    D, pos, theta = 16, 777, 10000.0
    v = rng.normal(size=D)
    out = O.rope(v, pos, theta)
    for i in range(D // 2):
        w = theta ** (-(2.0 * i) / D)
        z = complex(v[i], v[i + D // 2]) * cmath.exp(1j * pos * w)
        assert abs(out[i] - z.real) < 1e-12
        assert abs(out[i + D // 2] - z.imag) < 1e-12


def test_rope_frequency_closed_form():
    # D = 4, theta = 10^4: pair i = 1 has frequency 10^4^(-1/2) = 0.01, so at
    # position 100 the angle is exactly 1 radian.
    v = np.array([0.0, 1.0, 0.0, 0.0])
    out = O.rope(v, 100, 10000.0)
    np.testing.assert_allclose(out, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-15)
    # pair i = 0 always turns at one radian per position
    out = O.rope(np.array([1.0, 0.0, 0.0, 0.0]), 3, 10000.0)
    np.testing.assert_allclose(out, [math.cos(3), 0.0, math.sin(3), 0.0], atol=1e-15)


# ------------------------------------------------------------------ pooling

def test_pool_block_matches_torch_pooling():
    rng = np.random.default_rng(5)
    b, d, nb = 16, 8, 5
    keys = rng.normal(size=(nb * b, d))
    t = torch.from_numpy(keys.T.copy())[None]  # [1, d, L]
    mx = torch.nn.functional.max_pool1d(t, b, b)[0].T.numpy()
    mn = (-torch.nn.functional.max_pool1d(-t, b, b))[0].T.numpy()
    av = torch.nn.functional.avg_pool1d(t, b, b)[0].T.numpy()
    for j in range(nb):
        u = O.pool_block(keys[j * b:(j + 1) * b])
        np.testing.assert_array_equal(u[:d], mx[j])
        np.testing.assert_array_equal(u[d:2 * d], mn[j])
        np.testing.assert_allclose(u[2 * d:], av[j], rtol=1e-14, atol=1e-15)


def test_pool_block_closed_forms():
    d, b = 4, 8
    const = np.tile(np.array([1.5, -2.0, 0.25, 7.0]), (b, 1))
    u = O.pool_block(const)
    np.testing.assert_array_equal(u, np.concatenate([const[0]] * 3))
    ramp = np.arange(b, dtype=np.float64)[:, None] * np.ones((1, d))
    u = O.pool_block(ramp)
    np.testing.assert_array_equal(u[:d], ramp[-1])
    np.testing.assert_array_equal(u[d:2 * d], ramp[0])
    np.testing.assert_allclose(u[2 * d:], (b - 1) / 2.0)


def test_compress_block_selector_weights():
    rng = np.random.default_rng(6)
    b, d = 64, 8
    keys = O.round_to_bf16(rng.normal(size=(b, d)))
    eye, zero = np.eye(d), np.zeros((d, d))
    np.testing.assert_array_equal(
        O.compress_block(keys, np.hstack([zero, zero, eye]), 0, b),
        O.round_to_bf16(keys.mean(axis=0)))
    np.testing.assert_array_equal(
        O.compress_block(keys, np.hstack([eye, zero, zero]), 0, b),
        O.round_to_bf16(keys.max(axis=0)))
    np.testing.assert_array_equal(
        O.compress_block(keys, np.hstack([zero, eye, zero]), 0, b),
        O.round_to_bf16(keys.min(axis=0)))


def test_compress_block_position_is_first_token():
    # d = d_gate = 2: constant keys [1, 0] and W_k picking the max branch
    # give K_gate = [cos(j*b), sin(j*b)] -- the block's first-token position.
    b, j = 4, 3
    keys = np.tile([1.0, 0.0], (b, 1))
    w_k = np.hstack([np.eye(2), np.zeros((2, 4))])
    out = O.compress_block(keys, w_k, j, b)
    np.testing.assert_allclose(out, [math.cos(j * b), math.sin(j * b)], atol=2 ** -8)
    assert abs(out[0] - math.cos(j * b + b - 1)) > 0.1


# -------------------------------------------------------- cache bookkeeping

def test_incremental_cache_equals_bulk_and_never_rewrites():
    rng = np.random.default_rng(7)
    b, d, dg, N = 8, 4, 6, 70
    keys = O.round_to_bf16(rng.normal(size=(N, d)))
    w_k = O.round_to_bf16(rng.normal(size=(dg, 3 * d)) / math.sqrt(3 * d))
    cache, snapshots = [], []
    for L in range(1, N + 1):
        O.update_kcomp(cache, keys, w_k, L, b, max_new_blocks=1)
        assert len(cache) == L // b
        snapshots.append([c.copy() for c in cache])
    for snap in snapshots:  # entries, once written, never change
        for j, c in enumerate(snap):
            np.testing.assert_array_equal(c, cache[j])
    bulk = O.build_kcomp(keys, w_k, N, b)
    np.testing.assert_array_equal(np.array(cache), bulk)
    # catch-up from empty in one call also equals the bulk build
    np.testing.assert_array_equal(np.array(O.update_kcomp([], keys, w_k, N, b)), bulk)


def test_memory_ratio_is_page_value():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        gold = json.load(f)
    mr = gold["kcomp_memory_ratio"]
    assert O.memory_ratio(mr["d_gate"], mr["head_dim"], mr["block_size"]) == pytest.approx(
        mr["ratio_num"] / mr["ratio_den"], rel=0, abs=0)
    for case in gold["token_to_block_budget"]:
        assert O.topk_budget_blocks(case["token_budget"], case["block_size"]) == case["blocks"]


# ------------------------------------------------------------- gate query

def test_gate_query_identity_and_head_grouping():
    rng = np.random.default_rng(8)
    g, d = 4, 8
    q = rng.normal(size=(g, d))
    # g = 1 and W_q = I: Q_gate is the rotated query itself
    np.testing.assert_allclose(O.gate_query(q[:1], np.eye(d), 41), O.rope(q[0], 41), atol=1e-14)
    # W_q picking head i of the group: the concat order is head-major
    for i in range(g):
        w = np.zeros((d, g * d))
        w[:, i * d:(i + 1) * d] = np.eye(d)
        np.testing.assert_allclose(O.gate_query(q, w, 9), O.rope(q[i], 9), atol=1e-14)


def test_gate_logits_relative_positions_closed_form():
    # d = d_gate = 2, g = 1: constant keys [1, 0] per block and q_nope = [1, 0]
    # give z_j = cos((L-1) - j*b) / sqrt(2) up to the cache's bf16 rounding.
    b, L = 4, 23
    keys = np.tile([1.0, 0.0], (L, 1))
    w_k = np.hstack([np.eye(2), np.zeros((2, 4))])
    kc = O.build_kcomp(keys, w_k, L, b)
    res = O.decode_pair(np.array([[1.0, 0.0]]), np.array([[1.0, 0.0]]), keys, keys, keys,
                        np.eye(2), kc, L, b, mode="topk", topk=2)
    for j in range(L // b):
        expect = math.cos((L - 1) - j * b) / math.sqrt(2)
        assert abs(res["logits"][j] - expect) < 2 ** -7
    np.testing.assert_allclose(res["q_gate"], [math.cos(L - 1), math.sin(L - 1)], atol=1e-15)


def test_decode_pair_routes_pre_and_post_rope_inputs():
    """[CP Knowl 1, 2]: the gate scores with the *pre*-RoPE query (and a cache
    built from pre-RoPE keys), attention uses the model's post-RoPE q and K.
    Built so that the two queries pick different blocks: q_nope points along
    e0 and only block 2's pre-RoPE keys do too, while q points along e1 and
    only block 0's post-RoPE keys do.  With theta huge the gate's own RoPE is
    the identity at these positions, so the logits have the closed form
    z_j = <q_nope, mean key of block j> / sqrt(d_gate) (W_k = [0 0 I])."""
    d, b, L = 4, 4, 16
    e0, e1 = np.eye(d)[0], np.eye(d)[1]
    k_nope = np.zeros((L, d))
    k_nope[2 * b:3 * b] = 2.0 * e0     # block 2 aligned with q_nope
    k_post = np.zeros((L, d))
    k_post[0:b] = 5.0 * e1             # block 0 aligned with q
    v = np.arange(L * d, dtype=np.float64).reshape(L, d)
    w_k = np.hstack([np.zeros((d, 2 * d)), np.eye(d)])
    theta = 1e300  # every frequency but the first is 0; the first pair sees cos/sin of pos
    kc = O.build_kcomp(k_nope, w_k, L, b, theta)
    q_nope, q = e0[None, :], e1[None, :]
    res = O.decode_pair(q_nope, q, k_nope, k_post, v, np.eye(d), kc, L, b, mode="topk",
                        topk=1, theta=theta)
    # gate: only the pre-RoPE inputs count; frequency 0 rotates pair (0, 2)
    # by pos, so z_j = 2 cos((L-1) - j b) / 2 for block 2 and 0 elsewhere
    expect = np.zeros(L // b)
    expect[2] = 2.0 * math.cos((L - 1) - 2 * b) / math.sqrt(d)
    np.testing.assert_allclose(res["logits"], expect, atol=2 ** -7)
    assert res["blocks"].tolist() == [2]
    # attention: q over the post-RoPE keys of block 2 (all zero scores),
    # so the output is the mean of block 2's values
    np.testing.assert_allclose(res["o"][0], v[2 * b:3 * b].mean(axis=0), atol=1e-12)
    np.testing.assert_allclose(res["lse"][0], math.log(b), atol=1e-12)
    # swapping the roles changes both the selection and the output
    kc_swapped = O.build_kcomp(k_post, w_k, L, b, theta)
    swapped = O.decode_pair(q, q_nope, k_post, k_nope, v, np.eye(d), kc_swapped, L, b,
                            mode="topk", topk=1, theta=theta)
    assert swapped["blocks"].tolist() == [0]


# --------------------------------------------------------------- selection

def test_topk_matches_brute_force_subsets():
    rng = np.random.default_rng(9)
    nb, k, b = 16, 4, 64
    for _ in range(20):
        z = rng.normal(size=nb)
        best = max(itertools.combinations(range(nb), k), key=lambda s: sum(z[list(s)]))
        got = O.select_topk(z, k, nb * b, b)
        assert list(got) == sorted(best)
        # order-preserving transforms do not change the set
        sm = scipy.special.softmax(z)
        assert list(O.select_topk(sm, k, nb * b, b)) == list(got)
        assert list(O.select_topk(z + 3.7, k, nb * b, b)) == list(got)


def test_topk_ties_budget_and_partial_block():
    b = 64
    z = np.array([1.0, 2.0, 2.0, 2.0, 0.0])
    assert list(O.select_topk(z, 2, 5 * b, b)) == [1, 2]        # lower index wins
    assert list(O.select_topk(z, 9, 5 * b, b)) == [0, 1, 2, 3, 4]  # k > nb: all
    assert list(O.select_topk(z, 0, 5 * b, b)) == []
    assert list(O.select_topk(z, 2, 5 * b + 3, b)) == [1, 2, 5]  # partial block 5 forced
    assert list(O.select_topk(np.zeros(0), 4, 37, b)) == [0]     # L < b: only the partial
    # a row too short for k + forced: the forced partial block stays, k shrinks
    assert list(O.select_topk(z, 2, 5 * b + 3, b, capacity=2)) == [1, 5]


def test_capacity_keeps_forced_blocks_first():
    """[CP Knowl 5]: the incomplete last block is always selected.  With a
    cache that lags (complete blocks not yet scored, so more than one forced
    block) and an index row of k + 1, the forced blocks are kept and the
    scored part is the best subset that fits, by brute force over subsets."""
    rng = np.random.default_rng(21)
    b = 16
    for trial in range(40):
        n_cached = int(rng.integers(3, 10))
        lag = int(rng.integers(1, 3))              # complete blocks not yet cached
        L = (n_cached + lag) * b + int(rng.integers(1, b))  # ... plus a partial block
        forced = list(range(n_cached, n_cached + lag + 1))
        z = rng.normal(size=n_cached)
        k = int(rng.integers(1, n_cached))
        cap = k + 1
        for mode, got in (("topk", O.select_topk(z, k, L, b, capacity=cap)),
                          ("threshold", O.select_threshold(z, 0.0, L, b, capacity=cap)),
                          ("topp", O.select_topp(z, 1.0, L, b, capacity=cap))):
            got = list(got)
            assert len(got) == min(cap, n_cached + len(forced)), mode
            assert got[-1] == n_cached + lag, mode          # the partial block
            kept_forced = forced[max(0, len(forced) - cap):]
            assert [j for j in got if j >= n_cached] == kept_forced, mode
            room = cap - len(kept_forced)
            scored = [j for j in got if j < n_cached]
            if mode == "threshold":  # tau = 0 passes all: lowest indices fill the room
                assert scored == list(range(min(room, n_cached))), mode
            else:                    # top-k, and top-p at p = 1: the best `room`
                best = max(itertools.combinations(range(n_cached), room),
                           key=lambda s_: sum(z[list(s_)])) if room > 0 else ()
                assert scored == sorted(best), mode
    # more forced blocks than the row holds: the last ones, ending in the partial block
    z = np.array([3.0, 1.0])
    assert list(O.select_topk(z, 1, 6 * b + 5, b, capacity=2)) == [5, 6]


def test_threshold_matches_explicit_softmax():
    rng = np.random.default_rng(10)
    b = 128
    for trial in range(50):
        nb = int(rng.integers(1, 60))
        z = rng.normal(scale=2.0, size=nb)
        tau = float(rng.choice([0.001, 0.01, 0.05, 0.2]))
        p = scipy.special.softmax(z)
        if np.min(np.abs(p - tau)) < 1e-12:
            continue
        expect = [j for j in range(nb) if p[j] > tau]
        assert list(O.select_threshold(z, tau, nb * b, b)) == expect
        assert list(O.select_threshold(z, tau, nb * b + 5, b)) == expect + [nb]


def test_threshold_is_strict():
    b = 64
    assert list(O.select_threshold(np.array([0.0, 0.0]), 0.5, 2 * b, b)) == []
    assert list(O.select_threshold(np.array([0.0, 0.0]), 0.4999, 2 * b, b)) == [0, 1]
    assert list(O.select_threshold(np.array([0.3, -1.0, 2.0]), 0.0, 3 * b, b)) == [0, 1, 2]


def test_topp_matches_brute_force_smallest_set():
    """[CP Knowl 14] top-p read as the nucleus: among all block sets whose
    softmax mass reaches p, the smallest; among those the heaviest (unique for
    distinct scores).  Brute force over all subsets of 10 blocks."""
    import itertools
    rng = np.random.default_rng(14)
    b = 64
    for trial in range(12):
        n = 10
        z = rng.normal(scale=1.5, size=n)
        prob = scipy.special.softmax(z)
        for pmass in [0.05, 0.3, 0.5, 0.77, 0.9, 0.99]:
            best = None
            for r in range(0, n + 1):
                feas = [c for c in itertools.combinations(range(n), r)
                        if prob[list(c)].sum() >= pmass]
                if feas:
                    best = max(feas, key=lambda c: prob[list(c)].sum())
                    break
            cum = np.sort(prob)[::-1].cumsum()
            if np.min(np.abs(cum - pmass)) < 1e-12:
                continue  # the boundary itself is a rounding question
            assert list(O.select_topp(z, pmass, n * b, b)) == sorted(best), (trial, pmass)


def test_topp_special_cases_ties_and_partial_block():
    b = 64
    z = np.array([1.0, 2.0, 2.0, 0.0])
    p = scipy.special.softmax(z)
    assert list(O.select_topp(z, 0.0, 4 * b, b)) == []                  # nothing needed
    assert list(O.select_topp(z, 1e-12, 4 * b, b)) == [1]               # the top block, lower index
    assert list(O.select_topp(z, p[1] + 1e-9, 4 * b, b)) == [1, 2]      # its tie comes next
    assert list(O.select_topp(z, 1.0, 4 * b, b)) == [0, 1, 2, 3]        # all
    assert list(O.select_topp(z, 2.0, 4 * b, b)) == [0, 1, 2, 3]        # unreachable: all
    assert list(O.select_topp(z, 0.3, 4 * b + 7, b)) == [1, 4]          # partial block 4 forced
    assert list(O.select_topp(z, 0.5, 4 * b + 7, b)) == [1, 2, 4]
    assert list(O.select_topp(np.zeros(0), 0.9, 20, b)) == [0]          # L < b
    # the top-p set is the top-k set for its own size (distinct scores)
    rng = np.random.default_rng(15)
    for trial in range(30):
        zz = rng.normal(size=int(rng.integers(2, 40)))
        sel = O.select_topp(zz, float(rng.uniform(0.1, 0.99)), len(zz) * b, b)
        assert list(sel) == list(O.select_topk(zz, len(sel), len(zz) * b, b))


@pytest.mark.parametrize("mode", ["topk", "threshold"])
def test_partial_block_always_selected_even_if_disfavoured(mode):
    rng = np.random.default_rng(11)
    g, d, b = 2, 16, 16
    for L in [5 * b + 1, 5 * b + 7, 6 * b - 1, 3]:
        q = rng.normal(size=(g, d))
        keys = rng.normal(size=(L, d))
        u = q.mean(0) / np.linalg.norm(q.mean(0))
        nb = L // b
        keys[nb * b:] -= 10 * u  # the partial block's keys point away from q
        w_q = rng.normal(size=(d, g * d)) / math.sqrt(g * d)
        w_k = rng.normal(size=(d, 3 * d)) / math.sqrt(3 * d)
        kc = O.build_kcomp(keys, w_k, L, b)
        res = O.decode_pair(q, q, keys, keys, keys, w_q, kc, L, b, mode=mode, topk=1, tau=0.5)
        assert res["blocks"][-1] == nb
        assert nb in res["blocks"]
    # L a multiple of b: nothing is forced
    L = 4 * b
    keys = rng.normal(size=(L, d))
    kc = O.build_kcomp(keys, w_k, L, b)
    res = O.decode_pair(q, q, keys, keys, keys, w_q, kc, L, b, mode="topk", topk=1)
    assert len(res["blocks"]) == 1 and res["blocks"][0] < 4


# --------------------------------------------------------------- attention

def test_full_budget_equals_sdpa_dense():
    rng = np.random.default_rng(12)
    g, d, b = 4, 32, 16
    for L in [1, 15, 16, 17, 100, 128]:
        q = rng.normal(size=(g, d))
        k, v = rng.normal(size=(L, d)), rng.normal(size=(L, d))
        nblk = -(-L // b)
        o, lse = O.sparse_decode_pair(q, k, v, L, list(range(nblk)), b, 1 / math.sqrt(d))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :],
            torch.from_numpy(k)[None, None].expand(1, g, L, d),
            torch.from_numpy(v)[None, None].expand(1, g, L, d))[0, :, 0].numpy()
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=1e-12)
        s = q @ k.T / math.sqrt(d)
        np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), atol=1e-12)
        od, lsed = O.dense_decode_pair(q, k, v, L, 1 / math.sqrt(d))
        np.testing.assert_allclose(od, o, atol=1e-15)


def test_gathered_equals_masked_dense():
    rng = np.random.default_rng(13)
    g, d, b, L = 3, 16, 8, 77
    q = rng.normal(size=(g, d))
    k, v = rng.normal(size=(L, d)), rng.normal(size=(L, d))
    for blocks in [[0], [2, 5], [1, 3, 9], [9], list(range(10))]:
        toks = O.blocks_to_tokens(blocks, L, b)
        o1, l1 = O.attention_gathered(q, k, v, toks, 0.25)
        o2, l2 = O.attention_masked_dense(q, k, v, L, toks, 0.25)
        np.testing.assert_allclose(o1, o2, atol=1e-12)
        np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(14)
    g, d = 2, 8
    q = rng.normal(size=(g, d))
    k, v = rng.normal(size=(40, d)), rng.normal(size=(40, d))
    o, lse = O.attention_gathered(q, k, v, np.array([0]), 0.5)   # one token
    np.testing.assert_allclose(o, np.tile(v[0], (g, 1)), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]), atol=1e-14)
    kk = np.tile(k[3], (40, 1))                                  # identical keys
    toks = np.array([1, 4, 9, 16, 25])
    o, lse = O.attention_gathered(q, kk, v, toks, 0.5)
    np.testing.assert_allclose(o, np.tile(v[toks].mean(0), (g, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[3]) + math.log(5), atol=1e-13)
    o, lse = O.attention_gathered(q, k, v, np.array([], dtype=np.int64), 0.5)  # empty
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_invalid_block_entries_are_skipped():
    rng = np.random.default_rng(15)
    g, d, b, L = 2, 8, 8, 30
    q = rng.normal(size=(g, d))
    k, v = rng.normal(size=(L, d)), rng.normal(size=(L, d))
    a = O.sparse_decode_pair(q, k, v, L, [-1, 1, 3, 4, 99], b, 0.3)
    c = O.sparse_decode_pair(q, k, v, L, [1, 3], b, 0.3)
    np.testing.assert_array_equal(a[0], c[0])
